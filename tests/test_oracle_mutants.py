"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin of test_oracle.py fails for each.  This is what makes the pins worth
trusting: a dropped term, a wrong sign or index, a transposed operand or an
off-by-one in a mask must not slip through."""
import contextlib
import importlib

import numpy as np
import pytest

import oracle
import tests.test_oracle as T

OA = importlib.import_module("oracle.core")
OD = importlib.import_module("oracle.dropout")


@pytest.fixture(scope="module")
def ref(tmp_path_factory):
    # None without g++ or rocRAND's header: the two pins that need the
    # library engine are then left out, and the mutants only they catch skip
    return T.build_philox_ref(tmp_path_factory.mktemp("philox"))


def _pins(ref):
    yield "golden", T.test_golden_worked_examples
    yield "p1_ones", lambda: [T.test_p1_ones_value_gives_ones(c, w) for c, w in T.MASKS]
    yield "p2", lambda: [T.test_p2_identical_keys_average_visible_values(c, w) for c, w in T.MASKS]
    yield "p3_row0", T.test_p3_causal_row0_and_window0
    yield "p3_suffix", T.test_p3_bottom_right_alignment_is_suffix_of_square
    yield "p3_empty", T.test_p3_empty_rows
    yield "p4_closed", T.test_p4_closed_form_two_keys
    yield "p4_brute", lambda: [T.test_p4_brute_force_tiny(c, w, 3, 8) for c, w in T.MASKS]
    yield "p5", lambda: [T.test_p5_online_softmax_equals_full(c, w, 16) for c, w in T.MASKS]
    yield "p6", lambda: [T.test_p6_split_merge_equals_full(c, w, 7) for c, w in T.MASKS]
    yield "p7_shift", T.test_p7_key_shift_invariance
    yield "p8", lambda: T.test_p8_gqa_equals_mha_with_expanded_kv(4, 2)
    yield "p10", T.test_p10_paged_equals_dense_and_permutation_invariant
    yield "p11", lambda: [T.test_p11_library_sdpa_random_shapes(s) for s in range(6)]
    yield "p12", lambda: [T.test_p12_paged_prefill_equals_dense_and_library(c, w) for c, w in
                          ((True, -1), (True, 3), (False, -1), (False, 2))]
    yield "p12_decode", T.test_p12_paged_prefill_single_token_is_decode
    yield "p13_fd", lambda: [T.test_p13_backward_matches_finite_differences(c, w) for c, w in
                             ((False, -1), (True, 1))]
    yield "p13_torch", lambda: [T.test_p13_backward_matches_torch_autograd(s) for s in range(4)]
    yield "p13_sums", T.test_p13_backward_sum_identities_and_empty_rows
    if ref is not None:
        yield "p14_philox", lambda: T.test_p14_philox_matches_library_engine(ref)
        yield "p14_keep", lambda: T.test_p14_keep_convention_matches_library_engine(ref)
        yield "p14_keep_key0", lambda: T.test_p14_keep_with_key_offset(ref)
    yield "p14_rate", lambda: [T.test_p14_keep_rate_is_one_minus_p(p) for p in (0.1, 0.9)]
    yield "p14_zero", lambda: [T.test_p14_zero_probability_is_plain_attention(c, w) for c, w in T.MASKS]
    yield "p14_identity", T.test_p14_identity_values_expose_dropped_probabilities
    yield "p14_unbiased", T.test_p14_dropout_is_unbiased_over_seeds
    yield "p14_bwd_torch", lambda: [T.test_p14_dropout_backward_matches_torch_autograd(c, w) for c, w in
                                    ((False, -1), (True, 2))]
    yield "p14_bwd_zero", T.test_p14_dropout_backward_zero_probability_is_plain_backward


def _failing_pins(ref):
    failed = []
    for name, fn in _pins(ref):
        try:
            fn()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(name)
    return failed


@contextlib.contextmanager
def planted(attr, fn):
    """Replace oracle.core.<attr> or oracle.dropout.<attr> (and the package's
    re-export of it, which the pins call directly) for the duration of the
    block."""
    mod = OA if hasattr(OA, attr) else OD
    old = getattr(mod, attr)
    old_pkg = getattr(oracle, attr, None)
    setattr(mod, attr, fn)
    if old_pkg is not None:
        setattr(oracle, attr, fn)
    try:
        yield
    finally:
        setattr(mod, attr, old)
        if old_pkg is not None:
            setattr(oracle, attr, old_pkg)


_orig_mask = OA.allowed_mask
_orig_softmax = OA.row_softmax
_orig_gather = OA.gather_paged_kv
_orig_prefill = OA.prefill_paged


def _mask_strict_causal(Lq, Lk, causal, window, rows=None):
    ok = _orig_mask(Lq, Lk, causal, window, rows)
    if causal:  # j < i + off instead of j <= i + off
        i = np.arange(Lq) if rows is None else np.asarray(rows)
        ok &= np.arange(Lk)[None, :] != (i[:, None] + Lk - Lq)
    return ok


def _mask_top_left(Lq, Lk, causal, window, rows=None):
    i = np.arange(Lq) if rows is None else np.asarray(rows)
    rel = np.arange(Lk)[None, :] - i[:, None]  # forgets the Lk - Lq offset
    ok = np.ones((len(i), Lk), dtype=bool)
    if causal:
        ok &= rel <= 0
    if window >= 0:
        ok &= rel >= -window
        if not causal:
            ok &= rel <= window
    return ok


def _mask_window_short(Lq, Lk, causal, window, rows=None):
    return _orig_mask(Lq, Lk, causal, window - 1 if window > 0 else window, rows)


def _softmax_lse_log2(S, ok):
    P, lse = _orig_softmax(S, ok)
    return P, lse / np.log(2.0)


def _softmax_neg(S, ok):
    return _orig_softmax(-S, ok)


def _softmax_unnormalised(S, ok):
    P, lse = _orig_softmax(S, ok)
    return P * np.exp(lse)[:, None] / np.exp(np.where(ok, S, -np.inf).max(1))[:, None], lse


def _gather_ignores_table(k_cache, v_cache, block_table, ctx_lens, block_size, s):
    table = np.asarray(block_table)
    first = int(table[s, 0])
    c = int(ctx_lens[s])
    p = np.arange(c)
    kc, vc = np.asarray(k_cache, dtype=float), np.asarray(v_cache, dtype=float)
    blk = first + p // block_size  # assumes contiguous physical blocks
    blk = np.minimum(blk, kc.shape[0] - 1)
    return kc[blk, p % block_size], vc[blk, p % block_size]


def _prefill_ignores_causal(q, kc, vc, table, ctx, bs, scale, causal=True, window=-1):
    return _orig_prefill(q, kc, vc, table, ctx, bs, scale, False, window)


def _prefill_drops_last_position(q, kc, vc, table, ctx, bs, scale, causal=True, window=-1):
    return _orig_prefill(q, kc, vc, table, np.maximum(np.asarray(ctx) - 1, 0), bs, scale, causal, window)


def _bwd_variant(jacobian=True, scale_dk=True, sum_heads=True):
    """A backward with one planted mistake (see the MUTANTS below)."""
    def bwd(q, k, v, dout, scale, causal=False, window=-1):
        q, k, v, do = (np.asarray(x, dtype=float) for x in (q, k, v, dout))
        B, Lq, Hq, D = q.shape
        Lk, Hkv = k.shape[1], k.shape[2]
        sc = float(np.float32(scale))
        ok = OA.allowed_mask(Lq, Lk, causal, window)
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                P, _ = OA.row_softmax(sc * q[b, :, h] @ k[b, :, g].T, ok)
                dP = do[b, :, h] @ v[b, :, g].T
                dS = P * (dP - (P * dP).sum(axis=1, keepdims=True)) if jacobian else P * dP
                dq[b, :, h] = sc * dS @ k[b, :, g]
                gk = (sc if scale_dk else 1.0) * dS.T @ q[b, :, h]
                gv = P.T @ do[b, :, h]
                if sum_heads:
                    dk[b, :, g] += gk
                    dv[b, :, g] += gv
                else:
                    dk[b, :, g] = gk
                    dv[b, :, g] = gv
        return dq, dk, dv
    return bwd


_orig_philox = OD.philox4x32
_orig_keep = OD.dropout_keep
_orig_attn_drop = OD.attention_dropout


def _philox_variant(swap_m=False, bump=True, rounds=10, swap_hi_lo=False):
    """Philox4x32 with one planted mistake."""
    def philox(counter, key, rounds_=None):
        c = np.asarray(counter, dtype=np.uint64) & np.uint64(0xFFFFFFFF)
        x0, x1, x2, x3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
        k0 = np.asarray(key[0], dtype=np.uint64) & np.uint64(0xFFFFFFFF)
        k1 = np.asarray(key[1], dtype=np.uint64) & np.uint64(0xFFFFFFFF)
        m0, m1 = (np.uint64(0xCD9E8D57), np.uint64(0xD2511F53)) if swap_m else \
            (np.uint64(0xD2511F53), np.uint64(0xCD9E8D57))
        M, S = np.uint64(0xFFFFFFFF), np.uint64(32)
        for _ in range(rounds):
            p0, p1 = m0 * x0, m1 * x2
            h0, l0, h1, l1 = p0 >> S, p0 & M, p1 >> S, p1 & M
            if swap_hi_lo:
                h0, l0, h1, l1 = l0, h0, l1, h1
            x0, x1, x2, x3 = h1 ^ x1 ^ k0, l1, h0 ^ x3 ^ k1, l0
            if bump:
                k0 = (k0 + np.uint64(0x9E3779B9)) & M
                k1 = (k1 + np.uint64(0xBB67AE85)) & M
        return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)
    return philox


def _keep_inverted(bh, rows, Lk, p, seed, offset, key0=0):
    return ~_orig_keep(bh, rows, Lk, p, seed, offset, key0)


def _keep_halves(rows, words, flip=False):
    par = (np.asarray(rows) % 2).astype(np.uint64)
    if flip:
        par = np.uint64(1) - par
    return (words.astype(np.uint64) >> (np.uint64(16) * par)[:, None]) & np.uint64(0xFFFF)


def _keep_variant(bh, rows, Lk, p, seed, offset, key0=0, swap_row_key=False, flip_halves=False, full_row=False):
    rows = np.asarray(rows)
    thr = OD.dropout_threshold(p)
    g0, g1 = key0 // 4, (key0 + Lk + 3) // 4
    ctr = np.zeros((len(rows), g1 - g0, 4), dtype=np.uint64)
    rpair = rows if full_row else rows // 2
    ctr[..., 0] = rpair[:, None] if swap_row_key else np.arange(g0, g1)[None, :]
    ctr[..., 1] = np.arange(g0, g1)[None, :] if swap_row_key else rpair[:, None]
    ctr[..., 2] = bh
    ctr[..., 3] = offset
    w = OD.philox4x32(ctr, (seed & 0xFFFFFFFF, seed >> 32)).reshape(len(rows), 4 * (g1 - g0))
    return _keep_halves(rows, w[:, key0 - 4 * g0:key0 - 4 * g0 + Lk], flip_halves) >= thr


def _keep_row_key_swapped(bh, rows, Lk, p, seed, offset, key0=0):
    return _keep_variant(bh, rows, Lk, p, seed, offset, key0, swap_row_key=True)


def _keep_halves_swapped(bh, rows, Lk, p, seed, offset, key0=0):
    return _keep_variant(bh, rows, Lk, p, seed, offset, key0, flip_halves=True)


def _keep_row_not_paired(bh, rows, Lk, p, seed, offset, key0=0):
    return _keep_variant(bh, rows, Lk, p, seed, offset, key0, full_row=True)


def _keep_word_order_reversed(bh, rows, Lk, p, seed, offset, key0=0):
    g0 = key0 // 4
    full = _orig_keep(bh, rows, 4 * ((key0 + Lk + 3) // 4 - g0), p, seed, offset, 4 * g0)
    rev = full.reshape(len(full), -1, 4)[:, :, ::-1].reshape(len(full), -1)
    return rev[:, key0 - 4 * g0:key0 - 4 * g0 + Lk]


def _attn_drop_variant(mode):
    def fwd(q, k, v, scale, causal=False, window=-1, p=0.0, seed=0, offset=0, rows=None, key0=0):
        q, k, v = (np.asarray(x, dtype=float) for x in (q, k, v))
        B, Lq, Hq, D = q.shape
        Lk, Hkv = k.shape[1], k.shape[2]
        sc = float(np.float32(scale))
        rr = np.arange(Lq) if rows is None else np.asarray(rows)
        ok = OA.allowed_mask(Lq, Lk, causal, window, rr)
        out = np.zeros((B, len(rr), Hq, D))
        lse = np.full((B, Hq, len(rr)), -np.inf)
        for b in range(B):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                S = sc * q[b, rr, h] @ k[b, :, g].T
                keep = OD.dropout_keep(b * Hq + h, rr, Lk, p, seed, offset, key0)
                P, ls = OA.row_softmax(S, ok & keep if mode == "before_softmax" else ok)
                Pd = np.where(keep, P, 0.0)
                if mode == "renormalised":
                    s_ = Pd.sum(axis=1, keepdims=True)
                    Pd = Pd / np.where(s_ > 0, s_, 1.0)
                elif mode != "unscaled":
                    Pd = Pd / (1 - float(np.float32(p)))
                out[b, :, h] = Pd @ v[b, :, g]
                lse[b, h] = ls
        return out, lse
    return fwd


def _drop_bwd_variant(mask_dv=True, mask_dp=True):
    def bwd(q, k, v, dout, scale, causal=False, window=-1, p=0.0, seed=0, offset=0):
        q, k, v, do = (np.asarray(x, dtype=float) for x in (q, k, v, dout))
        B, Lq, Hq, D = q.shape
        Lk, Hkv = k.shape[1], k.shape[2]
        sc = float(np.float32(scale))
        ok = OA.allowed_mask(Lq, Lk, causal, window)
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                P, _ = OA.row_softmax(sc * q[b, :, h] @ k[b, :, g].T, ok)
                Mk = np.where(OD.dropout_keep(b * Hq + h, np.arange(Lq), Lk, p, seed, offset),
                              1 / (1 - float(np.float32(p))), 0.0)
                dv[b, :, g] += ((P * Mk) if mask_dv else P).T @ do[b, :, h]
                dP = do[b, :, h] @ v[b, :, g].T
                if mask_dp:
                    dP = dP * Mk
                dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
                dq[b, :, h] = sc * dS @ k[b, :, g]
                dk[b, :, g] += sc * dS.T @ q[b, :, h]
        return dq, dk, dv
    return bwd


MUTANTS = {
    "gqa_modulo": ("kv_head", lambda h, Hq, Hkv: h % Hkv),
    "no_scale": ("scores", lambda qr, kr, sc: qr @ kr.T),
    "scale_squared": ("scores", lambda qr, kr, sc: sc * sc * (qr @ kr.T)),
    "sign_flip": ("scores", lambda qr, kr, sc: -sc * (qr @ kr.T)),
    "strict_causal": ("allowed_mask", _mask_strict_causal),
    "top_left_causal": ("allowed_mask", _mask_top_left),
    "window_off_by_one": ("allowed_mask", _mask_window_short),
    "lse_log2": ("row_softmax", _softmax_lse_log2),
    "softmax_of_negated": ("row_softmax", _softmax_neg),
    "unnormalised": ("row_softmax", _softmax_unnormalised),
    "gather_ignores_table": ("gather_paged_kv", _gather_ignores_table),
    "prefill_ignores_causal": ("prefill_paged", _prefill_ignores_causal),
    "prefill_drops_last_position": ("prefill_paged", _prefill_drops_last_position),
    "bwd_no_jacobian_term": ("attention_backward", _bwd_variant(jacobian=False)),
    "bwd_dk_unscaled": ("attention_backward", _bwd_variant(scale_dk=False)),
    "bwd_gqa_not_summed": ("attention_backward", _bwd_variant(sum_heads=False)),
    "philox_swapped_multipliers": ("philox4x32", _philox_variant(swap_m=True)),
    "philox_no_key_bump": ("philox4x32", _philox_variant(bump=False)),
    "philox_nine_rounds": ("philox4x32", _philox_variant(rounds=9)),
    "philox_hi_lo_swapped": ("philox4x32", _philox_variant(swap_hi_lo=True)),
    "keep_inverted": ("dropout_keep", _keep_inverted),
    "keep_row_key_swapped": ("dropout_keep", _keep_row_key_swapped),
    "keep_halves_swapped": ("dropout_keep", _keep_halves_swapped),
    "keep_row_not_paired": ("dropout_keep", _keep_row_not_paired),
    "keep_word_order_reversed": ("dropout_keep", _keep_word_order_reversed),
    "dropout_renormalised": ("attention_dropout", _attn_drop_variant("renormalised")),
    "dropout_unscaled": ("attention_dropout", _attn_drop_variant("unscaled")),
    "dropout_before_softmax": ("attention_dropout", _attn_drop_variant("before_softmax")),
    "dropout_bwd_dv_unmasked": ("attention_dropout_backward", _drop_bwd_variant(mask_dv=False)),
    "dropout_bwd_dp_unmasked": ("attention_dropout_backward", _drop_bwd_variant(mask_dp=False)),
}


def test_unmutated_oracle_passes_every_pin(ref):
    assert _failing_pins(ref) == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(ref, mutant):
    attr, fn = MUTANTS[mutant]
    if ref is None and (attr == "philox4x32" or mutant in ("keep_row_key_swapped", "keep_word_order_reversed")):
        pytest.skip("caught only by the pins that need rocRAND's engine, which is not available")
    with np.errstate(all="ignore"), planted(attr, fn):
        failed = _failing_pins(ref)
    assert failed, f"mutant {mutant} passed every pin"
