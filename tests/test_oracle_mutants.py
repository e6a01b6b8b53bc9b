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


def _pins():
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


def _failing_pins():
    failed = []
    for name, fn in _pins():
        try:
            fn()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(name)
    return failed


@contextlib.contextmanager
def planted(attr, fn):
    """Replace oracle.core.<attr> (and the package's re-export of it, which the
    pins call directly) for the duration of the block."""
    old = getattr(OA, attr)
    old_pkg = getattr(oracle, attr, None)
    setattr(OA, attr, fn)
    if old_pkg is not None:
        setattr(oracle, attr, fn)
    try:
        yield
    finally:
        setattr(OA, attr, old)
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
}


def test_unmutated_oracle_passes_every_pin():
    assert _failing_pins() == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant):
    attr, fn = MUTANTS[mutant]
    with np.errstate(all="ignore"), planted(attr, fn):
        failed = _failing_pins()
    assert failed, f"mutant {mutant} passed every pin"
