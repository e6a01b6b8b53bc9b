"""Pins of the fp64 oracle against what the pages and the mathematics fix.

No GPU.  Every oracle function is pinned here by something other than itself:
hand-derived worked examples, closed forms, special cases, invariants of the
softmax, brute force in scalar Python, and a library routine (torch's CPU
float64 scaled_dot_product_attention).  test_oracle_mutants.py checks that
plausible planted mistakes fail at least one of these pins.

Page references:
  SA  = «Самовнимание, ядра CUDA и FlashAttention» (section 1: Scores and
        Attention equations, rows of the softmax sum to one; section 3: tiling
        and the online softmax).
  FA  = «Flash Attention» skill page (quick start; scenario 1, step 4: the
        explicit softmax(q@k^T/8)@v check; scenario 2, step 3: MQA/GQA and the
        (left, right) sliding window).
  NEWS = the-ai.news article, section «Внимание типа FlashAttention и
        постраничное внимание» (paged KV cache: block table, paging does not
        change the logical elements).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, dense_inputs, paged_inputs, random_dense

HERE = os.path.dirname(os.path.abspath(__file__))
TIGHT = 1e-12

MASKS = [(False, -1), (True, -1), (False, 3), (True, 3), (True, 0), (False, 0)]


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def small_case(B=2, Hq=4, Hkv=2, Lq=9, Lk=13, D=8, seed=0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Lq, Hq, D))
    k = r.standard_normal((B, Lk, Hkv, D))
    v = r.standard_normal((B, Lk, Hkv, D))
    return q, k, v


# ---------------------------------------------------------------- golden

def test_golden_worked_examples():
    """Hand-derived examples (SA section 1; bottom-right causal; window; GQA)."""
    with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
        data = json.load(f)
    for c in data["cases"]:
        out, lse = oracle.attention(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]),
                                    c["scale"], c["causal"], c["window"])
        np.testing.assert_allclose(out, np.array(c["out"]), atol=data["tolerance"], rtol=0, err_msg=c["name"])
        np.testing.assert_allclose(lse, np.array(c["lse"]), atol=data["tolerance"], rtol=0, err_msg=c["name"])


# ---------------------------------------------------------------- P1

def test_p1_probability_rows_sum_to_one():
    """SA section 1: the row softmax turns scores into probabilities summing to 1."""
    S = rnd((40, 57), 1) * 7
    ok = np.random.default_rng(2).random((40, 57)) < 0.3
    ok[np.arange(40), np.arange(40)] = True
    P, lse = oracle.row_softmax(S, ok)
    assert np.all(P[~ok] == 0)
    np.testing.assert_allclose(P.sum(1), 1.0, atol=TIGHT, rtol=0)
    # lse is the log of the sum of exponentials of the allowed entries
    ref = np.array([math.log(sum(math.exp(S[i, j]) for j in range(57) if ok[i, j])) for i in range(40)])
    np.testing.assert_allclose(lse, ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal,window", MASKS)
def test_p1_ones_value_gives_ones(causal, window):
    """Rows summing to one means V = 1 gives out = 1 on every non-empty row."""
    q, k, _ = small_case(seed=3)
    v = np.ones_like(k)
    out, lse = oracle.attention(q, k, v, 0.37, causal, window)
    np.testing.assert_allclose(out, 1.0, atol=TIGHT, rtol=0)
    assert np.all(np.isfinite(lse))


# ---------------------------------------------------------------- P2

@pytest.mark.parametrize("causal,window", MASKS)
def test_p2_identical_keys_average_visible_values(causal, window):
    """Identical keys give equal weights, so each row is the plain mean of the
    values it may see, and lse = score + ln(count)."""
    B, Hq, Hkv, Lq, Lk, D = 1, 2, 1, 7, 11, 3
    q = rnd((B, Lq, Hq, D), 4)
    k = np.broadcast_to(rnd((1, 1, Hkv, D), 5), (B, Lk, Hkv, D)).copy()
    v = rnd((B, Lk, Hkv, D), 6)
    out, lse = oracle.attention(q, k, v, 0.5, causal, window)
    off = Lk - Lq
    for i in range(Lq):
        lo, hi = 0, Lk - 1
        if causal:
            hi = min(hi, i + off)
        if window >= 0:
            lo = max(lo, i + off - window)
            if not causal:
                hi = min(hi, i + off + window)
        cnt = hi - lo + 1
        for h in range(Hq):
            np.testing.assert_allclose(out[0, i, h], v[0, lo:hi + 1, 0].mean(0), atol=TIGHT, rtol=0)
            s = 0.5 * float(np.dot(q[0, i, h], k[0, 0, 0]))
            assert abs(lse[0, h, i] - (s + math.log(cnt))) < 1e-12


# ---------------------------------------------------------------- P3

def test_p3_causal_row0_and_window0():
    q, k, v = small_case(Lq=10, Lk=10, seed=7)
    out, _ = oracle.attention(q, k, v, 0.3, causal=True)
    for h in range(4):
        assert np.array_equal(out[:, 0, h], v[:, 0, h // 2])  # row 0 sees only key 0: exact
    out0, lse0 = oracle.attention(q, k, v, 0.3, causal=True, window=0)
    for h in range(4):
        assert np.array_equal(out0[:, :, h], v[:, :, h // 2])  # W = 0: each row sees only itself
        s = float(np.float32(0.3)) * np.einsum("bid,bid->bi", q[:, :, h], k[:, :, h // 2])
        np.testing.assert_allclose(lse0[:, h], s, atol=TIGHT, rtol=0)


def test_p3_bottom_right_alignment_is_suffix_of_square():
    """Causal with Lq < Lk equals the last Lq rows of the square causal problem."""
    q, k, v = small_case(Lq=13, Lk=13, seed=8)
    full, lfull = oracle.attention(q, k, v, 0.4, causal=True, window=4)
    part, lpart = oracle.attention(q[:, 8:], k, v, 0.4, causal=True, window=4)
    np.testing.assert_allclose(part, full[:, 8:], atol=TIGHT, rtol=0)
    np.testing.assert_allclose(lpart, lfull[:, :, 8:], atol=TIGHT, rtol=0)


def test_p3_empty_rows():
    """Lq > Lk under causal alignment leaves the first Lq-Lk rows with no key."""
    q, k, v = small_case(Lq=9, Lk=4, seed=9)
    out, lse = oracle.attention(q, k, v, 0.4, causal=True)
    assert np.all(out[:, :5] == 0) and np.all(np.isneginf(lse[:, :, :5]))
    assert np.all(np.isfinite(lse[:, :, 5:]))


# ---------------------------------------------------------------- P4

def test_p4_closed_form_two_keys():
    """Lk = 2: out = v0 + sigmoid(s1 - s0) (v1 - v0), lse = logaddexp(s0, s1)."""
    r = np.random.default_rng(10)
    for _ in range(20):
        D = int(r.integers(1, 9))
        q = r.standard_normal((1, 1, 1, D)) * 2
        k = r.standard_normal((1, 2, 1, D)) * 2
        v = r.standard_normal((1, 2, 1, D))
        sc = float(np.float32(r.random() + 0.1))
        out, lse = oracle.attention(q, k, v, sc)
        s0 = sc * sum(q[0, 0, 0, d] * k[0, 0, 0, d] for d in range(D))
        s1 = sc * sum(q[0, 0, 0, d] * k[0, 1, 0, d] for d in range(D))
        sig = 1.0 / (1.0 + math.exp(-(s1 - s0)))
        np.testing.assert_allclose(out[0, 0, 0], v[0, 0, 0] + sig * (v[0, 1, 0] - v[0, 0, 0]), atol=1e-12, rtol=0)
        assert abs(lse[0, 0, 0] - np.logaddexp(s0, s1)) < 1e-12


def _brute(q, k, v, sc, causal, window):
    """Scalar Python attention: one query, one head at a time."""
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    out = np.zeros_like(q, shape=(B, Lq, Hq, D))
    lse = np.full((B, Hq, Lq), -math.inf)
    for b, i, h in itertools.product(range(B), range(Lq), range(Hq)):
        g = h * Hkv // Hq
        vis = []
        for j in range(Lk):
            diag = i + Lk - Lq
            if causal and j > diag:
                continue
            if window >= 0 and (j < diag - window or (not causal and j > diag + window)):
                continue
            vis.append(j)
        if not vis:
            continue
        s = {j: sc * sum(float(q[b, i, h, d]) * float(k[b, j, g, d]) for d in range(D)) for j in vis}
        mx = max(s.values())
        w = {j: math.exp(s[j] - mx) for j in vis}
        tot = sum(w.values())
        for d in range(D):
            out[b, i, h, d] = sum(w[j] * float(v[b, j, g, d]) for j in vis) / tot
        lse[b, h, i] = mx + math.log(tot)
    return out, lse


@pytest.mark.parametrize("causal,window", MASKS + [(False, 1), (True, 5)])
@pytest.mark.parametrize("Lq,Lk", [(1, 1), (5, 5), (3, 8), (8, 3), (7, 6)])
def test_p4_brute_force_tiny(causal, window, Lq, Lk):
    q, k, v = small_case(B=2, Hq=4, Hkv=2, Lq=Lq, Lk=Lk, D=4, seed=Lq * 31 + Lk)
    out, lse = oracle.attention(q, k, v, 0.45, causal, window)
    bo, bl = _brute(q, k, v, float(np.float32(0.45)), causal, window)
    np.testing.assert_allclose(out, bo, atol=1e-12, rtol=0)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(bl))
    fin = np.isfinite(bl)
    np.testing.assert_allclose(lse[fin], bl[fin], atol=1e-12, rtol=0)


# ---------------------------------------------------------------- P5 / P6

@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("block", [1, 5, 16, 64])
def test_p5_online_softmax_equals_full(causal, window, block):
    """SA section 3: block-by-block running max/normaliser with rescaling is
    the same softmax, only evaluated differently."""
    q, k, v = small_case(Lq=37, Lk=70, D=8, seed=11)
    ref = oracle.attention(q, k, v, 0.3, causal, window)
    got = oracle.online_attention(q, k, v, 0.3, causal, window, block_n=block)
    np.testing.assert_allclose(got[0], ref[0], atol=TIGHT, rtol=0)
    np.testing.assert_allclose(got[1][np.isfinite(ref[1])], ref[1][np.isfinite(ref[1])], atol=TIGHT, rtol=0)
    np.testing.assert_array_equal(np.isneginf(got[1]), np.isneginf(ref[1]))


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("chunk", [1, 7, 32, 100])
def test_p6_split_merge_equals_full(causal, window, chunk):
    q, k, v = small_case(Lq=21, Lk=70, D=8, seed=12)
    ref = oracle.attention(q, k, v, 0.3, causal, window)
    got = oracle.split_merge_attention(q, k, v, 0.3, causal, window, chunk=chunk)
    np.testing.assert_allclose(got[0], ref[0], atol=TIGHT, rtol=0)
    fin = np.isfinite(ref[1])
    np.testing.assert_allclose(got[1][fin], ref[1][fin], atol=TIGHT, rtol=0)


# ---------------------------------------------------------------- P7

def test_p7_key_shift_invariance():
    """k_j + c for every j adds sc*q.c to every score of the row: out is
    unchanged and lse shifts by sc*q.c."""
    q, k, v = small_case(seed=13)
    c = rnd((8,), 14)
    sc = float(np.float32(0.3))
    o1, l1 = oracle.attention(q, k, v, sc, True, 3)
    o2, l2 = oracle.attention(q, k + c, v, sc, True, 3)
    np.testing.assert_allclose(o2, o1, atol=1e-12, rtol=0)
    shift = sc * np.einsum("bihd,d->bhi", q, c)
    np.testing.assert_allclose(l2, l1 + shift, atol=1e-12, rtol=0)


def test_p7_value_affine_and_constant():
    q, k, v = small_case(seed=15)
    o1, _ = oracle.attention(q, k, v, 0.3, False, -1)
    o2, _ = oracle.attention(q, k, 2.5 * v - 1.25, 0.3, False, -1)
    np.testing.assert_allclose(o2, 2.5 * o1 - 1.25, atol=1e-12, rtol=0)
    const = np.broadcast_to(rnd((1, 1, 2, 8), 16), k.shape)
    o3, _ = oracle.attention(q, k, const, 0.3, True, -1)
    for h in range(4):
        np.testing.assert_allclose(o3[:, :, h], np.broadcast_to(const[:, :1, h // 2], o3[:, :, h].shape), atol=1e-13)


def test_p7_key_permutation_noncausal_and_zero_scale():
    q, k, v = small_case(seed=17)
    perm = np.random.default_rng(18).permutation(k.shape[1])
    o1, l1 = oracle.attention(q, k, v, 0.3)
    o2, l2 = oracle.attention(q, k[:, perm], v[:, perm], 0.3)
    np.testing.assert_allclose(o2, o1, atol=1e-12, rtol=0)
    np.testing.assert_allclose(l2, l1, atol=1e-12, rtol=0)
    o0, l0 = oracle.attention(q, k, v, 0.0)
    for h in range(4):
        np.testing.assert_allclose(o0[:, :, h], np.broadcast_to(v[:, :, h // 2].mean(1, keepdims=True), o0[:, :, h].shape), atol=1e-13)
    np.testing.assert_allclose(l0, math.log(k.shape[1]), atol=1e-13)


# ---------------------------------------------------------------- P8

@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (6, 1), (8, 8), (12, 2)])
def test_p8_gqa_equals_mha_with_expanded_kv(Hq, Hkv):
    """FA scenario 2, step 3: query heads of one group share one K/V head."""
    q, k, v = small_case(Hq=Hq, Hkv=Hkv, seed=19)
    o1, l1 = oracle.attention(q, k, v, 0.3, True, 5)
    rep = Hq // Hkv
    o2, l2 = oracle.attention(q, np.repeat(k, rep, axis=2), np.repeat(v, rep, axis=2), 0.3, True, 5)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ---------------------------------------------------------------- P9

def test_p9_wide_window_is_plain_mask():
    q, k, v = small_case(Lq=11, Lk=11, seed=20)
    for causal in (True, False):
        a = oracle.attention(q, k, v, 0.3, causal, -1)
        b = oracle.attention(q, k, v, 0.3, causal, 10)
        c = oracle.attention(q, k, v, 0.3, causal, 9)
        np.testing.assert_array_equal(a[0], b[0])
        assert not np.allclose(a[0], c[0])


# ---------------------------------------------------------------- P10

def _scatter_to_pool(K, V, ctx, bs, perm_seed, Hkv, D):
    """Write contiguous per-sequence K/V into a permuted block pool."""
    nblk = [-(-c // bs) for c in ctx]
    nb = sum(nblk)
    perm = np.random.default_rng(perm_seed).permutation(nb) if perm_seed is not None else np.arange(nb)
    kc = np.full((nb, bs, Hkv, D), np.nan)
    vc = np.full((nb, bs, Hkv, D), np.nan)
    table = np.zeros((len(ctx), max(nblk)), dtype=np.int32)
    o = 0
    for s, c in enumerate(ctx):
        for j in range(nblk[s]):
            phys = perm[o + j]
            table[s, j] = phys
            n = min(bs, c - j * bs)
            kc[phys, :n] = K[s][j * bs: j * bs + n]
            vc[phys, :n] = V[s][j * bs: j * bs + n]
        o += nblk[s]
    return kc, vc, table


def test_p10_paged_equals_dense_and_permutation_invariant():
    """NEWS: the table changes where elements live, not which are attended."""
    r = np.random.default_rng(21)
    S, Hq, Hkv, D, bs = 5, 6, 2, 8, 4
    ctx = [1, 4, 5, 13, 16]
    K = [r.standard_normal((c, Hkv, D)) for c in ctx]
    V = [r.standard_normal((c, Hkv, D)) for c in ctx]
    q = r.standard_normal((S, Hq, D))
    outs = []
    for perm_seed in (None, 22, 23):
        kc, vc, table = _scatter_to_pool(K, V, ctx, bs, perm_seed, Hkv, D)
        o, l = oracle.decode_paged(q, kc, vc, table, np.array(ctx), bs, 0.35)
        assert np.all(np.isfinite(o))  # NaN-filled unused slots are never read
        outs.append((o, l))
        for s in range(S):
            ro, rl = oracle.attention(q[s][None, None], K[s][None], V[s][None], 0.35)
            np.testing.assert_allclose(o[s], ro[0, 0], atol=TIGHT, rtol=0)
            np.testing.assert_allclose(l[s], rl[0, :, 0], atol=TIGHT, rtol=0)
    for o, l in outs[1:]:
        np.testing.assert_array_equal(o, outs[0][0])
        np.testing.assert_array_equal(l, outs[0][1])


def test_p10_workload_generator_table_is_consistent():
    cfg = CONFIGS["paged_decode"]
    inp = paged_inputs(cfg)
    ctx = inp.ctx_lens.numpy()
    assert ctx.min() >= 512 and ctx.max() <= 4096
    nblk = -(-ctx // 16)
    assert inp.num_blocks == nblk.sum()
    used = np.concatenate([inp.block_table[s, :nblk[s]].numpy() for s in range(cfg.num_seqs)])
    assert np.array_equal(np.sort(used), np.arange(inp.num_blocks))  # a permutation of the pool


# ---------------------------------------------------------------- P11

def _torch_sdpa(q, k, v, sc, causal, window):
    Lq, Lk = q.shape[1], k.shape[1]
    Hq, Hkv = q.shape[2], k.shape[2]
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(0, 2, 1, 3)))
    kt = torch.from_numpy(np.ascontiguousarray(np.repeat(k, Hq // Hkv, 2).transpose(0, 2, 1, 3)))
    vt = torch.from_numpy(np.ascontiguousarray(np.repeat(v, Hq // Hkv, 2).transpose(0, 2, 1, 3)))
    i = torch.arange(Lq)[:, None] + (Lk - Lq)
    j = torch.arange(Lk)[None, :]
    m = torch.ones(Lq, Lk, dtype=torch.bool)
    if causal:
        m &= j <= i
    if window >= 0:
        m &= j >= i - window
        if not causal:
            m &= j <= i + window
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=sc)
    return o.numpy().transpose(0, 2, 1, 3)


@pytest.mark.parametrize("name", ["tiny", "std512", "std512_causal", "vit"])
def test_p11_library_sdpa_on_workloads(name):
    """FA quick start / scenario 1: PyTorch's scaled_dot_product_attention is
    the pages' own reference; here it runs on the CPU in float64."""
    cfg = CONFIGS[name]
    q, k, v = dense_inputs(cfg)
    if name == "vit":  # a slice of the batch keeps the CPU suite short
        q, k, v = q[:4], k[:4], v[:4]
    q64, k64, v64 = (t.double().numpy() for t in (q, k, v))
    sc = float(np.float32(cfg.scale))
    out, _ = oracle.attention(q, k, v, cfg.scale, cfg.causal, cfg.window)
    ref = _torch_sdpa(q64, k64, v64, sc, cfg.causal, cfg.window)
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("seed", range(6))
def test_p11_library_sdpa_random_shapes(seed):
    r = np.random.default_rng(100 + seed)
    Hkv = int(r.choice([1, 2]))
    Hq = Hkv * int(r.choice([1, 3]))
    Lq, Lk = int(r.integers(1, 40)), int(r.integers(1, 40))
    causal = bool(r.integers(0, 2))
    window = int(r.choice([-1, 0, 2, 7]))
    if Lq > Lk and causal:
        Lq = Lk  # torch returns NaN for rows with no visible key
    if window >= 0 and not causal and Lq > Lk + window:
        Lq = Lk
    q, k, v = (t.double().numpy() for t in random_dense(2, Hq, Hkv, Lq, Lk, 16, "bf16", seed))
    out, _ = oracle.attention(q, k, v, 0.25, causal, window)
    ref = _torch_sdpa(q, k, v, 0.25, causal, window)
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- sampled rows

def test_rows_subset_matches_full():
    q, k, v = small_case(Lq=30, Lk=30, seed=24)
    full = oracle.attention(q, k, v, 0.3, True, 6)
    rows = [0, 5, 17, 29]
    part = oracle.attention(q, k, v, 0.3, True, 6, rows=rows)
    np.testing.assert_array_equal(part[0], full[0][:, rows])
    np.testing.assert_array_equal(part[1], full[1][:, :, rows])


# ---------------------------------------------------------------- P12: paged prefill

@pytest.mark.parametrize("causal,window", [(True, -1), (True, 3), (False, -1), (False, 2)])
def test_p12_paged_prefill_equals_dense_and_library(causal, window):
    """NEWS: paging changes where K/V live, not which are attended; the new
    Lq tokens are the last Lq positions of each sequence (bottom-right
    diagonal).  Checked against the oracle's dense attention on the unscattered
    K/V, against torch's CPU float64 SDPA with an explicit mask, and for
    invariance to the physical block permutation.  Contexts shorter than Lq
    leave the first rows without keys (out 0, lse -inf)."""
    r = np.random.default_rng(31)
    Hq, Hkv, D, bs, Lq = 4, 2, 8, 4, 5
    ctx = [1, 3, 5, 9, 16]
    B = len(ctx)
    K = [r.standard_normal((c, Hkv, D)) for c in ctx]
    V = [r.standard_normal((c, Hkv, D)) for c in ctx]
    q = r.standard_normal((B, Lq, Hq, D))
    sc = 0.3
    outs = []
    for perm_seed in (None, 32):
        kc, vc, table = _scatter_to_pool(K, V, ctx, bs, perm_seed, Hkv, D)
        o, l = oracle.prefill_paged(q, kc, vc, table, np.array(ctx), bs, sc, causal, window)
        outs.append((o, l))
        for b, c in enumerate(ctx):
            ro, rl = oracle.attention(q[b][None], K[b][None], V[b][None], sc, causal, window)
            np.testing.assert_allclose(o[b], ro[0], atol=TIGHT, rtol=0)
            np.testing.assert_allclose(l[b], rl[0], atol=TIGHT, rtol=0)
            empty = ~np.isfinite(l[b])  # [Hq, Lq]
            if causal:
                # exactly the rows before the context starts are empty
                assert np.array_equal(empty[0], np.arange(Lq) < Lq - c)
            assert np.all(o[b].transpose(1, 0, 2)[empty] == 0)
            rows = np.where(~empty[0])[0]
            if len(rows):
                sc32 = float(np.float32(sc))  # the oracle uses the float32 scale a kernel receives
                lib = _torch_sdpa(q[b][None], K[b][None], V[b][None], sc32, causal, window)[0]
                np.testing.assert_allclose(o[b][rows], lib[rows], atol=1e-12, rtol=0)
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


def test_p12_paged_prefill_single_token_is_decode():
    r = np.random.default_rng(33)
    Hq, Hkv, D, bs = 6, 2, 8, 4
    ctx = [2, 7, 12]
    K = [r.standard_normal((c, Hkv, D)) for c in ctx]
    V = [r.standard_normal((c, Hkv, D)) for c in ctx]
    kc, vc, table = _scatter_to_pool(K, V, ctx, bs, 34, Hkv, D)
    q = r.standard_normal((len(ctx), 1, Hq, D))
    o, l = oracle.prefill_paged(q, kc, vc, table, np.array(ctx), bs, 0.4)
    od, ld = oracle.decode_paged(q[:, 0], kc, vc, table, np.array(ctx), bs, 0.4)
    np.testing.assert_allclose(o[:, 0], od, atol=TIGHT, rtol=0)
    np.testing.assert_allclose(l[:, :, 0], ld, atol=TIGHT, rtol=0)


# ---------------------------------------------------------------- P13: backward

def _loss(q, k, v, do, sc, causal, window):
    o, _ = oracle.attention(q, k, v, sc, causal, window)
    return float((o * do).sum())


@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 1), (False, 1)])
def test_p13_backward_matches_finite_differences(causal, window):
    """Central differences of L = sum(dO * attention) on a tiny GQA case
    (3 query rows, 4 keys; the last row of the causal case sees all keys)."""
    r = np.random.default_rng(61)
    B, Hq, Hkv, Lq, Lk, D = 1, 2, 1, 3, 4, 3
    q = r.standard_normal((B, Lq, Hq, D))
    k = r.standard_normal((B, Lk, Hkv, D))
    v = r.standard_normal((B, Lk, Hkv, D))
    do = r.standard_normal((B, Lq, Hq, D))
    sc = 0.5  # exactly representable in float32
    dq, dk, dv = oracle.attention_backward(q, k, v, do, sc, causal, window)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], do, sc, causal, window)
                        - _loss(args_m["q"], args_m["k"], args_m["v"], do, sc, causal, window)) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=1e-7, rtol=0, err_msg=f"d{name}")


@pytest.mark.parametrize("seed", range(4))
def test_p13_backward_matches_torch_autograd(seed):
    """A library routine: torch CPU float64 autograd through
    scaled_dot_product_attention with an explicit mask (K/V expanded over the
    query heads of their group, gradients summed back)."""
    r = np.random.default_rng(70 + seed)
    Hkv = int(r.choice([1, 2]))
    Hq = Hkv * int(r.choice([1, 3]))
    Lk = int(r.integers(2, 30))
    Lq = int(r.integers(1, Lk + 1))
    causal = bool(r.integers(0, 2))
    window = int(r.choice([-1, 3, 9]))
    q, k, v = (t.double().numpy() for t in random_dense(2, Hq, Hkv, Lq, Lk, 16, "bf16", 80 + seed))
    do = r.standard_normal(q.shape)
    sc = 0.25
    dq, dk, dv = oracle.attention_backward(q, k, v, do, sc, causal, window)
    qt = torch.tensor(q.transpose(0, 2, 1, 3), requires_grad=True)
    kt = torch.tensor(k.transpose(0, 2, 1, 3), requires_grad=True)
    vt = torch.tensor(v.transpose(0, 2, 1, 3), requires_grad=True)
    i = torch.arange(Lq)[:, None] + (Lk - Lq)
    j = torch.arange(Lk)[None, :]
    m = torch.ones(Lq, Lk, dtype=torch.bool)
    if causal:
        m &= j <= i
    if window >= 0:
        m &= j >= i - window
        if not causal:
            m &= j <= i + window
    rep = Hq // Hkv
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(rep, 1), vt.repeat_interleave(rep, 1), attn_mask=m, scale=sc)
    (o * torch.tensor(do.transpose(0, 2, 1, 3))).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy().transpose(0, 2, 1, 3), atol=1e-10, rtol=0)
    np.testing.assert_allclose(dk, kt.grad.numpy().transpose(0, 2, 1, 3), atol=1e-10, rtol=0)
    np.testing.assert_allclose(dv, vt.grad.numpy().transpose(0, 2, 1, 3), atol=1e-10, rtol=0)


def test_p13_backward_sum_identities_and_empty_rows():
    """Rows of P sum to one, so sum_j dV_j = sum of dO over non-empty rows; the
    output does not change when every key of a head moves by the same vector
    (softmax shift invariance, P7), so sum_j dK_j = 0.  Rows with no visible
    key get dQ = 0 and contribute nothing."""
    r = np.random.default_rng(90)
    B, Hq, Hkv, Lq, Lk, D = 2, 4, 2, 9, 6, 5
    q = r.standard_normal((B, Lq, Hq, D))
    k = r.standard_normal((B, Lk, Hkv, D))
    v = r.standard_normal((B, Lk, Hkv, D))
    do = r.standard_normal((B, Lq, Hq, D))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.7, causal=True)
    empty = np.arange(Lq) < Lq - Lk  # causal, bottom-right: the first Lq-Lk rows see nothing
    assert np.all(dq[:, empty] == 0)
    for b in range(B):
        for g in range(Hkv):
            heads = [h for h in range(Hq) if oracle.kv_head(h, Hq, Hkv) == g]
            np.testing.assert_allclose(dv[b, :, g].sum(axis=0), do[b][~empty][:, heads].sum(axis=(0, 1)),
                                       atol=TIGHT)
            np.testing.assert_allclose(dk[b, :, g].sum(axis=0), 0.0, atol=TIGHT)


def test_p13_backward_gqa_is_sum_over_expanded_heads():
    r = np.random.default_rng(91)
    B, Hq, Hkv, L, D = 1, 6, 2, 7, 4
    q = r.standard_normal((B, L, Hq, D))
    k = r.standard_normal((B, L, Hkv, D))
    v = r.standard_normal((B, L, Hkv, D))
    do = r.standard_normal((B, L, Hq, D))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.3, causal=True)
    ke, ve = np.repeat(k, Hq // Hkv, axis=2), np.repeat(v, Hq // Hkv, axis=2)
    dq1, dk1, dv1 = oracle.attention_backward(q, ke, ve, do, 0.3, causal=True)
    np.testing.assert_allclose(dq, dq1, atol=TIGHT)
    np.testing.assert_allclose(dk, dk1.reshape(B, L, Hkv, Hq // Hkv, D).sum(axis=3), atol=TIGHT)
    np.testing.assert_allclose(dv, dv1.reshape(B, L, Hkv, Hq // Hkv, D).sum(axis=3), atol=TIGHT)


# ---------------------------------------------------------------- P14: dropout
# The generator is Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011); the
# oracle's numpy copy is pinned against rocRAND's engine, a library
# implementation compiled here for the host from its header.

import shutil
import subprocess

_ROCRAND_HDR = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"


def build_philox_ref(workdir):
    """Compile tests/philox_ref.cpp (rocRAND's engine) into workdir and return
    run(mode, rows) -> int64 array of its output lines; None without g++ or
    the header."""
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(_ROCRAND_HDR):
        return None
    exe = os.path.join(str(workdir), "philox_ref")
    subprocess.run([gxx, "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    os.path.join(HERE, "philox_ref.cpp"), "-o", exe], check=True)

    def run(mode, rows):
        text = "".join(" ".join(str(int(x)) for x in r) + "\n" for r in rows)
        res = subprocess.run([exe, mode], input=text, capture_output=True, text=True, check=True)
        return np.array([[int(w) for w in line.split()] for line in res.stdout.splitlines()], dtype=np.int64)
    return run


@pytest.fixture(scope="module")
def philox_ref(tmp_path_factory):
    run = build_philox_ref(tmp_path_factory.mktemp("philox"))
    if run is None:
        pytest.skip("g++ or rocRAND's Philox header not available")
    return run


def _philox_cases(n=300, seed=14):
    r = np.random.default_rng(seed)
    top = 2 ** 32 - 1
    rows = [(0, 0, 0, 0, 0, 0), (top, top, top, 2 ** 30 - 1, top, top), (1, 0, 0, 0, 0, 0),
            (0, 0, 1, 0, 0, 0), (0, 0, 0, 1, 0, 0), (0, 0, 0, 0, 1, 0), (0, 0, 0, 0, 0, 1)]
    for _ in range(n):
        rows.append((r.integers(0, 2 ** 32), r.integers(0, 2 ** 32), r.integers(0, 2 ** 32),
                     r.integers(0, 2 ** 30), r.integers(0, 2 ** 32), r.integers(0, 2 ** 32)))
    return np.array(rows, dtype=np.int64)


def test_p14_philox_matches_library_engine(philox_ref):
    cases = _philox_cases()
    want = philox_ref("words", cases)
    got = oracle.philox4x32(cases[:, 2:6], (cases[:, 0], cases[:, 1])).astype(np.int64)
    assert np.array_equal(got, want)


def test_p14_keep_convention_matches_library_engine(philox_ref):
    # element (bh, i, j) against the engine addressed per element, over rows and
    # keys that cross 4-key groups and row pairs, both rows of a pair, large
    # row and key indexes, offsets and seeds
    for (seed, off, p, bh, rows, Lk) in [(0, 0, 0.1, 0, [0, 1, 2, 3, 5], 13),
                                          (0x1234567890ABCDEF, 77, 0.5, 37, [0, 9, 8, 1000, 1001, 65535], 70),
                                          (2 ** 64 - 1, 2 ** 32 - 1, 0.9, 2 ** 20 + 3, [3, 2 ** 29, 2 ** 31 - 1], 9)]:
        thr = oracle.dropout_threshold(p)
        keep = oracle.dropout_keep(bh, rows, Lk, p, seed, off)
        qs = [(seed, off, thr, bh, i, j) for i in rows for j in range(Lk)]
        want = philox_ref("keep", qs).reshape(len(rows), Lk).astype(bool)
        assert np.array_equal(keep, want)


def test_p14_keep_with_key_offset(philox_ref):
    # key0 numbers the keys of a slice: the same columns of the full mask, and
    # the engine addressed per element at key indices near 2^30
    full = oracle.dropout_keep(3, [0, 7, 40], 150, 0.3, 99, 4)
    for key0 in (1, 4, 37, 101):
        part = oracle.dropout_keep(3, [0, 7, 40], 150 - key0, 0.3, 99, 4, key0=key0)
        assert np.array_equal(part, full[:, key0:])
    key0, n, rows = (1 << 30) + 3, 21, [5, 2 ** 20, 2 ** 20 + 1]
    thr = oracle.dropout_threshold(0.4)
    keep = oracle.dropout_keep(11, rows, n, 0.4, 77, 9, key0=key0)
    want = philox_ref("keep", [(77, 9, thr, 11, i, key0 + c) for i in rows for c in range(n)])
    assert np.array_equal(keep, want.reshape(len(rows), n).astype(bool))


def test_p14_threshold_and_validation():
    assert oracle.dropout_threshold(0.0) == 0
    assert oracle.dropout_threshold(0.5) == 2 ** 15
    assert oracle.dropout_threshold(0.25) == 2 ** 14
    assert oracle.dropout_threshold(np.nextafter(np.float32(1), np.float32(0))) == 2 ** 16 - 1
    p32 = float(np.float32(0.1))
    assert oracle.dropout_threshold(0.1) == math.floor(p32 * 2 ** 16) == 6553
    for bad in (1.0, -0.01, 1.5, float("nan")):
        with pytest.raises(ValueError):
            oracle.dropout_threshold(bad)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_p14_keep_rate_is_one_minus_p(p):
    # 2 heads x 300 rows x 700 keys = 420,000 independent decisions: the kept
    # fraction must lie within 5 binomial standard deviations of 1 - p, in
    # total, for each of the four words of a Philox output and for each of its
    # two 16-bit halves (even and odd rows)
    keep = np.concatenate([oracle.dropout_keep(bh, np.arange(300), 700, p, 99, 3) for bh in (0, 1)])
    n = keep.size
    sd = math.sqrt(p * (1 - p) / n)
    assert abs(keep.mean() - (1 - p)) < 5 * sd
    for w in range(4):
        kw = keep[:, w::4]
        assert abs(kw.mean() - (1 - p)) < 5 * math.sqrt(p * (1 - p) / kw.size)
    for half in range(2):
        kh = keep[half::2]
        assert abs(kh.mean() - (1 - p)) < 5 * math.sqrt(p * (1 - p) / kh.size)
    # the two rows of a pair share each generator call but not its bits
    x = keep.astype(float) - keep.mean()
    pair = (x[0::2] * x[1::2]).mean() / x.var()
    assert abs(pair) < 5 / math.sqrt(x[0::2].size)
    # neighbouring decisions are uncorrelated (lag-1 along keys and rows)
    x = keep.astype(float) - keep.mean()
    for a, b in ((x[:, 1:], x[:, :-1]), (x[1:], x[:-1])):
        corr = (a * b).mean() / x.var()
        assert abs(corr) < 5 / math.sqrt(a.size)


@pytest.mark.parametrize("causal,window", MASKS)
def test_p14_zero_probability_is_plain_attention(causal, window):
    q, k, v = small_case(seed=140)
    out, lse = oracle.attention_dropout(q, k, v, 0.4, causal, window, p=0.0, seed=5, offset=1)
    ref, rl = oracle.attention(q, k, v, 0.4, causal, window)
    assert np.array_equal(out, ref) and np.array_equal(lse, rl)


def test_p14_identity_values_expose_dropped_probabilities():
    # with V = I (one value dimension per key) row i of the output is
    # P_i * keep_i / (1 - p): the mask multiplies the normalised probabilities
    r = np.random.default_rng(141)
    B, Hq, Hkv, Lq, Lk = 1, 2, 1, 11, 16
    q = r.standard_normal((B, Lq, Hq, Lk))
    k = r.standard_normal((B, Lk, Hkv, Lk))
    v = np.eye(Lk)[None, :, None, :]
    p, seed, off = 0.3, 1234, 9
    out, lse = oracle.attention_dropout(q, k, v, 0.5, True, -1, p, seed, off)
    ref, rl = oracle.attention(q, k, v, 0.5, True, -1)  # = P itself
    assert np.array_equal(lse, rl)
    for h in range(Hq):
        keep = oracle.dropout_keep(h, np.arange(Lq), Lk, p, seed, off)
        want = np.where(keep, ref[0, :, h, :], 0.0) / (1 - float(np.float32(p)))
        np.testing.assert_allclose(out[0, :, h, :], want, rtol=1e-14, atol=1e-15)
    assert (out == 0).any() and (out > 0).any()


def test_p14_dropout_is_unbiased_over_seeds():
    # inverted dropout: averaged over independent draws the output tends to the
    # plain output (each element within 6 standard errors of the sample mean)
    q, k, v = small_case(B=1, Hq=2, Hkv=1, Lq=6, Lk=10, D=4, seed=142)
    ref, _ = oracle.attention(q, k, v, 0.7, False, -1)
    draws = np.stack([oracle.attention_dropout(q, k, v, 0.7, False, -1, 0.5, s, 0)[0] for s in range(600)])
    mean, se = draws.mean(axis=0), draws.std(axis=0) / math.sqrt(len(draws))
    assert np.all(np.abs(mean - ref) <= 6 * se + 1e-12)


def test_p14_dropout_rows_subset_matches_full():
    q, k, v = small_case(Lq=20, Lk=23, seed=143)
    out, lse = oracle.attention_dropout(q, k, v, 0.3, True, 4, 0.2, 77, 5)
    rows = [0, 3, 19, 7]
    o2, l2 = oracle.attention_dropout(q, k, v, 0.3, True, 4, 0.2, 77, 5, rows=rows)
    assert np.array_equal(o2, out[:, rows]) and np.array_equal(l2, lse[:, :, rows])


def _torch_dropout_grads(q, k, v, do, sc, causal, window, p, seed, off):
    """torch autograd (float64, CPU) of sum(do * ((softmax(S) * M) @ V)) with
    the mask M = keep / (1 - p) held fixed."""
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    grp = Hq // Hkv
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    ok = torch.tensor(oracle.allowed_mask(Lq, Lk, causal, window))
    loss = 0.0
    for b in range(B):
        for h in range(Hq):
            S = float(np.float32(sc)) * tq[b, :, h] @ tk[b, :, h // grp].T
            S = S.masked_fill(~ok, float("-inf"))
            P = torch.softmax(S, dim=1).nan_to_num(0.0)
            M = torch.tensor(np.where(oracle.dropout_keep(b * Hq + h, np.arange(Lq), Lk, p, seed, off),
                                      1.0 / (1.0 - float(np.float32(p))), 0.0))
            loss = loss + (torch.tensor(do[b, :, h]) * ((P * M) @ tv[b, :, h // grp])).sum()
    loss.backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 2)])
def test_p14_dropout_backward_matches_torch_autograd(causal, window):
    r = np.random.default_rng(144)
    q = r.standard_normal((2, 7, 4, 6))
    k = r.standard_normal((2, 9, 2, 6))
    v = r.standard_normal((2, 9, 2, 6))
    do = r.standard_normal(q.shape)
    got = oracle.attention_dropout_backward(q, k, v, do, 0.45, causal, window, 0.3, 31, 2)
    want = _torch_dropout_grads(q, k, v, do, 0.45, causal, window, 0.3, 31, 2)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=1e-11, atol=1e-12)


def test_p14_dropout_backward_zero_probability_is_plain_backward():
    r = np.random.default_rng(145)
    q = r.standard_normal((1, 5, 2, 4))
    k = r.standard_normal((1, 8, 1, 4))
    v = r.standard_normal((1, 8, 1, 4))
    do = r.standard_normal(q.shape)
    got = oracle.attention_dropout_backward(q, k, v, do, 0.6, True, -1, 0.0, 3, 0)
    want = oracle.attention_backward(q, k, v, do, 0.6, True, -1)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=0, atol=TIGHT)


def test_p14_dropout_backward_matches_finite_differences():
    r = np.random.default_rng(146)
    q = r.standard_normal((1, 4, 2, 3))
    k = r.standard_normal((1, 5, 1, 3))
    v = r.standard_normal((1, 5, 1, 3))
    do = r.standard_normal(q.shape)
    args = (0.8, True, 1, 0.4, 8, 1)

    def loss(q_, k_, v_):
        return float((do * oracle.attention_dropout(q_, k_, v_, *args)[0]).sum())
    grads = oracle.attention_dropout_backward(q, k, v, do, *args)
    eps = 1e-6
    for idx, x in enumerate((q, k, v)):
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[pos] += eps
            xm[pos] -= eps
            a = [q, k, v]
            a[idx] = xp
            lp = loss(*a)
            a[idx] = xm
            num[pos] = (lp - loss(*a)) / (2 * eps)
        np.testing.assert_allclose(grads[idx], num, rtol=1e-6, atol=1e-7)
