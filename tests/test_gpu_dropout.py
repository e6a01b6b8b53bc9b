"""GPU parity of the forward with dropout (attn_fwd_dropout) against the fp64
oracle (oracle.attention_dropout: the definition, with the keep decisions of
Philox4x32-10 at the per-element counter of include/attn.h).

Two kinds of checks:
  * the keep decisions themselves, bit for bit: with one-hot values
    v_j = e_{j mod D} and a causal window of D - 1 keys, every row sees D
    keys with distinct j mod D, so output column j mod D of row i is
    P_ij * keep_ij / (1 - p): nonzero exactly when the kernel kept (i, j);
  * the outputs, with the forward's per-dtype max-abs bound (2e-3 fp16,
    1.6e-2 bf16) times 1 / (1 - p), the factor by which dropout scales the
    kept terms (and their rounding errors); lse must match the undropped
    oracle within 1e-3.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, DTYPES, dense_inputs, random_dense

pytestmark = pytest.mark.gpu

TOL = {"fp16": 2e-3, "bf16": 1.6e-2}
LSE_TOL = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_drop(ta, q, k, v, p, seed, offset, scale, causal, window):
    qq, kk, vv = (t.to("cuda") for t in (q, k, v))
    out, lse = ta.attn_fwd_dropout(qq, kk, vv, p, seed, offset, scale=scale, causal=causal, window=window)
    torch.cuda.synchronize()
    return out, lse


def check_out(name, out, lse, q, k, v, scale, causal, window, p, seed, offset, dtype, rows=None):
    ref, rl = oracle.attention_dropout(q, k, v, scale, causal, window, p, seed, offset, rows=rows)
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    if rows is not None:
        o, l = o[:, rows], l[:, :, rows]
    assert not np.isnan(o).any(), f"{name}: NaN in output"
    err = float(np.max(np.abs(o - ref))) if o.size else 0.0
    tol = TOL[dtype] / (1.0 - float(np.float32(p)))
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(l), ~fin), f"{name}: lse -inf pattern differs"
    lerr = float(np.max(np.abs(l[fin] - rl[fin]))) if fin.any() else 0.0
    say(f"{name}: out max-abs {err:.3e} (tol {tol:.2e}); lse max-abs {lerr:.2e}")
    assert err <= tol, f"{name}: output error {err:.3e} > {tol:.3e}"
    assert lerr <= LSE_TOL, f"{name}: lse error {lerr:.3e}"


def one_hot_values(B, Lk, Hkv, D, dtype):
    v = np.zeros((B, Lk, Hkv, D), dtype=np.float32)
    v[:, np.arange(Lk), :, np.arange(Lk) % D] = 1.0
    return torch.from_numpy(v).to(DTYPES[dtype])


MASK_CASES = [
    # B, Hq, Hkv, Lq, Lk, D, dtype, p, seed, offset
    (1, 2, 1, 200, 200, 64, "bf16", 0.1, 7, 0),
    (2, 4, 2, 333, 400, 128, "fp16", 0.5, 0x1234567890ABCDEF, 3),
    (1, 3, 1, 129, 700, 64, "bf16", 0.9, 2 ** 64 - 1, 2 ** 32 - 1),
    (1, 8, 2, 600, 600, 128, "bf16", 0.25, 42, 12345),
]


@pytest.mark.parametrize("case", range(len(MASK_CASES)))
def test_dropout_keep_decisions_bit_exact(gpu_lib, case):
    B, Hq, Hkv, Lq, Lk, D, dtype, p, seed, offset = MASK_CASES[case]
    say(f"[case] dropout mask {case}: B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} D{D} {dtype} p{p} seed{seed} off{offset}")
    q, k, _ = random_dense(B, Hq, Hkv, Lq, Lk, D, dtype, 1000 + case)
    v = one_hot_values(B, Lk, Hkv, D, dtype)
    W = D - 1
    out, lse = run_drop(gpu_lib, q, k, v, p, seed, offset, 1.0 / np.sqrt(D), True, W)
    o = out.float().cpu().numpy()
    ok = oracle.allowed_mask(Lq, Lk, True, W)
    kept_total = seen_total = 0
    for b in range(B):
        for h in range(Hq):
            keep = oracle.dropout_keep(b * Hq + h, np.arange(Lq), Lk, p, seed, offset)
            i_idx, j_idx = np.nonzero(ok)
            got = o[b, i_idx, h, j_idx % D] > 0
            want = keep[i_idx, j_idx]
            bad = int(np.count_nonzero(got != want))
            assert bad == 0, f"(b={b}, h={h}): {bad} of {len(got)} keep decisions differ"
            kept_total += int(want.sum())
            seen_total += len(want)
    rate = kept_total / seen_total
    sd = np.sqrt(p * (1 - p) / seen_total)
    say(f"  {seen_total} decisions, kept fraction {rate:.4f} (1 - p = {1 - p})")
    assert abs(rate - (1 - p)) < 5 * sd
    check_out(f"dropout mask {case} values", out, lse, q, k, v, 1.0 / np.sqrt(D), True, W, p, seed, offset, dtype)


CASES = [
    # B, Hq, Hkv, Lq, Lk, D, dtype, causal, window, p
    (1, 2, 1, 128, 128, 64, "fp16", False, -1, 0.1),
    (2, 4, 2, 200, 333, 128, "bf16", True, -1, 0.2),
    (1, 4, 1, 300, 150, 64, "bf16", True, -1, 0.5),
    (1, 2, 2, 257, 257, 128, "fp16", True, 64, 0.1),
    (2, 6, 3, 100, 77, 64, "bf16", False, 20, 0.3),
    (1, 8, 2, 129, 1000, 128, "bf16", False, -1, 0.1),
    (1, 3, 1, 1, 65, 64, "fp16", True, -1, 0.7),
    (1, 2, 1, 70, 1, 128, "fp16", False, -1, 0.5),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_dropout_forward_cases(gpu_lib, case):
    B, Hq, Hkv, Lq, Lk, D, dtype, causal, window, p = CASES[case]
    say(f"[case] dropout fwd {case}: B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} D{D} {dtype} causal{causal} w{window} p{p}")
    q, k, v = random_dense(B, Hq, Hkv, Lq, Lk, D, dtype, 1100 + case)
    seed, offset = 9000 + case, case
    out, lse = run_drop(gpu_lib, q, k, v, p, seed, offset, 1.0 / np.sqrt(D), causal, window)
    check_out(f"dropout fwd {case}", out, lse, q, k, v, 1.0 / np.sqrt(D), causal, window, p, seed, offset, dtype)


@pytest.mark.parametrize("case", [0, 1, 3, 4])
def test_dropout_zero_probability_is_attn_fwd_bitwise(gpu_lib, case):
    B, Hq, Hkv, Lq, Lk, D, dtype, causal, window, _ = CASES[case]
    q, k, v = (t.to("cuda") for t in random_dense(B, Hq, Hkv, Lq, Lk, D, dtype, 1200 + case))
    a = gpu_lib.attn_fwd_dropout(q, k, v, 0.0, 5, 6, causal=causal, window=window)
    b = gpu_lib.attn_fwd(q, k, v, causal=causal, window=window)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("name,p", [("std512_causal", 0.1), ("gqa8k_causal", 0.1)])
def test_dropout_workloads_sampled_rows(gpu_lib, name, p):
    cfg = CONFIGS[name]
    say(f"[case] dropout workload {name} p{p} (sampled rows)")
    q, k, v = dense_inputs(cfg)
    out, lse = run_drop(gpu_lib, q, k, v, p, 77, 1, cfg.scale, cfg.causal, cfg.window)
    # one row from every 32-row wave group of every q-block, plus both ends
    per_group = np.arange(0, cfg.Lq, 32) + np.random.default_rng(cfg.seed).integers(0, 32, size=-(-cfg.Lq // 32))
    rows = np.unique(np.concatenate([np.arange(0, 40), np.minimum(per_group, cfg.Lq - 1),
                                     np.arange(cfg.Lq - 40, cfg.Lq)]))
    check_out(name, out, lse, q, k, v, cfg.scale, cfg.causal, cfg.window, p, 77, 1, cfg.dtype, rows=rows)


def test_dropout_long_gqa_first_kv_head_all_rows(gpu_lib):
    """The long causal GQA forward with dropout (p = 0.1) at its full size,
    every head run on the GPU; with B = 1 the first KV head's query heads are
    heads 0..3 of the problem, so the oracle on that slice draws the same keep
    decisions, and every output row of those heads is compared."""
    cfg = CONFIGS["gqa8k_causal"]
    say("[case] dropout workload gqa8k_causal p0.1 (KV head 0, all rows)")
    q, k, v = dense_inputs(cfg)
    out, lse = run_drop(gpu_lib, q, k, v, 0.1, 77, 1, cfg.scale, cfg.causal, cfg.window)
    hs = list(range(cfg.Hq // cfg.Hkv))
    check_out("gqa8k_causal dropout KV head 0", out[:, :, hs], lse[:, hs], q[:, :, hs], k[:, :, :1], v[:, :, :1],
              cfg.scale, cfg.causal, cfg.window, 0.1, 77, 1, cfg.dtype)


def test_dropout_deterministic_and_offset_changes_mask(gpu_lib):
    q, k, v = (t.to("cuda") for t in random_dense(1, 4, 2, 300, 300, 128, "bf16", 1300))
    a = gpu_lib.attn_fwd_dropout(q, k, v, 0.3, 11, 0, causal=True)
    b = gpu_lib.attn_fwd_dropout(q, k, v, 0.3, 11, 0, causal=True)
    c = gpu_lib.attn_fwd_dropout(q, k, v, 0.3, 11, 1, causal=True)
    d = gpu_lib.attn_fwd_dropout(q, k, v, 0.3, 12, 0, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert not torch.equal(a[0], c[0]) and not torch.equal(a[0], d[0])
    assert torch.equal(a[1], c[1]) and torch.equal(a[1], d[1])  # lse does not depend on the mask


def test_dropout_empty_keys_and_rows(gpu_lib):
    q, k, v = (t.to("cuda") for t in random_dense(1, 2, 1, 5, 7, 64, "fp16", 1301))
    o0, l0 = gpu_lib.attn_fwd_dropout(q, k[:, :0], v[:, :0], 0.5, 1, 0)
    torch.cuda.synchronize()
    assert torch.all(o0 == 0) and torch.all(torch.isneginf(l0))
    e, le = gpu_lib.attn_fwd_dropout(q[:, :0], k, v, 0.5, 1, 0)
    assert e.numel() == 0 and le.numel() == 0


# ---------------------------------------------------------------- backward

GTOL = {"fp16": 2e-3, "bf16": 1.6e-2}


def _dout(shape, dtype, seed):
    r = np.random.default_rng(seed)
    return torch.from_numpy(r.standard_normal(size=shape, dtype=np.float32)).to(DTYPES[dtype])


def run_bwd_drop(ta, q, k, v, do, p, seed, offset, scale, causal, window):
    qd, kd, vd, dod = (t.to("cuda") for t in (q, k, v, do))
    out, lse = ta.attn_fwd_dropout(qd, kd, vd, p, seed, offset, scale=scale, causal=causal, window=window)
    grads = ta.attn_bwd_dropout(qd, kd, vd, out, dod, lse, p, seed, offset, scale=scale, causal=causal,
                                window=window)
    torch.cuda.synchronize()
    return grads


BWD_CASES = [
    # B, Hq, Hkv, Lq, Lk, D, dtype, causal, window, p
    (1, 2, 1, 128, 128, 64, "fp16", False, -1, 0.1),
    (2, 4, 2, 200, 333, 128, "bf16", True, -1, 0.2),
    (1, 4, 1, 300, 150, 64, "bf16", True, -1, 0.5),
    (1, 2, 2, 257, 257, 128, "fp16", True, 64, 0.1),
    (2, 6, 3, 100, 77, 64, "bf16", False, 20, 0.3),
    (1, 3, 1, 1, 65, 64, "fp16", True, -1, 0.7),
    (1, 2, 1, 70, 1, 128, "fp16", False, -1, 0.5),
]


@pytest.mark.parametrize("case", range(len(BWD_CASES)))
def test_dropout_backward_cases(gpu_lib, case):
    """Tolerance: the backward's per-dtype bound times max(1, max|ref|), and
    times 1 / (1 - p), the factor dropout puts on the kept terms."""
    B, Hq, Hkv, Lq, Lk, D, dtype, causal, window, p = BWD_CASES[case]
    say(f"[case] dropout bwd {case}: B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} D{D} {dtype} causal{causal} w{window} p{p}")
    q, k, v = random_dense(B, Hq, Hkv, Lq, Lk, D, dtype, 1400 + case)
    do = _dout(q.shape, dtype, 1500 + case)
    scale = 1.0 / np.sqrt(D)
    seed, offset = 31 + case, 7 * case
    got = run_bwd_drop(gpu_lib, q, k, v, do, p, seed, offset, scale, causal, window)
    ref = oracle.attention_dropout_backward(q, k, v, do, scale, causal, window, p, seed, offset)
    msgs = []
    for n, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = g.double().cpu().numpy()
        assert not np.isnan(g).any(), f"{n}: NaN"
        err = float(np.max(np.abs(g - r))) if g.size else 0.0
        mag = max(1.0, float(np.max(np.abs(r)))) if r.size else 1.0
        tol = GTOL[dtype] * mag / (1.0 - float(np.float32(p)))
        msgs.append(f"{n} max-abs {err:.3e} (tol {tol:.2e})")
        assert err <= tol, "; ".join(msgs)
    say("  " + "; ".join(msgs))


@pytest.mark.parametrize("D,dtype,p,Lq,Lk", [(64, "fp16", 0.3, 300, 300), (128, "bf16", 0.6, 257, 400)])
def test_dropout_backward_keep_decisions(gpu_lib, D, dtype, p, Lq, Lk):
    """Both backward kernels' keep decisions, element by element.

    Keys, values and output gradients are one-hot, with a causal window of
    D - 1 keys, so that each row sees D keys of distinct j mod D and each key
    is seen by D rows of distinct i mod D:
      * dout_i = e_{i mod D}:  dv[j, i mod D] = P_ij M_ij, nonzero iff kept
        (the dK/dV kernel's decision);
      * dout = 1, k_j = v_j = e_{j mod D}: dq[i, j mod D] = scale * dS_ij with
        dS_ij = P_ij (M_ij - D_i), i.e. scale * P_ij (1/(1-p) - D_i) if kept and
        -scale * P_ij D_i if dropped; the kernel's value is classified by the
        nearer of the two (fp64 oracle values), which must give the oracle's
        decision (the dQ kernel's decision).
    """
    B, H, W = 1, 2, D - 1
    seed, offset = 0xC0FFEE, 17
    say(f"[case] dropout bwd decisions D{D} {dtype} p{p} Lq{Lq} Lk{Lk}")
    rng = np.random.default_rng(1600 + D)
    q = torch.from_numpy(rng.standard_normal((B, Lq, H, D), dtype=np.float32)).to(DTYPES[dtype])
    onehot_k = np.zeros((B, Lk, H, D), dtype=np.float32)
    onehot_k[:, np.arange(Lk), :, np.arange(Lk) % D] = 1.0
    kv = torch.from_numpy(onehot_k).to(DTYPES[dtype])
    scale = 1.0 / np.sqrt(D)
    ok = oracle.allowed_mask(Lq, Lk, True, W)
    i_idx, j_idx = np.nonzero(ok)

    # dK/dV kernel: dout_i = e_{i mod D}
    do_a = np.zeros((B, Lq, H, D), dtype=np.float32)
    do_a[:, np.arange(Lq), :, np.arange(Lq) % D] = 1.0
    k_rand = torch.from_numpy(rng.standard_normal((B, Lk, H, D), dtype=np.float32)).to(DTYPES[dtype])
    _, _, dv = run_bwd_drop(gpu_lib, q, k_rand, kv, torch.from_numpy(do_a).to(DTYPES[dtype]), p, seed, offset,
                            scale, True, W)
    dv = dv.float().cpu().numpy()
    for h in range(H):
        keep = oracle.dropout_keep(h, np.arange(Lq), Lk, p, seed, offset)
        got = dv[0, j_idx, h, i_idx % D] > 0
        bad = int(np.count_nonzero(got != keep[i_idx, j_idx]))
        assert bad == 0, f"dK/dV kernel, head {h}: {bad} of {len(got)} decisions differ"

    # dQ kernel: dout = 1, k = v = one-hot
    do_b = torch.ones((B, Lq, H, D), dtype=DTYPES[dtype])
    dq, _, _ = run_bwd_drop(gpu_lib, q, kv, kv, do_b, p, seed, offset, scale, True, W)
    dq = dq.double().cpu().numpy()
    Pm, _ = oracle.attention(q, kv, kv, scale, True, W)  # one-hot values: column j mod D of row i is P_ij
    inv = 1.0 / (1.0 - float(np.float32(p)))
    for h in range(H):
        keep = oracle.dropout_keep(h, np.arange(Lq), Lk, p, seed, offset)
        Pij = Pm[0, i_idx, h, j_idx % D]            # P_ij (values one-hot: column j mod D of row i)
        Di = np.zeros(Lq)
        np.add.at(Di, i_idx, Pij * np.where(keep[i_idx, j_idx], inv, 0.0))
        hyp_keep = scale * Pij * (inv - Di[i_idx])
        hyp_drop = -scale * Pij * Di[i_idx]
        g = dq[0, i_idx, h, j_idx % D]
        got = np.abs(g - hyp_keep) < np.abs(g - hyp_drop)
        bad = int(np.count_nonzero(got != keep[i_idx, j_idx]))
        assert bad == 0, f"dQ kernel, head {h}: {bad} of {len(got)} decisions differ"
    say(f"  {H * len(i_idx)} decisions per kernel agree")


def test_dropout_backward_zero_probability_is_attn_bwd_bitwise(gpu_lib):
    q, k, v = (t.to("cuda") for t in random_dense(1, 4, 2, 190, 230, 128, "bf16", 1700))
    do = _dout(q.shape, "bf16", 1701).to("cuda")
    out, lse = gpu_lib.attn_fwd(q, k, v, causal=True)
    a = gpu_lib.attn_bwd_dropout(q, k, v, out, do, lse, 0.0, 9, 9, causal=True)
    b = gpu_lib.attn_bwd(q, k, v, out, do, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_dropout_backward_workload_std2048(gpu_lib):
    cfg = CONFIGS["std2048"]
    say("[case] dropout bwd workload std2048 p0.1")
    q, k, v = dense_inputs(cfg)
    do = _dout(q.shape, cfg.dtype, 1800)
    got = run_bwd_drop(gpu_lib, q, k, v, do, 0.1, 5, 2, cfg.scale, cfg.causal, cfg.window)
    ref = oracle.attention_dropout_backward(q, k, v, do, cfg.scale, cfg.causal, cfg.window, 0.1, 5, 2)
    for n, g, r in zip(("dq", "dk", "dv"), got, ref):
        err = float(np.max(np.abs(g.double().cpu().numpy() - r)))
        tol = GTOL[cfg.dtype] * max(1.0, float(np.max(np.abs(r)))) / 0.9
        say(f"  {n} max-abs {err:.3e} (tol {tol:.2e})")
        assert err <= tol


def test_dropout_backward_long_gqa_first_kv_head_in_full(gpu_lib):
    """The long causal GQA backward with dropout (p = 0.1) at its full size
    (B1 Hq32 Hkv8 L8192 D128 bf16), every head run on the GPU.  With B = 1
    the first KV head's four query heads are heads 0..3 of the problem, so the
    oracle on that slice draws the same keep decisions (counter word 2 is
    b*Hq + h); every element of their dQ and of KV head 0's dK and dV is
    compared (about 30 s and 6 GB of CPU)."""
    cfg = CONFIGS["gqa8k_causal"]
    say("[case] dropout bwd workload gqa8k_causal p0.1 (KV head 0 in full)")
    q, k, v = dense_inputs(cfg)
    do = _dout(q.shape, cfg.dtype, 1801)
    dq, dk, dv = run_bwd_drop(gpu_lib, q, k, v, do, 0.1, 1234, 3, cfg.scale, cfg.causal, cfg.window)
    hs = list(range(cfg.Hq // cfg.Hkv))
    got = (dq[:, :, hs], dk[:, :, :1], dv[:, :, :1])
    ref = oracle.attention_dropout_backward(q[:, :, hs], k[:, :, :1], v[:, :, :1], do[:, :, hs], cfg.scale,
                                            cfg.causal, cfg.window, 0.1, 1234, 3)
    for n, g, r in zip(("dq", "dk", "dv"), got, ref):
        err = float(np.max(np.abs(g.double().cpu().numpy() - r)))
        tol = GTOL[cfg.dtype] * max(1.0, float(np.max(np.abs(r)))) / 0.9
        say(f"  {n} max-abs {err:.3e} (tol {tol:.2e})")
        assert err <= tol


def _rand_drop_cases(n=12):
    r = np.random.default_rng(8642)
    out = []
    for i in range(n):
        D = int(r.choice([64, 128]))
        dtype = str(r.choice(["fp16", "bf16"]))
        Hkv = int(r.choice([1, 2]))
        Hq = Hkv * int(r.choice([1, 2, 4]))
        Lq, Lk = int(r.integers(1, 300)), int(r.integers(1, 300))
        causal = bool(r.integers(0, 2))
        window = int(r.choice([-1, -1, 0, 7, 120]))
        p = float(r.choice([0.05, 0.1, 0.3, 0.5, 0.8]))
        seed = int(r.integers(0, 2 ** 63))
        offset = int(r.integers(0, 2 ** 32))
        out.append((i, int(r.integers(1, 3)), Hq, Hkv, Lq, Lk, D, dtype, causal, window, p, seed, offset))
    return out


@pytest.mark.parametrize("case", _rand_drop_cases(), ids=lambda c: f"r{c[0]}")
def test_dropout_random_forward_and_backward(gpu_lib, case):
    i, B, Hq, Hkv, Lq, Lk, D, dtype, causal, window, p, seed, offset = case
    say(f"[case] dropout random {i}: B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} D{D} {dtype} causal{causal} w{window} "
        f"p{p} seed{seed} off{offset}")
    q, k, v = random_dense(B, Hq, Hkv, Lq, Lk, D, dtype, 1900 + i)
    do = _dout(q.shape, dtype, 2000 + i)
    scale = 1.0 / np.sqrt(D)
    out, lse = run_drop(gpu_lib, q, k, v, p, seed, offset, scale, causal, window)
    check_out(f"dropout random {i}", out, lse, q, k, v, scale, causal, window, p, seed, offset, dtype)
    got = run_bwd_drop(gpu_lib, q, k, v, do, p, seed, offset, scale, causal, window)
    ref = oracle.attention_dropout_backward(q, k, v, do, scale, causal, window, p, seed, offset)
    for n, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = g.double().cpu().numpy()
        err = float(np.max(np.abs(g - r))) if g.size else 0.0
        mag = max(1.0, float(np.max(np.abs(r)))) if r.size else 1.0
        assert err <= GTOL[dtype] * mag / (1.0 - float(np.float32(p))), f"{n}: {err:.3e}"
