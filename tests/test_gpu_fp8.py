"""GPU parity of the FP8 forward (attn_fwd_fp8) against the fp64 oracle.

The oracle is plain attention on the e4m3 inputs decoded exactly (times their
descale factors).  The kernel's scores and row sums are exact up to fp32
summation; its probabilities enter the P*V product rounded to e4m3 (relative
error <= 2^-4 for normal values) and its output is rounded to bf16 (2^-8), so
each output element must lie within
    2^-4 * sum_j P_ij |v_jd| * v_descale  +  2^-8 * |ref_id|  +  2e-3
of the exact value (the 2e-3 covers the fp32 sums and the probabilities below
e4m3's normal range, which the kernel keeps at least 2^-14 below the row's
largest one).  The lse tolerance is the forward's 1e-3.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, DenseConfig, dense_inputs

pytestmark = pytest.mark.gpu

LSE_TOL = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_fp8(ta, q, k, v, scale, causal, window, qd=1.0, kd=1.0, vd=1.0):
    qq, kk, vv = (t.to("cuda") for t in (q, k, v))
    out, lse = ta.attn_fwd_fp8(qq, kk, vv, scale=scale, q_descale=qd, k_descale=kd, v_descale=vd,
                               causal=causal, window=window)
    torch.cuda.synchronize()
    return out, lse


def check_fp8(name, out, lse, q, k, v, scale, causal, window, qd=1.0, kd=1.0, vd=1.0, rows=None):
    q64, k64, v64 = (t.double().numpy() for t in (q, k, v))
    q64, k64, v64 = q64 * qd, k64 * kd, v64 * vd
    ref, rl = oracle.attention(q64, k64, v64, scale, causal, window, rows=rows)
    mag, _ = oracle.attention(q64, k64, np.abs(v64), scale, causal, window, rows=rows)
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    if rows is not None:
        o, l = o[:, rows], l[:, :, rows]
    assert not np.isnan(o).any(), f"{name}: NaN in output"
    bound = 2.0 ** -4 * mag + 2.0 ** -8 * np.abs(ref) + 2e-3
    err = np.abs(o - ref)
    worst = float(np.max(err / bound)) if o.size else 0.0
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(l), ~fin), f"{name}: lse -inf pattern differs"
    lerr = float(np.max(np.abs(l[fin] - rl[fin]))) if fin.any() else 0.0
    say(f"{name}: out max-abs {float(err.max()) if o.size else 0:.3e}, worst err/bound {worst:.3f}, "
        f"mean abs {float(err.mean()) if o.size else 0:.2e}; lse max-abs {lerr:.2e}")
    assert worst <= 1.0, f"{name}: output outside the derived bound (worst ratio {worst:.3f})"
    assert lerr <= LSE_TOL, f"{name}: lse error {lerr:.3e}"


CASES = [
    # B, Hq, Hkv, Lq, Lk, D, causal, window
    (1, 2, 1, 128, 128, 64, False, -1),
    (2, 4, 2, 200, 333, 128, True, -1),
    (1, 4, 1, 300, 150, 64, True, -1),
    (1, 2, 2, 257, 257, 128, True, 64),
    (2, 6, 3, 100, 77, 64, False, 20),
    (1, 8, 2, 129, 1000, 128, False, -1),
    (1, 3, 1, 1, 65, 64, True, -1),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fp8_cases(gpu_lib, case):
    B, Hq, Hkv, Lq, Lk, D, causal, window = CASES[case]
    say(f"[case] fp8 {case}: B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} D{D} causal{causal} w{window}")
    cfg = DenseConfig(f"fp8_{case}", B, Hq, Hkv, Lq, Lk, D, "fp8", causal, window, 900 + case)
    q, k, v = dense_inputs(cfg)
    out, lse = run_fp8(gpu_lib, q, k, v, cfg.scale, causal, window)
    check_fp8(f"fp8 {case}", out, lse, q, k, v, cfg.scale, causal, window)


def test_fp8_descale_factors(gpu_lib):
    cfg = DenseConfig("fp8_descale", 1, 4, 2, 190, 190, 128, "fp8", True, -1, 950)
    q, k, v = dense_inputs(cfg)
    say("[case] fp8 descale factors 0.5, 2.5, 0.25")
    out, lse = run_fp8(gpu_lib, q, k, v, cfg.scale, True, -1, 0.5, 2.5, 0.25)
    check_fp8("fp8 descale", out, lse, q, k, v, cfg.scale, True, -1, 0.5, 2.5, 0.25)


@pytest.mark.parametrize("name", ["fp8_causal", "gqa8k_causal_fp8"])
def test_fp8_workloads_sampled_rows(gpu_lib, name):
    cfg = CONFIGS[name]
    say(f"[case] fp8 workload {name} (sampled rows)")
    q, k, v = dense_inputs(cfg)
    out, lse = run_fp8(gpu_lib, q, k, v, cfg.scale, cfg.causal, cfg.window)
    # one row from every 32-row wave group of every q-block, plus both ends
    per_group = np.arange(0, cfg.Lq, 32) + np.random.default_rng(cfg.seed).integers(0, 32, size=-(-cfg.Lq // 32))
    rows = np.unique(np.concatenate([np.arange(0, 130), np.minimum(per_group, cfg.Lq - 1),
                                     np.arange(cfg.Lq - 70, cfg.Lq)]))
    check_fp8(name, out, lse, q, k, v, cfg.scale, cfg.causal, cfg.window, rows=rows)


@pytest.mark.parametrize("name", ["fp8_causal", "gqa8k_causal_fp8"])
def test_fp8_workloads_first_and_last_kv_head_all_rows(gpu_lib, name):
    """The FP8 workloads at full size, every head run on the GPU; heads are
    independent, so the query heads of the first and the last KV head are
    compared with the oracle on every row."""
    cfg = CONFIGS[name]
    q, k, v = dense_inputs(cfg)
    out, lse = run_fp8(gpu_lib, q, k, v, cfg.scale, cfg.causal, cfg.window)
    group = cfg.Hq // cfg.Hkv
    gs = [0, cfg.Hkv - 1]
    hs = [h for h in range(cfg.Hq) if h // group in gs]
    say(f"[case] fp8 workload {name} (KV heads {gs}, all rows)")
    check_fp8(f"{name} KV heads {gs}", out[:, :, hs], lse[:, hs], q[:, :, hs], k[:, :, gs], v[:, :, gs], cfg.scale,
              cfg.causal, cfg.window)


def test_fp8_deterministic_bitwise(gpu_lib):
    cfg = DenseConfig("fp8_det", 1, 8, 2, 300, 300, 128, "fp8", True, -1, 960)
    q, k, v = dense_inputs(cfg)
    a = run_fp8(gpu_lib, q, k, v, cfg.scale, True, -1)
    b = run_fp8(gpu_lib, q, k, v, cfg.scale, True, -1)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("scale", [-0.09, 0.0])
def test_fp8_negative_and_zero_scale(gpu_lib, scale):
    # the kernel moves a negative scale into Q (sign flip of every e4m3 byte)
    # and zeroes Q for a zero scale (uniform attention over the visible keys)
    cfg = DenseConfig("fp8_sign", 1, 4, 2, 150, 190, 128, "fp8", True, -1, 970)
    q, k, v = dense_inputs(cfg)
    say(f"[case] fp8 scale {scale}")
    out, lse = run_fp8(gpu_lib, q, k, v, scale, True, -1, 1.5, 1.0, 0.5)
    check_fp8(f"fp8 scale {scale}", out, lse, q, k, v, scale, True, -1, 1.5, 1.0, 0.5)


def _rand_fp8_cases(n=10):
    r = np.random.default_rng(9753)
    out = []
    for i in range(n):
        D = int(r.choice([64, 128]))
        Hkv = int(r.choice([1, 2]))
        Hq = Hkv * int(r.choice([1, 2, 4]))
        Lq, Lk = int(r.integers(1, 400)), int(r.integers(1, 400))
        causal = bool(r.integers(0, 2))
        window = int(r.choice([-1, -1, 0, 9, 150]))
        qd, kd, vd = (float(x) for x in r.choice([0.25, 0.5, 1.0, 2.0], size=3))
        out.append((i, int(r.integers(1, 3)), Hq, Hkv, Lq, Lk, D, causal, window, qd, kd, vd))
    return out


@pytest.mark.parametrize("case", _rand_fp8_cases(), ids=lambda c: f"r{c[0]}")
def test_fp8_random(gpu_lib, case):
    i, B, Hq, Hkv, Lq, Lk, D, causal, window, qd, kd, vd = case
    say(f"[case] fp8 random {i}: B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} D{D} causal{causal} w{window} "
        f"descale {qd},{kd},{vd}")
    cfg = DenseConfig(f"fp8_r{i}", B, Hq, Hkv, Lq, Lk, D, "fp8", causal, window, 980 + i)
    q, k, v = dense_inputs(cfg)
    out, lse = run_fp8(gpu_lib, q, k, v, cfg.scale, causal, window, qd, kd, vd)
    check_fp8(f"fp8 random {i}", out, lse, q, k, v, cfg.scale, causal, window, qd, kd, vd)
