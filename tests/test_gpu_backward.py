"""GPU parity of the attention backward (attn_bwd) against the fp64 oracle.

The forward runs on the GPU (its out and lse feed the backward, as in
training); the oracle differentiates the definition on the same rounded
inputs (oracle.attention_backward).  Tolerance: the forward's per-dtype bound
(2e-3 fp16, 1.6e-2 bf16) scaled by the gradient's magnitude, max(1, max|ref|):
each gradient is a sum of products whose 16-bit factors (P, dS and the saved
output) carry one rounding each, plus one rounding of the result.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, DTYPES, dense_inputs, random_dense

pytestmark = pytest.mark.gpu

GTOL = {"fp16": 2e-3, "bf16": 1.6e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _dout(shape, dtype, seed):
    r = np.random.default_rng(seed)
    return torch.from_numpy(r.standard_normal(size=shape, dtype=np.float32)).to(DTYPES[dtype])


def run_bwd(ta, q, k, v, do, scale, causal, window):
    qd, kd, vd, dod = (t.to("cuda") for t in (q, k, v, do))
    out, lse = ta.attn_fwd(qd, kd, vd, scale=scale, causal=causal, window=window)
    dq, dk, dv = ta.attn_bwd(qd, kd, vd, out, dod, lse, scale=scale, causal=causal, window=window)
    torch.cuda.synchronize()
    return dq, dk, dv


def check_grads(name, got, ref, dtype):
    msgs = []
    for n, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = g.double().cpu().numpy()
        assert not np.isnan(g).any(), f"{name}: NaN in {n}"
        err = float(np.max(np.abs(g - r))) if g.size else 0.0
        mag = max(1.0, float(np.max(np.abs(r)))) if r.size else 1.0
        msgs.append(f"{n} max-abs {err:.3e} (|ref| max {mag:.2f}, tol {GTOL[dtype] * mag:.2e})")
        assert err <= GTOL[dtype] * mag, f"{name}: " + "; ".join(msgs)
    say(f"{name}: " + "; ".join(msgs))


CASES = [
    # B, Hq, Hkv, Lq, Lk, D, dtype, causal, window
    (1, 2, 1, 128, 128, 64, "fp16", False, -1),
    (2, 4, 2, 200, 333, 128, "bf16", True, -1),
    (1, 4, 1, 300, 150, 64, "bf16", True, -1),
    (1, 2, 2, 257, 257, 128, "fp16", True, 64),
    (2, 6, 3, 100, 77, 64, "bf16", False, 20),
    (1, 8, 2, 129, 129, 128, "bf16", False, -1),
    (1, 3, 1, 1, 65, 64, "fp16", True, -1),
    (1, 2, 1, 70, 1, 128, "fp16", False, -1),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_backward_cases(gpu_lib, case):
    B, Hq, Hkv, Lq, Lk, D, dtype, causal, window = CASES[case]
    say(f"[case] backward {case}: B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} D{D} {dtype} causal{causal} w{window}")
    q, k, v = random_dense(B, Hq, Hkv, Lq, Lk, D, dtype, 300 + case)
    do = _dout(q.shape, dtype, 400 + case)
    scale = 1.0 / np.sqrt(D)
    got = run_bwd(gpu_lib, q, k, v, do, scale, causal, window)
    ref = oracle.attention_backward(q, k, v, do, scale, causal, window)
    check_grads(f"backward {case}", got, ref, dtype)


def _rand_cases(n=16):
    r = np.random.default_rng(4321)
    out = []
    for i in range(n):
        D = int(r.choice([64, 128]))
        dtype = str(r.choice(["fp16", "bf16"]))
        Hkv = int(r.choice([1, 2]))
        Hq = Hkv * int(r.choice([1, 2, 4]))
        Lq = int(r.integers(1, 260))
        Lk = int(r.integers(1, 260))
        causal = bool(r.integers(0, 2))
        window = int(r.choice([-1, -1, 0, 5, 100]))
        out.append((i, int(r.integers(1, 3)), Hq, Hkv, Lq, Lk, D, dtype, causal, window))
    return out


@pytest.mark.parametrize("case", _rand_cases(), ids=lambda c: f"r{c[0]}")
def test_backward_random(gpu_lib, case):
    i, B, Hq, Hkv, Lq, Lk, D, dtype, causal, window = case
    say(f"[case] backward random {i}: B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} D{D} {dtype} causal{causal} w{window}")
    q, k, v = random_dense(B, Hq, Hkv, Lq, Lk, D, dtype, 500 + i)
    do = _dout(q.shape, dtype, 600 + i)
    got = run_bwd(gpu_lib, q, k, v, do, 0.125, causal, window)
    ref = oracle.attention_backward(q, k, v, do, 0.125, causal, window)
    check_grads(f"backward random {i}", got, ref, dtype)


@pytest.mark.parametrize("name", ["std512_causal", "std2048"])
def test_backward_workloads(gpu_lib, name):
    cfg = CONFIGS[name]
    say(f"[case] backward workload {name}")
    q, k, v = dense_inputs(cfg)
    do = _dout(q.shape, cfg.dtype, 700)
    got = run_bwd(gpu_lib, q, k, v, do, cfg.scale, cfg.causal, cfg.window)
    ref = oracle.attention_backward(q, k, v, do, cfg.scale, cfg.causal, cfg.window)
    check_grads(f"backward {name}", got, ref, cfg.dtype)


@pytest.mark.parametrize("name", ["gqa8k_causal", "gqa8k_window"])
def test_backward_long_gqa_two_kv_heads_in_full(gpu_lib, name):
    """The long GQA backward at its full size (B1 Hq32 Hkv8 L8192 D128 bf16,
    causal, and with the 4096-key window), every head run on the GPU in the
    launch configuration the bench times.  Heads are independent, so the
    oracle differentiates the first and the last KV head with their query
    heads (8 of the 32, about 20 s of CPU) and every element of their dQ, dK
    and dV is compared: all rows and all keys."""
    cfg = CONFIGS[name]
    say(f"[case] backward workload {name} (KV heads 0 and {cfg.Hkv - 1} in full)")
    q, k, v = dense_inputs(cfg)
    do = _dout(q.shape, cfg.dtype, 701)
    dq, dk, dv = run_bwd(gpu_lib, q, k, v, do, cfg.scale, cfg.causal, cfg.window)
    group = cfg.Hq // cfg.Hkv
    gs = [0, cfg.Hkv - 1]
    hs = [h for h in range(cfg.Hq) if h // group in gs]
    got = (dq[:, :, hs].cpu(), dk[:, :, gs].cpu(), dv[:, :, gs].cpu())
    del dq, dk, dv
    ref = oracle.attention_backward(q[:, :, hs], k[:, :, gs], v[:, :, gs], do[:, :, hs], cfg.scale, cfg.causal,
                                    cfg.window)
    check_grads(f"backward {name} (KV heads {gs})", got, ref, cfg.dtype)


def test_backward_deterministic_bitwise(gpu_lib):
    q, k, v = random_dense(2, 8, 2, 300, 300, 128, "bf16", 801)
    do = _dout(q.shape, "bf16", 802)
    a = run_bwd(gpu_lib, q, k, v, do, 0.1, True, -1)
    b = run_bwd(gpu_lib, q, k, v, do, 0.1, True, -1)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_empty_sizes(gpu_lib):
    ta = gpu_lib
    q, k, v = (t.to("cuda") for t in random_dense(1, 2, 1, 5, 7, 64, "fp16", 803))
    out, lse = ta.attn_fwd(q, k, v, causal=False)
    do = torch.ones_like(q)
    # Lq = 0: dk and dv are empty sums
    dk = torch.full_like(k, 3.0)
    dv = torch.full_like(v, 3.0)
    ta.attn_bwd(q[:, :0], k, v, out[:, :0], do[:, :0], lse[:, :, :0], dk=dk, dv=dv)
    # Lk = 0: dq is an empty sum (the rows see no key: lse = -inf)
    o0, l0 = ta.attn_fwd(q, k[:, :0], v[:, :0])
    dq = torch.full_like(q, 3.0)
    ta.attn_bwd(q, k[:, :0], v[:, :0], o0, do, l0, dq=dq)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0) and torch.all(dq == 0)
