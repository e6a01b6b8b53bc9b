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
    rows = np.unique(np.concatenate([np.arange(0, 40), np.linspace(0, cfg.Lq - 1, 24).astype(np.int64),
                                     np.arange(cfg.Lq - 40, cfg.Lq)]))
    check_out(name, out, lse, q, k, v, cfg.scale, cfg.causal, cfg.window, p, 77, 1, cfg.dtype, rows=rows)


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
