"""GPU parity of every kernel instance the host can dispatch, against the oracle.

The host picks an instance by grid size: a grid of at most one work-group per
CU runs the key-split instance (two 4-wave halves over alternate key tiles),
a larger grid the plain one.  Most small parity cases have small grids, so
this file holds, for each entry point and each (dtype, head dim) pair, a case
whose grid exceeds the CU count (the plain instance), and checks it against
the fp64 oracle with the usual bars:
  * forward: max-abs 2e-3 (fp16) / 1.6e-2 (bf16) on the output, 1e-3 on lse;
  * dropout: the same bound times 1 / (1 - p);
  * backward: the per-dtype bound times max(1, max|ref|) (times 1 / (1 - p)
    with dropout).
Each case asserts its own grid size so that a change of tile shape cannot
silently move it back under the CU count.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import DTYPES, PrefillConfig, prefill_inputs, random_dense

pytestmark = pytest.mark.gpu

TOL = {"fp16": 2e-3, "bf16": 1.6e-2}
LSE_TOL = 1e-3
BLOCK_M = 128  # query rows per forward / dQ work-group
BLOCK_N_BWD = 128  # keys per dK/dV work-group


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def q_grid(B, Hq, Lq):
    return -(-Lq // BLOCK_M) * Hq * B


def check_fwd(name, out, lse, ro, rl, tol):
    o = out.double().cpu().numpy()
    assert not np.isnan(o).any(), f"{name}: NaN in output"
    err = float(np.max(np.abs(o - ro)))
    l = lse.double().cpu().numpy()
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(l), ~fin), f"{name}: lse -inf pattern differs"
    lerr = float(np.max(np.abs(l[fin] - rl[fin]))) if fin.any() else 0.0
    msg = f"{name}: out max-abs {err:.3e} (tol {tol:.2e}); lse max-abs {lerr:.3e}"
    say(msg)
    assert err <= tol and lerr <= LSE_TOL, msg


def _dout(shape, dtype, seed):
    r = np.random.default_rng(seed)
    return torch.from_numpy(r.standard_normal(size=shape, dtype=np.float32)).to(DTYPES[dtype])


def check_grads(name, got, ref, tol):
    msgs = []
    for n, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = g.double().cpu().numpy()
        assert not np.isnan(g).any(), f"{name}: NaN in {n}"
        err = float(np.max(np.abs(g - r)))
        mag = max(1.0, float(np.max(np.abs(r))))
        msgs.append(f"{n} max-abs {err:.3e} (tol {tol * mag:.2e})")
        assert err <= tol * mag, f"{name}: " + "; ".join(msgs)
    say(f"{name}: " + "; ".join(msgs))


# Shapes with more work-groups than CUs: 9 q-blocks x 16 heads x 2 = 288.
PLAIN = [
    # B, Hq, Hkv, L, D, dtype, causal, window
    (2, 16, 4, 1100, 128, "fp16", True, -1),
    (2, 16, 4, 1100, 128, "fp16", False, 300),
    (2, 16, 4, 1100, 64, "fp16", False, -1),
    (2, 16, 4, 1100, 128, "bf16", False, -1),
    (2, 16, 4, 1100, 64, "bf16", True, 200),
]


@pytest.mark.parametrize("case", range(len(PLAIN)))
def test_dense_forward_plain_instance(gpu_lib, case):
    B, Hq, Hkv, L, D, dtype, causal, window = PLAIN[case]
    assert q_grid(B, Hq, L) > cus()
    say(f"[case] dense fwd plain instance: B{B} Hq{Hq} Hkv{Hkv} L{L} D{D} {dtype} causal{causal} w{window}")
    q, k, v = random_dense(B, Hq, Hkv, L, L, D, dtype, 2100 + case)
    scale = 1.0 / math.sqrt(D)
    out, lse = gpu_lib.attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal, window=window)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, scale, causal, window)
    check_fwd(f"dense plain {case}", out, lse, ro, rl, TOL[dtype])


DROP = [
    # B, Hq, Hkv, L, D, dtype, causal, window, p
    (2, 16, 4, 1100, 64, "fp16", True, -1, 0.1),
    (2, 16, 4, 1100, 128, "fp16", False, 250, 0.3),
    (2, 16, 4, 1100, 64, "bf16", False, -1, 0.2),
    (2, 16, 4, 1100, 128, "bf16", True, -1, 0.1),
]


@pytest.mark.parametrize("case", range(len(DROP)))
def test_dropout_forward_plain_instance(gpu_lib, case):
    B, Hq, Hkv, L, D, dtype, causal, window, p = DROP[case]
    assert q_grid(B, Hq, L) > cus()
    say(f"[case] dropout fwd plain instance: B{B} Hq{Hq} Hkv{Hkv} L{L} D{D} {dtype} causal{causal} w{window} p{p}")
    q, k, v = random_dense(B, Hq, Hkv, L, L, D, dtype, 2200 + case)
    scale = 1.0 / math.sqrt(D)
    seed, offset = 4242 + case, 3 * case
    out, lse = gpu_lib.attn_fwd_dropout(q.cuda(), k.cuda(), v.cuda(), p, seed, offset, scale=scale, causal=causal,
                                        window=window)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_dropout(q, k, v, scale, causal, window, p, seed, offset)
    check_fwd(f"dropout plain {case}", out, lse, ro, rl, TOL[dtype] / (1.0 - float(np.float32(p))))


PAGED = [
    # B, Lq, Hq, Hkv, D, dtype, ctx_min, ctx_max, causal
    (4, 600, 16, 4, 64, "fp16", 600, 1500, True),
    (4, 600, 16, 4, 128, "fp16", 600, 1500, True),
    (4, 600, 16, 4, 64, "bf16", 600, 1500, False),
    (4, 600, 16, 4, 128, "bf16", 600, 1500, True),
]


@pytest.mark.parametrize("case", range(len(PAGED)))
def test_paged_prefill_plain_instance(gpu_lib, case):
    B, Lq, Hq, Hkv, D, dtype, cmin, cmax, causal = PAGED[case]
    assert q_grid(B, Hq, Lq) > cus()
    say(f"[case] paged prefill plain instance: B{B} Lq{Lq} Hq{Hq} Hkv{Hkv} D{D} {dtype} ctx[{cmin},{cmax}] "
        f"causal{causal}")
    cfg = PrefillConfig(f"pp_plain{case}", B, Lq, Hq, Hkv, D, dtype, cmin, cmax, 16, causal, 2300 + case)
    inp = prefill_inputs(cfg)
    out, lse = gpu_lib.attn_fwd_paged(inp.q.cuda(), inp.k_cache.cuda(), inp.v_cache.cuda(),
                                      inp.block_table.cuda(), inp.ctx_lens.cuda(), scale=cfg.scale, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, 16, cfg.scale,
                                  causal)
    check_fwd(f"paged plain {case}", out, lse, ro, rl, TOL[dtype])


BWD = [
    # B, Hq, Hkv, L, D, dtype, causal, window
    (2, 16, 4, 1100, 128, "bf16", True, -1),
    (2, 16, 4, 1100, 128, "bf16", True, 300),
    (2, 16, 4, 1100, 64, "fp16", True, -1),
    (2, 16, 4, 1100, 64, "fp16", False, -1),
    (2, 16, 4, 1100, 128, "fp16", False, 200),
]


@pytest.mark.parametrize("case", range(len(BWD)))
def test_backward_plain_dq_instance(gpu_lib, case):
    """dQ grids above the CU count run the non-split dQ kernel."""
    B, Hq, Hkv, L, D, dtype, causal, window = BWD[case]
    assert q_grid(B, Hq, L) > cus()
    say(f"[case] backward plain dQ instance: B{B} Hq{Hq} Hkv{Hkv} L{L} D{D} {dtype} causal{causal} w{window}")
    q, k, v = random_dense(B, Hq, Hkv, L, L, D, dtype, 2400 + case)
    do = _dout(q.shape, dtype, 2500 + case)
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    out, lse = gpu_lib.attn_fwd(qd, kd, vd, scale=scale, causal=causal, window=window)
    got = gpu_lib.attn_bwd(qd, kd, vd, out, dod, lse, scale=scale, causal=causal, window=window)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(q, k, v, do, scale, causal, window)
    check_grads(f"backward plain {case}", got, ref, TOL[dtype])


BWD_DROP = [
    # B, Hq, Hkv, L, D, dtype, causal, window, p
    (2, 16, 4, 1100, 128, "bf16", True, -1, 0.1),
    (2, 16, 4, 1100, 64, "fp16", False, 300, 0.2),
    (2, 16, 4, 1100, 128, "fp16", True, -1, 0.3),
    (2, 16, 4, 1100, 64, "bf16", True, 150, 0.1),
]


@pytest.mark.parametrize("case", range(len(BWD_DROP)))
def test_dropout_backward_plain_dq_instance(gpu_lib, case):
    B, Hq, Hkv, L, D, dtype, causal, window, p = BWD_DROP[case]
    assert q_grid(B, Hq, L) > cus()
    say(f"[case] dropout backward plain dQ instance: B{B} Hq{Hq} Hkv{Hkv} L{L} D{D} {dtype} causal{causal} "
        f"w{window} p{p}")
    q, k, v = random_dense(B, Hq, Hkv, L, L, D, dtype, 2600 + case)
    do = _dout(q.shape, dtype, 2700 + case)
    scale = 1.0 / math.sqrt(D)
    seed, offset = 777 + case, 11 * case
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    out, lse = gpu_lib.attn_fwd_dropout(qd, kd, vd, p, seed, offset, scale=scale, causal=causal, window=window)
    got = gpu_lib.attn_bwd_dropout(qd, kd, vd, out, dod, lse, p, seed, offset, scale=scale, causal=causal,
                                   window=window)
    torch.cuda.synchronize()
    ref = oracle.attention_dropout_backward(q, k, v, do, scale, causal, window, p, seed, offset)
    check_grads(f"dropout backward plain {case}", got, ref, TOL[dtype] / (1.0 - float(np.float32(p))))
