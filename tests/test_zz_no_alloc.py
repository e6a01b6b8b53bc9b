"""The allocation-free decode (attn_decode_paged_static) through the C ABI.

It runs the same kernels as attn_decode_paged over a static device array
instead of a caller workspace, so on the same inputs its output and lse must
equal attn_decode_paged's bit for bit.  Two calls in a row, the second on a
smaller input, check that what the first call left in the array does not
leak into the second; a call too large for the array is refused on the host.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, PagedConfig, paged_inputs

pytestmark = pytest.mark.gpu

SCRATCH_ERR = -8


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def call_static(ta, inp, scale):
    """attn_decode_paged_static called directly through ctypes."""
    q, kc, vc, bt, cl = (t.cuda() for t in (inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens))
    S, Hq, D = q.shape
    out = torch.full_like(q, float("nan"))
    lse = torch.full((S, Hq), float("nan"), dtype=torch.float32, device="cuda")
    dtype = 1 if q.dtype == torch.bfloat16 else 0
    st = ta.load_library().attn_decode_paged_static(
        q.data_ptr(), kc.data_ptr(), vc.data_ptr(), bt.data_ptr(), cl.data_ptr(), 16, out.data_ptr(),
        lse.data_ptr(), S, Hq, kc.shape[2], D, bt.shape[1], kc.shape[0], ctypes.c_float(scale), dtype, None)
    assert st == 0, ta.attn_status_string(st)
    torch.cuda.synchronize()
    return out, lse


def call_workspace(ta, inp, scale):
    q, kc, vc, bt, cl = (t.cuda() for t in (inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens))
    out, lse = ta.attn_decode_paged(q, kc, vc, bt, cl, scale=scale)
    torch.cuda.synchronize()
    return out, lse


def test_static_decode_matches_workspace_decode_twice(gpu_lib):
    big_cfg = CONFIGS["paged_decode"]
    small_cfg = PagedConfig("static_small", 5, 12, 2, 128, "bf16", 20, 700, 16, 31)
    for name, cfg in (("paged_decode", big_cfg), ("smaller", small_cfg)):
        say(f"[case] static decode {name}: {cfg.num_seqs} seqs Hq{cfg.Hq} Hkv{cfg.Hkv} D{cfg.D}")
        inp = paged_inputs(cfg)
        so, sl = call_static(gpu_lib, inp, cfg.scale)
        wo, wl = call_workspace(gpu_lib, inp, cfg.scale)
        assert torch.equal(so, wo), f"{name}: output differs from attn_decode_paged"
        assert torch.equal(sl, wl), f"{name}: lse differs from attn_decode_paged"
        ro, rl = oracle.decode_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, 16, cfg.scale)
        err = float(np.max(np.abs(so.double().cpu().numpy() - ro)))
        lerr = float(np.max(np.abs(sl.double().cpu().numpy() - rl)))
        say(f"  bit-identical to attn_decode_paged; oracle max-abs {err:.2e}, lse {lerr:.2e}")
        assert err <= 1.6e-2 and lerr <= 1e-3


def test_static_decode_fp16_d64(gpu_lib):
    cfg = PagedConfig("static_f16", 9, 8, 1, 64, "fp16", 1, 900, 16, 32)
    say("[case] static decode fp16 D64")
    inp = paged_inputs(cfg)
    so, sl = call_static(gpu_lib, inp, cfg.scale)
    wo, wl = call_workspace(gpu_lib, inp, cfg.scale)
    assert torch.equal(so, wo) and torch.equal(sl, wl)


def test_static_decode_refuses_calls_beyond_its_scratch(gpu_lib):
    """2048 sequences of 64 query heads need far more than the array holds;
    the host refuses before any launch (the buffers below would also be a
    valid call: one 16-token block per sequence)."""
    S, Hq, Hkv, D = 2048, 64, 1, 128
    q = torch.zeros((S, Hq, D), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, 16, Hkv, D), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((S, 1), dtype=torch.int32, device="cuda")
    cl = torch.full((S,), 16, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 7.0)
    st = gpu_lib.load_library().attn_decode_paged_static(
        q.data_ptr(), kc.data_ptr(), kc.data_ptr(), bt.data_ptr(), cl.data_ptr(), 16, out.data_ptr(), None,
        S, Hq, Hkv, D, 1, 1, ctypes.c_float(0.1), 1, None)
    torch.cuda.synchronize()
    assert st == SCRATCH_ERR, gpu_lib.attn_status_string(st)
    assert torch.all(out == 7.0), "a refused call wrote its output"
