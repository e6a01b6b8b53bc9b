"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Tolerances are the stated bar for N(0,1) inputs: max-abs error of the output
<= 2e-3 (fp16) or 1.6e-2 (bf16), and of the log-sum-exp <= 1e-3.  Every
comparison also reports the irreducible floor |round_dtype(ref) - ref|.
Inputs come from the seeded generators in workloads/ (shared with the
oracle); small cases span several tiles and a ragged tail; every workload,
the long causal GQA ones included, is compared on all of its rows.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import (CONFIGS, DTYPES, PrefillConfig, dense_inputs, paged_inputs, poison_unused_slots,
                       prefill_inputs, random_dense)

pytestmark = pytest.mark.gpu

TOL = {"fp16": 2e-3, "bf16": 1.6e-2}
LSE_TOL = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(*ts):
    return [t.to("cuda") for t in ts]


def floor_err(ref, dtype):
    r = torch.from_numpy(ref).to(DTYPES[dtype]).double().numpy()
    return float(np.max(np.abs(r - ref))) if ref.size else 0.0


def check(name, out, lse, ref_out, ref_lse, dtype):
    o = out.double().cpu().numpy()
    assert not np.isnan(o).any(), f"{name}: NaN in output"
    err = float(np.max(np.abs(o - ref_out))) if o.size else 0.0
    fl = floor_err(ref_out, dtype)
    msg = f"{name}: out max-abs {err:.3e} (floor {fl:.3e}, tol {TOL[dtype]:.1e})"
    if lse is not None:
        l = lse.double().cpu().numpy()
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isneginf(l), ~fin), f"{name}: lse -inf pattern differs"
        lerr = float(np.max(np.abs(l[fin] - ref_lse[fin]))) if fin.any() else 0.0
        msg += f"; lse max-abs {lerr:.3e}"
        assert lerr <= LSE_TOL, msg
    say(msg)
    assert err <= TOL[dtype], msg


def run_fwd(gpu_lib, q, k, v, scale, causal, window):
    qd, kd, vd = dev(q, k, v)
    out, lse = gpu_lib.attn_fwd(qd, kd, vd, scale=scale, causal=causal, window=window)
    torch.cuda.synchronize()
    return out, lse


# ------------------------------------------------------------ the five workloads

@pytest.mark.parametrize("name", ["tiny", "std512", "std512_causal", "std2048", "std2048_causal", "vit"])
def test_workload_full(gpu_lib, name):
    cfg = CONFIGS[name]
    say(f"[case] workload {name}")
    q, k, v = dense_inputs(cfg)
    out, lse = run_fwd(gpu_lib, q, k, v, cfg.scale, cfg.causal, cfg.window)
    ro, rl = oracle.attention(q, k, v, cfg.scale, cfg.causal, cfg.window)
    check(name, out, lse, ro, rl, cfg.dtype)


def oracle_by_kv_group(q, k, v, scale, causal, window, workers=None):
    """oracle.attention on every row, one KV group (its K/V head and the query
    heads that share it) per worker thread.  The groups are independent, so
    the result is the same array as one call over all heads; numpy's matmul
    and elementwise work release the GIL, and BLAS runs one thread per worker."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    import threadpoolctl

    q64, k64, v64 = (t.double().numpy() for t in (q, k, v))
    Hq, Hkv = q64.shape[2], k64.shape[2]
    rep = Hq // Hkv
    n = workers or max(1, min(16, len(os.sched_getaffinity(0)), Hkv))

    def one(g):
        return oracle.attention(q64[:, :, rep * g:rep * (g + 1)], k64[:, :, g:g + 1], v64[:, :, g:g + 1], scale,
                                causal, window)

    with threadpoolctl.threadpool_limits(1), ThreadPoolExecutor(n) as ex:
        parts = list(ex.map(one, range(Hkv)))
    return np.concatenate([p[0] for p in parts], axis=2), np.concatenate([p[1] for p in parts], axis=1)


@pytest.mark.parametrize("name", ["gqa8k_causal", "gqa8k_window"])
def test_workload_gqa8k_all_rows(gpu_lib, name):
    """The long causal GQA workload, plain and with the 4096-key window:
    every one of the 8192 query rows of all 32 heads against the oracle."""
    cfg = CONFIGS[name]
    say(f"[case] workload {name} (all rows)")
    q, k, v = dense_inputs(cfg)
    out, lse = run_fwd(gpu_lib, q, k, v, cfg.scale, cfg.causal, cfg.window)
    ro, rl = oracle_by_kv_group(q, k, v, cfg.scale, cfg.causal, cfg.window)
    check(name, out, lse, ro, rl, cfg.dtype)


def test_workload_gqa8k_properties_all_rows(gpu_lib):
    """Every row at full size: finite, and for the causal run the first row is
    exactly v_0 of its KV head (one visible key)."""
    cfg = CONFIGS["gqa8k_causal"]
    q, k, v = dense_inputs(cfg)
    out, lse = run_fwd(gpu_lib, q, k, v, cfg.scale, True, -1)
    o = out.float().cpu()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    rep = cfg.Hq // cfg.Hkv
    assert torch.equal(out[0, 0].cpu(), v[0, 0].repeat_interleave(rep, dim=0))


def run_decode(gpu_lib, inp, scale, workspace=None):
    qd, kc, vc, bt, cl = dev(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens)
    out, lse = gpu_lib.attn_decode_paged(qd, kc, vc, bt, cl, scale=scale, workspace=workspace, check_table=True)
    torch.cuda.synchronize()
    return out, lse


def test_workload_paged_decode(gpu_lib):
    cfg = CONFIGS["paged_decode"]
    say("[case] workload paged_decode")
    inp = paged_inputs(cfg)
    out, lse = run_decode(gpu_lib, inp, cfg.scale)
    ro, rl = oracle.decode_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, 16, cfg.scale)
    check("paged_decode", out, lse, ro, rl, cfg.dtype)


# ------------------------------------------------------------ randomised small shapes

def _rand_cases(n=48):
    r = np.random.default_rng(1234)
    cases = []
    for i in range(n):
        D = int(r.choice([64, 128]))
        dtype = str(r.choice(["fp16", "bf16"]))
        Hkv = int(r.choice([1, 2, 3]))
        Hq = Hkv * int(r.choice([1, 2, 4]))
        Lq = int(r.integers(1, 301))
        Lk = int(r.integers(1, 301))
        if i % 4 == 0:
            Lk = Lq
        causal = bool(r.integers(0, 2))
        window = int(r.choice([-1, -1, 0, 1, 17, 64, 130]))
        B = int(r.integers(1, 3))
        cases.append((i, B, Hq, Hkv, Lq, Lk, D, dtype, causal, window))
    return cases


@pytest.mark.parametrize("case", _rand_cases(), ids=lambda c: "r{}_B{}_H{}-{}_L{}x{}_D{}_{}_c{}_w{}".format(*c))
def test_random_small(gpu_lib, case):
    i, B, Hq, Hkv, Lq, Lk, D, dtype, causal, window = case
    say(f"[case] random {case}")
    q, k, v = random_dense(B, Hq, Hkv, Lq, Lk, D, dtype, seed=1000 + i)
    scale = 1.0 / math.sqrt(D)
    out, lse = run_fwd(gpu_lib, q, k, v, scale, causal, window)
    ro, rl = oracle.attention(q, k, v, scale, causal, window)
    check(f"random{i}", out, lse, ro, rl, dtype)


@pytest.mark.parametrize("B,H,Lq,Lk,D,dtype,window", [(8, 3, 200, 300, 128, "bf16", 100), (16, 24, 130, 77, 64, "fp16", -1),
                                                      (24, 2, 257, 257, 64, "bf16", -1)])
def test_batch_rows_per_xcd(gpu_lib, B, H, Lq, Lk, D, dtype, window):
    """Multi-head (no GQA), non-causal, batch a multiple of 8: the work-groups
    of each batch row go to one XCD.  Small grids (key-split instance) and
    large ones, against the oracle on a few batch rows."""
    say(f"[case] batch rows per XCD: B{B} H{H} Lq{Lq} Lk{Lk} D{D} {dtype} window {window}")
    q, k, v = random_dense(B, H, H, Lq, Lk, D, dtype, seed=B + H)
    scale = 1.0 / math.sqrt(D)
    out, lse = run_fwd(gpu_lib, q, k, v, scale, False, window)
    rows = [0, 5, B - 1]
    ro, rl = oracle.attention(q[rows], k[rows], v[rows], scale, False, window)
    check("batch rows per XCD", out[rows], lse[rows], ro, rl, dtype)


# ------------------------------------------------------------ edge cases

@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_no_keys_gives_zero_and_neg_inf(gpu_lib, dtype):
    q, _, _ = random_dense(2, 4, 2, 37, 1, 64, dtype, seed=5)
    k = torch.zeros(2, 0, 2, 64, dtype=q.dtype)
    kd = torch.empty(2, 0, 2, 64, dtype=q.dtype, device="cuda")
    out, lse = gpu_lib.attn_fwd(q.cuda(), kd, kd.clone(), scale=0.125)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
    assert torch.isneginf(lse).all()
    del k


def test_empty_rows_when_lq_exceeds_lk_causal(gpu_lib):
    q, k, v = random_dense(1, 2, 1, 200, 70, 128, "bf16", seed=6)
    out, lse = run_fwd(gpu_lib, q, k, v, 0.1, True, -1)
    ro, rl = oracle.attention(q, k, v, 0.1, True, -1)
    check("lq>lk causal", out, lse, ro, rl, "bf16")
    assert torch.count_nonzero(out[:, :130]) == 0


def test_zero_batch_and_zero_rows_are_noops(gpu_lib):
    q = torch.empty(0, 16, 2, 64, dtype=torch.float16, device="cuda")
    out, lse = gpu_lib.attn_fwd(q, q, q)
    assert out.shape == q.shape
    q = torch.empty(2, 0, 2, 64, dtype=torch.float16, device="cuda")
    k = torch.randn(2, 5, 2, 64, dtype=torch.float16, device="cuda")
    gpu_lib.attn_fwd(q, k, k)


@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 127, 128, 129, 255, 257])
def test_tile_boundaries_causal(gpu_lib, L):
    q, k, v = random_dense(1, 2, 1, L, L, 128, "bf16", seed=L)
    out, lse = run_fwd(gpu_lib, q, k, v, 0.0884, True, -1)
    ro, rl = oracle.attention(q, k, v, 0.0884, True, -1)
    check(f"causal L={L}", out, lse, ro, rl, "bf16")


# ------------------------------------------------------------ invariances

def test_gqa_equals_mha_with_expanded_kv_bitwise(gpu_lib):
    q, k, v = random_dense(1, 8, 2, 300, 300, 128, "bf16", seed=7)
    a, la = run_fwd(gpu_lib, q, k, v, 0.09, True, 100)
    b, lb = run_fwd(gpu_lib, q, k.repeat_interleave(4, 2), v.repeat_interleave(4, 2), 0.09, True, 100)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_deterministic_bitwise(gpu_lib):
    q, k, v = random_dense(2, 4, 2, 333, 333, 64, "fp16", seed=8)
    a, la = run_fwd(gpu_lib, q, k, v, 0.125, False, -1)
    b, lb = run_fwd(gpu_lib, q, k, v, 0.125, False, -1)
    assert torch.equal(a, b) and torch.equal(la, lb)


@pytest.mark.parametrize("Lk,causal,window", [(150, False, -1), (200, True, -1), (321, False, 70), (64, True, 0)])
def test_key_split_boundary(gpu_lib, Lk, causal, window):
    """A grid of exactly one work-group per CU runs the key-split instance
    (two 4-wave halves over alternate key tiles); one more work-group runs
    the plain one.  The same heads go through both: each result matches the
    oracle, and the shared heads agree with each other to the tolerance.
    Odd tile counts (150 keys: 3 tiles) leave half 1 a tile past the range."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    Lq, D, dtype = 128, 64, "fp16"
    say(f"[case] key split boundary: {cus} vs {cus + 1} work-groups, Lk {Lk} causal {causal} window {window}")
    q, k, v = random_dense(1, cus + 1, 1, Lq, Lk, D, dtype, seed=77)
    scale = 1.0 / math.sqrt(D)
    split_o, split_l = run_fwd(gpu_lib, q[:, :, :cus].contiguous(), k, v, scale, causal, window)
    full_o, full_l = run_fwd(gpu_lib, q, k, v, scale, causal, window)
    heads = np.unique(np.r_[0, 1, cus // 2, cus - 1, np.random.default_rng(Lk).integers(0, cus, 12)])
    ro, rl = oracle.attention(q[:, :, heads].contiguous(), k, v, scale, causal, window)
    check("split instance", split_o[:, :, heads], split_l[:, heads], ro, rl, dtype)
    check("plain instance", full_o[:, :, heads], full_l[:, heads], ro, rl, dtype)
    d = (split_o.double() - full_o[:, :, :cus].double()).abs().max().item()
    assert d <= TOL[dtype], f"split and plain instances differ by {d:.3e}"


def test_constant_v_gives_v(gpu_lib):
    q, k, _ = random_dense(1, 4, 4, 190, 190, 64, "bf16", seed=9)
    v = torch.full((1, 190, 4, 64), 0.8125, dtype=torch.bfloat16)
    out, _ = run_fwd(gpu_lib, q, k, v, 0.125, True, 37)
    assert torch.all(out.cpu() == v[0, 0, 0, 0])


def test_wide_window_equals_causal(gpu_lib):
    q, k, v = random_dense(1, 4, 2, 250, 250, 128, "bf16", seed=10)
    a, la = run_fwd(gpu_lib, q, k, v, 0.09, True, -1)
    b, lb = run_fwd(gpu_lib, q, k, v, 0.09, True, 249)
    assert torch.equal(a, b) and torch.equal(la, lb)


# ------------------------------------------------------------ paged decode variants

def _identity_placement(inp):
    """The same logical cache with physical block i holding the i-th logical
    block in sequence order (the permutation undone)."""
    import dataclasses
    nblk = [-(-int(c) // 16) for c in inp.ctx_lens]
    order = torch.cat([inp.block_table[s, :n].long() for s, n in enumerate(nblk)])
    table = torch.zeros_like(inp.block_table)
    o = 0
    for s, n in enumerate(nblk):
        table[s, :n] = torch.arange(o, o + n, dtype=torch.int32)
        o += n
    return dataclasses.replace(inp, k_cache=inp.k_cache[order].contiguous(), v_cache=inp.v_cache[order].contiguous(),
                               block_table=table)


def test_paged_permutation_invariance_bitwise(gpu_lib):
    cfg = CONFIGS["paged_decode"]
    a = paged_inputs(cfg, seed=11)
    b = _identity_placement(a)
    oa, la = run_decode(gpu_lib, a, cfg.scale)
    ob, lb = run_decode(gpu_lib, b, cfg.scale)
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    ro, rl = oracle.decode_paged(a.q, a.k_cache, a.v_cache, a.block_table, a.ctx_lens, 16, cfg.scale)
    check("paged perm", oa, la, ro, rl, "bf16")


def test_paged_nan_poisoned_unused_slots(gpu_lib):
    cfg = CONFIGS["paged_decode"]
    inp = poison_unused_slots(paged_inputs(cfg, seed=12, extra_blocks=3))
    out, lse = run_decode(gpu_lib, inp, cfg.scale)
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()
    ro, rl = oracle.decode_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, 16, cfg.scale)
    check("paged nan-poison", out, lse, ro, rl, "bf16")


@pytest.mark.parametrize("Hq,Hkv,D,dtype", [(12, 2, 128, "bf16"), (8, 8, 64, "fp16"), (32, 1, 128, "fp16"),
                                            (20, 1, 64, "bf16"), (4, 2, 128, "fp16")])
def test_paged_shapes_and_lengths(gpu_lib, Hq, Hkv, D, dtype):
    from workloads import PagedConfig
    ctx = np.array([1, 15, 16, 17, 255, 256, 257, 511, 600, 1000, 4096, 3], dtype=np.int64)
    cfg = PagedConfig("adhoc", len(ctx), Hq, Hkv, D, dtype, 1, 4096, 16, 13)
    inp = paged_inputs(cfg, ctx_lens=ctx)
    out, lse = run_decode(gpu_lib, inp, cfg.scale)
    ro, rl = oracle.decode_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, 16, cfg.scale)
    check(f"paged H{Hq}/{Hkv} D{D} {dtype}", out, lse, ro, rl, dtype)


def test_paged_zero_length_sequence(gpu_lib):
    from workloads import PagedConfig
    ctx = np.array([5, 0, 40], dtype=np.int64)
    cfg = PagedConfig("adhoc", 3, 6, 2, 128, "bf16", 0, 64, 16, 14)
    inp = paged_inputs(cfg, ctx_lens=ctx)
    out, lse = run_decode(gpu_lib, inp, cfg.scale)
    assert torch.count_nonzero(out[1]) == 0 and torch.isneginf(lse[1]).all()
    ro, rl = oracle.decode_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, 16, cfg.scale)
    check("paged with empty sequence", out, lse, ro, rl, "bf16")


def test_paged_matches_dense_forward(gpu_lib):
    """Decode of the last token equals the dense forward's last row (both GPU)."""
    from workloads import PagedConfig
    ctx = np.array([700, 333], dtype=np.int64)
    cfg = PagedConfig("adhoc", 2, 12, 2, 128, "bf16", 1, 1024, 16, 15)
    inp = paged_inputs(cfg, ctx_lens=ctx)
    out, lse = run_decode(gpu_lib, inp, cfg.scale)
    for s in range(2):
        K, V = oracle.gather_paged_kv(inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, 16, s)
        kt = torch.from_numpy(K).to(torch.bfloat16)[None]
        vt = torch.from_numpy(V).to(torch.bfloat16)[None]
        o2, l2 = run_fwd(gpu_lib, inp.q[s][None, None], kt, vt, cfg.scale, False, -1)
        assert (o2[0, 0].float() - out[s].float()).abs().max().item() <= 2 * TOL["bf16"]
        assert (l2[0, :, 0] - lse[s]).abs().max().item() <= 2 * LSE_TOL


def _paged_case(name, ctx, Hq, Hkv, D, dtype, seed):
    from workloads import PagedConfig
    ctx = np.asarray(ctx, dtype=np.int64)
    cfg = PagedConfig("adhoc", len(ctx), Hq, Hkv, D, dtype, 0, int(max(ctx.max(), 1)), 16, seed)
    return cfg, paged_inputs(cfg, ctx_lens=ctx)


def test_paged_many_tiny_sequences(gpu_lib):
    """Lengths 0..40: ranges hold several whole sequences (direct output) and
    sequences split over ranges (merged partials) in one launch."""
    say("[case] paged many tiny sequences")
    ctx = np.random.default_rng(16).integers(0, 41, size=300)
    cfg, inp = _paged_case("tiny", ctx, 8, 2, 64, "bf16", 16)
    out, lse = run_decode(gpu_lib, inp, cfg.scale)
    ro, rl = oracle.decode_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, 16, cfg.scale)
    check("paged tiny seqs", out, lse, ro, rl, "bf16")


def test_paged_more_sequences_than_one_launch(gpu_lib):
    """2100 sequences: the call is cut into launches of at most 2048."""
    say("[case] paged 2100 sequences")
    ctx = np.random.default_rng(17).integers(1, 50, size=2100)
    cfg, inp = _paged_case("many", ctx, 4, 2, 64, "fp16", 17)
    out, lse = run_decode(gpu_lib, inp, cfg.scale)
    ro, rl = oracle.decode_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, 16, cfg.scale)
    check("paged 2100 seqs", out, lse, ro, rl, "fp16")


def test_paged_long_ranges_and_wide_groups(gpu_lib):
    """256 query heads on one KV head (16 head groups of 16): few ranges per
    group, each longer than one 64-block window."""
    say("[case] paged long ranges")
    ctx = np.array([16400, 5, 20000, 16, 30001], dtype=np.int64)
    cfg, inp = _paged_case("long", ctx, 256, 1, 128, "bf16", 18)
    out, lse = run_decode(gpu_lib, inp, cfg.scale)
    ro, rl = oracle.decode_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, 16, cfg.scale)
    check("paged long ranges", out, lse, ro, rl, "bf16")


def test_paged_deterministic_bitwise(gpu_lib):
    cfg = CONFIGS["paged_decode"]
    inp = paged_inputs(cfg, seed=19)
    a, la = run_decode(gpu_lib, inp, cfg.scale)
    b, lb = run_decode(gpu_lib, inp, cfg.scale)
    assert torch.equal(a, b) and torch.equal(la, lb)


# ------------------------------------------------------------ paged prefill

def run_prefill(gpu_lib, inp, scale, causal=True, window=-1):
    q, kc, vc, bt, cl = dev(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens)
    out, lse = gpu_lib.attn_fwd_paged(q, kc, vc, bt, cl, scale=scale, causal=causal, window=window,
                                      check_table=True)
    torch.cuda.synchronize()
    return out, lse


def test_workload_paged_prefill(gpu_lib):
    cfg = CONFIGS["paged_prefill"]
    say("[case] workload paged_prefill")
    inp = prefill_inputs(cfg)
    out, lse = run_prefill(gpu_lib, inp, cfg.scale, cfg.causal)
    ro, rl = oracle.prefill_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, 16, cfg.scale,
                                  cfg.causal)
    check("paged_prefill", out, lse, ro, rl, cfg.dtype)


def _gathered(inp, b):
    """Contiguous K/V [1, ctx, Hkv, D] of sequence b (an index gather on the host)."""
    c = int(inp.ctx_lens[b])
    p = torch.arange(c)
    blk = inp.block_table[b, (p // 16)].long()
    return inp.k_cache[blk, p % 16][None], inp.v_cache[blk, p % 16][None]


@pytest.mark.parametrize("window", [-1, 300])
def test_paged_prefill_bitwise_equals_dense_kernel(gpu_lib, window):
    """Paging moves K/V, nothing else: per sequence, the dense kernel on the
    gathered K/V (Lk = ctx_len) produces the same bits."""
    cfg = PrefillConfig("pp_bitwise", 6, 200, 8, 2, 128, "bf16", 1, 900, 16, True, 41)
    say(f"[case] paged prefill bitwise vs dense, window {window}")
    inp = prefill_inputs(cfg, ctx_lens=np.array([200, 201, 64, 900, 333, 17]))
    out, lse = run_prefill(gpu_lib, inp, cfg.scale, True, window)
    for b in range(cfg.B):
        k, v = _gathered(inp, b)
        od, ld = run_fwd(gpu_lib, inp.q[b:b + 1], k, v, cfg.scale, True, window)
        assert torch.equal(out[b:b + 1], od), f"sequence {b}: output differs from the dense kernel"
        assert torch.equal(lse[b:b + 1], ld), f"sequence {b}: lse differs from the dense kernel"


PREFILL_CASES = [
    # D, dtype, Hq, Hkv, Lq, ctx_lens, causal, window
    (64, "fp16", 4, 2, 70, [1, 15, 16, 17, 63, 64, 65, 200], True, -1),
    (128, "bf16", 8, 1, 130, [130, 131, 257, 500, 1000], True, 100),
    (128, "fp16", 6, 3, 33, [33, 40, 700, 0], False, -1),
    (64, "bf16", 2, 2, 256, [1, 128, 300, 1024], False, 50),
    (128, "bf16", 12, 2, 1, [5, 4096, 16, 17], True, -1),
    (64, "fp16", 4, 4, 129, [129, 128, 0, 2000], True, 0),
    # item counts around the kernel's 64-item longest-first ordering: exactly
    # 64 (sequence, q-block) items, and 70 (the plain order)
    (128, "fp16", 2, 1, 200, [int(x) for x in np.random.default_rng(77).integers(200, 900, 32)], True, -1),
    (64, "bf16", 4, 2, 10, [int(x) for x in np.random.default_rng(78).integers(0, 300, 70)], True, -1),
]


@pytest.mark.parametrize("case", range(len(PREFILL_CASES)))
def test_paged_prefill_ragged(gpu_lib, case):
    D, dtype, Hq, Hkv, Lq, ctx, causal, window = PREFILL_CASES[case]
    cfg = PrefillConfig(f"pp{case}", len(ctx), Lq, Hq, Hkv, D, dtype, 0, max(max(ctx), 1), 16, causal, 50 + case)
    say(f"[case] paged prefill {case}: D{D} {dtype} Hq{Hq} Hkv{Hkv} Lq{Lq} ctx{ctx} causal{causal} w{window}")
    inp = poison_unused_slots(prefill_inputs(cfg, ctx_lens=np.array(ctx), extra_blocks=3))
    out, lse = run_prefill(gpu_lib, inp, cfg.scale, causal, window)
    ro, rl = oracle.prefill_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, 16, cfg.scale,
                                  causal, window)
    check(f"paged prefill {case}", out, lse, ro, rl, dtype)
