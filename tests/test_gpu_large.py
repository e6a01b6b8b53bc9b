"""GPU checks at sizes past 2 GiB per tensor, where byte offsets and buffer
ranges no longer fit 31 bits.

The oracle cannot hold such inputs whole, so each case is built so that its
exact result needs only a small part of them:
  * a sliding window at the far end of a 2^23 + 2^22-key sequence: only the
    last few hundred keys (past byte 2^31 of K and V) are visible, random,
    and the oracle runs on that slice (same bottom-right alignment);
  * the same sequence, causal without a window and with all keys zero: every
    visible key has probability 1/n, so the output is the mean of the values,
    which are constant per region (one value per head-dim column before byte
    2^31, another after it).  A tile read from the wrong region, or a buffer
    range cut at 31 bits, moves the mean by far more than the tolerance;
    the lse is ln(n);
  * a paged KV pool of more than 2 GiB whose sequences sit in its last blocks,
    random, with the oracle run on a compact copy of the blocks they use;
  * the backward of the windowed case: the oracle's gradients on the slice,
    and exactly zero dk, dv for every key outside the window;
  * the FP8 forward's windowed case over 2^24 + 4096 one-byte keys, within
    that forward's derived bound;
  * the dropout forward's windowed case, whose keep decisions use the keys'
    absolute indices (the oracle numbers the slice's keys from its start).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

TOL_BF16 = 1.6e-2
LSE_TOL = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def randn(shape, seed, dtype=torch.bfloat16):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype)


LK = (1 << 23) + (1 << 22)  # 12,582,912 keys: 3.2 GB per K or V at Hkv=1, D=128 bf16
SPLIT = 1 << 23             # first key at byte 2^31


def test_forward_window_past_2gib(gpu_lib):
    Lq, Hq, Hkv, D, W = 96, 4, 1, 128, 300
    say(f"[case] forward window {W} at the end of {LK} keys ({LK * D * 2 / 1e9:.2f} GB per K/V)")
    s0 = LK - Lq - W - 64                      # the slice that holds every visible key
    ks, vs = randn((1, LK - s0, Hkv, D), 31), randn((1, LK - s0, Hkv, D), 32)
    q = randn((1, Lq, Hq, D), 33)
    k = torch.zeros((1, LK, Hkv, D), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    k[:, s0:] = ks.to("cuda")
    v[:, s0:] = vs.to("cuda")
    scale = 1.0 / math.sqrt(D)
    out, lse = gpu_lib.attn_fwd(q.to("cuda"), k, v, scale=scale, causal=True, window=W)
    torch.cuda.synchronize()
    ref, rl = oracle.attention(q, ks, vs, scale, True, W)
    err = float(np.max(np.abs(out.double().cpu().numpy() - ref)))
    lerr = float(np.max(np.abs(lse.double().cpu().numpy() - rl)))
    say(f"  out max-abs {err:.3e}, lse max-abs {lerr:.2e}")
    assert err <= TOL_BF16 and lerr <= LSE_TOL


def test_forward_all_keys_past_2gib(gpu_lib):
    Lq, Hq, Hkv, D = 64, 2, 1, 128
    say(f"[case] forward causal over all {LK} keys, region-constant values")
    d = torch.arange(D)
    lo_val = ((d % 3) - 1).to(torch.bfloat16)        # keys before byte 2^31
    hi_val = ((d % 5) - 2).to(torch.bfloat16) * 0.5  # keys at and after it
    k = torch.zeros((1, LK, Hkv, D), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    v[:, :SPLIT] = lo_val.to("cuda")
    v[:, SPLIT:] = hi_val.to("cuda")
    q = randn((1, Lq, Hq, D), 34).to("cuda")
    out, lse = gpu_lib.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    o, l = out.double().cpu().numpy(), lse.double().cpu().numpy()
    off = LK - Lq
    worst = 0.0
    for i in (0, 1, 31, 63):
        n = i + off + 1
        ref = (SPLIT * lo_val.double().numpy() + (n - SPLIT) * hi_val.double().numpy()) / n
        for h in range(Hq):
            worst = max(worst, float(np.max(np.abs(o[0, i, h] - ref))))
            assert abs(l[0, h, i] - math.log(n)) < LSE_TOL
    say(f"  max-abs vs the exact region means {worst:.2e}")
    assert worst <= TOL_BF16


def test_paged_pool_past_2gib(gpu_lib):
    Hq, Hkv, D, bs = 4, 1, 128, 16
    n_blocks = (1 << 19) + 200                 # 2.15 GB per cache
    seqs = [3000, 17, 1, 600]
    say(f"[case] paged pool of {n_blocks} blocks, sequences in its last blocks")
    nbs = [(c + bs - 1) // bs for c in seqs]
    used = sum(nbs)
    kloc = randn((used, bs, Hkv, D), 35)
    vloc = randn((used, bs, Hkv, D), 36)
    # compact table (for the oracle) and the same blocks at the pool's end
    table_c = torch.zeros((len(seqs), max(nbs)), dtype=torch.int32)
    nxt = 0
    for s, nb in enumerate(nbs):
        table_c[s, :nb] = torch.arange(nxt, nxt + nb, dtype=torch.int32)
        nxt += nb
    base = n_blocks - used
    kc = torch.zeros((n_blocks, bs, Hkv, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kc[base:] = kloc.to("cuda")
    vc[base:] = vloc.to("cuda")
    table = (table_c + base).to("cuda")
    ctx = torch.tensor(seqs, dtype=torch.int32)
    scale = 1.0 / math.sqrt(D)

    q = randn((len(seqs), Hq, D), 37)
    out, lse = gpu_lib.attn_decode_paged(q.to("cuda"), kc, vc, table, ctx.to("cuda"), scale=scale)
    torch.cuda.synchronize()
    ref, rl = oracle.decode_paged(q, kloc, vloc, table_c, ctx, bs, scale)
    err = float(np.max(np.abs(out.double().cpu().numpy() - ref)))
    lerr = float(np.max(np.abs(lse.double().cpu().numpy() - rl)))
    say(f"  decode: out max-abs {err:.3e}, lse max-abs {lerr:.2e}")
    assert err <= TOL_BF16 and lerr <= LSE_TOL

    Lq = 16
    qp = randn((len(seqs), Lq, Hq, D), 38)
    outp, lsep = gpu_lib.attn_fwd_paged(qp.to("cuda"), kc, vc, table, ctx.to("cuda"), scale=scale, causal=True)
    torch.cuda.synchronize()
    refp, rlp = oracle.prefill_paged(qp, kloc, vloc, table_c, ctx, bs, scale, True)
    op, lp = outp.double().cpu().numpy(), lsep.double().cpu().numpy()
    err = float(np.max(np.abs(op - refp)))
    fin = np.isfinite(rlp)
    assert np.array_equal(np.isneginf(lp), ~fin)
    lerr = float(np.max(np.abs(lp[fin] - rlp[fin])))
    say(f"  prefill: out max-abs {err:.3e}, lse max-abs {lerr:.2e}")
    assert err <= TOL_BF16 and lerr <= LSE_TOL


def test_backward_window_past_2gib(gpu_lib):
    Lq, Hq, Hkv, D, W = 96, 4, 2, 128, 300
    say(f"[case] backward window {W} at the end of {LK} keys")
    s0 = LK - Lq - W - 64
    ks, vs = randn((1, LK - s0, Hkv, D), 41), randn((1, LK - s0, Hkv, D), 42)
    q, do = randn((1, Lq, Hq, D), 43), randn((1, Lq, Hq, D), 44)
    k = torch.zeros((1, LK, Hkv, D), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    k[:, s0:] = ks.to("cuda")
    v[:, s0:] = vs.to("cuda")
    qd, dod = q.to("cuda"), do.to("cuda")
    scale = 1.0 / math.sqrt(D)
    out, lse = gpu_lib.attn_fwd(qd, k, v, scale=scale, causal=True, window=W)
    dq, dk, dv = gpu_lib.attn_bwd(qd, k, v, out, dod, lse, scale=scale, causal=True, window=W)
    torch.cuda.synchronize()
    # keys outside the window get exactly zero gradients
    assert int(torch.count_nonzero(dk[:, :s0])) == 0 and int(torch.count_nonzero(dv[:, :s0])) == 0
    rq, rk, rv = oracle.attention_backward(q, ks, vs, do, scale, True, W)
    for n, g, r in (("dq", dq, rq), ("dk", dk[:, s0:], rk), ("dv", dv[:, s0:], rv)):
        err = float(np.max(np.abs(g.double().cpu().numpy() - r)))
        tol = TOL_BF16 * max(1.0, float(np.max(np.abs(r))))
        say(f"  {n} max-abs {err:.3e} (tol {tol:.2e})")
        assert err <= tol


def test_fp8_window_past_2gib(gpu_lib):
    # e4m3 keys are one byte per element: 2^24 + 4096 keys x 128 = 2.15 GB per K/V
    Lk, Lq, Hq, Hkv, D, W = (1 << 24) + 4096, 64, 2, 1, 128, 200
    say(f"[case] fp8 forward window {W} at the end of {Lk} keys")
    s0 = Lk - Lq - W - 64
    ks = randn((1, Lk - s0, Hkv, D), 51, torch.float32).to(torch.float8_e4m3fn)
    vs = randn((1, Lk - s0, Hkv, D), 52, torch.float32).to(torch.float8_e4m3fn)
    q = randn((1, Lq, Hq, D), 53, torch.float32).to(torch.float8_e4m3fn)
    k = torch.zeros((1, Lk, Hkv, D), dtype=torch.float8_e4m3fn, device="cuda")
    v = torch.zeros_like(k)
    k[:, s0:] = ks.to("cuda")
    v[:, s0:] = vs.to("cuda")
    scale = 1.0 / math.sqrt(D)
    out, lse = gpu_lib.attn_fwd_fp8(q.to("cuda"), k, v, scale=scale, causal=True, window=W)
    torch.cuda.synchronize()
    q64, k64, v64 = (t.double().numpy() for t in (q, ks, vs))
    ref, rl = oracle.attention(q64, k64, v64, scale, True, W)
    mag, _ = oracle.attention(q64, k64, np.abs(v64), scale, True, W)
    # the FP8 forward's derived bound (e4m3 probabilities, bf16 output)
    bound = 2.0 ** -4 * mag + 2.0 ** -8 * np.abs(ref) + 2e-3
    o = out.double().cpu().numpy()
    worst = float(np.max(np.abs(o - ref) / bound))
    lerr = float(np.max(np.abs(lse.double().cpu().numpy() - rl)))
    say(f"  worst err/bound {worst:.3f}, lse max-abs {lerr:.2e}")
    assert worst <= 1.0 and lerr <= LSE_TOL


def test_dropout_window_past_2gib(gpu_lib):
    # keep decisions at key indices past 12.5M (Philox counter word 0 past
    # 3.1M) and K/V addresses past byte 2^31, bit for bit: with one-hot values
    # v_j = e_(j mod D) and a causal window of D - 1 keys, output column
    # j mod D of row i is P_ij * keep_ij / (1 - p), nonzero iff (i, j) was kept
    Lq, Hq, Hkv, D, p = 96, 2, 1, 128, 0.2
    W = D - 1
    say(f"[case] dropout forward window {W} at the end of {LK} keys")
    s0 = LK - Lq - W - 64
    n = LK - s0
    ks = randn((1, n, Hkv, D), 61)
    onehot = torch.zeros((1, n, Hkv, D), dtype=torch.bfloat16)
    j = torch.arange(s0, LK)
    onehot[0, torch.arange(n), :, j % D] = 1.0
    q = randn((1, Lq, Hq, D), 63)
    k = torch.zeros((1, LK, Hkv, D), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    k[:, s0:] = ks.to("cuda")
    v[:, s0:] = onehot.to("cuda")
    scale = 1.0 / math.sqrt(D)
    seed, offset = 0xABCDEF0123, 5
    out, lse = gpu_lib.attn_fwd_dropout(q.to("cuda"), k, v, p, seed, offset, scale=scale, causal=True, window=W)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    ok = oracle.allowed_mask(Lq, n, True, W)   # the slice's own masks (bottom-right, window)
    i_idx, c_idx = np.nonzero(ok)
    total = 0
    for h in range(Hq):
        keep = oracle.dropout_keep(h, np.arange(Lq), n, p, seed, offset, key0=s0)
        got = o[0, i_idx, h, (s0 + c_idx) % D] > 0
        bad = int(np.count_nonzero(got != keep[i_idx, c_idx]))
        assert bad == 0, f"head {h}: {bad} of {len(got)} keep decisions differ"
        total += len(got)
    ref, rl = oracle.attention_dropout(q, ks, onehot, scale, True, W, p, seed, offset, key0=s0)
    err = float(np.max(np.abs(out.double().cpu().numpy() - ref)))
    lerr = float(np.max(np.abs(lse.double().cpu().numpy() - rl)))
    say(f"  {total} decisions agree; out max-abs {err:.3e}, lse max-abs {lerr:.2e}")
    assert err <= TOL_BF16 / (1.0 - float(np.float32(p))) and lerr <= LSE_TOL
