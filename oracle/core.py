"""Plain fp64 attention (definition), its blocked/online and split forms, and
the paged gather.  Test infrastructure only; see the package docstring."""
from __future__ import annotations

import numpy as np

_ROW_CHUNK = 1024  # rows of the explicit score matrix held at once


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: upcast exactly on the CPU
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def _scale64(scale: float) -> float:
    """The fp32 value a kernel receives, widened exactly to fp64."""
    return float(np.float32(scale))


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """KV head used by query head h: contiguous groups of Hq // Hkv query
    heads share one K/V head (MQA/GQA of the "Flash Attention" page,
    scenario 2, step 3)."""
    return h // (Hq // Hkv)


def scores(q_rows: np.ndarray, k_rows: np.ndarray, sc: float) -> np.ndarray:
    """Scaled scores q_i . k_j * sc for a block of query rows and keys (the
    Scores equation, "Самовнимание, ядра CUDA и FlashAttention", section 1)."""
    return sc * (q_rows @ k_rows.T)


def allowed_mask(Lq: int, Lk: int, causal: bool, window: int, rows=None) -> np.ndarray:
    """Boolean [R, Lk]: may query row i see key j.

    Causal ("causal=True" of the flash-attn call on the "Flash Attention"
    page, quick start and scenario 2) is aligned bottom-right; the sliding
    window is scenario 2, step 3's window_size=(W, W) (left only when causal).
    """
    i = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    j = np.arange(Lk)
    rel = j[None, :] - (i[:, None] + (Lk - Lq))  # key position relative to the query's diagonal
    ok = np.ones((len(i), Lk), dtype=bool)
    if causal:
        ok &= rel <= 0
    if window >= 0:
        ok &= rel >= -window
        if not causal:
            ok &= rel <= window
    return ok


def row_softmax(S: np.ndarray, ok: np.ndarray):
    """Row softmax over the allowed entries of a score block.

    Returns (P, lse): P's allowed entries in each non-empty row sum to one
    ("Самовнимание, ядра CUDA и FlashAttention", section 1); lse is the
    natural log of each row's sum of exponentials; empty rows give P = 0 and
    lse = -inf.
    """
    S = np.where(ok, S, -np.inf)
    m = S.max(axis=1) if S.shape[1] else np.full(S.shape[0], -np.inf)
    has = np.isfinite(m)
    base = np.where(has, m, 0.0)
    e = np.where(ok, np.exp(S - base[:, None]), 0.0)
    l = e.sum(axis=1)
    P = e / np.where(has, l, 1.0)[:, None]
    lse = np.where(has, base + np.log(np.where(has, l, 1.0)), -np.inf)
    return P, lse


def attention(q, k, v, scale: float, causal: bool = False, window: int = -1, rows=None):
    """softmax(Q K^T * scale) V per (batch, query head), explicitly.

    q [B,Lq,Hq,D], k/v [B,Lk,Hkv,D] (any float dtype, upcast exactly).
    rows: optional subset of query rows (for sampled checks at full size).
    Returns (out [B,R,Hq,D], lse [B,Hq,R]) in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    assert k.shape == (B, Lk, Hkv, D) and v.shape == k.shape and Hq % Hkv == 0
    sc = _scale64(scale)
    rr = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rr)
    out = np.zeros((B, R, Hq, D))
    lse = np.full((B, Hq, R), -np.inf)
    for r0 in range(0, R, _ROW_CHUNK):
        sel = rr[r0:r0 + _ROW_CHUNK]
        ok = allowed_mask(Lq, Lk, causal, window, sel)
        for b in range(B):
            for h in range(Hq):
                g = kv_head(h, Hq, Hkv)
                S = scores(q[b, sel, h, :], k[b, :, g, :], sc)
                P, ls = row_softmax(S, ok)
                out[b, r0:r0 + len(sel), h, :] = P @ v[b, :, g, :]
                lse[b, h, r0:r0 + len(sel)] = ls
    return out, lse


def online_attention(q, k, v, scale: float, causal: bool = False, window: int = -1, block_n: int = 64):
    """The blocked evaluation the pages describe, in fp64.

    Keys/values are visited block by block; each row keeps a running maximum m
    and normaliser l, rescales its partial output when m grows, and is
    normalised once at the end ("Самовнимание, ядра CUDA и FlashAttention",
    section 3, the online-softmax trick; the-ai.news article, section on
    FlashAttention: per block, partial scores, updated softmax statistics and
    an output accumulated on chip).  Must equal `attention` up to rounding.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    assert Hq % Hkv == 0
    sc = _scale64(scale)
    ok_all = allowed_mask(Lq, Lk, causal, window)
    out = np.zeros((B, Lq, Hq, D))
    lse = np.full((B, Hq, Lq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            m = np.full(Lq, -np.inf)
            l = np.zeros(Lq)
            acc = np.zeros((Lq, D))
            for j0 in range(0, Lk, block_n):
                j1 = min(Lk, j0 + block_n)
                ok = ok_all[:, j0:j1]
                S = np.where(ok, scores(q[b, :, h, :], k[b, j0:j1, g, :], sc), -np.inf)
                m_new = np.maximum(m, S.max(axis=1))
                live = np.isfinite(m_new)
                base = np.where(live, m_new, 0.0)
                alpha = np.where(np.isfinite(m), np.exp(m - base), 0.0)
                p = np.where(ok, np.exp(S - base[:, None]), 0.0)
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ v[b, j0:j1, g, :]
                m = m_new
            has = l > 0
            out[b, :, h, :] = acc / np.where(has, l, 1.0)[:, None]
            lse[b, h, :] = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    return out, lse


def split_merge_attention(q, k, v, scale: float, causal: bool = False, window: int = -1, chunk: int = 64):
    """Attention over key chunks evaluated independently, then merged.

    Each chunk c yields a normalised partial o_c and its lse_c; the merge is
    the online-softmax rescaling applied across chunks:
        M = max_c lse_c,  w_c = exp(lse_c - M),
        out = sum_c w_c o_c / sum_c w_c,  lse = M + ln sum_c w_c.
    This is the split-K combine used by the paged decode.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    assert Hq % Hkv == 0
    sc = _scale64(scale)
    ok_all = allowed_mask(Lq, Lk, causal, window)
    parts_o, parts_lse = [], []
    for j0 in range(0, Lk, chunk):
        j1 = min(Lk, j0 + chunk)
        o_c = np.zeros((B, Lq, Hq, D))
        lse_c = np.full((B, Hq, Lq), -np.inf)
        for b in range(B):
            for h in range(Hq):
                g = kv_head(h, Hq, Hkv)
                S = scores(q[b, :, h, :], k[b, j0:j1, g, :], sc)
                P, ls = row_softmax(S, ok_all[:, j0:j1])
                o_c[b, :, h, :] = P @ v[b, j0:j1, g, :]
                lse_c[b, h, :] = ls
        parts_o.append(o_c)
        parts_lse.append(lse_c)
    L = np.stack(parts_lse)                      # [C, B, Hq, Lq]
    M = L.max(axis=0)
    has = np.isfinite(M)
    w = np.where(np.isfinite(L), np.exp(L - np.where(has, M, 0.0)), 0.0)
    wsum = w.sum(axis=0)
    wo = np.einsum("cbhi,cbihd->bihd", w, np.stack(parts_o))
    out = wo / np.where(has, wsum, 1.0).transpose(0, 2, 1)[..., None]
    lse = np.where(has, M + np.log(np.where(has, wsum, 1.0)), -np.inf)
    return out, lse


def gather_paged_kv(k_cache, v_cache, block_table, ctx_lens, block_size: int, s: int):
    """Contiguous K/V [ctx, Hkv, D] of sequence s: logical position p lives in
    physical block block_table[s, p // block_size] at slot p % block_size
    (the block table of the the-ai.news article, section on FlashAttention and
    paged attention)."""
    kc, vc = _f64(k_cache), _f64(v_cache)
    table = np.asarray(block_table.cpu() if hasattr(block_table, "cpu") else block_table)
    c = int(ctx_lens[s])
    p = np.arange(c)
    blk = table[s, p // block_size].astype(np.int64)
    slot = p % block_size
    return kc[blk, slot], vc[blk, slot]


def decode_paged(q, k_cache, v_cache, block_table, ctx_lens, block_size: int, scale: float):
    """One query token per sequence against its paged context [0, ctx_len).

    q [S,Hq,D]; caches [num_blocks, block_size, Hkv, D]; returns
    (out [S,Hq,D], lse [S,Hq]) in float64.  Paging changes where elements
    live, not which elements are attended, so this is plain attention on the
    gathered K/V.
    """
    q = _f64(q)
    S_, Hq, D = q.shape
    out = np.zeros((S_, Hq, D))
    lse = np.full((S_, Hq), -np.inf)
    for s in range(S_):
        K, V = gather_paged_kv(k_cache, v_cache, block_table, ctx_lens, block_size, s)
        o, ls = attention(q[s][None, None], K[None], V[None], scale)
        out[s] = o[0, 0]
        lse[s] = ls[0, :, 0]
    return out, lse


def prefill_paged(q, k_cache, v_cache, block_table, ctx_lens, block_size: int, scale: float,
                  causal: bool = True, window: int = -1):
    """Lq new query tokens per sequence against that sequence's paged context.

    q [B,Lq,Hq,D]: the last Lq positions of each sequence, i.e. query i of
    sequence b sits at position ctx_lens[b] - Lq + i (the causal diagonal is
    aligned bottom-right, as for dense attention with Lk = ctx_lens[b]).
    K/V of positions [0, ctx_lens[b]) come through the block table exactly as
    for decode_paged; then this is plain attention.  Returns
    (out [B,Lq,Hq,D], lse [B,Hq,Lq]) in float64.
    """
    q = _f64(q)
    B, Lq, Hq, D = q.shape
    out = np.zeros((B, Lq, Hq, D))
    lse = np.full((B, Hq, Lq), -np.inf)
    for b in range(B):
        K, V = gather_paged_kv(k_cache, v_cache, block_table, ctx_lens, block_size, b)
        o, ls = attention(q[b][None], K[None], V[None], scale, causal=causal, window=window)
        out[b] = o[0]
        lse[b] = ls[0]
    return out, lse


def attention_backward(q, k, v, dout, scale: float, causal: bool = False, window: int = -1):
    """Gradients of L = sum(dout * attention(q, k, v)) with respect to q, k, v.

    The chain rule applied to the definition ("Самовнимание, ядра CUDA и
    FlashAttention", section 1; section 3 keeps only the normalisation
    statistics and recomputes the tiles in the backward pass, which must give
    these same values): with S = scale * Q K^T and P its row softmax over the
    visible keys,
        dV = P^T dO,   dP = dO V^T,
        dS = P * (dP - sum_j P_ij dP_ij)     (the softmax Jacobian),
        dQ = scale * dS K,   dK = scale * dS^T Q,
    per (batch, query head); a K/V head's gradients sum over the query heads
    that share it.  Rows without a visible key contribute nothing.
    Returns (dq, dk, dv) in float64, shaped like q, k, v.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    assert k.shape == (B, Lk, Hkv, D) and v.shape == k.shape and do.shape == q.shape and Hq % Hkv == 0
    sc = _scale64(scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, Lq, _ROW_CHUNK):
        sel = np.arange(r0, min(Lq, r0 + _ROW_CHUNK))
        ok = allowed_mask(Lq, Lk, causal, window, sel)
        for b in range(B):
            for h in range(Hq):
                g = kv_head(h, Hq, Hkv)
                S = scores(q[b, sel, h, :], k[b, :, g, :], sc)
                P, _ = row_softmax(S, ok)
                dO = do[b, sel, h, :]
                dv[b, :, g, :] += P.T @ dO
                dP = dO @ v[b, :, g, :].T
                dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
                dq[b, sel, h, :] = sc * (dS @ k[b, :, g, :])
                dk[b, :, g, :] += sc * (dS.T @ q[b, sel, h, :])
    return dq, dk, dv
