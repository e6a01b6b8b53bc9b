"""Attention with dropout on the probabilities, and the counter-based random
generator that decides which probabilities are dropped.  Test infrastructure
only (see the package docstring).

The "Flash Attention" page passes dropout_p to flash_attn_func (quick start:
dropout_p=0.0; scenario 2: dropout_p=0.1 in a causal call) without saying
more.  The readings taken here:
  * dropout acts on the normalised attention probabilities P (after the row
    softmax, before the product with V), each entry kept independently with
    probability 1 - p and the kept ones multiplied by 1 / (1 - p) ("inverted"
    dropout, so that the expectation of the output is the plain output);
  * the log-sum-exp the forward exports is that of the undropped scores;
  * the random numbers come from Philox4x32-10, the counter-based generator
    of Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as
    1, 2, 3" (SC 2011), so that any element's decision can be computed on its
    own, in any order, on either side;
  * element (b, h, i, j) (batch, query head, query row, key) takes word
    j mod 4 of Philox4x32-10 at counter (floor(j / 4), floor(i / 2),
    b * Hq + h, offset) under the key (seed mod 2^32, floor(seed / 2^32)),
    and of that word the low 16 bits for even i, the high 16 bits for odd i;
    it is kept iff that 16-bit number is >= floor(p * 2^16), with p the
    float32 value of dropout_p and 0 <= p < 1.  One generator call thus
    decides four keys of two neighbouring rows.  The keep probability is
    1 - floor(p * 2^16) / 2^16, which is 1 - p for p a multiple of 2^-16 and
    otherwise above 1 - p by less than 2^-16; the kept values are still
    scaled by 1 / (1 - p).
"""
from __future__ import annotations

import math

import numpy as np

from .core import _f64, _scale64, allowed_mask, kv_head, row_softmax, scores

# Philox4x32 constants (Salmon et al. 2011, section on the Philox S-box):
# the two round multipliers and the two Weyl key increments.
PHILOX_M = (0xD2511F53, 0xCD9E8D57)
PHILOX_W = (0x9E3779B9, 0xBB67AE85)
PHILOX_ROUNDS = 10
_M32 = np.uint64(0xFFFFFFFF)


def philox4x32(counter, key, rounds: int = PHILOX_ROUNDS) -> np.ndarray:
    """Philox4x32-R of each counter under its key.

    counter: integer array [..., 4] of 32-bit words (x0, x1, x2, x3);
    key: pair (k0, k1) of 32-bit words, scalars or arrays broadcasting
    against counter[..., 0].  Returns uint32 [..., 4].

    One round multiplies x0 by M0 and x2 by M1 as 32 x 32 -> 64-bit products
    (hi, lo) and outputs (hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0); the key
    then advances by (W0, W1) modulo 2^32.  The first round uses the key as
    given.
    """
    c = np.asarray(counter, dtype=np.uint64) & _M32
    x0, x1, x2, x3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0 = np.asarray(key[0], dtype=np.uint64) & _M32
    k1 = np.asarray(key[1], dtype=np.uint64) & _M32
    m0, m1 = np.uint64(PHILOX_M[0]), np.uint64(PHILOX_M[1])
    w0, w1 = np.uint64(PHILOX_W[0]), np.uint64(PHILOX_W[1])
    for _ in range(rounds):
        p0 = m0 * x0  # both factors < 2^32: the 64-bit product is exact
        p1 = m1 * x2
        x0, x1, x2, x3 = (p1 >> np.uint64(32)) ^ x1 ^ k0, p1 & _M32, (p0 >> np.uint64(32)) ^ x3 ^ k1, p0 & _M32
        k0 = (k0 + w0) & _M32
        k1 = (k1 + w1) & _M32
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def dropout_threshold(p: float) -> int:
    """The 16-bit threshold of dropout probability p (as float32): floor(p * 2^16)."""
    p32 = float(np.float32(p))
    if not (0.0 <= p32 < 1.0):
        raise ValueError(f"dropout probability must lie in [0, 1), got {p}")
    return int(math.floor(p32 * 2.0 ** 16))


def dropout_keep(bh: int, rows, Lk: int, p: float, seed: int, offset: int, key0: int = 0) -> np.ndarray:
    """Boolean [R, Lk]: is probability (row i, key key0 + c) of the (batch,
    head) pair with linear index bh = b * Hq + h kept, for c = 0..Lk-1."""
    thr = dropout_threshold(p)
    i = np.asarray(rows, dtype=np.int64)
    g0, g1 = key0 // 4, (key0 + Lk + 3) // 4  # the 4-key groups that cover the keys
    ctr = np.empty((len(i), g1 - g0, 4), dtype=np.uint64)
    ctr[..., 0] = np.arange(g0, g1, dtype=np.uint64)[None, :]
    ctr[..., 1] = (i // 2).astype(np.uint64)[:, None]
    ctr[..., 2] = np.uint64(bh)
    ctr[..., 3] = np.uint64(offset & 0xFFFFFFFF)
    words = philox4x32(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    first = key0 - 4 * g0
    words = words.reshape(len(i), 4 * (g1 - g0))[:, first:first + Lk].astype(np.uint64)
    halves = (words >> (np.uint64(16) * (i % 2).astype(np.uint64))[:, None]) & np.uint64(0xFFFF)
    return halves >= np.uint64(thr)


def attention_dropout(q, k, v, scale: float, causal: bool = False, window: int = -1,
                      p: float = 0.0, seed: int = 0, offset: int = 0, rows=None, key0: int = 0):
    """softmax(Q K^T * scale) with dropout on the probabilities, times V.

    out_i = sum_j P_ij * keep_ij * v_j / (1 - p), with P the row softmax over
    the visible keys and keep from dropout_keep; lse is the undropped one.
    Shapes as in attention().  key0 numbers the given keys key0, key0 + 1, ...
    in the keep decisions (a slice of a longer key sequence whose earlier keys
    are invisible to every row); the masks are those of the slice.  Returns
    (out, lse) in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    assert k.shape == (B, Lk, Hkv, D) and v.shape == k.shape and Hq % Hkv == 0
    sc = _scale64(scale)
    inv_keep = 1.0 / (1.0 - float(np.float32(p)))
    dropout_threshold(p)  # validates p
    rr = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((B, len(rr), Hq, D))
    lse = np.full((B, Hq, len(rr)), -np.inf)
    ok = allowed_mask(Lq, Lk, causal, window, rr)
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            P, ls = row_softmax(scores(q[b, rr, h, :], k[b, :, g, :], sc), ok)
            keep = dropout_keep(b * Hq + h, rr, Lk, p, seed, offset, key0)
            out[b, :, h, :] = (np.where(keep, P, 0.0) @ v[b, :, g, :]) * inv_keep
            lse[b, h, :] = ls
    return out, lse


def attention_dropout_backward(q, k, v, dout, scale: float, causal: bool = False, window: int = -1,
                               p: float = 0.0, seed: int = 0, offset: int = 0):
    """Gradients of L = sum(dout * attention_dropout(q, k, v, ...)) for a
    fixed draw of the dropout mask (same seed and offset).

    With M = keep / (1 - p) the forward is O = (P * M) V, so the chain rule
    gives dV = (P * M)^T dO and dP = (dO V^T) * M; the softmax Jacobian and
    the score products are those of the plain backward:
        dS = P * (dP - sum_j P_ij dP_ij),  dQ = scale * dS K,  dK = scale * dS^T Q.
    (sum_j P_ij dP_ij equals sum_d dO_id O_id, the dropped output's row dot
    product, as without dropout.)  Returns (dq, dk, dv) in float64.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    assert k.shape == (B, Lk, Hkv, D) and v.shape == k.shape and do.shape == q.shape and Hq % Hkv == 0
    sc = _scale64(scale)
    inv_keep = 1.0 / (1.0 - float(np.float32(p)))
    dropout_threshold(p)
    rr = np.arange(Lq)
    ok = allowed_mask(Lq, Lk, causal, window, rr)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            P, _ = row_softmax(scores(q[b, :, h, :], k[b, :, g, :], sc), ok)
            Mk = np.where(dropout_keep(b * Hq + h, rr, Lk, p, seed, offset), inv_keep, 0.0)
            dO = do[b, :, h, :]
            dv[b, :, g, :] += (P * Mk).T @ dO
            dP = (dO @ v[b, :, g, :].T) * Mk
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dq[b, :, h, :] = sc * (dS @ k[b, :, g, :])
            dk[b, :, g, :] += sc * (dS.T @ q[b, :, h, :])
    return dq, dk, dv
