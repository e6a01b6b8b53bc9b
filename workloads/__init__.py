"""Seeded synthetic inputs for the attention forward and the paged decode.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  The fp64 oracle, the GPU parity tests and the benchmark
all take their inputs from here, so both sides see identical bits.

Workload shapes follow the pages:
  * [batch, seq, heads, dim] layout and the MQA/GQA and sliding-window options
    of the "Flash Attention" skill page, scenario 2 (steps 2 and 3);
  * the [2, 8, 512|2048, 64] fp16 tensors of its quick start and scenario 1;
  * ViT-B/16: N = 196 patch tokens, 12 heads, model dim 768, from
    "Самовнимание, ядра CUDA и FlashAttention", section 1;
  * a paged KV cache of 16-token blocks behind a block table, from the
    the-ai.news article, section "Внимание типа FlashAttention и постраничное
    внимание".

Recipe (identical for every consumer):
  * rng = numpy.random.default_rng(seed);
  * dense workloads draw q, k, v in that order as float32 standard normals
    and cast them to fp16/bf16/float8_e4m3fn with round-to-nearest-even
    (torch's cast);
  * the paged workload draws ctx_lens (integers, inclusive range), then the
    physical-block permutation, then q, then the K pool, then the V pool;
  * the paged prefill workload (Lq new tokens per sequence, the last Lq
    positions of its context) follows the same order, with q [B, Lq, Hq, D].
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


@dataclasses.dataclass(frozen=True)
class DenseConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lk: int
    D: int
    dtype: str
    causal: bool
    window: int  # -1: no sliding window
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


@dataclasses.dataclass(frozen=True)
class PagedConfig:
    name: str
    num_seqs: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    ctx_min: int
    ctx_max: int  # inclusive
    block_size: int
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def max_blocks_per_seq(self) -> int:
        return -(-self.ctx_max // self.block_size)


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    """Paged prefill: Lq new query tokens per sequence over a paged context of
    ctx_lens[b] >= Lq positions (the new tokens are the last Lq of them)."""
    name: str
    B: int
    Lq: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    ctx_min: int
    ctx_max: int  # inclusive
    block_size: int
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def max_blocks_per_seq(self) -> int:
        return -(-self.ctx_max // self.block_size)


# The five workloads.  Seeds: 1 tiny, 2/3 standard L=512/2048, 4 ViT,
# 5 long GQA, 6 paged decode.
CONFIGS = {
    "tiny": DenseConfig("tiny", 1, 2, 2, 128, 128, 64, "fp16", False, -1, 1),
    "std512": DenseConfig("std512", 2, 8, 8, 512, 512, 64, "fp16", False, -1, 2),
    "std512_causal": DenseConfig("std512_causal", 2, 8, 8, 512, 512, 64, "fp16", True, -1, 2),
    "std2048": DenseConfig("std2048", 2, 8, 8, 2048, 2048, 64, "fp16", False, -1, 3),
    "std2048_causal": DenseConfig("std2048_causal", 2, 8, 8, 2048, 2048, 64, "fp16", True, -1, 3),
    "vit": DenseConfig("vit", 64, 12, 12, 196, 196, 64, "bf16", False, -1, 4),
    "gqa8k_causal": DenseConfig("gqa8k_causal", 1, 32, 8, 8192, 8192, 128, "bf16", True, -1, 5),
    "gqa8k_window": DenseConfig("gqa8k_window", 1, 32, 8, 8192, 8192, 128, "bf16", True, 4096, 5),
    "paged_decode": PagedConfig("paged_decode", 64, 12, 2, 128, "bf16", 512, 4096, 16, 6),
    # FP8 (e4m3fn) forward: the [2, 4096, 32, 64] causal shape of the skill
    # page's FP8 scenario, and the long causal GQA workload in fp8
    "fp8_causal": DenseConfig("fp8_causal", 2, 32, 32, 4096, 4096, 64, "fp8", True, -1, 8),
    "gqa8k_causal_fp8": DenseConfig("gqa8k_causal_fp8", 1, 32, 8, 8192, 8192, 128, "fp8", True, -1, 5),
    # chunked prefill on the same model shape: 512 new tokens per sequence
    "paged_prefill": PrefillConfig("paged_prefill", 16, 512, 12, 2, 128, "bf16", 512, 4096, 16, True, 7),
}


def _normals(rng: np.random.Generator, shape, dtype: str) -> torch.Tensor:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(DTYPES[dtype])


def dense_inputs(cfg: DenseConfig, seed: Optional[int] = None):
    """q [B,Lq,Hq,D], k/v [B,Lk,Hkv,D] as CPU tensors of cfg.dtype."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    q = _normals(rng, (cfg.B, cfg.Lq, cfg.Hq, cfg.D), cfg.dtype)
    k = _normals(rng, (cfg.B, cfg.Lk, cfg.Hkv, cfg.D), cfg.dtype)
    v = _normals(rng, (cfg.B, cfg.Lk, cfg.Hkv, cfg.D), cfg.dtype)
    return q, k, v


def random_dense(B, Hq, Hkv, Lq, Lk, D, dtype, seed):
    """Ad-hoc dense inputs with the same recipe (for randomised small cases)."""
    cfg = DenseConfig("adhoc", B, Hq, Hkv, Lq, Lk, D, dtype, False, -1, seed)
    return dense_inputs(cfg)


@dataclasses.dataclass
class PagedInputs:
    q: torch.Tensor            # [num_seqs, Hq, D]
    k_cache: torch.Tensor      # [num_blocks, block_size, Hkv, D]
    v_cache: torch.Tensor      # [num_blocks, block_size, Hkv, D]
    block_table: torch.Tensor  # int32 [num_seqs, max_blocks_per_seq]
    ctx_lens: torch.Tensor     # int32 [num_seqs]
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int


def paged_inputs(cfg: PagedConfig, seed: Optional[int] = None, identity_perm: bool = False,
                 ctx_lens: Optional[np.ndarray] = None, extra_blocks: int = 0) -> PagedInputs:
    """A shared KV pool holding exactly sum(ceil(ctx/bs)) blocks (+extra_blocks).

    Logical block j of sequence s lives in physical block
    perm[offset_s + j], where offset_s is the running block count of the
    sequences before s; unused table entries are 0.
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    if ctx_lens is None:
        ctx = rng.integers(cfg.ctx_min, cfg.ctx_max + 1, size=cfg.num_seqs)
    else:
        ctx = np.asarray(ctx_lens, dtype=np.int64)
        assert ctx.shape == (cfg.num_seqs,)
    bs = cfg.block_size
    nblk = -(-ctx // bs)
    num_blocks = int(nblk.sum()) + extra_blocks
    perm = np.arange(num_blocks) if identity_perm else rng.permutation(num_blocks)
    mbps = max(cfg.max_blocks_per_seq, int(nblk.max()) if len(nblk) else 0)
    table = np.zeros((cfg.num_seqs, mbps), dtype=np.int32)
    off = 0
    for s in range(cfg.num_seqs):
        table[s, : nblk[s]] = perm[off: off + nblk[s]]
        off += nblk[s]
    q = _normals(rng, (cfg.num_seqs, cfg.Hq, cfg.D), cfg.dtype)
    kc = _normals(rng, (num_blocks, bs, cfg.Hkv, cfg.D), cfg.dtype)
    vc = _normals(rng, (num_blocks, bs, cfg.Hkv, cfg.D), cfg.dtype)
    return PagedInputs(q, kc, vc, torch.from_numpy(table), torch.from_numpy(ctx.astype(np.int32)),
                       bs, num_blocks, mbps)


def poison_unused_slots(inp: PagedInputs, value: float = float("nan")) -> PagedInputs:
    """Fill every cache slot that no sequence attends (the tail of each
    sequence's last block and any extra blocks) with `value`."""
    kc = inp.k_cache.clone()
    vc = inp.v_cache.clone()
    used = torch.zeros(inp.num_blocks, inp.block_size, dtype=torch.bool)
    for s in range(inp.q.shape[0]):
        c = int(inp.ctx_lens[s])
        for j in range(-(-c // inp.block_size)):
            n = min(inp.block_size, c - j * inp.block_size)
            used[int(inp.block_table[s, j]), :n] = True
    kc[~used] = value
    vc[~used] = value
    return dataclasses.replace(inp, k_cache=kc, v_cache=vc)


def prefill_inputs(cfg: PrefillConfig, seed: Optional[int] = None, identity_perm: bool = False,
                   ctx_lens: Optional[np.ndarray] = None, extra_blocks: int = 0) -> PagedInputs:
    """Paged prefill inputs: a pool of sum(ceil(ctx/bs)) (+extra_blocks)
    permuted blocks as in paged_inputs, and q [B, Lq, Hq, D]."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    if ctx_lens is None:
        ctx = rng.integers(cfg.ctx_min, cfg.ctx_max + 1, size=cfg.B)
    else:
        ctx = np.asarray(ctx_lens, dtype=np.int64)
        assert ctx.shape == (cfg.B,)
    bs = cfg.block_size
    nblk = -(-ctx // bs)
    num_blocks = max(int(nblk.sum()) + extra_blocks, 1)
    perm = np.arange(num_blocks) if identity_perm else rng.permutation(num_blocks)
    mbps = max(cfg.max_blocks_per_seq, int(nblk.max()) if len(nblk) else 0, 1)
    table = np.zeros((cfg.B, mbps), dtype=np.int32)
    off = 0
    for s in range(cfg.B):
        table[s, : nblk[s]] = perm[off: off + nblk[s]]
        off += nblk[s]
    q = _normals(rng, (cfg.B, cfg.Lq, cfg.Hq, cfg.D), cfg.dtype)
    kc = _normals(rng, (num_blocks, bs, cfg.Hkv, cfg.D), cfg.dtype)
    vc = _normals(rng, (num_blocks, bs, cfg.Hkv, cfg.D), cfg.dtype)
    return PagedInputs(q, kc, vc, torch.from_numpy(table), torch.from_numpy(ctx.astype(np.int32)),
                       bs, num_blocks, mbps)
