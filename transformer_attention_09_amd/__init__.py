"""Fused attention for AMD Instinct MI355X (gfx950): Python binding of libattn.so.

Every step of the computation runs in the HIP kernels of libattn.so; this
module only marshals torch tensors (device memory and the current stream) into
the C ABI declared in include/attn.h, with the same entry-point names:

    attn_fwd(q, k, v, ...)                  q [B,Lq,Hq,D], k/v [B,Lk,Hkv,D]
    attn_fwd_dropout(q, k, v, p, seed, ...) the same with dropout on the probabilities
    attn_decode_paged(q, k_cache, ...)      q [S,Hq,D], caches [N,16,Hkv,D]
    attn_decode_paged_static(q, k_cache, ...)  the same without a workspace (no allocation)
    attn_fwd_paged(q, k_cache, ...)         q [B,Lq,Hq,D] over paged caches [N,16,Hkv,D]
    attn_bwd(q, k, v, out, dout, lse, ...)  gradients dq, dk, dv
    attn_bwd_dropout(..., p, seed, ...)     gradients of attn_fwd_dropout's output
    attn_fwd_fp8(q, k, v, ...)              float8_e4m3fn inputs, bf16 output
    attn_bwd_workspace_size(B, Hq, Lq)
    attn_decode_paged_workspace_size(...)
    attn_status_string(status)
    attn_hbm_read_probe(buf, sink)          plain streaming read (include/attn_measure.h)

There is no fallback: if the library is missing or the device is not a
gfx950 GPU the calls raise.  Build the library with
``python -m transformer_attention_09_amd.build``.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_F16, ATTN_BF16 = 0, 1
STATUS = {
    0: "ATTN_OK",
    -1: "ATTN_ERR_NULL",
    -2: "ATTN_ERR_SHAPE",
    -3: "ATTN_ERR_UNSUPPORTED",
    -4: "ATTN_ERR_ALIGN",
    -5: "ATTN_ERR_WORKSPACE",
    -6: "ATTN_ERR_DEVICE",
    -7: "ATTN_ERR_HIP",
    -8: "ATTN_ERR_SCRATCH",
}
EXPORTED = ("attn_fwd", "attn_decode_paged", "attn_decode_paged_workspace_size", "attn_status_string",
            "attn_fwd_paged", "attn_bwd", "attn_bwd_workspace_size", "attn_fwd_fp8", "attn_hbm_read_probe",
            "attn_fwd_dropout", "attn_bwd_dropout", "attn_decode_paged_static")

_lib = None
_lock = threading.Lock()


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_status_text(status)})")


def load_library() -> ctypes.CDLL:
    """Load libattn.so once; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m transformer_attention_09_amd.build`")
            lib = ctypes.CDLL(LIB_PATH)
            vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
            lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32, i32, vp]
            lib.attn_fwd.restype = i32
            lib.attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32,
                                              f32, i32, vp, sz, vp]
            lib.attn_decode_paged.restype = i32
            lib.attn_decode_paged_static.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32,
                                                     i32, f32, i32, vp]
            lib.attn_decode_paged_static.restype = i32
            lib.attn_decode_paged_workspace_size.argtypes = [i32, i32, i32, i32, i32]
            lib.attn_decode_paged_workspace_size.restype = sz
            lib.attn_status_string.argtypes = [i32]
            lib.attn_status_string.restype = ctypes.c_char_p
            lib.attn_fwd_paged.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                           f32, i32, i32, i32, vp]
            lib.attn_fwd_paged.restype = i32
            lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                     f32, i32, i32, i32, vp, sz, vp]
            lib.attn_bwd.restype = i32
            lib.attn_bwd_workspace_size.argtypes = [i32, i32, i32]
            lib.attn_bwd_workspace_size.restype = sz
            lib.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, f32, f32, f32,
                                         i32, i32, vp]
            lib.attn_fwd_fp8.restype = i32
            lib.attn_hbm_read_probe.argtypes = [vp, sz, vp, vp]
            lib.attn_hbm_read_probe.restype = i32
            lib.attn_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32,
                                             f32, ctypes.c_uint64, ctypes.c_uint32, i32, vp]
            lib.attn_fwd_dropout.restype = i32
            lib.attn_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                             f32, i32, i32, f32, ctypes.c_uint64, ctypes.c_uint32, i32,
                                             vp, sz, vp]
            lib.attn_bwd_dropout.restype = i32
            _lib = lib
    return _lib


def _status_text(status: int) -> str:
    try:
        return load_library().attn_status_string(status).decode()
    except Exception:  # noqa: BLE001 - message only
        return "?"


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float16:
        return ATTN_F16
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float16 or bfloat16")


def _stream_handle(stream) -> Optional[int]:
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream if hasattr(s, "cuda_stream") else int(s)


def _require_cuda(name, t):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _fwd_tensors(q, k, v, out, lse, scale, return_lse):
    """Check the dense forward's tensors; allocate out/lse if not given."""
    import torch

    for n, t in (("q", q), ("k", k), ("v", v)):
        _require_cuda(n, t)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("expected q [B,Lq,Hq,D] and k, v [B,Lk,Hkv,D] of equal shape")
    B, Lq, Hq, D = q.shape
    Bk, Lk, Hkv, Dk = k.shape
    if Bk != B or Dk != D or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v disagree in batch, head dim or dtype")
    if out is None:
        out = torch.empty_like(q)
    _require_cuda("out", out)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _require_cuda("lse", lse)
        if lse.shape != (B, Hq, Lq) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [B,Hq,Lq]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return out, lse, (B, Hq, Hkv, Lq, Lk, D), float(scale)


def attn_fwd(q, k, v, out=None, lse=None, scale: Optional[float] = None, causal: bool = False,
             window: int = -1, stream=None, return_lse: bool = True):
    """Fused attention forward; returns (out, lse) (lse None if not requested).

    q [B,Lq,Hq,D], k/v [B,Lk,Hkv,D]; scale defaults to 1/sqrt(D); window < 0
    disables the sliding window; causal masking is aligned bottom-right.
    """
    out, lse, dims, scale = _fwd_tensors(q, k, v, out, lse, scale, return_lse)
    st = load_library().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr() if lse is not None else None,
                                 *dims, scale, int(bool(causal)), int(window),
                                 _dtype_code(q), _stream_handle(stream))
    if st != 0:
        raise AttnError(st, "attn_fwd")
    return out, lse


def attn_fwd_dropout(q, k, v, dropout_p: float, seed: int, offset: int = 0, out=None, lse=None,
                     scale: Optional[float] = None, causal: bool = False, window: int = -1,
                     stream=None, return_lse: bool = True):
    """attn_fwd with dropout on the probabilities; returns (out, lse).

    Each probability is kept with probability 1 - dropout_p and the kept ones
    are scaled by 1 / (1 - dropout_p); the decisions come from Philox4x32-10
    keyed by the 64-bit seed, with the 32-bit offset selecting the stream
    (contract in include/attn.h).  lse is the undropped one.
    """
    out, lse, dims, scale = _fwd_tensors(q, k, v, out, lse, scale, return_lse)
    st = load_library().attn_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                         lse.data_ptr() if lse is not None else None,
                                         *dims, scale, int(bool(causal)), int(window),
                                         float(dropout_p), int(seed) & (2 ** 64 - 1), int(offset) & 0xFFFFFFFF,
                                         _dtype_code(q), _stream_handle(stream))
    if st != 0:
        raise AttnError(st, "attn_fwd_dropout")
    return out, lse


def attn_decode_paged_workspace_size(num_seqs: int, Hq: int, D: int, max_blocks_per_seq: int,
                                     block_size: int = 16) -> int:
    return int(load_library().attn_decode_paged_workspace_size(num_seqs, Hq, D, max_blocks_per_seq, block_size))


def attn_decode_paged(q, k_cache, v_cache, block_table, ctx_lens, out=None, lse=None,
                      scale: Optional[float] = None, workspace=None, stream=None,
                      return_lse: bool = True, check_table: bool = False):
    """Paged-KV decode; returns (out, lse).

    q [S,Hq,D]; k_cache/v_cache [num_blocks, block_size, Hkv, D]; block_table
    int32 [S, max_blocks_per_seq]; ctx_lens int32 [S].  check_table=True
    copies the table and lengths to the host and validates them first (it
    synchronises; meant for tests).
    """
    import torch

    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("block_table", block_table),
                 ("ctx_lens", ctx_lens)):
        _require_cuda(n, t)
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("expected q [S,Hq,D] and caches [N,block_size,Hkv,D] of equal shape")
    S, Hq, D = q.shape
    num_blocks, bs, Hkv, Dk = k_cache.shape
    if Dk != D or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and caches disagree in head dim or dtype")
    if block_table.dtype != torch.int32 or ctx_lens.dtype != torch.int32:
        raise ValueError("block_table and ctx_lens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != S or ctx_lens.shape != (S,):
        raise ValueError("block_table must be [S, max_blocks_per_seq] and ctx_lens [S]")
    mbps = block_table.shape[1]
    if check_table:
        ctx = ctx_lens.cpu()
        tab = block_table.cpu()
        if ctx.numel() and (int(ctx.min()) < 0 or int(ctx.max()) > mbps * bs):
            raise ValueError("ctx_lens outside [0, max_blocks_per_seq * block_size]")
        for s in range(S):
            n = -(-int(ctx[s]) // bs)
            if n and (int(tab[s, :n].min()) < 0 or int(tab[s, :n].max()) >= num_blocks):
                raise ValueError(f"block_table row {s} points outside the pool")
    if out is None:
        out = torch.empty_like(q)
    _require_cuda("out", out)
    if lse is None and return_lse:
        lse = torch.empty((S, Hq), dtype=torch.float32, device=q.device)
    need = attn_decode_paged_workspace_size(S, Hq, D, mbps, bs) if S else 0
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = load_library().attn_decode_paged(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                          block_table.data_ptr(), ctx_lens.data_ptr(), bs,
                                          out.data_ptr(), lse.data_ptr() if lse is not None else None,
                                          S, Hq, Hkv, D, mbps, num_blocks, float(scale), _dtype_code(q),
                                          ws_ptr, ws_bytes, _stream_handle(stream))
    if st != 0:
        raise AttnError(st, "attn_decode_paged")
    return out, lse


def attn_decode_paged_static(q, k_cache, v_cache, block_table, ctx_lens, out, lse=None,
                             scale: Optional[float] = None, stream=None):
    """Paged-KV decode that allocates nothing: the caller passes out (and lse,
    optional) and the library keeps its partial results in a static device
    array (attn_decode_paged_static in include/attn.h).  Calls that overlap in
    time on one device race; calls ordered on one stream do not."""
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("block_table", block_table),
                 ("ctx_lens", ctx_lens), ("out", out)):
        _require_cuda(n, t)
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape or out.shape != q.shape:
        raise ValueError("expected q, out [S,Hq,D] and caches [N,block_size,Hkv,D] of equal shape")
    S, Hq, D = q.shape
    num_blocks, bs, Hkv, Dk = k_cache.shape
    if Dk != D or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype or out.dtype != q.dtype:
        raise ValueError("q, out and caches disagree in head dim or dtype")
    if block_table.dim() != 2 or block_table.shape[0] != S or ctx_lens.shape != (S,):
        raise ValueError("block_table must be [S, max_blocks_per_seq] and ctx_lens [S]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = load_library().attn_decode_paged_static(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                                 block_table.data_ptr(), ctx_lens.data_ptr(), bs,
                                                 out.data_ptr(), lse.data_ptr() if lse is not None else None,
                                                 S, Hq, Hkv, D, block_table.shape[1], num_blocks, float(scale),
                                                 _dtype_code(q), _stream_handle(stream))
    if st != 0:
        raise AttnError(st, "attn_decode_paged_static")
    return out, lse


def _check_paged_table(block_table, ctx_lens, bs, num_blocks):
    """Host-side check of the device-resident table and lengths (synchronises)."""
    ctx = ctx_lens.cpu()
    tab = block_table.cpu()
    mbps = tab.shape[1]
    if ctx.numel() and (int(ctx.min()) < 0 or int(ctx.max()) > mbps * bs):
        raise ValueError("ctx_lens outside [0, max_blocks_per_seq * block_size]")
    for s in range(tab.shape[0]):
        n = -(-int(ctx[s]) // bs)
        if n and (int(tab[s, :n].min()) < 0 or int(tab[s, :n].max()) >= num_blocks):
            raise ValueError(f"block_table row {s} points outside the pool")


def attn_fwd_paged(q, k_cache, v_cache, block_table, ctx_lens, out=None, lse=None,
                   scale: Optional[float] = None, causal: bool = True, window: int = -1, stream=None,
                   return_lse: bool = True, check_table: bool = False):
    """Paged prefill; returns (out, lse).

    q [B,Lq,Hq,D]: the last Lq positions of each sequence; k_cache/v_cache
    [num_blocks, block_size, Hkv, D]; block_table int32 [B, max_blocks_per_seq];
    ctx_lens int32 [B] (context lengths including the Lq new tokens).
    check_table=True validates the table and lengths on the host first (it
    synchronises; meant for tests).
    """
    import torch

    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("block_table", block_table),
                 ("ctx_lens", ctx_lens)):
        _require_cuda(n, t)
    if q.dim() != 4 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("expected q [B,Lq,Hq,D] and caches [N,block_size,Hkv,D] of equal shape")
    B, Lq, Hq, D = q.shape
    num_blocks, bs, Hkv, Dk = k_cache.shape
    if Dk != D or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and caches disagree in head dim or dtype")
    if block_table.dtype != torch.int32 or ctx_lens.dtype != torch.int32:
        raise ValueError("block_table and ctx_lens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != B or ctx_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_blocks_per_seq] and ctx_lens [B]")
    mbps = block_table.shape[1]
    if check_table:
        _check_paged_table(block_table, ctx_lens, bs, num_blocks)
    if out is None:
        out = torch.empty_like(q)
    _require_cuda("out", out)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _require_cuda("lse", lse)
        if lse.shape != (B, Hq, Lq) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [B,Hq,Lq]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = load_library().attn_fwd_paged(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                       block_table.data_ptr(), ctx_lens.data_ptr(), bs,
                                       out.data_ptr(), lse.data_ptr() if lse is not None else None,
                                       B, Hq, Hkv, Lq, D, mbps, num_blocks, float(scale), int(bool(causal)),
                                       int(window), _dtype_code(q), _stream_handle(stream))
    if st != 0:
        raise AttnError(st, "attn_fwd_paged")
    return out, lse


def attn_bwd_workspace_size(B: int, Hq: int, Lq: int) -> int:
    return int(load_library().attn_bwd_workspace_size(B, Hq, Lq))


def _bwd_tensors(q, k, v, out, dout, lse, dq, dk, dv, scale, workspace):
    """Check the backward's tensors; allocate gradients and workspace if not given."""
    import torch

    for n, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout), ("lse", lse)):
        _require_cuda(n, t)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("expected q/out/dout [B,Lq,Hq,D] and k, v [B,Lk,Hkv,D]")
    B, Lq, Hq, D = q.shape
    Bk, Lk, Hkv, Dk = k.shape
    if Bk != B or Dk != D or any(t.dtype != q.dtype for t in (k, v, out, dout)):
        raise ValueError("q, k, v, out, dout disagree in batch, head dim or dtype")
    if lse.shape != (B, Hq, Lq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B,Hq,Lq]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for n, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _require_cuda(n, t)
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError(f"{n} must match the shape and dtype of its input")
    need = attn_bwd_workspace_size(B, Hq, Lq)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return dq, dk, dv, (B, Hq, Hkv, Lq, Lk, D), float(scale), ws_ptr, ws_bytes


def attn_bwd(q, k, v, out, dout, lse, dq=None, dk=None, dv=None, scale: Optional[float] = None,
             causal: bool = False, window: int = -1, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of sum(dout * out) for out, lse = attn_fwd(q, k, v, ...)
    called with the same scale, causal and window."""
    dq, dk, dv, dims, scale, ws_ptr, ws_bytes = _bwd_tensors(q, k, v, out, dout, lse, dq, dk, dv, scale, workspace)
    st = load_library().attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                                 lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                 *dims, scale, int(bool(causal)), int(window),
                                 _dtype_code(q), ws_ptr, ws_bytes, _stream_handle(stream))
    if st != 0:
        raise AttnError(st, "attn_bwd")
    return dq, dk, dv


def attn_bwd_dropout(q, k, v, out, dout, lse, dropout_p: float, seed: int, offset: int = 0, dq=None, dk=None,
                     dv=None, scale: Optional[float] = None, causal: bool = False, window: int = -1,
                     workspace=None, stream=None):
    """Gradients (dq, dk, dv) of sum(dout * out) for out, lse =
    attn_fwd_dropout(q, k, v, dropout_p, seed, offset, ...) called with the same
    arguments; the keep decisions are recomputed from (seed, offset)."""
    dq, dk, dv, dims, scale, ws_ptr, ws_bytes = _bwd_tensors(q, k, v, out, dout, lse, dq, dk, dv, scale, workspace)
    st = load_library().attn_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                         dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                         dv.data_ptr(), *dims, scale, int(bool(causal)), int(window),
                                         float(dropout_p), int(seed) & (2 ** 64 - 1), int(offset) & 0xFFFFFFFF,
                                         _dtype_code(q), ws_ptr, ws_bytes, _stream_handle(stream))
    if st != 0:
        raise AttnError(st, "attn_bwd_dropout")
    return dq, dk, dv


def attn_fwd_fp8(q, k, v, out=None, lse=None, scale: Optional[float] = None, q_descale: float = 1.0,
                 k_descale: float = 1.0, v_descale: float = 1.0, causal: bool = False, window: int = -1,
                 stream=None, return_lse: bool = True):
    """FP8 forward: q [B,Lq,Hq,D], k/v [B,Lk,Hkv,D] as torch.float8_e4m3fn; returns
    (out bf16 [B,Lq,Hq,D], lse fp32 [B,Hq,Lq]).  The inputs stand for
    q*q_descale, k*k_descale, v*v_descale."""
    import torch

    for n, t in (("q", q), ("k", k), ("v", v)):
        _require_cuda(n, t)
        if t.dtype != torch.float8_e4m3fn:
            raise TypeError(f"{n} must be torch.float8_e4m3fn")
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("expected q [B,Lq,Hq,D] and k, v [B,Lk,Hkv,D] of equal shape")
    B, Lq, Hq, D = q.shape
    Bk, Lk, Hkv, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError("q, k, v disagree in batch or head dim")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _require_cuda("out", out)
    if out.shape != q.shape or out.dtype != torch.bfloat16:
        raise ValueError("out must be bfloat16 shaped like q")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _require_cuda("lse", lse)
        if lse.shape != (B, Hq, Lq) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [B,Hq,Lq]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = load_library().attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     lse.data_ptr() if lse is not None else None,
                                     B, Hq, Hkv, Lq, Lk, D, float(scale), float(q_descale), float(k_descale),
                                     float(v_descale), int(bool(causal)), int(window), _stream_handle(stream))
    if st != 0:
        raise AttnError(st, "attn_fwd_fp8")
    return out, lse


def attn_hbm_read_probe(buf, sink, stream=None) -> None:
    """Read the whole device tensor `buf` once (a plain streaming read, the
    attainable-bandwidth reference for the HBM-bound decode).  `sink` is a
    device tensor of at least 4 bytes that the kernel may write."""
    _require_cuda("buf", buf)
    _require_cuda("sink", sink)
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must hold at least 4 bytes")
    st = load_library().attn_hbm_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                            _stream_handle(stream))
    if st != 0:
        raise AttnError(st, "attn_hbm_read_probe")
