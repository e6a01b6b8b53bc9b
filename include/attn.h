/*
 * attn.h - C ABI of the MI355X (gfx950) fused attention library (libattn.so).
 *
 * Two operations, both the scaled dot-product attention
 *     out = softmax(Q K^T * scale) V
 * of «Самовнимание, ядра CUDA и FlashAttention», section 1 (the Scores and
 * Attention equations), evaluated the way its section 3 describes: Q, K and V
 * are processed tile by tile on chip with an online softmax (running row
 * maximum and row sum, partial outputs rescaled as the maximum grows), so the
 * score matrix never reaches device memory; only the output and a small
 * per-row statistic (the log-sum-exp) are written.
 *
 *   attn_fwd           - prefill/forward over dense [batch, seq, heads, dim]
 *                        tensors, with the causal, sliding-window and MQA/GQA
 *                        options of the flash-attn call on the «Flash
 *                        Attention» page (quick start; scenario 2, steps 2-3).
 *   attn_decode_paged  - one query token per sequence against a paged KV cache
 *                        (fixed-size blocks plus a block table that maps each
 *                        sequence's logical block to a physical block), as in
 *                        the the-ai.news article, section «Внимание типа
 *                        FlashAttention и постраничное внимание».
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or synchronises.  Calls enqueue work on `stream`
 *    (a hipStream_t; NULL = the null stream) and return after the enqueue.
 *  - Tensors are contiguous, row-major, last dimension innermost.  Element
 *    type of q/k/v/out/caches is `dtype` (ATTN_F16 or ATTN_BF16); lse is fp32.
 *  - Arguments are validated on the host before anything is launched.  On
 *    failure the call returns a negative status, launches nothing and leaves
 *    every output untouched.  No exception crosses this ABI.
 *  - Supported: D in {64, 128}; Hq % Hkv == 0; block_size == 16 for decode;
 *    tensor base pointers 16-byte aligned (lse 4-byte aligned).  The device
 *    current on the calling thread must be a gfx950 GPU.
 *  - Results: accumulation in fp32, probabilities rounded to `dtype` (round to
 *    nearest even) before the P.V product, output rounded to `dtype` once.
 *  - Calls are re-entrant; the library keeps no mutable state besides a
 *    thread-safe per-device architecture check.
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_F16 = 0, ATTN_BF16 = 1 } attn_dtype;

enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,        /* a required pointer is NULL                        */
  ATTN_ERR_SHAPE = -2,       /* a size is negative/zero where it may not be, sizes
                                are inconsistent (Hq % Hkv), a size product
                                overflows, or scale is not finite                 */
  ATTN_ERR_UNSUPPORTED = -3, /* D, dtype or block_size outside the supported set  */
  ATTN_ERR_ALIGN = -4,       /* a tensor pointer is not suitably aligned          */
  ATTN_ERR_WORKSPACE = -5,   /* decode workspace missing, misaligned or too small  */
  ATTN_ERR_DEVICE = -6,      /* no current HIP device, or it is not gfx950         */
  ATTN_ERR_HIP = -7,         /* the HIP runtime reported an error at launch        */
  ATTN_ERR_SCRATCH = -8      /* attn_decode_paged_static: the call needs more than
                                the library's static scratch holds                */
};

/*
 * attn_fwd - fused attention forward.
 *
 *   q    [B, Lq, Hq,  D]  dtype      k, v [B, Lk, Hkv, D]  dtype
 *   out  [B, Lq, Hq,  D]  dtype      lse  [B, Hq, Lq] fp32, may be NULL
 *
 * out[b,i,h,:] = sum_j P[i,j] v[b,j,g,:] with g = h / (Hq/Hkv) (contiguous
 * groups of query heads share a K/V head: MQA when Hkv = 1, GQA otherwise),
 * P = row softmax of scale * q[b,i,h,:].k[b,j,g,:] over the keys j that row i
 * may see:
 *   - causal != 0: j <= i + (Lk - Lq)  (bottom-right alignment);
 *   - window >= 0: j >= i + (Lk - Lq) - window, and, when not causal, also
 *     j <= i + (Lk - Lq) + window (window_size = (window, window));
 *   - window < 0: no sliding window.
 * lse[b,h,i] = ln sum_j exp(scale * q.k_j) over the same keys.  A row that may
 * see no key gets out = 0 and lse = -inf.  `scale` is used as given (the usual
 * value is 1/sqrt(D)).
 *
 * B, Lq, Lk may be 0 (B = 0 or Lq = 0: nothing to do, returns ATTN_OK).  A
 * pointer may be NULL only when its tensor is empty (q/out when B*Lq = 0,
 * k/v when B*Lk = 0).
 * Errors: ATTN_ERR_NULL (a non-empty q, k, v or out is NULL), ATTN_ERR_SHAPE,
 * ATTN_ERR_UNSUPPORTED, ATTN_ERR_ALIGN, ATTN_ERR_DEVICE, ATTN_ERR_HIP.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int B, int Hq, int Hkv, int Lq, int Lk, int D,
             float scale, int causal, int window, int dtype, void* stream);

/*
 * attn_fwd_dropout - attn_fwd with dropout on the attention probabilities
 * (the training-time forward; the dropout_p argument of the flash-attn call on
 * the «Flash Attention» page, quick start and scenario 2).
 *
 * Same tensors, masks and errors as attn_fwd, plus:
 *   dropout_p  probability of dropping each probability, 0 <= dropout_p < 1
 *              (else ATTN_ERR_SHAPE; 0 gives attn_fwd's result);
 *   seed       64-bit key of the random generator;
 *   offset     32-bit stream selector (e.g. the training step), so one seed
 *              can serve many calls without reusing a mask.
 *
 *   out[b,i,h,:] = sum_j P[i,j] * keep(b,h,i,j) * v[b,j,g,:] / (1 - dropout_p)
 *
 * with P the row softmax of attn_fwd; lse is attn_fwd's (the undropped row
 * statistic), which attn_bwd_dropout needs.  keep(b,h,i,j) is 1 iff the
 * 16-bit half (low for even i, high for odd i) of word j%4 of Philox4x32-10
 * (Salmon, Moraes, Dror, Shaw: "Parallel Random Numbers: As Easy as 1, 2, 3",
 * SC 2011) at the counter (j/4, i/2, b*Hq + h, offset) under the key
 * (seed mod 2^32, seed / 2^32) is >= floor(dropout_p * 2^16): one generator
 * call decides four keys of two neighbouring rows.  Each probability is kept
 * with probability 1 - floor(dropout_p * 2^16) / 2^16 (1 - dropout_p exactly
 * for dropout_p a multiple of 2^-16, and never more than 2^-16 above it),
 * independently of the others, and any element's decision can be recomputed
 * on its own (the backward does).  1 / (1 - dropout_p) is applied in fp32
 * with the output normalisation.
 */
int attn_fwd_dropout(const void* q, const void* k, const void* v, void* out, float* lse,
                     int B, int Hq, int Hkv, int Lq, int Lk, int D,
                     float scale, int causal, int window,
                     float dropout_p, uint64_t seed, uint32_t offset, int dtype, void* stream);

/*
 * attn_decode_paged - one new query token per sequence against its paged
 * KV cache.
 *
 *   q, out       [num_seqs, Hq, D]                       dtype
 *   k_cache,
 *   v_cache      [num_blocks, block_size, Hkv, D]         dtype
 *   block_table  [num_seqs, max_blocks_per_seq]           int32
 *   ctx_lens     [num_seqs]                               int32
 *   lse          [num_seqs, Hq]  fp32, may be NULL
 *   workspace    >= attn_decode_paged_workspace_size(...) bytes, 16-byte aligned
 *
 * Sequence s attends the positions p in [0, ctx_lens[s]) of its own cache;
 * position p lives in physical block block_table[s, p / block_size] at slot
 * p % block_size.  The result equals attn_fwd on the gathered contiguous K/V
 * with Lq = 1 (paging moves elements, it does not change which are attended).
 *
 * block_table and ctx_lens live in device memory, so their contents are caller
 * preconditions that the host cannot check without a synchronisation:
 * 0 <= ctx_lens[s] <= max_blocks_per_seq * block_size and every entry used by a
 * sequence in [0, num_blocks).  Violations never make the kernels read outside
 * the given buffers (lengths and block ids are clamped) but give unspecified
 * values.  A sequence with ctx_len = 0 gets out = 0 and lse = -inf.
 * The workspace holds per-chunk partial results between the two kernels of
 * one call; calls that share a workspace must be ordered on one stream.
 * num_seqs = 0 is a no-op (pointers may then be NULL).
 * Errors: ATTN_ERR_NULL, ATTN_ERR_SHAPE, ATTN_ERR_UNSUPPORTED, ATTN_ERR_ALIGN,
 * ATTN_ERR_WORKSPACE, ATTN_ERR_DEVICE, ATTN_ERR_HIP.
 */
int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* ctx_lens, int block_size,
                      void* out, float* lse,
                      int num_seqs, int Hq, int Hkv, int D, int max_blocks_per_seq, int num_blocks,
                      float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged_static - attn_decode_paged without a caller workspace and
 * without any allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).
 *
 * Arguments, layouts, preconditions and results are those of
 * attn_decode_paged (the same kernels run, so outputs are bit-identical); the
 * partial results between its two kernels live instead in a static device
 * array of ATTN_DECODE_STATIC_SCRATCH_BYTES that the library holds on every
 * device it runs on until the process ends.  A call needs
 * (R + min(num_seqs, 2048)) * Hq * (D + 1) * 4 bytes of it, where R, the
 * number of ranges per KV head, is at most 4 * (CU count) / Hkv (512 for
 * Hkv = 2 on a 256-CU device): 3.6 MB for 64 sequences with Hq = 12,
 * D = 128; larger calls return ATTN_ERR_SCRATCH and launch nothing.
 * Every call on one device shares that device's array: calls that overlap in
 * time on one device (different streams, or different host threads without
 * ordering) race and give unspecified results; calls ordered on one stream
 * are safe.  Nothing in the array needs clearing between calls.
 * Errors: those of attn_decode_paged except ATTN_ERR_WORKSPACE, plus
 * ATTN_ERR_SCRATCH.
 */
#define ATTN_DECODE_STATIC_SCRATCH_BYTES (16u << 20)
int attn_decode_paged_static(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* ctx_lens, int block_size,
                             void* out, float* lse,
                             int num_seqs, int Hq, int Hkv, int D, int max_blocks_per_seq, int num_blocks,
                             float scale, int dtype, void* stream);

/*
 * attn_fwd_paged - fused attention forward for Lq new query tokens per
 * sequence over a paged KV cache (chunked / paged prefill).
 *
 *   q, out       [B, Lq, Hq, D]                          dtype
 *   k_cache,
 *   v_cache      [num_blocks, block_size, Hkv, D]         dtype
 *   block_table  [B, max_blocks_per_seq]                  int32
 *   ctx_lens     [B]                                      int32
 *   lse          [B, Hq, Lq]  fp32, may be NULL
 *
 * The FlashAttention forward of a (long) prefill, with keys and values
 * addressed through the paged cache's block table (the-ai.news article,
 * section "Внимание типа FlashAttention и постраничное внимание": blockwise
 * attention for prefill; a block table maps logical positions to physical
 * blocks and the kernel translates every position through it).  Sequence b
 * has the keys at positions [0, ctx_lens[b]); position p lives in physical
 * block block_table[b, p / block_size] at slot p % block_size.  Its Lq query
 * rows are the last Lq positions, so the result equals attn_fwd on the
 * gathered contiguous K/V with Lk = ctx_lens[b], including the bottom-right
 * causal alignment, the window and the rows that see no key when
 * ctx_lens[b] < Lq (out = 0, lse = -inf).
 *
 * block_table and ctx_lens are device memory: 0 <= ctx_lens[b] <=
 * max_blocks_per_seq * block_size and entries in [0, num_blocks) are caller
 * preconditions, as for attn_decode_paged (violations never make the kernel
 * read outside the given buffers, but give unspecified values).  No workspace;
 * B = 0 or Lq = 0 is a no-op (pointers may then be NULL).
 * Errors: ATTN_ERR_NULL, ATTN_ERR_SHAPE, ATTN_ERR_UNSUPPORTED (D, dtype,
 * block_size != 16), ATTN_ERR_ALIGN, ATTN_ERR_DEVICE, ATTN_ERR_HIP.
 */
int attn_fwd_paged(const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_table, const int32_t* ctx_lens, int block_size,
                   void* out, float* lse,
                   int B, int Hq, int Hkv, int Lq, int D, int max_blocks_per_seq, int num_blocks,
                   float scale, int causal, int window, int dtype, void* stream);

/*
 * attn_fwd_fp8 - FP8 attention forward (inference / forward only).
 *
 *   q    [B, Lq, Hq,  D]  float8 e4m3 (OCP e4m3fn)   k, v [B, Lk, Hkv, D]  e4m3
 *   out  [B, Lq, Hq,  D]  bf16                       lse  [B, Hq, Lq] fp32, may be NULL
 *
 * The FP8 forward of the "Flash Attention" skill page, scenario 3 (inputs cast
 * to float8_e4m3fn, forward pass only), with per-tensor descale factors:
 * the inputs stand for q*q_descale, k*k_descale, v*v_descale, so
 *   out = softmax(scale * q_descale * k_descale * q k^T) * (v_descale * v),
 * with the masks, GQA mapping, empty-row rule and lse of attn_fwd (lse is that
 * of the scaled scores).  The scores and the row sums are exact fp32 sums of
 * the fp8 products; the probabilities enter the P*V product rounded to e4m3
 * (3 mantissa bits), so each output element is within about
 * 2^-4 * sum_j P_ij |v_j| of the exact value, plus its bf16 rounding.
 * Errors as attn_fwd (D in {64, 128}).
 */
int attn_fwd_fp8(const void* q, const void* k, const void* v, void* out, float* lse,
                 int B, int Hq, int Hkv, int Lq, int Lk, int D,
                 float scale, float q_descale, float k_descale, float v_descale,
                 int causal, int window, void* stream);

/*
 * attn_bwd - gradients of attention: dq, dk, dv of L = sum(dout * out) for
 * the out = attn_fwd(q, k, v, ...) computed with the same arguments.
 *
 *   q, out, dout, dq   [B, Lq, Hq,  D]   dtype
 *   k, v, dk, dv       [B, Lk, Hkv, D]   dtype
 *   lse                [B, Hq, Lq] fp32, as attn_fwd wrote it (required)
 *   workspace          >= attn_bwd_workspace_size(B, Hq, Lq) bytes, 16-byte aligned
 *
 * The forward keeps only the per-row log-sum-exp, and the backward recomputes
 * the probability tiles from q and k ("Самовнимание, ядра CUDA и
 * FlashAttention", section 3, recomputation in the backward pass).  With
 * P = softmax(scale * q k^T) over the visible keys (same masks as attn_fwd):
 *   dv = P^T dout;  dS = P * (dout v^T - rowsum(dout * out));
 *   dq = scale * dS k;  dk = scale * dS^T q.
 * A K/V head's dk, dv sum over the query heads sharing it (GQA/MQA).  Rows
 * that see no key (lse = -inf) contribute nothing and get dq = 0.  Results
 * are rounded once to dtype; no atomics, so repeated calls give the same bits.
 * The workspace holds two fp32 values per (b, h, row) between the kernels of
 * one call; calls sharing a workspace must be ordered on one stream.
 * Empty sizes: B = 0 is a no-op; Lq = 0 writes dk = dv = 0 (no workspace
 * needed); Lk = 0 writes dq = 0.  Pointers of empty tensors may be NULL.
 * Errors: ATTN_ERR_NULL, ATTN_ERR_SHAPE, ATTN_ERR_UNSUPPORTED, ATTN_ERR_ALIGN,
 * ATTN_ERR_WORKSPACE, ATTN_ERR_DEVICE, ATTN_ERR_HIP.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
             void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int Lq, int Lk, int D,
             float scale, int causal, int window, int dtype,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_bwd_dropout - gradients of L = sum(dout * out) for the out of
 * attn_fwd_dropout(q, k, v, ..., dropout_p, seed, offset) called with the
 * same arguments (out and lse are that call's).
 *
 * The keep decisions are recomputed from (seed, offset) with the forward's
 * counter, so no mask is stored.  With M = keep / (1 - dropout_p):
 *   dv = (P * M)^T dout;  dS = P * (M * (dout v^T) - rowsum(dout * out));
 *   dq = scale * dS k;  dk = scale * dS^T q
 * (the row sum of dout * out equals sum_j P_ij M_ij (dout v^T)_ij, as without
 * dropout).  Tensors, workspace, determinism, empty sizes and errors as
 * attn_bwd; dropout_p outside [0, 1) is ATTN_ERR_SHAPE, and dropout_p = 0
 * gives attn_bwd's result.
 */
int attn_bwd_dropout(const void* q, const void* k, const void* v, const void* out, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv,
                     int B, int Hq, int Hkv, int Lq, int Lk, int D,
                     float scale, int causal, int window,
                     float dropout_p, uint64_t seed, uint32_t offset, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace attn_bwd needs (a pure host function); 0 when B*Hq*Lq = 0
 * or the arguments are invalid. */
size_t attn_bwd_workspace_size(int B, int Hq, int Lq);

/*
 * Bytes of workspace attn_decode_paged needs for these sizes (a pure host
 * function; no device is touched).  Returns 0 when nothing needs a workspace
 * (num_seqs = 0) or when the arguments are invalid.
 */
size_t attn_decode_paged_workspace_size(int num_seqs, int Hq, int D, int max_blocks_per_seq,
                                        int block_size);

/* A static, human-readable description of a status code (never NULL). */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */
