// C ABI of libattn.so: host-side validation, instance selection and launch.
// Declarations and the full contract are in include/attn.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>

#include "../../include/attn.h"
#include "../../include/attn_measure.h"
#include "internal.h"

#define ATTN_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxDevices = 64;
// 0 = not checked yet, 1 = gfx950, 2 = something else.
std::atomic<int> g_arch_ok[kMaxDevices];
std::atomic<int> g_cu_count[kMaxDevices];

// The device current on this thread must be gfx950 (CDNA4).  The result and
// the device's CU count are cached per device id; racing first calls just
// both query.
int check_device(int* cus = nullptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ERR_DEVICE;
  if (dev >= kMaxDevices) return ATTN_ERR_DEVICE;
  int st = g_arch_ok[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_DEVICE;
    g_cu_count[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1, std::memory_order_relaxed);
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_release);
  }
  if (cus) *cus = g_cu_count[dev].load(std::memory_order_relaxed);
  return st == 1 ? ATTN_OK : ATTN_ERR_DEVICE;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_dtype(int dtype) { return dtype == ATTN_F16 || dtype == ATTN_BF16; }
bool supported_d(int D) { return D == 64 || D == 128; }

// a*b*c*d fits comfortably in a signed 64-bit element count
bool prod_ok(long long a, long long b, long long c, long long d) {
  const long long lim = (1LL << 62);
  long long p = 1;
  for (long long x : {a, b, c, d}) {
    if (x < 0) return false;
    if (x != 0 && p > lim / x) return false;
    p *= x;
  }
  return true;
}

// Sequences per decode launch: at most kDecodeMaxSeqsPerLaunch, and few
// enough that their block count fits the kernels' 32-bit counters.
int decode_seqs_per_launch(int max_blocks_per_seq) {
  const long long by_blocks = 0x7fffffffLL / max_blocks_per_seq;
  return (int)std::min<long long>(attn::kDecodeMaxSeqsPerLaunch, std::max<long long>(1, by_blocks));
}

}  // namespace

ATTN_API const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid or inconsistent sizes (or non-finite scale)";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dim, dtype or block size";
    case ATTN_ERR_ALIGN: return "tensor pointer not 16-byte aligned (lse: 4-byte)";
    case ATTN_ERR_WORKSPACE: return "decode workspace missing, misaligned or too small";
    case ATTN_ERR_DEVICE: return "no current HIP device, or it is not gfx950";
    case ATTN_ERR_HIP: return "HIP runtime error at launch";
    case ATTN_ERR_SCRATCH: return "the call needs more than the library's static decode scratch holds";
    default: return "unknown status";
  }
}

namespace {

// Validation and launch shared by attn_fwd and attn_fwd_dropout.
int fwd_dense(const void* q, const void* k, const void* v, void* out, float* lse,
              int B, int Hq, int Hkv, int Lq, int Lk, int D,
              float scale, int causal, int window, int dtype, void* stream,
              bool drop, float dropout_p, uint64_t seed, uint32_t offset) {
  if (B < 0 || Lq < 0 || Lk < 0 || Hq <= 0 || Hkv <= 0) return ATTN_ERR_SHAPE;
  // A pointer may be NULL only when the tensor it describes is empty.
  const bool q_empty = (B == 0 || Lq == 0), kv_empty = (B == 0 || Lk == 0);
  if ((!q_empty && (!q || !out)) || (!kv_empty && (!k || !v))) return ATTN_ERR_NULL;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (!std::isfinite(scale)) return ATTN_ERR_SHAPE;
  if (drop && !(dropout_p >= 0.f && dropout_p < 1.f)) return ATTN_ERR_SHAPE;  // NaN fails too
  if (!supported_d(D) || !supported_dtype(dtype)) return ATTN_ERR_UNSUPPORTED;
  if (!prod_ok(B, Lq, Hq, D) || !prod_ok(B, Lk, Hkv, D)) return ATTN_ERR_SHAPE;
  const long long n_qblocks = ((long long)Lq + attn::kPrefillBlockM - 1) / attn::kPrefillBlockM;
  if (n_qblocks * Hq * (long long)B > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return ATTN_ERR_ALIGN;
  if (lse && !aligned(lse, 4)) return ATTN_ERR_ALIGN;
  if (q_empty) return ATTN_OK;  // nothing to compute
  int cus = 0;
  const int dev = check_device(&cus);
  if (dev != ATTN_OK) return dev;

  attn::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = out; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = Lq; a.Lk = Lk;
  a.group = Hq / Hkv;
  a.causal = causal ? 1 : 0;
  a.window = window < 0 ? -1 : window;
  a.scale_log2 = scale * attn::kLog2e;
  a.n_qblocks = (int)n_qblocks;
  a.block_table = nullptr;
  a.ctx_lens = nullptr;
  a.max_blocks_per_seq = 0;
  a.num_blocks = 0;
  // threshold floor(p * 2^16): exact in double, below 2^16 for p < 1
  a.drop_thr = drop ? (uint32_t)std::floor((double)dropout_p * 65536.0) : 0u;
  a.drop_scale = drop ? (float)(1.0 / (1.0 - (double)dropout_p)) : 1.f;
  a.seed_lo = (uint32_t)seed;
  a.seed_hi = (uint32_t)(seed >> 32);
  a.drop_offset = offset;
  // A grid of at most one work-group per CU leaves each SIMD one wave; the
  // key-split instance then gives every work-group 8 waves.
  a.kv_split = n_qblocks * Hq * (long long)B <= cus ? 1 : 0;
  hipError_t e = drop ? attn::launch_fwd_dropout(a, D, dtype, (hipStream_t)stream)
                      : attn::launch_fwd(a, D, dtype, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

ATTN_API int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                      int B, int Hq, int Hkv, int Lq, int Lk, int D,
                      float scale, int causal, int window, int dtype, void* stream) {
  return fwd_dense(q, k, v, out, lse, B, Hq, Hkv, Lq, Lk, D, scale, causal, window, dtype, stream,
                   false, 0.f, 0u, 0u);
}

ATTN_API int attn_fwd_dropout(const void* q, const void* k, const void* v, void* out, float* lse,
                              int B, int Hq, int Hkv, int Lq, int Lk, int D,
                              float scale, int causal, int window,
                              float dropout_p, uint64_t seed, uint32_t offset, int dtype, void* stream) {
  return fwd_dense(q, k, v, out, lse, B, Hq, Hkv, Lq, Lk, D, scale, causal, window, dtype, stream,
                   true, dropout_p, seed, offset);
}

ATTN_API int attn_fwd_fp8(const void* q, const void* k, const void* v, void* out, float* lse,
                          int B, int Hq, int Hkv, int Lq, int Lk, int D,
                          float scale, float q_descale, float k_descale, float v_descale,
                          int causal, int window, void* stream) {
  if (B < 0 || Lq < 0 || Lk < 0 || Hq <= 0 || Hkv <= 0) return ATTN_ERR_SHAPE;
  const bool q_empty = (B == 0 || Lq == 0), kv_empty = (B == 0 || Lk == 0);
  if ((!q_empty && (!q || !out)) || (!kv_empty && (!k || !v))) return ATTN_ERR_NULL;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  const float sl = scale * q_descale * k_descale;
  if (!std::isfinite(scale) || !std::isfinite(q_descale) || !std::isfinite(k_descale) ||
      !std::isfinite(v_descale) || !std::isfinite(sl))
    return ATTN_ERR_SHAPE;
  if (!supported_d(D)) return ATTN_ERR_UNSUPPORTED;
  if (!prod_ok(B, Lq, Hq, D) || !prod_ok(B, Lk, Hkv, D)) return ATTN_ERR_SHAPE;
  const long long n_qblocks = ((long long)Lq + attn::kPrefillBlockM - 1) / attn::kPrefillBlockM;
  if (n_qblocks * Hq * (long long)B > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return ATTN_ERR_ALIGN;
  if (lse && !aligned(lse, 4)) return ATTN_ERR_ALIGN;
  if (q_empty) return ATTN_OK;
  const int dev = check_device();
  if (dev != ATTN_OK) return dev;

  attn::F8Args a;
  a.q = q; a.k = k; a.v = v; a.o = out; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = Lq; a.Lk = Lk;
  a.group = Hq / Hkv;
  a.causal = causal ? 1 : 0;
  a.window = window < 0 ? -1 : window;
  a.scale_log2 = sl * attn::kLog2e;
  a.v_descale = v_descale;
  a.n_qblocks = (int)n_qblocks;
  hipError_t e = attn::launch_fwd_fp8(a, D, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

ATTN_API int attn_fwd_paged(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_table, const int32_t* ctx_lens, int block_size,
                            void* out, float* lse,
                            int B, int Hq, int Hkv, int Lq, int D, int max_blocks_per_seq, int num_blocks,
                            float scale, int causal, int window, int dtype, void* stream) {
  if (B < 0 || Lq < 0 || Hq <= 0 || Hkv <= 0) return ATTN_ERR_SHAPE;
  const bool empty = (B == 0 || Lq == 0);
  if (!empty && (!q || !out || !k_cache || !v_cache || !block_table || !ctx_lens)) return ATTN_ERR_NULL;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (!std::isfinite(scale)) return ATTN_ERR_SHAPE;
  if (!supported_d(D) || !supported_dtype(dtype) || block_size != attn::kPagedBlock) return ATTN_ERR_UNSUPPORTED;
  if (!empty && (max_blocks_per_seq <= 0 || num_blocks <= 0)) return ATTN_ERR_SHAPE;
  if (!prod_ok(B, Lq, Hq, D) || !prod_ok(num_blocks, block_size, Hkv, D) || !prod_ok(B, max_blocks_per_seq, 1, 1))
    return ATTN_ERR_SHAPE;
  // the longest context must fit the kernel's 32-bit key positions
  if ((long long)max_blocks_per_seq * block_size > 0x3fffffffLL) return ATTN_ERR_SHAPE;
  const long long n_qblocks = ((long long)Lq + attn::kPrefillBlockM - 1) / attn::kPrefillBlockM;
  if (n_qblocks * Hq * (long long)B > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16)) return ATTN_ERR_ALIGN;
  if (!aligned(block_table, 4) || !aligned(ctx_lens, 4)) return ATTN_ERR_ALIGN;
  if (lse && !aligned(lse, 4)) return ATTN_ERR_ALIGN;
  if (empty) return ATTN_OK;
  int cus = 0;
  const int dev = check_device(&cus);
  if (dev != ATTN_OK) return dev;

  attn::FwdArgs a;
  a.q = q; a.k = k_cache; a.v = v_cache; a.o = out; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = Lq; a.Lk = 0;
  a.group = Hq / Hkv;
  a.causal = causal ? 1 : 0;
  a.window = window < 0 ? -1 : window;
  a.scale_log2 = scale * attn::kLog2e;
  a.n_qblocks = (int)n_qblocks;
  a.block_table = block_table;
  a.ctx_lens = ctx_lens;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.drop_thr = a.seed_lo = a.seed_hi = a.drop_offset = 0u;
  a.drop_scale = 1.f;
  a.kv_split = n_qblocks * Hq * (long long)B <= cus ? 1 : 0;
  hipError_t e = attn::launch_fwd_paged(a, D, dtype, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

ATTN_API size_t attn_bwd_workspace_size(int B, int Hq, int Lq) {
  if (B <= 0 || Hq <= 0 || Lq <= 0 || !prod_ok(B, Hq, Lq, 8)) return 0;
  const size_t n = (size_t)B * Hq * Lq;
  return ((n * 4 + 15) & ~(size_t)15) * 2;  // D, then the base-2 lse, each 16-byte aligned
}

namespace {

// Validation and launch shared by attn_bwd and attn_bwd_dropout.
int bwd_common(const void* q, const void* k, const void* v, const void* out, const void* dout,
               const float* lse, void* dq, void* dk, void* dv,
               int B, int Hq, int Hkv, int Lq, int Lk, int D,
               float scale, int causal, int window, int dtype,
               void* workspace, size_t workspace_bytes, void* stream,
               bool drop, float dropout_p, uint64_t seed, uint32_t offset) {
  if (B < 0 || Lq < 0 || Lk < 0 || Hq <= 0 || Hkv <= 0) return ATTN_ERR_SHAPE;
  const bool q_empty = (B == 0 || Lq == 0), kv_empty = (B == 0 || Lk == 0);
  if (!q_empty && (!q || !out || !dout || !lse || !dq)) return ATTN_ERR_NULL;
  if (!kv_empty && (!k || !v || !dk || !dv)) return ATTN_ERR_NULL;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (!std::isfinite(scale)) return ATTN_ERR_SHAPE;
  if (drop && !(dropout_p >= 0.f && dropout_p < 1.f)) return ATTN_ERR_SHAPE;  // NaN fails too
  if (!supported_d(D) || !supported_dtype(dtype)) return ATTN_ERR_UNSUPPORTED;
  if (!prod_ok(B, Lq, Hq, D) || !prod_ok(B, Lk, Hkv, D)) return ATTN_ERR_SHAPE;
  const long long n_qblocks = ((long long)Lq + attn::kPrefillBlockM - 1) / attn::kPrefillBlockM;
  if (n_qblocks * Hq * (long long)B > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  if ((((long long)Lk + 127) / 128) * Hkv * (long long)B > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  for (const void* p : {q, k, v, out, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned(p, 16)) return ATTN_ERR_ALIGN;
  if (!aligned(lse, 4)) return ATTN_ERR_ALIGN;
  if (q_empty && kv_empty) return ATTN_OK;  // nothing to write
  const size_t need = attn_bwd_workspace_size(B, Hq, Lq);
  if (need > 0 && (!workspace || !aligned(workspace, 16) || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  int cus = 0;
  const int dev = check_device(&cus);
  if (dev != ATTN_OK) return dev;

  attn::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = out; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.Dv = static_cast<float*>(workspace);
  a.L2 = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) + need / 2) : nullptr;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = Lq; a.Lk = Lk;
  a.group = Hq / Hkv;
  a.causal = causal ? 1 : 0;
  a.window = window < 0 ? -1 : window;
  a.scale = scale;
  a.scale_log2 = scale * attn::kLog2e;
  a.n_qblocks = (int)n_qblocks;
  // the forward's threshold and scale (attn_fwd_dropout)
  a.drop_thr = drop ? (uint32_t)std::floor((double)dropout_p * 65536.0) : 0u;
  a.drop_scale = drop ? (float)(1.0 / (1.0 - (double)dropout_p)) : 1.f;
  a.d_mult = drop ? (float)(1.0 - (double)dropout_p) : 1.f;
  a.seed_lo = (uint32_t)seed;
  a.seed_hi = (uint32_t)(seed >> 32);
  a.drop_offset = offset;
  // The dQ kernel's grid; at most one work-group per CU leaves each SIMD one
  // wave, and the key-split instance then gives every work-group 8 waves.
  a.kv_split = n_qblocks * Hq * (long long)B <= cus ? 1 : 0;
  hipError_t e = drop ? attn::launch_bwd_dropout(a, D, dtype, (hipStream_t)stream)
                      : attn::launch_bwd(a, D, dtype, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

ATTN_API int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv,
                      int B, int Hq, int Hkv, int Lq, int Lk, int D,
                      float scale, int causal, int window, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_common(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Lq, Lk, D, scale, causal, window, dtype,
                    workspace, workspace_bytes, stream, false, 0.f, 0u, 0u);
}

ATTN_API int attn_bwd_dropout(const void* q, const void* k, const void* v, const void* out, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv,
                              int B, int Hq, int Hkv, int Lq, int Lk, int D,
                              float scale, int causal, int window,
                              float dropout_p, uint64_t seed, uint32_t offset, int dtype,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_common(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Lq, Lk, D, scale, causal, window, dtype,
                    workspace, workspace_bytes, stream, true, dropout_p, seed, offset);
}

// Workspace slots of one decode launch: one per (range, sequence) pair that
// can leave a partial, indexed range + sequence, so fewer than
// ranges + sequences; ranges never outnumber the launch's cache blocks.
static long long decode_slots(int num_seqs, int max_blocks_per_seq) {
  const long long n = std::min(num_seqs, decode_seqs_per_launch(max_blocks_per_seq));
  return std::min<long long>(attn::kDecodeMaxStreams, n * max_blocks_per_seq) + n;
}

ATTN_API size_t attn_decode_paged_workspace_size(int num_seqs, int Hq, int D, int max_blocks_per_seq,
                                                 int block_size) {
  if (num_seqs <= 0 || Hq <= 0 || max_blocks_per_seq <= 0 || block_size != 16 || !supported_d(D)) return 0;
  // One partial (D outputs + a log2-sum-exp) per query head and slot.
  const long long slots = decode_slots(num_seqs, max_blocks_per_seq);
  if (!prod_ok(slots, Hq, D + 1, (long long)sizeof(float))) return 0;
  return (size_t)slots * Hq * (D + 1) * sizeof(float);
}

namespace {

// Host checks shared by the decode entry points (everything but the workspace).
int decode_validate(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                    const int32_t* ctx_lens, int block_size, void* out, float* lse, int num_seqs, int Hq, int Hkv,
                    int D, int max_blocks_per_seq, int num_blocks, float scale, int dtype) {
  if (num_seqs < 0 || Hq <= 0 || Hkv <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0) return ATTN_ERR_SHAPE;
  if (num_seqs > 0 && (!q || !k_cache || !v_cache || !block_table || !ctx_lens || !out)) return ATTN_ERR_NULL;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (!std::isfinite(scale)) return ATTN_ERR_SHAPE;
  if (!supported_d(D) || !supported_dtype(dtype) || block_size != 16) return ATTN_ERR_UNSUPPORTED;
  if (!prod_ok(num_blocks, block_size, Hkv, D) || !prod_ok(num_seqs, max_blocks_per_seq, 1, 1) ||
      !prod_ok(num_seqs, Hq, D, 1))
    return ATTN_ERR_SHAPE;
  if ((long long)max_blocks_per_seq * block_size > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_table, 4) || !aligned(ctx_lens, 4))
    return ATTN_ERR_ALIGN;
  if (lse && !aligned(lse, 4)) return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

// Ranges per (KV head, head group) of one decode launch: enough waves to give
// every CU one resident work-group, never more ranges than blocks.
long long decode_streams(int cus, int Hkv, int n_hgroups, int num_seqs, int max_blocks_per_seq) {
  const int per_launch = decode_seqs_per_launch(max_blocks_per_seq);
  long long streams = (long long)cus * attn::kDecodeWavesPerCU / ((long long)Hkv * n_hgroups);
  streams = std::min<long long>(streams, (long long)std::min(num_seqs, per_launch) * max_blocks_per_seq);
  return std::max<long long>(1, std::min<long long>(streams, attn::kDecodeMaxStreams));
}

// Launches of the decode over `workspace`, laid out as `slots` partial
// outputs [slots, Hq, D] followed by their log2-sum-exps [slots, Hq].
int decode_launch(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                  const int32_t* ctx_lens, void* out, float* lse, int num_seqs, int Hq, int Hkv, int D,
                  int max_blocks_per_seq, int num_blocks, float scale, int dtype, float* workspace, size_t slots,
                  long long streams, void* stream) {
  const int group = Hq / Hkv;
  const int per_launch = decode_seqs_per_launch(max_blocks_per_seq);
  const size_t esz = 2;  // fp16 / bf16
  attn::DecArgs a;
  a.k_cache = k_cache; a.v_cache = v_cache;
  a.ws_o = workspace;
  a.ws_lse = workspace + slots * Hq * D;
  a.Hq = Hq; a.Hkv = Hkv; a.group = group;
  a.max_blocks_per_seq = max_blocks_per_seq; a.num_blocks = num_blocks;
  a.n_hgroups = (group + 15) / 16;
  a.streams = (int)streams;
  a.scale_log2 = scale * attn::kLog2e;
  // Launches of successive sequence batches share the workspace; the stream
  // orders them.
  for (int s0 = 0; s0 < num_seqs; s0 += per_launch) {
    const int n = std::min(per_launch, num_seqs - s0);
    a.q = (const char*)q + (size_t)s0 * Hq * D * esz;
    a.o = (char*)out + (size_t)s0 * Hq * D * esz;
    a.lse = lse ? lse + (size_t)s0 * Hq : nullptr;
    a.block_table = block_table + (size_t)s0 * max_blocks_per_seq;
    a.ctx_lens = ctx_lens + s0;
    a.num_seqs = n;
    hipError_t e = attn::launch_decode(a, D, dtype, (hipStream_t)stream);
    if (e != hipSuccess) return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

}  // namespace

ATTN_API int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* ctx_lens, int block_size,
                               void* out, float* lse,
                               int num_seqs, int Hq, int Hkv, int D, int max_blocks_per_seq, int num_blocks,
                               float scale, int dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
  const int v = decode_validate(q, k_cache, v_cache, block_table, ctx_lens, block_size, out, lse, num_seqs, Hq,
                                Hkv, D, max_blocks_per_seq, num_blocks, scale, dtype);
  if (v != ATTN_OK) return v;
  if (num_seqs == 0) return ATTN_OK;
  const size_t need = attn_decode_paged_workspace_size(num_seqs, Hq, D, max_blocks_per_seq, block_size);
  if (need == 0 || !workspace || workspace_bytes < need || !aligned(workspace, 16)) return ATTN_ERR_WORKSPACE;
  int cus = 0;
  const int dev = check_device(&cus);
  if (dev != ATTN_OK) return dev;
  const long long streams = decode_streams(cus, Hkv, (Hq / Hkv + 15) / 16, num_seqs, max_blocks_per_seq);
  return decode_launch(q, k_cache, v_cache, block_table, ctx_lens, out, lse, num_seqs, Hq, Hkv, D,
                       max_blocks_per_seq, num_blocks, scale, dtype, (float*)workspace,
                       (size_t)decode_slots(num_seqs, max_blocks_per_seq), streams, stream);
}

// ---------------------------------------------------------------- no-alloc decode
//
// attn_decode_paged_static keeps the decode's partial results in `scratch`, a
// static device array of ATTN_DECODE_STATIC_SCRATCH_BYTES that every device
// the library runs on holds until the process ends.  On the host the array's
// name is only a stand-in for the device address, so its address on each
// device is looked up once (with that device current) and only that pointer
// is handed to kernels.
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_STATIC_SCRATCH_BYTES];

namespace {

std::atomic<void*> g_scratch[kMaxDevices];

// This device's address of `scratch` (nullptr if the lookup fails).  Racing
// first calls on one device both look it up and store the same value.
void* scratch_ptr(int dev) {
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* found = nullptr;
    if (hipGetSymbolAddress(&found, HIP_SYMBOL(scratch)) != hipSuccess || found == nullptr) return nullptr;
    g_scratch[dev].store(found, std::memory_order_release);
    p = found;
  }
  return p;
}

}  // namespace

ATTN_API int attn_decode_paged_static(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* ctx_lens, int block_size,
                                      void* out, float* lse,
                                      int num_seqs, int Hq, int Hkv, int D, int max_blocks_per_seq,
                                      int num_blocks, float scale, int dtype, void* stream) {
  const int v = decode_validate(q, k_cache, v_cache, block_table, ctx_lens, block_size, out, lse, num_seqs, Hq,
                                Hkv, D, max_blocks_per_seq, num_blocks, scale, dtype);
  if (v != ATTN_OK) return v;
  if (num_seqs == 0) return ATTN_OK;
  int cus = 0;
  const int st = check_device(&cus);
  if (st != ATTN_OK) return st;
  // Slots actually addressed: range index + sequence index of one launch.
  const long long streams = decode_streams(cus, Hkv, (Hq / Hkv + 15) / 16, num_seqs, max_blocks_per_seq);
  const long long slots = streams + std::min(num_seqs, decode_seqs_per_launch(max_blocks_per_seq));
  if (!prod_ok(slots, Hq, D + 1, (long long)sizeof(float)) ||
      slots * Hq * (D + 1) * (long long)sizeof(float) > (long long)ATTN_DECODE_STATIC_SCRATCH_BYTES)
    return ATTN_ERR_SCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_DEVICE;
  void* ws = scratch_ptr(dev);
  if (ws == nullptr) return ATTN_ERR_HIP;
  return decode_launch(q, k_cache, v_cache, block_table, ctx_lens, out, lse, num_seqs, Hq, Hkv, D,
                       max_blocks_per_seq, num_blocks, scale, dtype, (float*)ws, (size_t)slots, streams, stream);
}

ATTN_API int attn_hbm_read_probe(const void* p, size_t bytes, unsigned int* sink, void* stream) {
  if (!p || !sink) return ATTN_ERR_NULL;
  if (bytes < 16 || bytes % 16 != 0) return ATTN_ERR_SHAPE;
  if (!aligned(p, 16)) return ATTN_ERR_ALIGN;
  int cus = 1;
  const int dev = check_device(&cus);
  if (dev != ATTN_OK) return dev;
  const hipError_t e = attn::launch_hbm_read(p, bytes, sink, cus, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}
