// C ABI of libattn.so: host-side validation, instance selection and launch.
// Declarations and the full contract are in include/attn.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>

#include "../../include/attn.h"
#include "internal.h"

#define ATTN_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxDevices = 64;
// 0 = not checked yet, 1 = gfx950, 2 = something else.
std::atomic<int> g_arch_ok[kMaxDevices];

// The device current on this thread must be gfx950 (CDNA4).  The result is
// cached per device id; racing first calls just both query.
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ERR_DEVICE;
  if (dev >= kMaxDevices) return ATTN_ERR_DEVICE;
  int st = g_arch_ok[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_DEVICE;
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_release);
  }
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

int decode_n_split(int max_blocks_per_seq, int block_size) {
  const long long toks = (long long)max_blocks_per_seq * block_size;
  return (int)((toks + attn::kDecodeChunk - 1) / attn::kDecodeChunk);
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
    default: return "unknown status";
  }
}

ATTN_API int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                      int B, int Hq, int Hkv, int Lq, int Lk, int D,
                      float scale, int causal, int window, int dtype, void* stream) {
  if (B < 0 || Lq < 0 || Lk < 0 || Hq <= 0 || Hkv <= 0) return ATTN_ERR_SHAPE;
  // A pointer may be NULL only when the tensor it describes is empty.
  const bool q_empty = (B == 0 || Lq == 0), kv_empty = (B == 0 || Lk == 0);
  if ((!q_empty && (!q || !out)) || (!kv_empty && (!k || !v))) return ATTN_ERR_NULL;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (!std::isfinite(scale)) return ATTN_ERR_SHAPE;
  if (!supported_d(D) || !supported_dtype(dtype)) return ATTN_ERR_UNSUPPORTED;
  if (!prod_ok(B, Lq, Hq, D) || !prod_ok(B, Lk, Hkv, D)) return ATTN_ERR_SHAPE;
  const long long n_qblocks = ((long long)Lq + attn::kPrefillBlockM - 1) / attn::kPrefillBlockM;
  if (n_qblocks * Hq * (long long)B > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return ATTN_ERR_ALIGN;
  if (lse && !aligned(lse, 4)) return ATTN_ERR_ALIGN;
  if (q_empty) return ATTN_OK;  // nothing to compute
  const int dev = check_device();
  if (dev != ATTN_OK) return dev;

  attn::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = out; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = Lq; a.Lk = Lk;
  a.group = Hq / Hkv;
  a.causal = causal ? 1 : 0;
  a.window = window < 0 ? -1 : window;
  a.scale_log2 = scale * attn::kLog2e;
  a.n_qblocks = (int)n_qblocks;
  hipError_t e = attn::launch_fwd(a, D, dtype, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

ATTN_API size_t attn_decode_paged_workspace_size(int num_seqs, int Hq, int D, int max_blocks_per_seq,
                                                 int block_size) {
  if (num_seqs <= 0 || Hq <= 0 || max_blocks_per_seq <= 0 || block_size != 16 || !supported_d(D)) return 0;
  const long long n_split = decode_n_split(max_blocks_per_seq, block_size);
  if (!prod_ok(num_seqs, Hq, n_split, D + 1)) return 0;
  return (size_t)num_seqs * Hq * n_split * (D + 1) * sizeof(float);
}

ATTN_API int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* ctx_lens, int block_size,
                               void* out, float* lse,
                               int num_seqs, int Hq, int Hkv, int D, int max_blocks_per_seq, int num_blocks,
                               float scale, int dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
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
  if (num_seqs == 0) return ATTN_OK;
  const size_t need = attn_decode_paged_workspace_size(num_seqs, Hq, D, max_blocks_per_seq, block_size);
  if (need == 0 || !workspace || workspace_bytes < need || !aligned(workspace, 16)) return ATTN_ERR_WORKSPACE;
  const int group = Hq / Hkv;
  const int n_split = decode_n_split(max_blocks_per_seq, block_size);
  const int n_hgroups = (group + 15) / 16;
  if ((long long)num_seqs * Hkv * n_hgroups * n_split > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  const int dev = check_device();
  if (dev != ATTN_OK) return dev;

  attn::DecArgs a;
  a.q = q; a.k_cache = k_cache; a.v_cache = v_cache;
  a.block_table = block_table; a.ctx_lens = ctx_lens;
  a.o = out; a.lse = lse;
  a.ws_o = (float*)workspace;
  a.ws_lse = (float*)workspace + (size_t)num_seqs * Hq * n_split * D;
  a.num_seqs = num_seqs; a.Hq = Hq; a.Hkv = Hkv; a.group = group;
  a.max_blocks_per_seq = max_blocks_per_seq; a.num_blocks = num_blocks;
  a.n_split = n_split; a.n_hgroups = n_hgroups;
  a.scale_log2 = scale * attn::kLog2e;
  hipError_t e = attn::launch_decode(a, D, dtype, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}
