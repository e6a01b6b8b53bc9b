// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  int B, Hq, Hkv, Lq, Lk;
  int group;       // Hq / Hkv
  int causal;
  int window;      // < 0: none
  float scale_log2;  // scale * log2(e): scores are handled in base 2
  int n_qblocks;
};

struct DecArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  void* o;
  float* lse;  // may be null
  float* ws_o;    // [num_seqs, Hq, n_split, D] partial outputs (normalised)
  float* ws_lse;  // [num_seqs, Hq, n_split] partial log2-sum-exp
  int num_seqs, Hq, Hkv, group, max_blocks_per_seq, num_blocks;
  int n_split;     // context chunks per sequence
  int n_hgroups;   // ceil(group / 16): query-head groups of one KV head
  float scale_log2;
};

// Tokens handled by one decode work-group (4 waves x 4 blocks x 16 tokens).
constexpr int kDecodeChunk = 256;
constexpr int kPrefillBlockM = 128;
constexpr float kLog2e = 1.44269504088896340736f;

hipError_t launch_fwd(const FwdArgs& a, int D, int dtype, hipStream_t stream);
hipError_t launch_decode(const DecArgs& a, int D, int dtype, hipStream_t stream);

}  // namespace attn
