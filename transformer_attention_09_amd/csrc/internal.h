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
  // Paged K/V (attn_fwd_paged): k and v are caches [num_blocks, 16, Hkv, D],
  // sequence b's keys are positions [0, ctx_lens[b]) behind block_table[b],
  // and Lk is unused.  Null for the dense layout.
  const int32_t* block_table;
  const int32_t* ctx_lens;
  int max_blocks_per_seq, num_blocks;
  // Dropout on the probabilities (attn_fwd_dropout): element (b, h, i, j) is
  // kept iff the 16-bit half (low for even i, high for odd i) of word j%4 of
  // Philox4x32-10 at counter (j/4, i/2, b*Hq+h, drop_offset) under key
  // (seed_lo, seed_hi) is >= drop_thr (= floor(p * 2^16)); kept ones are
  // scaled by drop_scale = 1/(1-p).  Unused by the other entry points.
  uint32_t drop_thr, seed_lo, seed_hi, drop_offset;
  float drop_scale;
  // Split each work-group's key tiles between two 4-wave halves (set when
  // the grid has no more work-groups than the device has CUs).
  int kv_split;
};

// Paged decode.  The cache blocks of all sequences, taken in sequence order,
// form one list of NB = sum_s ceil(ctx_s / 16) blocks; it is cut into
// `streams` equal contiguous ranges per (KV head, query-head group), and each
// range is one wave's work.  A wave whose range holds a whole sequence writes
// that sequence's output directly; otherwise it leaves a partial (normalised
// output, log2-sum-exp) in the workspace slot (range index + sequence index),
// and the combine kernel merges the partials of each sequence.
struct DecArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  void* o;
  float* lse;     // may be null
  float* ws_o;    // [slots, Hq, D] partial outputs (normalised)
  float* ws_lse;  // [slots, Hq] partial log2-sum-exp
  int num_seqs, Hq, Hkv, group, max_blocks_per_seq, num_blocks;
  int n_hgroups;  // ceil(group / 16): query-head groups of one KV head
  int streams;    // ranges per (KV head, head group)
  float scale_log2;
};

// Backward.  dout, out and lse come from the forward; Dv and L2 are the
// workspace rows written by the preprocess kernel ([B, Hq, Lq] fp32 each).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* Dv;  // sum_d dO * O per row
  float* L2;  // lse * log2(e), +inf for rows that see no key
  int B, Hq, Hkv, Lq, Lk;
  int group;
  int causal;
  int window;
  float scale;
  float scale_log2;
  int n_qblocks;
  // Dropout (attn_bwd_dropout): the forward's keep decisions, recomputed
  // with the same Philox counter, key and threshold as FwdArgs.  The kernels
  // accumulate with 0/1 keep factors and D * (1 - p) (d_mult = 1 - p; 1
  // without dropout), and multiply dQ, dK and dV by drop_scale = 1/(1-p)
  // once when they store them.
  uint32_t drop_thr, seed_lo, seed_hi, drop_offset;
  float drop_scale;
  float d_mult;
  // The dQ kernel splits each work-group's key tiles between two 4-wave
  // halves (set when its grid has no more work-groups than the device has CUs).
  int kv_split;
};

// FP8 forward: q, k, v e4m3 (OCP float8_e4m3fn), out bf16; scale_log2 holds
// scale * q_descale * k_descale * log2(e), v_descale multiplies the output.
struct F8Args {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  int B, Hq, Hkv, Lq, Lk;
  int group;
  int causal;
  int window;
  float scale_log2;
  float v_descale;
  int n_qblocks;
};

constexpr int kPrefillBlockM = 128;
constexpr int kPagedBlock = 16;  // tokens per cache block (both paged entry points)
constexpr float kLog2e = 1.44269504088896340736f;

// Decode launch limits.  Larger batches are cut into several launches.
constexpr int kDecodeMaxSeqsPerLaunch = 2048;
constexpr int kDecodeMaxStreams = 2048;
// Waves of the split kernel resident on one CU (one 4-wave work-group).
constexpr int kDecodeWavesPerCU = 4;

hipError_t launch_fwd(const FwdArgs& a, int D, int dtype, hipStream_t stream);
hipError_t launch_fwd_dropout(const FwdArgs& a, int D, int dtype, hipStream_t stream);
hipError_t launch_fwd_paged(const FwdArgs& a, int D, int dtype, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, int D, int dtype, hipStream_t stream);
hipError_t launch_bwd_dropout(const BwdArgs& a, int D, int dtype, hipStream_t stream);
hipError_t launch_fwd_fp8(const F8Args& a, int D, hipStream_t stream);
hipError_t launch_decode(const DecArgs& a, int D, int dtype, hipStream_t stream);
hipError_t launch_hbm_read(const void* p, size_t bytes, unsigned* sink, int cus, hipStream_t stream);

}  // namespace attn
