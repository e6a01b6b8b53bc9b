// Paged-KV decode for gfx950: one query token per sequence against a KV cache
// stored in fixed-size blocks behind a block table (the-ai.news article,
// section «Внимание типа FlashAttention и постраничное внимание»: the kernel
// translates every logical position through the table to a physical block;
// paging leaves the set of attended elements unchanged).
//
// The work is bound by HBM bandwidth: every K/V byte of every context is read
// once per KV head and used by the Hq/Hkv query heads of its group.  To give
// the 256 CUs enough independent streams, each sequence's context is split
// into chunks of 256 tokens ("split-K"):
//
//   decode_split_kernel: one work-group = (sequence, KV head, query-head group
//     of up to 16, chunk).  Each of its 4 waves takes 4 cache blocks (64
//     tokens): it resolves the block ids, issues all K and V loads at once
//     (64 B per lane per block and tensor, coalesced along D), computes
//     S^T = K Q^T with 16x16x32 MFMA (tokens x query heads), a per-wave
//     softmax in base 2, stages its V blocks in LDS and accumulates
//     O^T = V^T P^T with MFMA, fetching V^T with the LDS transpose read.  The
//     4 wave partials are merged in LDS with the online-softmax rescaling and
//     one normalised partial (o, log2-sum-exp) per chunk goes to the
//     workspace.
//   decode_combine_kernel: merges the chunk partials of each (sequence, query
//     head): M = max_c lse_c, w_c = 2^(lse_c - M), out = sum w_c o_c / sum w_c.
//     This is the same rescaling identity the online softmax uses («Самовнимание,
//     ядра CUDA и FlashAttention», section 3), applied across chunks.
//
// Slots past a sequence's length are masked to -inf before the softmax and
// their V rows are zeroed in LDS, so stale or non-finite cache contents never
// reach the result.
#include "common.h"
#include "internal.h"

namespace attn {

template <int D>
struct DecCfg {
  static constexpr int NT = 256, WAVES = 4;
  static constexpr int BS = 16;                       // tokens per cache block
  static constexpr int BPW = 4;                       // cache blocks per wave
  static constexpr int CHUNK = WAVES * BPW * BS;      // tokens per work-group
  static constexpr int DSTEPS = D / 32;               // k-steps of S^T
  static constexpr int DB = D / 16;                   // 16-row blocks of O^T
  static constexpr int LPT = D / 4;                   // elements per lane per token row
  static constexpr int WAVE_ELEMS = BPW * BS * D;     // LDS elements of one wave's V
  static_assert(CHUNK == kDecodeChunk, "chunk size mismatch");
};

// Chunk swizzle of V rows in LDS.  A transposed read covers 16 rows (one per
// slot) x 2 adjacent chunks per instruction; rows r..r+7 land on distinct
// chunk pairs.
template <int D>
__device__ __forceinline__ int dv_swz(int r) {
  if constexpr (D == 128) return (r & 7) << 1;
  else return (r & 3) << 1;
}

template <typename TT, int D>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecArgs a) {
  using C = DecCfg<D>;
  using E = typename TT::elem;
  using V8 = typename TT::vec8;
  using V4 = typename TT::vec4;
  __shared__ __attribute__((aligned(16))) E sv[C::WAVES * C::WAVE_ELEMS];
  __shared__ float sm_m[C::WAVES][16], sm_l[C::WAVES][16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;

  int id = blockIdx.x;
  const int c = id % a.n_split;
  id /= a.n_split;
  const int hg = id % a.n_hgroups;
  id /= a.n_hgroups;
  const int g = id % a.Hkv;
  const int s = id / a.Hkv;

  const int ctx = min(max(a.ctx_lens[s], 0), a.max_blocks_per_seq * C::BS);
  if (c * C::CHUNK >= ctx) return;  // uniform over the work-group: no barrier reached

  // Query heads of this work-group: hq = g*group + hg*16 + (lane % 16).
  const int hj = hg * 16 + l16;
  const bool head_ok = hj < a.group;
  const int hq = g * a.group + hj;

  // Q operand (B of S^T): lane holds head l16, d = LPT*g4 + 8*ds + e.
  V8 qf[C::DSTEPS];
  {
    const E* qrow = (const E*)a.q + ((size_t)s * a.Hq + hq) * D + C::LPT * g4;
#pragma unroll
    for (int ds = 0; ds < C::DSTEPS; ++ds) qf[ds] = head_ok ? *(const V8*)(qrow + 8 * ds) : V8{};
  }

  // This wave's cache blocks: logical lb = chunk*16 + wave*4 + i.
  const int lb0 = c * (C::CHUNK / C::BS) + wave * C::BPW;
  int pb[C::BPW];
  bool bvalid[C::BPW];
#pragma unroll
  for (int i = 0; i < C::BPW; ++i) {
    const int lb = lb0 + i;
    bvalid[i] = lb * C::BS < ctx;
    int p = bvalid[i] ? a.block_table[(size_t)s * a.max_blocks_per_seq + lb] : 0;
    pb[i] = min(max(p, 0), a.num_blocks - 1);
  }

  // Issue every K and V load of the wave: lane -> (slot l16, d-range LPT*g4).
  const size_t tok_rs = (size_t)a.Hkv * D;     // elements between slots
  const size_t blk_rs = (size_t)C::BS * tok_rs;  // elements between blocks
  uint4 kr[C::BPW][C::DSTEPS], vr[C::BPW][C::DSTEPS];
#pragma unroll
  for (int i = 0; i < C::BPW; ++i) {
    const size_t o = pb[i] * blk_rs + l16 * tok_rs + (size_t)g * D + C::LPT * g4;
#pragma unroll
    for (int ds = 0; ds < C::DSTEPS; ++ds) {
      if (bvalid[i]) {
        kr[i][ds] = *(const uint4*)((const E*)a.k_cache + o + 8 * ds);
        vr[i][ds] = *(const uint4*)((const E*)a.v_cache + o + 8 * ds);
      } else {
        kr[i][ds] = make_uint4(0, 0, 0, 0);
        vr[i][ds] = make_uint4(0, 0, 0, 0);
      }
    }
  }

  // S^T = K Q^T per block: register r of lane = (slot 4*g4 + r, head l16).
  f32x4 sacc[C::BPW];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < C::BPW; ++i) {
    sacc[i] = f32x4{};
#pragma unroll
    for (int ds = 0; ds < C::DSTEPS; ++ds) {
      const V8 kf = __builtin_bit_cast(V8, kr[i][ds]);
      sacc[i] = TT::mfma16(kf, qf[ds], sacc[i]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pos = (lb0 + i) * C::BS + 4 * g4 + r;
      const float x = pos < ctx ? sacc[i][r] * a.scale_log2 : -INFINITY;
      sacc[i][r] = x;
      mx = fmaxf(mx, x);
    }
  }
  mx = max_xor16(mx);
  mx = max_xor32(mx);
  const float base = (mx == -INFINITY) ? 0.f : mx;

  // P (B operand of O^T = V^T P^T): k index 8*g4 + e is
  // (block 2*ks + e/4, slot 4*g4 + e%4).
  V8 pf[C::BPW / 2];
  float lsum = 0.f;
#pragma unroll
  for (int i = 0; i < C::BPW; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = fast_exp2(sacc[i][r] - base);
      lsum += p;
      pf[i >> 1][4 * (i & 1) + r] = TT::cvt(p);
    }
  }
  lsum = sum_xor16(lsum);
  lsum = sum_xor32(lsum);

  // Stage this wave's V blocks in LDS ([block][slot][d], chunk-swizzled);
  // slots past the context are written as zeros.
  E* wv = sv + wave * C::WAVE_ELEMS;
#pragma unroll
  for (int i = 0; i < C::BPW; ++i) {
    const int row = i * C::BS + l16;
    const bool live = (lb0 + i) * C::BS + l16 < ctx;
#pragma unroll
    for (int ds = 0; ds < C::DSTEPS; ++ds) {
      const int ch = (C::LPT / 8) * g4 + ds;
      *(uint4*)(wv + row * D + ((ch ^ dv_swz<D>(row)) << 3)) = live ? vr[i][ds] : make_uint4(0, 0, 0, 0);
    }
  }
  __syncthreads();

  // O^T = V^T P^T: 32 tokens (two blocks) per k-step, 16 d per MFMA.
  f32x4 oacc[C::DB];
#pragma unroll
  for (int d = 0; d < C::DB; ++d) oacc[d] = f32x4{};
#pragma unroll
  for (int ks = 0; ks < C::BPW / 2; ++ks) {
    const int r0 = (2 * ks) * C::BS + 4 * g4 + (l16 >> 2);
    const int r1 = r0 + C::BS;
#pragma unroll
    for (int d = 0; d < C::DB; ++d) {
      const int col = 16 * d + 4 * (l16 & 3);
      const int ch = col >> 3, hf = (col >> 2) & 1;
      const E* p0 = wv + r0 * D + (((ch ^ dv_swz<D>(r0)) << 3) + 4 * hf);
      const E* p1 = wv + r1 * D + (((ch ^ dv_swz<D>(r1)) << 3) + 4 * hf);
      const V8 vf = cat4<V4, V8>(TT::read_tr(p0), TT::read_tr(p1));
      oacc[d] = TT::mfma16(vf, pf[ks], oacc[d]);
    }
  }

  // Merge the 4 wave partials of this chunk.
  if (g4 == 0) {
    sm_m[wave][l16] = mx;
    sm_l[wave][l16] = lsum;
  }
  __syncthreads();  // also: every wave is done reading its V from LDS
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < C::WAVES; ++w) M = fmaxf(M, sm_m[w][l16]);
  const float mb = (M == -INFINITY) ? 0.f : M;
  const float wscale = fast_exp2(mx - mb);

  float* so = (float*)sv;  // [wave][head 16][D] fp32, reuses the V area
#pragma unroll
  for (int d = 0; d < C::DB; ++d)
    *(f32x4*)(so + (wave * 16 + l16) * D + 16 * d + 4 * g4) = oacc[d] * wscale;
  __syncthreads();

  // 16 heads x D outputs, D/16 per thread; thread -> (head, 16 consecutive d / (128/D)).
  constexpr int PER = 16 * D / C::NT;
  const int oh = tid / (D / PER), od = (tid % (D / PER)) * PER;
  const int ohj = hg * 16 + oh;
  if (ohj < a.group) {
    const int ohq = g * a.group + ohj;
    float Lh = 0.f, Mh = -INFINITY;
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w) Mh = fmaxf(Mh, sm_m[w][oh]);
    const float mbh = (Mh == -INFINITY) ? 0.f : Mh;
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w) Lh += sm_l[w][oh] * fast_exp2(sm_m[w][oh] - mbh);
    const float inv = Lh > 0.f ? 1.f / Lh : 0.f;
    const size_t pidx = ((size_t)s * a.Hq + ohq) * a.n_split + c;
    float* dst = a.ws_o + pidx * D + od;
#pragma unroll
    for (int e = 0; e < PER; e += 4) {
      f32x4 acc = f32x4{};
#pragma unroll
      for (int w = 0; w < C::WAVES; ++w) acc += *(const f32x4*)(so + (w * 16 + oh) * D + od + e);
      *(f32x4*)(dst + e) = acc * inv;
    }
    if (od == 0) a.ws_lse[pidx] = Lh > 0.f ? mbh + log2f(Lh) : -INFINITY;
  }
}

template <typename TT, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecArgs a) {
  using E = typename TT::elem;
  const int s = blockIdx.x / a.Hq, hq = blockIdx.x % a.Hq;
  const int d = threadIdx.x;
  const int ctx = min(max(a.ctx_lens[s], 0), a.max_blocks_per_seq * 16);
  const int nc = (ctx + kDecodeChunk - 1) / kDecodeChunk;
  const size_t pbase = ((size_t)s * a.Hq + hq) * a.n_split;
  float M = -INFINITY;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, a.ws_lse[pbase + c]);
  const float mb = (M == -INFINITY) ? 0.f : M;
  float acc = 0.f, wsum = 0.f;
  for (int c = 0; c < nc; ++c) {
    const float w = fast_exp2(a.ws_lse[pbase + c] - mb);
    wsum += w;
    acc += w * a.ws_o[(pbase + c) * D + d];
  }
  const float o = wsum > 0.f ? acc / wsum : 0.f;
  ((E*)a.o)[((size_t)s * a.Hq + hq) * D + d] = TT::cvt(o);
  if (a.lse != nullptr && d == 0)
    a.lse[(size_t)s * a.Hq + hq] = wsum > 0.f ? (mb + log2f(wsum)) * kLn2 : -INFINITY;
}

template <typename TT, int D>
static hipError_t launch_decode_t(const DecArgs& a, hipStream_t stream) {
  const long long blocks = (long long)a.num_seqs * a.Hkv * a.n_hgroups * a.n_split;
  hipLaunchKernelGGL((decode_split_kernel<TT, D>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<TT, D>), dim3((unsigned)(a.num_seqs * a.Hq)), dim3(D), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecArgs& a, int D, int dtype, hipStream_t stream) {
  if (dtype == 1) return D == 128 ? launch_decode_t<BF16, 128>(a, stream) : launch_decode_t<BF16, 64>(a, stream);
  return D == 128 ? launch_decode_t<F16, 128>(a, stream) : launch_decode_t<F16, 64>(a, stream);
}

}  // namespace attn
