// Paged-KV decode for gfx950: one query token per sequence against a KV cache
// stored in fixed-size blocks behind a block table (the-ai.news article,
// section «Внимание типа FlashAttention и постраничное внимание»: the kernel
// translates every logical position through the table to a physical block;
// paging leaves the set of attended elements unchanged).
//
// The work is bound by HBM bandwidth: every K/V byte of every context is read
// once and used by the Hq/Hkv query heads of its KV head.  The kernel is
// shaped so that every CU streams the same number of bytes, with several
// cache blocks in flight per wave, and so that the two halves of a block that
// belong to different KV heads are read at the same time:
//
//   decode_split_kernel: the cache blocks of all sequences, in sequence order,
//     form one list of NB blocks.  Each (KV head, query-head group of <= 16)
//     cuts it into `streams` equal contiguous ranges; one wave owns one range
//     (a work-group's 4 waves are neighbouring ranges/KV heads).  The unit of
//     work is one 16-token block of one KV head: its K and V tiles go
//     global->LDS with direct-to-LDS loads (range-checked, so slots past the
//     sequence's length arrive as zeros), DEPTH units ahead of the one being
//     computed.  Per unit, S^T = K Q^T (16 tokens x 16 query heads) on a
//     16x16x32 MFMA, an online softmax in base 2 over the tokens, and
//     O^T += V^T P^T on 16x16x16 MFMAs with V^T fetched by the LDS transpose
//     read and P^T taken straight from the S^T accumulators.  At the end of a
//     sequence's run inside the range, the wave writes either the final
//     output (the range holds the whole sequence) or a partial (normalised
//     output and log2-sum-exp) into workspace slot (range + sequence).
//   decode_combine_kernel: merges the partials of each split sequence:
//     M = max_c lse_c, w_c = 2^(lse_c - M), out = sum w_c o_c / sum w_c.  This
//     is the online-softmax rescaling («Самовнимание, ядра CUDA и
//     FlashAttention», section 3) applied across ranges.
//
// The LDS reads of a unit are inline assembly preceded by an explicit wait
// for that unit's own loads only (the compiler cannot tell which in-flight
// direct-to-LDS load a read depends on and would otherwise wait for all of
// them), so DEPTH-1 units stay in flight while one computes.
#include "common.h"
#include "internal.h"

namespace attn {

template <int D>
struct DecCfg {
  static constexpr int BS = 16;           // tokens per cache block
  static constexpr int WAVES = 4;         // ranges per work-group
  static constexpr int DEPTH = 4;         // units in flight per wave
  static constexpr int ROW = D * 2;       // bytes of one token of one KV head
  static constexpr int TILE = BS * D;     // elements of one K or V tile
  static constexpr int CPR = ROW / 16;    // 16-byte chunks per row
  static constexpr int LPI = 1024 / ROW;  // rows per 1 KiB direct-to-LDS load
  static constexpr int IPT = BS / LPI;    // loads per tile
  static constexpr int KS = D / 32;       // k-steps of S^T = K Q^T (16x16x32)
  static constexpr int DB = D / 16;       // 16-row blocks of O^T (16x16x16)
  static constexpr int OPS = 2 * IPT;     // vector-memory loads issued per unit
  static_assert(DEPTH == 4, "the unit loop below is unrolled for 4 slots");
};

// Chunk swizzles.  K: the 16 lanes of a K-operand read fetch one chunk from
// each of 16 rows; row t holds logical chunk c at c ^ (t mod CPR), so they hit
// distinct chunks.  V: a transposed read fetches a chunk pair from 16 rows;
// row t shifts pairs by 2*t mod CPR, so 8 consecutive rows use distinct pairs.
template <int D>
__device__ __forceinline__ int dk_swz(int t) { return t & (DecCfg<D>::CPR - 1); }
template <int D>
__device__ __forceinline__ int dv_swz(int t) { return (2 * t) & (DecCfg<D>::CPR - 1); }

// The running maximum used as the exponent base only moves when a head's new
// maximum exceeds it by more than this (base-2 units); the output rescale is
// then skipped on most units.
constexpr float kDecRescaleThreshold = 8.0f;

// Direct global->LDS load of 16 bytes per lane marked non-temporal: every
// K/V byte of the decode is read exactly once, so it should not displace
// other lines from the caches (10% faster per call on the decode workload,
// measured side by side).
__device__ __forceinline__ void buf_load16_lds_nt(rsrc_t r, uint32_t byte_off, void* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, byte_off, 0,
                                           0, kCachePolicyNT);
}

template <int J>
struct Slot {
  static constexpr int value = J;
};

template <typename TT, int D>
__global__ __launch_bounds__(256, 1) void decode_split_kernel(DecArgs a) {
  using C = DecCfg<D>;
  using E = typename TT::elem;
  using V8 = typename TT::vec8;
  using V4 = typename TT::vec4;
  __shared__ __attribute__((aligned(16))) E kb0[C::WAVES * C::TILE];
  __shared__ __attribute__((aligned(16))) E kb1[C::WAVES * C::TILE];
  __shared__ __attribute__((aligned(16))) E kb2[C::WAVES * C::TILE];
  __shared__ __attribute__((aligned(16))) E kb3[C::WAVES * C::TILE];
  __shared__ __attribute__((aligned(16))) E vb0[C::WAVES * C::TILE];
  __shared__ __attribute__((aligned(16))) E vb1[C::WAVES * C::TILE];
  __shared__ __attribute__((aligned(16))) E vb2[C::WAVES * C::TILE];
  __shared__ __attribute__((aligned(16))) E vb3[C::WAVES * C::TILE];
  __shared__ int pref[kDecodeMaxSeqsPerLaunch];  // inclusive prefix of per-sequence block counts
  __shared__ int wtot[C::WAVES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 4, c16 = lane & 15;
  const int ns = a.num_seqs;
  const int cap = a.max_blocks_per_seq * C::BS;

  // ---- 1. block counts of all sequences -> inclusive prefix in LDS.
  // Thread t takes the run of up to 8 sequences [8t, 8t+8).  Every load is
  // unconditional at an index clamped into [0, ns) (ns >= 1), so all eight
  // are in flight together instead of one guarded load after another;
  // entries past the launch's last sequence then count as empty.
  int nbv[8];
  int local = 0;
  const int s_beg = tid * 8;
  {
    int cl[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) cl[i] = a.ctx_lens[min(s_beg + i, ns - 1)];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      nbv[i] = s_beg + i < ns ? (min(max(cl[i], 0), cap) + C::BS - 1) / C::BS : 0;
      local += nbv[i];
    }
  }
  int x = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wtot[wave] = x;
  __syncthreads();
  int before = 0, NB = 0;
#pragma unroll
  for (int w = 0; w < C::WAVES; ++w) {
    before += w < wave ? wtot[w] : 0;
    NB += wtot[w];
  }
  {
    int run = before + x - local;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      run += nbv[i];
      if (s_beg + i < ns) pref[s_beg + i] = run;
    }
  }
  __syncthreads();  // the last barrier: from here on every wave runs alone

  // ---- 2. this wave's range
  const int n_eff = a.Hkv * a.n_hgroups;
  const int gid = blockIdx.x * C::WAVES + wave;
  const int geff = gid % n_eff, w = gid / n_eff;
  if (w >= a.streams) return;
  const long long nstreams = a.streams;
  const int r_beg = (int)((long long)w * NB / nstreams);
  const int r_end = (int)((long long)(w + 1) * NB / nstreams);
  if (r_beg >= r_end) return;
  const int g = geff / a.n_hgroups, hg = geff % a.n_hgroups;
  const int hj = hg * 16 + c16;  // this lane's query head inside the KV head's group
  const bool head_ok = hj < a.group;
  const int hq = g * a.group + (head_ok ? hj : 0);

  // Per-lane offsets.  Direct-to-LDS load j of a tile: lane -> row
  // LPI*j + lane/CPR, physical chunk lane%CPR holding logical chunk
  // (lane%CPR) ^ swizzle(row).
  const uint32_t tok_stride = (uint32_t)a.Hkv * C::ROW;  // bytes between tokens
  uint32_t kdo[C::IPT], vdo[C::IPT];
#pragma unroll
  for (int j = 0; j < C::IPT; ++j) {
    const int t = C::LPI * j + lane / C::CPR, pc = lane % C::CPR;
    kdo[j] = t * tok_stride + ((pc ^ dk_swz<D>(t)) << 4);
    vdo[j] = t * tok_stride + ((pc ^ dv_swz<D>(t)) << 4);
  }
  // K operand of k-step ks: row c16, logical chunk KS*G + ks (the lane group G
  // owns head-dim elements [D/4*G, D/4*(G+1)); Q uses the same order).
  int koff[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) koff[ks] = c16 * D + (((C::KS * G + ks) ^ dk_swz<D>(c16)) << 3);
  // V^T operand of d-block db: rows 4G + c16/4, columns 16*db + 4*(c16%4)..+3.
  int voff[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    const int r = 4 * G + (c16 >> 2), col = 16 * db + 4 * (c16 & 3);
    voff[db] = r * D + ((((col >> 3) ^ dv_swz<D>(r)) << 3) + 4 * ((col >> 2) & 1));
  }
  // Query operand of k-step ks: head hj, head-dim chunk KS*G + ks (byte
  // offset inside the KV head's group of query rows).
  const uint32_t qoff = (uint32_t)((head_ok ? hj : 0) * C::ROW + ((D / 4) * G) * 2);
  const E* kbase = (const E*)a.k_cache + (size_t)g * D;
  const E* vbase = (const E*)a.v_cache + (size_t)g * D;
  const size_t blk_elems = (size_t)C::BS * a.Hkv * D;
  const float sl2 = a.scale_log2;

  f32x4 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x4{};
  float m_ref = -INFINITY, l_run = 0.f;
  // Query operand of the sequence being computed (qcur), and one landing
  // buffer per pipeline slot: a unit that starts a sequence (or a window)
  // loads that sequence's query rows into its slot's buffer together with
  // its K/V tiles, so the load overlaps the units ahead of it, and its
  // compute step takes them over.  These are compiler-visible loads, so the
  // compiler places the wait before their first use.
  u32x4_t qcur[C::KS];
  u32x4_t qs[C::DEPTH][C::KS];
  // Query operand for sequence s: 16-byte chunks KS*G + ks of head hj.
  auto load_q = [&](int s, u32x4_t(&dst)[C::KS]) {
    const rsrc_t rq = make_rsrc((const E*)a.q + ((size_t)s * a.Hq + g * a.group) * D, (uint32_t)(a.group * C::ROW));
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) dst[ks] = __builtin_bit_cast(u32x4_t, buf_load16(rq, qoff + 16 * ks));
  };

  // Windows of up to 64 units: lane i describes unit i.  The loads of the
  // unit DEPTH-1 ahead are issued before each unit is computed; a unit's LDS
  // reads wait until only the loads of the units issued after it (up to
  // DEPTH-1 of them, OPS each) remain outstanding.  Stores issued in between
  // only make that wait longer, never too short.
  for (int wb = r_beg; wb < r_end; wb += 64) {
    const int n = min(64, r_end - wb);
    int u_pb = 0, u_ntok = 0, u_s = 0, u_fl = 0;
    if (lane < n) {
      const int B = wb + lane;
      int lo = 0, hi = ns - 1;  // first sequence whose inclusive prefix exceeds B
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (pref[mid] > B) hi = mid;
        else lo = mid + 1;
      }
      const int s = lo;
      const int incl = pref[s], excl = s ? pref[s - 1] : 0;
      const int b = B - excl;
      const int ctx = min(max(a.ctx_lens[s], 0), cap);
      const int pb = a.block_table[(size_t)s * a.max_blocks_per_seq + b];
      u_pb = min(max(pb, 0), a.num_blocks - 1);
      u_ntok = min(C::BS, ctx - C::BS * b);
      u_s = s;
      const int first = (B == r_beg) || (B == excl);   // the range's first unit of this sequence
      const int last = (B + 1 == r_end) || (B + 1 == incl);
      const int whole = (r_beg <= excl) && (r_end >= incl);
      u_fl = first | (last << 1) | (whole << 2);
    }
    // K and V tiles of unit u into pipeline slot J, preceded by the query
    // rows when the unit starts a sequence or the window.
    auto issue = [&](int u, auto slot) {
      constexpr int J = decltype(slot)::value;
      if (u == 0 || (__builtin_amdgcn_readlane(u_fl, u) & 1)) load_q(__builtin_amdgcn_readlane(u_s, u), qs[J]);
      E* kd = (J == 0 ? kb0 : J == 1 ? kb1 : J == 2 ? kb2 : kb3) + wave * C::TILE;
      E* vd = (J == 0 ? vb0 : J == 1 ? vb1 : J == 2 ? vb2 : vb3) + wave * C::TILE;
      const int pb = __builtin_amdgcn_readlane(u_pb, u);
      const int ntok = __builtin_amdgcn_readlane(u_ntok, u);
      const uint32_t range = (uint32_t)(ntok - 1) * tok_stride + C::ROW;
      const rsrc_t rk = make_rsrc(kbase + (size_t)pb * blk_elems, range);
      const rsrc_t rv = make_rsrc(vbase + (size_t)pb * blk_elems, range);
#pragma unroll
      for (int j = 0; j < C::IPT; ++j) buf_load16_lds_nt(rk, kdo[j], kd + j * 512);
#pragma unroll
      for (int j = 0; j < C::IPT; ++j) buf_load16_lds_nt(rv, vdo[j], vd + j * 512);
    };

    auto compute = [&](int u, auto slot) {
      constexpr int J = decltype(slot)::value;
      const uint32_t kt = lds_addr((J == 0 ? kb0 : J == 1 ? kb1 : J == 2 ? kb2 : kb3) + wave * C::TILE);
      const uint32_t vt = lds_addr((J == 0 ? vb0 : J == 1 ? vb1 : J == 2 ? vb2 : vb3) + wave * C::TILE);
      const int ntok = __builtin_amdgcn_readlane(u_ntok, u);
      const int fl = __builtin_amdgcn_readlane(u_fl, u);
      const int s = __builtin_amdgcn_readlane(u_s, u);
      if (u == 0 || (fl & 1)) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) qcur[ks] = qs[J][ks];
      }
      const int after = min(n - 1 - u, C::DEPTH - 1);  // units issued after this one
      if (after >= 3) wait_vm<3 * C::OPS>();
      else if (after == 2) wait_vm<2 * C::OPS>();
      else if (after == 1) wait_vm<C::OPS>();
      else wait_vm<0>();
      u32x4_t kf[C::KS];
      {
        uint32_t ka[C::KS];
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) ka[ks] = kt + 2 * koff[ks];
        if constexpr (C::KS == 4) lds_read16_x4(kf, ka);
        else lds_read16_x2(kf, ka);
      }
      // S^T = K Q^T: register r of lane = (token 4G + r, head c16)
      f32x4 sacc = f32x4{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        sacc = TT::mfma16(__builtin_bit_cast(V8, kf[ks]), __builtin_bit_cast(V8, qcur[ks]), sacc);
      float xs[4];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        xs[r] = (4 * G + r < ntok) ? sacc[r] * sl2 : -INFINITY;
        mx = fmaxf(mx, xs[r]);
      }
      mx = max_xor16(mx);
      mx = max_xor32(mx);  // finite: every unit holds at least one token
      const bool need = mx > m_ref + kDecRescaleThreshold;
      if (__any(need)) {
        const float alpha = need ? fast_exp2(m_ref - mx) : 1.f;
        m_ref = need ? mx : m_ref;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
      }
      V4 pf;
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(xs[r] - m_ref);
        ps += p;
        pf[r] = TT::cvt(p);
      }
      l_run += ps;
      // O^T += V^T P^T: P^T's operand is exactly the S^T register layout.
      u32x2_t vf[C::DB];
      {
        uint32_t va[C::DB];
#pragma unroll
        for (int db = 0; db < C::DB; ++db) va[db] = vt + 2 * voff[db];
        if constexpr (C::DB == 8) lds_read_tr8_x8(vf, va);
        else lds_read_tr8_x4(vf, va);
      }
#pragma unroll
      for (int db = 0; db < C::DB; ++db) oacc[db] = TT::mfma16k16(__builtin_bit_cast(V4, vf[db]), pf, oacc[db]);

      // End of a sequence's run inside this range: write the output (the
      // range holds the whole sequence) or a partial, and restart the state.
      if (fl & 2) {
        float lt = sum_xor16(l_run);
        lt = sum_xor32(lt);
        const float inv = 1.f / lt;
        const float lse2 = m_ref + log2f(lt);
        if (head_ok) {
          if (fl & 4) {
            E* orow = (E*)a.o + ((size_t)s * a.Hq + hq) * D + 4 * G;
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
              V4 o4;
#pragma unroll
              for (int r = 0; r < 4; ++r) o4[r] = TT::cvt(oacc[db][r] * inv);
              *(V4*)(orow + 16 * db) = o4;
            }
            if (G == 0 && a.lse != nullptr) a.lse[(size_t)s * a.Hq + hq] = lse2 * kLn2;
          } else {
            const size_t slot_id = (size_t)w + s;
            float* dst = a.ws_o + (slot_id * a.Hq + hq) * D + 4 * G;
#pragma unroll
            for (int db = 0; db < C::DB; ++db) *(f32x4*)(dst + 16 * db) = oacc[db] * inv;
            if (G == 0) a.ws_lse[slot_id * a.Hq + hq] = lse2;
          }
        }
        m_ref = -INFINITY;
        l_run = 0.f;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) oacc[db] = f32x4{};
      }
    };

    auto step = [&](int u, auto slot) {
      constexpr int J = decltype(slot)::value;
      if (u < n) {
        if (u + C::DEPTH - 1 < n) issue(u + C::DEPTH - 1, Slot<(J + C::DEPTH - 1) % C::DEPTH>{});
        compute(u, slot);
      }
    };

    issue(0, Slot<0>{});
    if (1 < n) issue(1, Slot<1>{});
    if (2 < n) issue(2, Slot<2>{});
    for (int u0 = 0; u0 < n; u0 += C::DEPTH) {
      step(u0, Slot<0>{});
      step(u0 + 1, Slot<1>{});
      step(u0 + 2, Slot<2>{});
      step(u0 + 3, Slot<3>{});
    }
  }
}

// Merge of split sequences: one wave per (sequence, HPW query heads), each
// lane owning 4 consecutive outputs of one head.  The wave loads the partials
// of up to 16 ranges at once, so a sequence spread over <= 16 ranges costs one
// round trip to memory after the block counts.
template <typename TT, int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecArgs a) {
  using E = typename TT::elem;
  using V4 = typename TT::vec4;
  constexpr int D4 = D / 4, HPW = 64 / D4;
  const int n_hb = (a.Hq + HPW - 1) / HPW;
  const int s = blockIdx.x / n_hb, hb = blockIdx.x % n_hb;
  const int lane = threadIdx.x;
  const int hq = hb * HPW + lane / D4, d4 = lane % D4;
  const bool lane_ok = hq < a.Hq;
  const int cap = a.max_blocks_per_seq * 16;

  // NB (all sequences) and the blocks before sequence s, as the split kernel
  // counted them.
  int tot = 0, bef = 0;
  for (int j0 = 0; j0 < a.num_seqs; j0 += 8 * 64) {
    int c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = j0 + 64 * i + lane;
      c[i] = a.ctx_lens[min(j, a.num_seqs - 1)];  // unconditional, so the 8 loads overlap
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = j0 + 64 * i + lane;
      const int nb = j < a.num_seqs ? (min(max(c[i], 0), cap) + 15) >> 4 : 0;
      tot += nb;
      bef += j < s ? nb : 0;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    tot += __shfl_xor(tot, off);
    bef += __shfl_xor(bef, off);
  }
  const int NB = tot, S0 = bef;
  const int nb_s = (min(max(a.ctx_lens[s], 0), cap) + 15) >> 4;
  E* orow = (E*)a.o + ((size_t)s * a.Hq + hq) * D + 4 * d4;
  if (nb_s == 0) {  // no context: out = 0, lse = -inf
    if (lane_ok) {
      *(V4*)orow = V4{};
      if (d4 == 0 && a.lse != nullptr) a.lse[(size_t)s * a.Hq + hq] = -INFINITY;
    }
    return;
  }
  const long long W = a.streams;
  // Range holding global block X: the largest w with floor(w*NB/W) <= X.
  const int w_lo = (int)(((long long)(S0 + 1) * W + NB - 1) / NB) - 1;
  const int w_hi = (int)(((long long)(S0 + nb_s) * W + NB - 1) / NB) - 1;
  if (w_lo == w_hi || !lane_ok) return;  // one range held the whole sequence and wrote it

  // With NB >= W every range holds a block.  Otherwise (NB * W < W^2 fits
  // 32 bits) a range w holds one iff floor(w*NB/W) < floor((w+1)*NB/W).
  const bool all_live = NB >= a.streams;
  const unsigned nb32 = (unsigned)NB, w32 = (unsigned)a.streams;
  float M = -INFINITY, wsum = 0.f;
  f32x4 acc = f32x4{};
  for (int base = w_lo; base <= w_hi; base += 16) {
    float L[16];
    f32x4 O[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int w = base + k;
      // a range that holds no block left no partial
      const bool ok = w <= w_hi && (all_live || ((unsigned)w * nb32) / w32 < ((unsigned)(w + 1) * nb32) / w32);
      const size_t slot = (size_t)w + s;
      L[k] = ok ? a.ws_lse[slot * a.Hq + hq] : -INFINITY;
      O[k] = ok ? *(const f32x4*)(a.ws_o + (slot * a.Hq + hq) * D + 4 * d4) : f32x4{};
    }
    float mloc = M;
#pragma unroll
    for (int k = 0; k < 16; ++k) mloc = fmaxf(mloc, L[k]);
    const float sc = M == -INFINITY ? 0.f : fast_exp2(M - mloc);
    wsum *= sc;
    acc *= sc;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float wt = L[k] == -INFINITY ? 0.f : fast_exp2(L[k] - mloc);
      wsum += wt;
      acc += wt * O[k];
    }
    M = mloc;
  }
  const float inv = 1.f / wsum;
  V4 o4;
#pragma unroll
  for (int r = 0; r < 4; ++r) o4[r] = TT::cvt(acc[r] * inv);
  *(V4*)orow = o4;
  if (d4 == 0 && a.lse != nullptr) a.lse[(size_t)s * a.Hq + hq] = (M + log2f(wsum)) * kLn2;
}

template <typename TT, int D>
static hipError_t launch_decode_t(const DecArgs& a, hipStream_t stream) {
  const long long waves = (long long)a.streams * a.Hkv * a.n_hgroups;
  const long long blocks = (waves + DecCfg<D>::WAVES - 1) / DecCfg<D>::WAVES;
  hipLaunchKernelGGL((decode_split_kernel<TT, D>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int HPW = 64 / (D / 4);
  const long long cblocks = (long long)a.num_seqs * ((a.Hq + HPW - 1) / HPW);
  hipLaunchKernelGGL((decode_combine_kernel<TT, D>), dim3((unsigned)cblocks), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecArgs& a, int D, int dtype, hipStream_t stream) {
  if (dtype == 1) return D == 128 ? launch_decode_t<BF16, 128>(a, stream) : launch_decode_t<BF16, 64>(a, stream);
  return D == 128 ? launch_decode_t<F16, 128>(a, stream) : launch_decode_t<F16, 64>(a, stream);
}

}  // namespace attn
