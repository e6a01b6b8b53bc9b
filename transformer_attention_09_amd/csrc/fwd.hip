// Fused attention forward for gfx950 (CDNA4): softmax(Q K^T * scale) V.
//
// The method is the tiled, fused evaluation of «Самовнимание, ядра CUDA и
// FlashAttention», section 3: Q, K and V are cut into blocks that live on
// chip, each K/V block updates a running row maximum and row sum (the online
// softmax) and rescales the partial output, and only the final output plus
// the per-row log-sum-exp ("small normalisation statistics") go back to
// device memory.  The the-ai.news article (section «Внимание типа
// FlashAttention и постраничное внимание») states the same per-block loop:
// partial scores, updated softmax statistics, output accumulated on chip.
// The pages' kernels (64x64 tiles, a K-loop matmul on tensor cores, «Как
// ускорить нейросети…», section on kernel internals) are prior art for other
// hardware; this kernel is laid out for CDNA4 as follows.
//
// Work decomposition
//   One work-group = 4 waves = 128 query rows of one (batch, query head); each
//   wave owns 32 rows.  K/V tiles of 64 keys are staged through LDS (double
//   buffered; global loads for tile t+1 are in flight while tile t computes)
//   and shared by the 4 waves.  Causal and sliding-window masks are applied
//   as a key-tile range [t_lo, t_hi) per work-group, so fully masked tiles are
//   never loaded, and only tiles that straddle a mask edge (or the end of the
//   keys) pay for an element-wise mask.  Work-group ids go round-robin over
//   the 8 XCDs; when the KV groups divide evenly, each XCD takes whole KV
//   groups (the query heads sharing one K/V stay in one L2) and issues its
//   q-blocks heaviest first (causal).  Without GQA and without the causal
//   mask, whole batch rows go to one XCD instead (all heads of a token range
//   are read there together).
//
// Per 64-key tile and wave (all MFMA 32x32x16, fp32 accumulate):
//   S^T = K Q^T  : A = K rows from LDS, B = the wave's Q rows (registers).
//                  The transposed product puts one query per lane column, so
//                  a row's maximum and sum need one cross-lane step (lane ^ 32).
//   online softmax in base 2: x = s * scale * log2(e), p = 2^(x - m).
//   O^T += V^T P^T: A = V^T fetched from the natural [key][d] LDS tile with
//                  the LDS transpose read, B = P straight from the S^T
//                  accumulators (rounded to the input type), no shuffles.
// The loop is software-pipelined: while tile t's exponentials run on the
// vector ALU, the MFMA unit works on tile t's P.V (16 keys at a time, each
// step right after its probabilities) and on tile t+1's scores, so the two
// units overlap inside one wave.
//
// Instances of the same kernel:
//   PAGED  K/V come through a block table from 16-token cache blocks (the
//          paged prefill); each wave's 16 rows of a tile are one block, and
//          (sequence, q-block) items of different context lengths are taken
//          longest first when there are at most 64 of them;
//   DROP   dropout on the probabilities ("dropout_p" of the flash-attn call
//          on the «Flash Attention» page): each tile's keep decisions come
//          from Philox4x32-10, one call per four keys of two neighbouring
//          rows, drawn a round at a time between the previous tile's MFMAs;
//          dropped probabilities still enter the row sum;
//   SPLIT  for grids of at most one work-group per CU (any of the above):
//          8 waves, two 4-wave halves over alternate key tiles of the same
//          rows, merged through LDS at the end (two waves per SIMD).
//
// LDS: 2 stages x (K tile + V tile) x 64 x D x 2 B = 64 KiB at D = 128, so two
// work-groups fit in the 160 KiB of a CU.  16-byte chunks of each row are
// XOR-swizzled by row so the MFMA operand reads hit distinct banks.  Each of
// the four tile buffers is an LDS array of its own and the loop is unrolled
// by two, so every read names its buffer and the compiler waits only for the
// global->LDS loads that fill it, never for the ones landing in the others.
#include "common.h"
#include "internal.h"

namespace attn {

template <int D>
struct FwdCfg {
  static constexpr int BM = kPrefillBlockM;  // query rows per work-group
  static constexpr int BN = 64;              // keys per tile
  static constexpr int NT = 256;             // threads (4 waves)
  static constexpr int CPR = D / 8;          // 16-byte chunks per K/V row
  static constexpr int RPP = NT / CPR;       // rows per staging pass
  static constexpr int KPT = BN / RPP;       // staging passes per tile
  static constexpr int KSTEPS = D / 16;      // k-steps of S^T = K Q^T
  static constexpr int DB = D / 32;          // 32-row blocks of O^T
  static constexpr int TILE = BN * D;        // elements per K or V tile
};

// Swizzle of the 16-byte chunk index inside a K row.  K operand reads take
// one chunk from 32 consecutive rows; any 16 consecutive rows map to distinct
// chunks (and any 8 to distinct chunks mod 8).
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  // Depends on r % 32 only, so the two 32-row halves of a tile share offsets.
  if constexpr (D == 128) return r & 15;
  else return (r ^ ((r >> 3) & 3)) & 7;
}
// Swizzle inside a V row.  A transposed read of a 16-lane group touches 4
// consecutive rows (r % 4 = 0..3) x 2 adjacent chunks; two groups of a half
// wave touch 4 adjacent chunks.  For D = 128 the offsets {0, 6, 10, 12} keep
// both the 8 and the 16 touched chunks of a row quad on distinct banks.
// Depends on r % 4 only.
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  if constexpr (D == 128) return ((r & 1) * 6) ^ (((r >> 1) & 1) * 10);
  else return (r & 3) << 1;
}

// The running maximum used as the exponent base is only moved when a row's
// new maximum exceeds it by more than this (base-2 units): probabilities then
// stay below 2^8, exact enough in fp32 and in the 16-bit P operand, and the
// rescale of the output accumulator is skipped on almost every tile.
constexpr float kRescaleThreshold = 8.0f;


template <typename TT, int D, bool PAGED, bool DROP, bool SPLIT>
__global__ __launch_bounds__(SPLIT ? 512 : 256, SPLIT ? 1 : 2) void fwd_kernel(FwdArgs a) {
  using C = FwdCfg<D>;
  using E = typename TT::elem;
  using V8 = typename TT::vec8;
  using V4 = typename TT::vec4;
  // SPLIT: 8 waves; waves 4h..4h+3 (half h) take the key tiles t_lo + h,
  // t_lo + h + 2, ... of the same 128 query rows, each half with its own
  // tile buffers, and half 1 hands its (max, sum, output) to half 0 through
  // LDS at the end.  Used when the grid is too small to give every SIMD two
  // waves; otherwise SPLIT is false and each work-group walks all tiles.
  constexpr int NH = SPLIT ? 2 : 1;  // key halves
  constexpr int TS = NH;             // tile stride of one half
  __shared__ __attribute__((aligned(16))) E kt0[NH * C::TILE];
  __shared__ __attribute__((aligned(16))) E kt1[NH * C::TILE];
  __shared__ __attribute__((aligned(16))) E vt0[NH * C::TILE];
  __shared__ __attribute__((aligned(16))) E vt1[NH * C::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep it scalar
  const int wave = wave_id & 3;                  // 32-row group of the work-group's 128 rows
  const int hf = SPLIT ? (wave_id >> 2) : 0;     // key half
  const int hoff = hf * C::TILE;                 // this half's tile buffers
  const int hh = lane >> 5, l32 = lane & 31;
  const int j16 = lane & 15, grp = lane >> 4;

  // ---- which (q-block, head, batch)
  int qb_rank, gid, hj;
  {
    const int n_groups = a.B * a.Hkv;
    if (!PAGED && !a.causal && a.group == 1 && (a.B & 7) == 0) {
      // No K/V is shared between heads, and no q-block outweighs another:
      // XCD x takes the batch rows x, x+8, ... and walks (batch, q-block,
      // head), so the heads of one token range, which sit side by side in
      // memory, are read by one XCD at about the same time.
      const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
      const int per_b = a.n_qblocks * a.Hq;
      const int bl = k / per_b, r = k - bl * per_b;
      qb_rank = r / a.Hq;
      gid = (x + 8 * bl) * a.Hkv + (r - qb_rank * a.Hq);
      hj = 0;
    } else if ((n_groups & 7) == 0) {
      // XCD x (= blockIdx mod 8) takes the KV groups x, x+8, ...; its
      // work-groups walk q-block ranks, heaviest first when causal.
      const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
      const int row = (n_groups >> 3) * a.group;  // work-groups per q-block rank on one XCD
      qb_rank = k / row;
      const int r = k - qb_rank * row;
      gid = x + 8 * (r / a.group);
      hj = r % a.group;
    } else {
      const int row = n_groups * a.group;
      qb_rank = blockIdx.x / row;
      const int r = blockIdx.x - qb_rank * row;
      gid = r / a.group;
      hj = r % a.group;
    }
  }
  int b = gid / a.Hkv;
  const int g = gid % a.Hkv;
  const int hq = g * a.group + hj;
  const int W = a.window;
  // Key-tile range [t_lo, t_hi) of the q-block starting at row q0 over Lk keys.
  auto tile_range = [&](int q0_, int Lk_, int& t_lo_, int& t_hi_) {
    const int off_ = Lk_ - a.Lq;
    const int row_hi = min(q0_ + C::BM, a.Lq) - 1;
    int j_lo = 0, j_hi = Lk_ - 1;
    if (a.causal) j_hi = min(j_hi, row_hi + off_);
    if (W >= 0) {
      j_lo = max(j_lo, q0_ + off_ - W);
      if (!a.causal) j_hi = min(j_hi, row_hi + off_ + W);
    }
    t_lo_ = j_lo / C::BN;
    t_hi_ = (j_hi >= j_lo) ? j_hi / C::BN + 1 : t_lo_;
  };
  auto ctx_len = [&](int bb) { return min(max(a.ctx_lens[bb], 0), a.max_blocks_per_seq * kPagedBlock); };
  int qbr = qb_rank;
  if constexpr (PAGED) {
    // Paged contexts differ in length, so the (sequence, q-block) items
    // differ in work.  With at most 64 items the work-groups take them
    // longest first: item i = (q-block rank i / B, sequence i % B) goes to
    // the work-groups of the item whose rank in descending tile count (ties
    // by index) is i.  Every wave ranks the items in one pass, a lane each.
    const int n_items = a.B * a.n_qblocks;
    if (n_items <= 64) {
      int w = -1;
      if (lane < n_items) {
        const int r = lane / a.B, qbl = a.causal ? (a.n_qblocks - 1 - r) : r;
        int tl, th;
        tile_range(qbl * C::BM, ctx_len(lane % a.B), tl, th);
        w = th - tl;
      }
      int rank = 0;
      for (int j = 0; j < n_items; ++j) {
        const int wj = __builtin_amdgcn_readlane(w, j);
        rank += (wj > w || (wj == w && j < lane)) ? 1 : 0;
      }
      const int it = qb_rank * a.B + b;
      const unsigned long long hit = __ballot(lane < n_items && rank == it);
      const int item = __builtin_amdgcn_readfirstlane(__builtin_ffsll((long long)hit) - 1);
      qbr = item / a.B;
      b = item % a.B;
    }
  }
  // Keys of batch row b: Lk of the dense layout, or the paged context length.
  int Lk = a.Lk;
  if constexpr (PAGED) Lk = ctx_len(b);
  const int qb = a.causal ? (a.n_qblocks - 1 - qbr) : qbr;
  const int q0 = qb * C::BM;
  const int off = Lk - a.Lq;  // bottom-right alignment of the causal diagonal

  // ---- key-tile range of the whole work-group
  int t_lo, t_hi;
  tile_range(q0, Lk, t_lo, t_hi);

  // ---- this lane's query row and its Q operand (B of S^T = K Q^T).
  // The kernel keeps the base-2 scale positive: a negative scale is moved
  // into Q (an exact sign flip) and a zero scale zeroes Q.
  const int qi = q0 + wave * 32 + l32;
  float sl2 = a.scale_log2;
  uint32_t qsign = 0u, qkeep = 0xffffffffu;
  if (sl2 < 0.f) { qsign = 0x80008000u; sl2 = -sl2; }
  if (sl2 == 0.f) { qkeep = 0u; sl2 = 1.f; }
  // The loads are issued here and their values used only after the first
  // K/V tiles have been requested, so the two memory round trips overlap.
  uint4 qw[C::KSTEPS];
  {
    // Rows q0.. of this head: row i at (i - q0) * Hq * D elements; rows past
    // Lq read as zeros through the resource range.
    const E* qbase = (const E*)a.q + ((size_t)((size_t)b * a.Lq + q0) * a.Hq + hq) * D;
    const rsrc_t qr = make_rsrc(qbase, rows_range(a.Lq - q0, (size_t)a.Hq * D, D, sizeof(E)));
    const uint32_t qo = (uint32_t)(((size_t)(wave * 32 + l32) * a.Hq * D + 8 * hh) * sizeof(E));
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) qw[s] = buf_load16(qr, qo + 32 * s);
  }
  V8 qf[C::KSTEPS];
  auto finish_q = [&]() {
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
      uint4 w = qw[s];
      w.x = (w.x ^ qsign) & qkeep; w.y = (w.y ^ qsign) & qkeep;
      w.z = (w.z ^ qsign) & qkeep; w.w = (w.w ^ qsign) & qkeep;
      qf[s] = __builtin_bit_cast(V8, w);
    }
  };
  // Keys this row may see: [jlo_row, jhi_row] (empty when jhi_row < jlo_row).
  int jlo_row = 0, jhi_row = Lk - 1;
  if (a.causal) jhi_row = min(jhi_row, qi + off);
  if (W >= 0) {
    jlo_row = max(jlo_row, qi + off - W);
    if (!a.causal) jhi_row = min(jhi_row, qi + off + W);
  }
  const int wr_lo = q0 + wave * 32;
  const int wr_hi = min(wr_lo + 31, a.Lq - 1);
  // Dropout: the Philox counter of this row's keys j..j+3 (j = 4c) is
  // (c, qi, b*Hq + hq, offset); see philox4x32_10.
  const uint32_t drop_bh = (uint32_t)(b * a.Hq + hq);

  // ---- per-lane LDS element offsets inside a tile
  int koff[C::KSTEPS];  // K operand of k-step s, first 32-key half (+32*D for the second)
#pragma unroll
  for (int s = 0; s < C::KSTEPS; ++s) koff[s] = hoff + l32 * D + (((2 * s + hh) ^ k_swz<D>(l32)) << 3);
  int voff[C::DB];      // V transposed read for d-block d, rows 4*hh + j16/4 (+16*s, +8)
  {
    const int r = 4 * hh + (j16 >> 2);
#pragma unroll
    for (int d = 0; d < C::DB; ++d) {
      const int col = 32 * d + 16 * (grp & 1) + 4 * (j16 & 3);
      voff[d] = hoff + r * D + ((((col >> 3) ^ v_swz<D>(r)) << 3) + 4 * ((col >> 2) & 1));
    }
  }

  // ---- staging: direct global->LDS loads, 1 KiB (RPI rows) per wave-instruction.
  // Lane -> row RPI*i + lane/CPR of the tile, physical chunk lane%CPR, which
  // holds logical chunk (lane%CPR) ^ swizzle(row).
  constexpr int RPI = 1024 / (D * (int)sizeof(E));  // rows per instruction
  constexpr int IPW = C::BN / RPI / 4;              // instructions per wave per tile
  const size_t kv_rs = (size_t)a.Hkv * D;           // elements between consecutive keys
  // Paged: the IPW*RPI = 16 tile rows of wave w are exactly one cache block,
  // logical block (BN/16)*t + w of the sequence, so each load instruction
  // addresses rows of one block and the wave needs one table entry per tile.
  static_assert(!PAGED || IPW * RPI == kPagedBlock, "a wave's tile rows are one cache block");
  const E* kb;
  const E* vb;
  if constexpr (PAGED) {
    kb = (const E*)a.k + (size_t)g * D;
    vb = (const E*)a.v + (size_t)g * D;
  } else {
    kb = (const E*)a.k + ((size_t)b * Lk * a.Hkv + g) * D;
    vb = (const E*)a.v + ((size_t)b * Lk * a.Hkv + g) * D;
  }
  uint32_t ksrc[IPW], vsrc[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int rw = i * RPI + lane / C::CPR;  // row among the wave's 16
    const int r = wave * IPW * RPI + rw;     // row of the tile
    const int p = lane % C::CPR;
    const size_t src_row = PAGED ? (size_t)rw : (size_t)r;
    ksrc[i] = (uint32_t)((src_row * kv_rs + ((p ^ k_swz<D>(r)) << 3)) * sizeof(E));
    vsrc[i] = (uint32_t)((src_row * kv_rs + ((p ^ v_swz<D>(r)) << 3)) * sizeof(E));
  }
  auto tile_bytes = [&](int t) -> uint32_t {
    // Resources start at the tile's first key and end after key Lk-1, so
    // rows past the end of the keys load as zeros; tiles past the range get
    // an empty resource (the loads then only write zeros to a free buffer).
    if (t >= t_hi) return 0u;
    return rows_range((long long)Lk - (long long)t * C::BN, kv_rs, D, sizeof(E));
  };
  // Paged: the table row of sequence b (entries past its end read as 0) and
  // the resource of this wave's block of tile t.  A block holding no visible
  // key, or of a tile past the range, gets an empty resource.
  const rsrc_t trow = make_rsrc(PAGED ? (const void*)(a.block_table + (size_t)b * a.max_blocks_per_seq) : a.q,
                                PAGED ? (uint32_t)a.max_blocks_per_seq * 4u : 0u);
  auto fetch_entry = [&](int t) -> int {  // a vector load, so it is counted with the tile loads
    return buf_load4(trow, (uint32_t)(t * (C::BN / kPagedBlock) + wave) * 4u);
  };
  const size_t blk_elems = (size_t)kPagedBlock * kv_rs;
  auto block_rsrc = [&](const E* base, int t, int entry) -> rsrc_t {
    const int lb = t * (C::BN / kPagedBlock) + wave;
    const int ntok = t < t_hi ? min(kPagedBlock, Lk - kPagedBlock * lb) : 0;
    const int e = min(max(__builtin_amdgcn_readfirstlane(entry), 0), a.num_blocks - 1);
    return make_rsrc(base + (size_t)e * blk_elems, ntok > 0 ? (uint32_t)(((ntok - 1) * kv_rs + D) * sizeof(E)) : 0u);
  };
  auto load_k = [&](int t, E* dst, int entry) {
    rsrc_t r;
    if constexpr (PAGED) r = block_rsrc(kb, t, entry);
    else r = make_rsrc(kb + (size_t)t * C::BN * kv_rs, tile_bytes(t));
#pragma unroll
    for (int i = 0; i < IPW; ++i) buf_load16_lds(r, ksrc[i], dst + hoff + (wave * IPW + i) * RPI * D);
  };
  auto load_v = [&](int t, E* dst, int entry) {
    rsrc_t r;
    if constexpr (PAGED) r = block_rsrc(vb, t, entry);
    else r = make_rsrc(vb + (size_t)t * C::BN * kv_rs, tile_bytes(t));
#pragma unroll
    for (int i = 0; i < IPW; ++i) buf_load16_lds(r, vsrc[i], dst + hoff + (wave * IPW + i) * RPI * D);
  };
  // Paged: table entries for the next K and V tile loads (K(t+2) and V(t+1)
  // at tile t); each tile fetches the entry of K(t+3), one tile ahead of use
  // (with SPLIT, the tiles of this half: t+4, t+2 and t+6).
  int eK = 0, eV = 0;

  // Does every row of this wave see every key of tile t?  (Wave-uniform.)
  auto tile_full = [&](int t) {
    const int jt = t * C::BN;
    return (jt + C::BN <= Lk) && (!a.causal || jt + C::BN - 1 <= wr_lo + off) &&
           (W < 0 || jt >= wr_hi + off - W) && (W < 0 || a.causal || jt + C::BN - 1 <= wr_lo + off + W);
  };
  // Element-wise mask of tile t's scores: key (kh*32 + 8*(r/4) + 4*hh + r%4)
  // of the tile is visible to row qi iff it lies in [jlo_row, jhi_row].
  auto mask_tile = [&](int t, f32x16* s) {
    const int base = t * C::BN + 4 * hh;
    const int lo = jlo_row - base, hi = jhi_row - base;
    const uint32_t span = (uint32_t)(hi - lo);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rel = kh * 32 + 8 * (r >> 2) + (r & 3);
        const bool ok = hi >= lo && (uint32_t)(rel - lo) <= span;
        s[kh][r] = ok ? s[kh][r] : -INFINITY;
      }
    }
  };
  // Row maximum of raw scores (lane and lane^32 share a row).
  auto row_max = [&](const f32x16* s) {
    float mx = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kh][r]);
    return max_xor32(mx);
  };

  // Dropout decisions of a tile's 32 elements in this lane, element e at
  // bit keep_bit(e).  Element e is key 8*(e/4) + 4*hh + e%4 of the tile, so the
  // elements 4g..4g+3 are the four words of the call whose counter word 0 is
  // 16*t + 2*g + hh; the two rows of a pair sit in lanes l and l^1.
  // The empty asm statement makes the counter and the key opaque at each
  // call, so the compiler can neither hoist the parts of the rounds that do
  // not depend on the tile out of the key loop nor turn the products of
  // word 0 into induction variables: either would keep values live across
  // the loop, which has no registers to spare.
  auto draw_tile = [&](int t) -> uint32_t {
    uint32_t c0 = (uint32_t)(16 * t + hh), row = (uint32_t)qi, bh = drop_bh, k0 = a.seed_lo, k1 = a.seed_hi;
    asm volatile("" : "+v"(c0), "+v"(row), "+s"(bh), "+s"(k0), "+s"(k1));
    return keep_bits_row_pair(c0, row, bh, a.drop_offset, k0, k1, a.drop_thr);
  };
  uint32_t kbits = 0u;  // decisions of the current tile (dropout only)

  f32x16 oacc[C::DB];
#pragma unroll
  for (int d = 0; d < C::DB; ++d) oacc[d] = f32x16{};
  float m_ref = -INFINITY;  // exponent base of this row (base-2 units)
  float l_run = 0.f;        // this lane's share of the row sum
  f32x16 scur[2];           // raw scores of the current tile, masked
  float mx_cur = -INFINITY; // their row maximum

  // One tile (with SPLIT, "t+1" and "t+2" below are this half's next tiles,
  // t+2 and t+4): K(t+2) and V(t+1) start loading into the buffers K(t) and
  // V(t-1) left; tile t's statistics update; then, per 16-key step s, the
  // step's probabilities (exp2 of one FMA on the raw scores), its P.V MFMAs,
  // and a quarter of tile t+1's S^T = K Q^T.  The key order inside a step is
  // the one the S^T accumulator hands out: operand index 8*hh + e is key
  // 16*s + 8*(e/4) + 4*hh + e%4, and the two transposed reads fetch exactly
  // those V rows for column d = 32*db + 16*(group&1) + (lane&15).
  auto body = [&](int t, auto par) {
    constexpr int P = decltype(par)::value;
    const E* kn = P ? kt0 : kt1;  // K(t+1)
    const E* vc = P ? vt1 : vt0;  // V(t)
    constexpr int G = C::DB;         // MFMAs per group (KSTEPS/2 == D/32)
    V8 kop[4][G];
    auto read_k = [&](int q) {
#pragma unroll
      for (int k = 0; k < G; ++k) kop[q][k] = *(const V8*)(kn + koff[(q & 1) * G + k] + (q >> 1) * 32 * D);
    };
    // The first K operands go first: their LDS latency then overlaps the
    // loads issued next and the rescale test instead of stalling the first
    // MFMA.  (K(t+1) was completed before the barrier; the loads below fill
    // the other buffers.)
    read_k(0);
    read_k(1);
    __builtin_amdgcn_sched_barrier(0);
    load_k(t + 2 * TS, P ? kt1 : kt0, eK);
    load_v(t + TS, P ? vt0 : vt1, eV);
    int eN = 0;
    if constexpr (PAGED) eN = fetch_entry(t + 3 * TS);

    // Move the exponent base only when the maximum has grown by more than
    // the threshold somewhere in the wave; rescale those rows.
    const float m_new = mx_cur * sl2;  // sl2 > 0 keeps the order; -inf stays -inf
    const bool need = m_new > m_ref + kRescaleThreshold;
    if (__any(need)) {
      if (need) {
        const float alpha = fast_exp2(m_ref - m_new);
        m_ref = m_new;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < C::DB; ++d) oacc[d] *= alpha;
      }
    }
    const float nb = (m_ref == -INFINITY) ? 0.f : -m_ref;

    // The tile as 8 groups of G MFMAs (G = D/32), in the order
    //   Q0 Q1 P0 Q2 P1 Q3 P2 P3
    // Qk = 1/4 of the next tile's S^T (Q0-Q1 build keys 0-31, Q2-Q3 keys
    // 32-63, so the second half takes over the registers of this tile's first
    // half); Ps = P.V of key step s (16 keys).  A wave issues in order and an
    // MFMA waits for the matrix unit, so the vector-ALU work sits between
    // MFMAs in small portions, and each piece of it is split over consecutive
    // MFMAs so that no MFMA waits behind a dependent chain: a probability's
    // FMA, its exp2 and its sum/pack go after three successive MFMAs.  This
    // tile's 32 probabilities are spread so that each step's are packed
    // before its P.V group; the next tile's row maximum (two interleaved
    // chains) follows its Q groups.  Each group's LDS operands are read two
    // groups ahead; sched_barrier keeps every MFMA in its own scheduling
    // region.
    constexpr int NSLOT = 8 * G;     // MFMAs per tile
    constexpr int SA = G == 4 ? 26 : 9;  // slots that start a probability
    static_assert(C::KSTEPS / 2 == G && (G == 4 || G == 2), "Q and P groups have the same size");
    f32x16 snext[2];
    float rs = 0.f, mx_a = -INFINITY, mx_b = -INFINITY;
    float px[32];  // probabilities in flight: exponent argument, then value
    uint32_t pw[4][4];
    V8 vop[4][G];

    auto read_v = [&](int st) {
#pragma unroll
      for (int d = 0; d < G; ++d) {
        const E* p0 = vc + voff[d] + 16 * st * D;
        vop[st][d] = cat4<V4, V8>(TT::read_tr(p0), TT::read_tr(p0 + 8 * D));
      }
    };
    // Element e: key step e/8, register 8*(step&1) + e%8 of the S^T half
    // step/2 (which holds key 8*(r/4) + 4*hh + r%4 of that half).
    auto stage_a = [&](int e) {
      const int st = e >> 3, r = 8 * (st & 1) + (e & 7);
      px[e] = __builtin_fmaf(scur[st >> 1][r], sl2, nb);
    };
    auto stage_b = [&](int e) { px[e] = fast_exp2(px[e]); };
    auto stage_c = [&](int e) {
      rs += px[e];
      // keep the sum here, between the MFMAs, instead of letting it sink
      // below the loop's barrier where nothing overlaps it
      asm volatile("" : "+v"(rs));
      if (e & 1) {
        uint32_t w = pack2<TT>(px[e - 1], px[e]);
        // Dropped probabilities are zeroed in the packed operand only (the
        // row sum keeps every probability): the pair's two keep bits (pair
        // order) multiply its two 16-bit halves.
        if constexpr (DROP) {
          // (opaque first: seen through, the packed conversion was split
          // into two single conversions and a byte permute)
          asm("" : "+v"(w));
          const uint32_t b = (kbits >> keep_bit(e - 1)) & 0x00010001u;
          w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2_t, w) * __builtin_bit_cast(u16x2_t, b));
        }
        pw[e >> 3][(e & 7) >> 1] = w;
      }
    };
    // Dropout: the next tile's decisions are drawn during this tile's
    // schedule, one Philox round at a time between the MFMAs (call k's round
    // r in slot (10k + r) * NSLOT / 40), so the generator's vector work
    // overlaps the matrix unit instead of running after the schedule.  The
    // counter, the row and the key are opaque here so that no part of a round
    // is hoisted out of the key loop (its registers are all in use).
    uint4 dcall = make_uint4(0u, 0u, 0u, 0u);
    uint32_t dacc_e = 0u, dacc_o = 0u;
    uint32_t dc0 = (uint32_t)(16 * (t + TS) + hh), drow = (uint32_t)qi, dbh = drop_bh;
    uint32_t dk0 = a.seed_lo, dk1 = a.seed_hi;
    if constexpr (DROP) asm volatile("" : "+v"(dc0), "+v"(drow), "+s"(dbh), "+s"(dk0), "+s"(dk1));
    const uint32_t dthr2 = a.drop_thr | (a.drop_thr << 16);
    __builtin_amdgcn_sched_barrier(0);
    static_for<NSLOT + 2>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int grp_id = i / G, m = i % G;
      constexpr int q_of[9] = {0, 1, -1, 2, -1, 3, -1, -1, -1};
      constexpr int p_of[9] = {-1, -1, 0, -1, 1, -1, 2, 3, -1};
      // From the first P.V group to the barrier this wave outranks the other
      // work-group's wave on its SIMD that is still early in its tile: the
      // four waves of a work-group then reach the barrier closer together,
      // and the early wave has slack to give.
      if constexpr (i == 2 * G) __builtin_amdgcn_s_setprio(1);
      if constexpr (i < NSLOT) {
        if constexpr (m == 0) {  // operands two groups ahead
          if constexpr (grp_id == 0) read_v(0);
          if constexpr (grp_id == 1) read_k(2);
          if constexpr (grp_id == 2) read_v(1);
          if constexpr (grp_id == 3) read_k(3);
          if constexpr (grp_id == 4) read_v(2);
          if constexpr (grp_id == 5) read_v(3);
        }
        if constexpr (q_of[grp_id] >= 0) {
          constexpr int q = q_of[grp_id];
          const f32x16 acc = (m == 0 && (q & 1) == 0) ? f32x16{} : snext[q >> 1];
          snext[q >> 1] = TT::mfma32(kop[q][m], qf[(q & 1) * G + m], acc);
        } else {
          constexpr int st = p_of[grp_id];
          const V8 pf = __builtin_bit_cast(V8, make_uint4(pw[st][0], pw[st][1], pw[st][2], pw[st][3]));
          oacc[m] = TT::mfma32(vop[st][m], pf, oacc[m]);
        }
      }
      // probability stages: elements started at slot i-2 finish, at i-1 exp, at i start
      static_for<32>([&](auto ec) {
        constexpr int e = decltype(ec)::value;
        constexpr int sa = (e * SA) / 32;  // slot of stage A
        if constexpr (sa + 2 == i) stage_c(e);
        if constexpr (sa + 1 == i) stage_b(e);
        if constexpr (sa == i) stage_a(e);
      });
      // next tile's row maximum: half 0 after Q1 (one slot later), half 1 after Q3
      if constexpr (i > 2 * G && i < 6 * G) {
        constexpr int r0 = (16 * (i - 2 * G - 1)) / (4 * G - 1), r1 = (16 * (i - 2 * G)) / (4 * G - 1);
#pragma unroll
        for (int r = r0; r < r1; ++r) {
          if (r & 1) mx_b = fmaxf(mx_b, snext[0][r]);
          else mx_a = fmaxf(mx_a, snext[0][r]);
        }
      }
      if constexpr (i > 6 * G && i <= NSLOT) {
        constexpr int r0 = (16 * (i - 6 * G - 1)) / (2 * G), r1 = (16 * (i - 6 * G)) / (2 * G);
#pragma unroll
        for (int r = r0; r < r1; ++r) {
          if (r & 1) mx_b = fmaxf(mx_b, snext[1][r]);
          else mx_a = fmaxf(mx_a, snext[1][r]);
        }
      }
      if constexpr (DROP) {
        static_for<40>([&](auto jc) {
          constexpr int j = decltype(jc)::value, k = j / 10, r = j % 10;
          if constexpr ((j * NSLOT) / 40 == i) {
            if constexpr (r == 0) dcall = keep_call(dc0, drow, dbh, a.drop_offset, k);
            philox_round(dcall, dk0 + (uint32_t)r * kPhiloxW0, dk1 + (uint32_t)r * kPhiloxW1);
            if constexpr (r == 9) keep_fold(dacc_e, dacc_o, dcall, dthr2, k);
          }
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    const float mnext = max_xor32(fmaxf(mx_a, mx_b));
    l_run += rs;
    mx_cur = mnext;
    if (!tile_full(t + TS)) {
      asm volatile("" ::: "memory");  // a real branch: the mask is rare, do not speculate it
      mask_tile(t + TS, snext);
      mx_cur = row_max(snext);
    }
    scur[0] = snext[0];
    scur[1] = snext[1];
    if constexpr (DROP) kbits = keep_finish(dacc_e, dacc_o, drow);
    wait_vmem();
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);
    if constexpr (PAGED) {
      eV = eK;
      eK = eN;
    }
  };

  if (t_lo < t_hi) {
    if constexpr (PAGED) {
      const int e0 = fetch_entry(t_lo + hf), e1 = fetch_entry(t_lo + hf + TS);
      eK = fetch_entry(t_lo + hf + 2 * TS);
      eV = e1;
      load_k(t_lo + hf, kt0, e0);
      load_v(t_lo + hf, vt0, e0);
      load_k(t_lo + hf + TS, kt1, e1);
    } else {
      load_k(t_lo + hf, kt0, 0);
      load_v(t_lo + hf, vt0, 0);
      load_k(t_lo + hf + TS, kt1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    finish_q();
    wait_vmem();
    __syncthreads();
    scur[0] = f32x16{};
    scur[1] = f32x16{};
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const V8 kf = *(const V8*)(kt0 + koff[s] + kh * 32 * D);
        scur[kh] = TT::mfma32(kf, qf[s], scur[kh]);
      }
    }
    // (SPLIT: half 1's first tile may lie past the range when the range
    // holds one tile; it then loaded zeros and is masked whole.)
    if (!tile_full(t_lo + hf)) mask_tile(t_lo + hf, scur);
    mx_cur = row_max(scur);
    if constexpr (DROP) kbits = draw_tile(t_lo + hf);
    __syncthreads();  // K(t_lo)'s buffer is refilled by the first tile
  }
  // Both halves run the same number of bodies (the barriers inside are the
  // work-group's): with an odd tile count half 1's last one lies past the
  // range, loads zeros and is masked whole, so it adds nothing.
  const int n_it = (t_hi - t_lo + NH - 1) / NH;
  for (int i = 0; i < n_it; i += 2) {
    body(t_lo + hf + i * TS, Par<0>{});
    if (i + 1 < n_it) body(t_lo + hf + (i + 1) * TS, Par<1>{});
  }

  if constexpr (SPLIT) {
    // Every load has landed and every wave has passed the last barrier, so
    // the tile buffers are free.  Half 1 leaves, per lane, its output block
    // d in buffer d (kt0, kt1, vt0, vt1 in turn) and its exponent base and
    // sum after that; half 0's wave of the same rows reads them lane for
    // lane and merges: m = max(m0, m1), each side scaled by 2^(m_side - m).
    float* xo[4] = {(float*)kt0, (float*)kt1, (float*)vt0, (float*)vt1};
    float* xs = (float*)(C::DB == 4 ? vt1 : vt0) + (C::DB == 4 ? 16 : 0) * 256;
    const int xi = wave * 64 + lane;  // 256 lanes of a half
    if (hf == 1) {
#pragma unroll
      for (int d = 0; d < C::DB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[d][r * 256 + xi] = oacc[d][r];
      xs[xi] = m_ref;
      xs[256 + xi] = l_run;
    }
    __syncthreads();
    if (hf == 1) return;
    const float m1 = xs[xi], l1 = xs[256 + xi];
    const float mm = fmaxf(m_ref, m1);
    const float a0 = m_ref == -INFINITY ? 0.f : fast_exp2(m_ref - mm);
    const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - mm);
    l_run = a0 * l_run + a1 * l1;
#pragma unroll
    for (int d = 0; d < C::DB; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[d][r] = a0 * oacc[d][r] + a1 * xo[d][r * 256 + xi];
    m_ref = mm;
  }

  // ---- epilogue: normalise, store O in the input type, and the log-sum-exp
  const float lt = sum_xor32(l_run);
  float inv = lt > 0.f ? 1.f / lt : 0.f;
  if constexpr (DROP) inv *= a.drop_scale;
  store_row16<TT, C::DB>((E*)a.o + ((size_t)((size_t)b * a.Lq + qi) * a.Hq + hq) * D, oacc, inv, hh, qi < a.Lq);
  if (qi < a.Lq) {
    if (a.lse != nullptr && hh == 0)
      a.lse[((size_t)b * a.Hq + hq) * a.Lq + qi] = lt > 0.f ? (m_ref + log2f(lt)) * kLn2 : -INFINITY;
  }
}

template <typename TT, int D, bool PAGED, bool DROP = false, bool SPLIT = false>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const long long blocks = (long long)a.n_qblocks * a.Hq * a.B;
  hipLaunchKernelGGL((fwd_kernel<TT, D, PAGED, DROP, SPLIT>), dim3((unsigned)blocks), dim3(SPLIT ? 512 : 256), 0,
                     stream, a);
  return hipGetLastError();
}

// The key-split instance serves grids of at most one work-group per CU
// (kv_split), for every entry point of this kernel, so that the dense,
// paged and dropout forwards of one shape stay the same arithmetic.
template <typename TT, int D, bool PAGED, bool DROP>
static hipError_t launch_fwd_s(const FwdArgs& a, hipStream_t stream) {
  return a.kv_split ? launch_fwd_t<TT, D, PAGED, DROP, true>(a, stream) : launch_fwd_t<TT, D, PAGED, DROP>(a, stream);
}

template <bool PAGED, bool DROP>
static hipError_t launch_fwd_any(const FwdArgs& a, int D, int dtype, hipStream_t stream) {
  if (dtype == 1)
    return D == 128 ? launch_fwd_s<BF16, 128, PAGED, DROP>(a, stream) : launch_fwd_s<BF16, 64, PAGED, DROP>(a, stream);
  return D == 128 ? launch_fwd_s<F16, 128, PAGED, DROP>(a, stream) : launch_fwd_s<F16, 64, PAGED, DROP>(a, stream);
}

hipError_t launch_fwd(const FwdArgs& a, int D, int dtype, hipStream_t stream) {
  return launch_fwd_any<false, false>(a, D, dtype, stream);
}

hipError_t launch_fwd_dropout(const FwdArgs& a, int D, int dtype, hipStream_t stream) {
  return launch_fwd_any<false, true>(a, D, dtype, stream);
}

hipError_t launch_fwd_paged(const FwdArgs& a, int D, int dtype, hipStream_t stream) {
  return launch_fwd_any<true, false>(a, D, dtype, stream);
}

}  // namespace attn
