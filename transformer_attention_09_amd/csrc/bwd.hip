// Attention backward: dQ, dK, dV of L = sum(dO * out) by recomputation.
//
// Only the forward's per-row log-sum-exp is kept; every probability tile is
// recomputed from Q and K ("Самовнимание, ядра CUDA и FlashAttention",
// section 3: the normalisation statistics are saved and the attention tiles
// are recomputed on chip in the backward pass).  With S = scale * Q K^T,
// P = exp(S - lse) (row softmax) and D_i = sum_d dO_id * O_id (which equals
// sum_j P_ij dP_ij):
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),
//   dK = scale * dS^T Q,   dQ = scale * dS K.
//
// Three kernels, no atomics (results are deterministic):
//   bwd_pre_kernel   D_i per (batch, head, row), and the base-2 lse with +inf
//                    for rows that see no key (their P is then exactly 0);
//   bwd_dkdv_kernel  one work-group per (batch, KV head, 128-key block), 8 waves:
//                    wave w takes keys 32*(w%4).. and row half w/4 of every
//                    64-row tile, so each SIMD runs two waves.  The block's K
//                    and V sit in LDS, the Q/dO tiles of every query head of
//                    the group stream through LDS, dK and dV accumulate in
//                    registers, and the two row halves' sums meet in LDS once
//                    at the end.  S = Q K^T puts one key in each lane column,
//                    so P and dS feed dV^T += dO^T P and dK^T += Q^T dS as
//                    B operands straight from the accumulators; the A operands
//                    dO^T and Q^T are transposed LDS reads (ds_read_b64_tr_b16)
//                    that fetch rows in the accumulators' order;
//   bwd_dq_kernel    one work-group per (batch, head, 128-row block), the
//                    forward's layout: S^T = K Q^T and dP^T = V dO^T with Q and
//                    dO in registers, dQ^T += K^T dS^T with K^T read transposed.
// All MFMAs are v_mfma_f32_32x32x16 on 16-bit operands (P and dS are rounded
// to the input type), accumulating in fp32.
//
// With dropout (the DROP instances) the forward computed O = (P * M) V with
// M = keep / (1 - p); then dV = (P * M)^T dO and dS = P * (M * dP - D), where
// D_i = sum_d dO_id O_id still equals sum_j P_ij M_ij dP_ij.  The factor
// 1/(1 - p) comes out of all three gradients: the kernels use the 0/1 keep
// factor K, dV' = (P * K)^T dO and dS' = P * (K * dP - (1 - p) D) (the
// preprocess stores D (1 - p)), and scale dQ, dK and dV by 1/(1 - p) once,
// when they are stored.  Both kernels
// recompute the keep decisions with the forward's Philox counter
// (j/4, i/2, b*Hq + h, offset): one call gives the four keys 4c..4c+3 of the
// rows 2m (low 16 bits of each word) and 2m+1 (high 16 bits).  The dQ kernel
// holds a row per lane and four consecutive keys per register group, as the
// forward does, and the two lanes of a row pair split the calls; the dK/dV
// kernel holds a key per lane, so the four lanes of a quad (four consecutive
// keys) each draw two row pairs' calls and trade words with a 4x4 quad
// transpose.
#include <hip/hip_runtime.h>

#include "common.h"
#include "internal.h"

namespace attn {

template <int D>
struct BwdCfg {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int RPI = 1024 / (D * 2);        // rows per 1 KiB direct-to-LDS load
  static constexpr int DSTEPS = D / 16;             // k-steps over the head dimension
  static constexpr int DT = D / 32;                 // 32-wide head-dimension tiles
  static constexpr int BQ = 64;                     // query rows per tile (dK/dV kernel)
  static constexpr int BK = 128;                    // keys per work-group (dK/dV kernel)
  static constexpr int BN = 64;                     // keys per tile (dQ kernel)
  static constexpr int BM = kPrefillBlockM;         // query rows per work-group (dQ kernel)
  static constexpr int TILE = 64 * D;               // elements of a 64-row tile
  static constexpr int IPW = 64 / RPI / 4;          // load instructions per wave per 64-row tile
};

// One swizzle for every backward tile.  Tiles are read both along rows (k
// over the head dimension: one 16-byte chunk from 32 consecutive rows) and
// transposed (k over rows); the 8-row period keeps the transposed reads'
// fixed +8 and +16 row steps on the same chunk pattern.
__device__ __forceinline__ int bswz(int r) { return r & 7; }

// ------------------------------------------------------------------ preprocess

template <typename TT, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  using E = typename TT::elem;
  constexpr int LPR = D / 8;          // lanes per row, 8 elements each
  constexpr int RPB = 256 / LPR;      // rows per work-group
  const int tid = threadIdx.x;
  const long long row = (long long)blockIdx.x * RPB + tid / LPR;  // ((b*Lq + i)*Hq + h)
  const long long nrows = (long long)a.B * a.Lq * a.Hq;
  const int c = tid % LPR;
  float acc = 0.f;
  if (row < nrows) {
    using V8 = typename TT::vec8;
    const V8 o = *(const V8*)((const E*)a.o + row * D + 8 * c);
    const V8 g = *(const V8*)((const E*)a.dout + row * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(TT::to_f32(o[e]), TT::to_f32(g[e]), acc);
  }
#pragma unroll
  for (int m = LPR / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m);
  if (row < nrows && c == 0) {
    const long long h = row % a.Hq, bi = row / a.Hq, i = bi % a.Lq, b = bi / a.Lq;
    const size_t o = ((size_t)b * a.Hq + h) * a.Lq + i;
    a.Dv[o] = acc * a.d_mult;
    const float l = a.lse[o];
    a.L2[o] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
}

// ------------------------------------------------------------------ dK, dV

template <typename TT, int D, bool DROP>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(BwdArgs a) {
  using C = BwdCfg<D>;
  using E = typename TT::elem;
  using V8 = typename TT::vec8;
  using V4 = typename TT::vec4;
  __shared__ __attribute__((aligned(16))) E qt0[C::TILE];
  __shared__ __attribute__((aligned(16))) E qt1[C::TILE];
  __shared__ __attribute__((aligned(16))) E gt0[C::TILE];   // dO tiles
  __shared__ __attribute__((aligned(16))) E gt1[C::TILE];
  __shared__ __attribute__((aligned(16))) float lt0[C::BQ];  // base-2 lse of the tile's rows
  __shared__ __attribute__((aligned(16))) float lt1[C::BQ];
  __shared__ __attribute__((aligned(16))) float dt0[C::BQ];  // D of the tile's rows
  __shared__ __attribute__((aligned(16))) float dt1[C::BQ];
  __shared__ __attribute__((aligned(16))) E kblk[C::BK * D];  // the work-group's K and V rows
  __shared__ __attribute__((aligned(16))) E vblk[C::BK * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
  const int ks = wave & 3, rh = wave >> 2;                      // key slice, row half
  const int hh = lane >> 5, l32 = lane & 31, j16 = lane & 15, grp = lane >> 4;

  // Key blocks in order (block 0 has the most visible rows when causal).
  const int n_groups = a.B * a.Hkv;
  const int kb = blockIdx.x / n_groups, gid = blockIdx.x % n_groups;
  const int b = gid / a.Hkv, g = gid % a.Hkv;
  const int k0 = kb * C::BK, kw0 = k0 + ks * 32;
  const int off = a.Lk - a.Lq;
  const int W = a.window;

  // Query rows that see at least one key of [k0, k0 + BK) (bottom-right
  // causal alignment; the window as in the forward).
  int i_lo = 0, i_hi = a.Lq - 1;
  const int kl = k0, kh = min(k0 + C::BK, a.Lk) - 1;
  if (a.causal) i_lo = max(i_lo, kl - off);
  if (W >= 0) {
    i_hi = min(i_hi, kh - off + W);
    if (!a.causal) i_lo = max(i_lo, kl - off - W);
  }
  const int qt_lo = i_lo / C::BQ;
  const int nq = (i_hi >= i_lo) ? i_hi / C::BQ + 1 - qt_lo : 0;
  const int n_items = nq * a.group;

  // K and V of the block's keys go to LDS once (rows past Lk load as zeros);
  // each wave reads its 32 keys' rows as B operands (k over the head dim).
  const size_t kv_rs = (size_t)a.Hkv * D;
  {
    const uint32_t bytes = rows_range((long long)a.Lk - k0, kv_rs, D, sizeof(E));
    const rsrc_t rk = make_rsrc((const E*)a.k + ((size_t)b * a.Lk + k0) * kv_rs + (size_t)g * D, bytes);
    const rsrc_t rv = make_rsrc((const E*)a.v + ((size_t)b * a.Lk + k0) * kv_rs + (size_t)g * D, bytes);
    constexpr int IPB = C::BK / C::RPI / 8;  // load instructions per wave for 128 rows
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      const int r = (wave * IPB + i) * C::RPI + lane / C::CPR;
      const int p = lane % C::CPR;
      const uint32_t o = (uint32_t)(((size_t)r * kv_rs + ((p ^ bswz(r)) << 3)) * sizeof(E));
      buf_load16_lds(rk, o, kblk + (wave * IPB + i) * C::RPI * D);
      buf_load16_lds(rv, o, vblk + (wave * IPB + i) * C::RPI * D);
    }
  }

  // LDS offsets.  Row read: row l32 of a 32-row block, chunk 2s + hh.
  int noff[C::DSTEPS];
#pragma unroll
  for (int s = 0; s < C::DSTEPS; ++s) noff[s] = l32 * D + (((2 * s + hh) ^ bswz(l32)) << 3);
  const int koff = ks * 32 * D;  // the wave's 32 keys inside the K/V block
  // Transposed read of d-tile dt: rows 4*hh + j16/4 (+16*s, +8), columns
  // 32*dt + 16*(grp&1) + 4*(j16&3)..+3, so that operand index 8*hh + e is
  // row 16*s + 8*(e/4) + 4*hh + e%4 -- the accumulators' row order.
  int toff[C::DT];
  {
    const int r = 4 * hh + (j16 >> 2);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const int col = 32 * dt + 16 * (grp & 1) + 4 * (j16 & 3);
      toff[dt] = r * D + ((((col >> 3) ^ bswz(r)) << 3) + 4 * ((col >> 2) & 1));
    }
  }

  // Staging of item it (query head h, 64-row tile qt) into buffer set P.
  constexpr int IPT8 = C::BQ / C::RPI / 8;  // load instructions per wave per tile
  uint32_t src[IPT8];
#pragma unroll
  for (int i = 0; i < IPT8; ++i) {
    const int r = (wave * IPT8 + i) * C::RPI + lane / C::CPR;
    const int p = lane % C::CPR;
    src[i] = (uint32_t)(((size_t)r * a.Hq * D + ((p ^ bswz(r)) << 3)) * sizeof(E));
  }
  auto issue = [&](int it, auto par) {
    constexpr int P = decltype(par)::value;
    const int h = g * a.group + it / nq;
    const int i0 = (qt_lo + it % nq) * C::BQ;
    const uint32_t bytes = rows_range((long long)a.Lq - i0, (size_t)a.Hq * D, D, sizeof(E));
    const size_t base = (((size_t)b * a.Lq + i0) * a.Hq + h) * D;
    const rsrc_t rq = make_rsrc((const E*)a.q + base, bytes);
    const rsrc_t rg = make_rsrc((const E*)a.dout + base, bytes);
#pragma unroll
    for (int i = 0; i < IPT8; ++i) {
      buf_load16_lds(rq, src[i], (P ? qt1 : qt0) + (wave * IPT8 + i) * C::RPI * D);
      buf_load16_lds(rg, src[i], (P ? gt1 : gt0) + (wave * IPT8 + i) * C::RPI * D);
    }
    {
      // Every wave loads the 64 rows' statistics (identical bytes), so no
      // wave-dependent branch sits among the loads.
      const size_t so = ((size_t)b * a.Hq + h) * a.Lq + i0;
      const uint32_t sb = (uint32_t)(a.Lq - i0) * 4u;
      buf_load4_lds(make_rsrc(a.L2 + so, sb), 4u * lane, P ? lt1 : lt0);
      buf_load4_lds(make_rsrc(a.Dv + so, sb), 4u * lane, P ? dt1 : dt0);
    }
  };

  f32x16 dkacc[C::DT], dvacc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    dkacc[dt] = f32x16{};
    dvacc[dt] = f32x16{};
  }
  const float sl2 = a.scale_log2;

  auto body = [&](int it, auto par) {
    constexpr int P = decltype(par)::value;
    if (it + 1 < n_items) issue(it + 1, Par<1 - P>{});
    const E* qs = P ? qt1 : qt0;
    const E* gs = P ? gt1 : gt0;
    const float* ls = P ? lt1 : lt0;
    const float* ds = P ? dt1 : dt0;
    const int i0 = (qt_lo + it % nq) * C::BQ;
    const uint32_t drop_bh = (uint32_t)(b * a.Hq + g * a.group + it / nq);
    if constexpr (DROP) {
      // With the draws below the loop is short of registers: make the LDS
      // offsets opaque here so that their sums with the buffer bases are
      // formed in the loop instead of being hoisted (and spilled) outside it.
#pragma unroll
      for (int s2 = 0; s2 < C::DSTEPS; ++s2) asm volatile("" : "+v"(noff[s2]));
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) asm volatile("" : "+v"(toff[dt]));
    }

    // This wave's 32-row block rb = rh: S = Q K^T and dP = dO V^T (32 rows x
    // 32 keys), then P = exp2(S * scale * log2(e) - lse2) and dS = P (dP - D),
    // masked, then dV^T += dO^T P and dK^T += Q^T dS over its two row steps
    // of 16.  Register r of the accumulators is row 8*(r/4) + 4*hh + r%4.
    const int r0 = i0 + 32 * rh;
    const bool full = (r0 + 32 <= a.Lq) && (kw0 + 32 <= a.Lk) && (!a.causal || kw0 + 31 <= r0 + off) &&
                      (W < 0 || kw0 >= r0 + 31 + off - W) && (W < 0 || a.causal || kw0 + 31 <= r0 + off + W);
    const int key = kw0 + l32;
    {
      const int rb = rh;
      // Dropout: bit r of kbits keeps the element of accumulator register r
      // (row 8*(r/4) + 4*hh + r%4 of the block, this lane's key).  A call
      // decides the quad's four keys for a pair of rows (registers 2m, 2m+1):
      // lane q of a quad draws the pairs of registers 8s + 2q (s = 0, 1), and
      // the transpose hands each lane its key's word of the four lanes' calls,
      // so the word of lane c in round s holds registers 8s + 2c (low half)
      // and 8s + 2c + 1 (high half).  The two calls' twenty rounds run between
      // the S and dP products (round j after the products of k-step
      // j * DSTEPS / 20), one call in flight, so the generator's vector work
      // overlaps the matrix unit.
      uint32_t kbits = 0u;
      f32x16 sacc = f32x16{}, pacc = f32x16{};
      if constexpr (DROP) {
        // The S and dP products read their operands (Q, K, dO and V rows) one
        // k-step ahead, into alternating registers, so that the reads overlap
        // the previous step's products and the draws.
        V8 op[2][4];
        auto read_op = [&](int s, V8 (&o)[4]) {
          o[0] = *(const V8*)(qs + noff[s] + rb * 32 * D);
          o[1] = *(const V8*)(kblk + koff + noff[s]);
          o[2] = *(const V8*)(gs + noff[s] + rb * 32 * D);
          o[3] = *(const V8*)(vblk + koff + noff[s]);
        };
        const uint32_t thr2 = a.drop_thr | (a.drop_thr << 16);
        const int q = l32 & 3;
        uint32_t drop = 0u;
        uint4 dc = make_uint4(0u, 0u, 0u, 0u);
        uint32_t c0 = (uint32_t)(key >> 2), rowq = (uint32_t)(i0 + rb * 32 + 4 * hh + 8 * (q >> 1) + 2 * (q & 1));
        uint32_t k0 = a.seed_lo, k1 = a.seed_hi, dbh = drop_bh;
        asm volatile("" : "+v"(rowq), "+v"(c0), "+s"(k0), "+s"(k1), "+s"(dbh));
        read_op(0, op[0]);
        static_for<C::DSTEPS>([&](auto sc) {
          constexpr int s = decltype(sc)::value;
          if constexpr (s + 1 < C::DSTEPS) read_op(s + 1, op[(s + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
          sacc = TT::mfma32(op[s & 1][0], op[s & 1][1], sacc);
          pacc = TT::mfma32(op[s & 1][2], op[s & 1][3], pacc);
          static_for<20>([&](auto jc) {
            constexpr int j = decltype(jc)::value, s2 = j / 10, r = j % 10;
            if constexpr ((j * C::DSTEPS) / 20 == s) {
              if constexpr (r == 0) {
                const uint32_t row = rowq + 16u * s2;
                dc = make_uint4(c0, row >> 1, dbh, a.drop_offset);
              }
              philox_round(dc, k0 + (uint32_t)r * kPhiloxW0, k1 + (uint32_t)r * kPhiloxW1);
              if constexpr (r == 9) {
                uint32_t w[4] = {dc.x, dc.y, dc.z, dc.w};
                quad_transpose(w, q);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                  const uint32_t f = drop_flags2(w[c], thr2, 0x00010001u);
                  drop |= ((f & 1u) | ((f >> 15) & 2u)) << (8 * s2 + 2 * c);
                }
              }
            }
          });
          __builtin_amdgcn_sched_barrier(0);
        });
        kbits = ~drop & 0xFFFFu;
      } else {
#pragma unroll
        for (int s = 0; s < C::DSTEPS; ++s) {
          sacc = TT::mfma32(*(const V8*)(qs + noff[s] + rb * 32 * D), *(const V8*)(kblk + koff + noff[s]), sacc);
          pacc = TT::mfma32(*(const V8*)(gs + noff[s] + rb * 32 * D), *(const V8*)(vblk + koff + noff[s]), pacc);
        }
      }
      // Two row steps of 16 (registers 8*h2 .. 8*h2+7): their P and dS, packed
      // to the input type, then the step's dV and dK products.
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int s = 2 * rb + h2;
        float pv[8], sv[8];
        const f32x4 lA = *(const f32x4*)(ls + rb * 32 + 16 * h2 + 4 * hh);
        const f32x4 lB = *(const f32x4*)(ls + rb * 32 + 16 * h2 + 8 + 4 * hh);
        const f32x4 dA = *(const f32x4*)(ds + rb * 32 + 16 * h2 + 4 * hh);
        const f32x4 dB = *(const f32x4*)(ds + rb * 32 + 16 * h2 + 8 + 4 * hh);
        if (full) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * h2 + e;
            const float lv = e < 4 ? lA[e] : lB[e - 4], dv = e < 4 ? dA[e] : dB[e - 4];
            pv[e] = fast_exp2(__builtin_fmaf(sacc[r], sl2, -lv));
            if constexpr (DROP) {
              const float kf = (float)((kbits >> r) & 1u);
              sv[e] = pv[e] * __builtin_fmaf(kf, pacc[r], -dv);
              pv[e] *= kf;
            } else {
              sv[e] = pv[e] * (pacc[r] - dv);
            }
          }
        } else {
          asm volatile("" ::: "memory");  // a real branch: edge tiles are rare
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * h2 + e;
            const float lv = e < 4 ? lA[e] : lB[e - 4], dv = e < 4 ? dA[e] : dB[e - 4];
            const int i = i0 + rb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
            const int rel = key - (i + off);
            const bool vis = (i < a.Lq) & (key < a.Lk) & (!a.causal | (rel <= 0)) & ((W < 0) | (rel >= -W)) &
                             ((W < 0) | a.causal | (rel <= W));
            const float x = __builtin_fmaf(sacc[r], sl2, -lv);
            pv[e] = fast_exp2(vis ? x : -INFINITY);
            if constexpr (DROP) {
              const float kf = (float)((kbits >> r) & 1u);
              sv[e] = pv[e] * __builtin_fmaf(kf, pacc[r], -dv);
              pv[e] *= kf;
            } else {
              sv[e] = pv[e] * (pacc[r] - dv);
            }
          }
        }
        const V8 bp = __builtin_bit_cast(V8, make_uint4(pack2<TT>(pv[0], pv[1]), pack2<TT>(pv[2], pv[3]),
                                                        pack2<TT>(pv[4], pv[5]), pack2<TT>(pv[6], pv[7])));
        const V8 bs = __builtin_bit_cast(V8, make_uint4(pack2<TT>(sv[0], sv[1]), pack2<TT>(sv[2], sv[3]),
                                                        pack2<TT>(sv[4], sv[5]), pack2<TT>(sv[6], sv[7])));
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const E* g0 = gs + toff[dt] + 16 * s * D;
          const E* q0p = qs + toff[dt] + 16 * s * D;
          dvacc[dt] = TT::mfma32(cat4<V4, V8>(TT::read_tr(g0), TT::read_tr(g0 + 8 * D)), bp, dvacc[dt]);
          dkacc[dt] = TT::mfma32(cat4<V4, V8>(TT::read_tr(q0p), TT::read_tr(q0p + 8 * D)), bs, dkacc[dt]);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  };

  if (n_items > 0) {
    issue(0, Par<0>{});
    wait_vmem();
    __syncthreads();
    for (int it = 0; it < n_items; it += 2) {
      body(it, Par<0>{});
      if (it + 1 < n_items) body(it + 1, Par<1>{});
    }
  }

  // The two row halves' sums meet in LDS: row half 1 parks its dK^T, dV^T
  // (each lane its own 16-byte slots) in the freed tile and K/V buffers, row
  // half 0 adds them and stores.  Register r of d-tile dt is head-dim element
  // 32*dt + 8*(r/4) + 4*hh + r%4 of this lane's key.
  wait_vmem();
  __syncthreads();
  {
    static_assert(C::DT * 16 * 64 * 4 <= C::TILE * (int)sizeof(E), "a slice's partial sums fit a tile buffer");
    float* pk = (float*)(ks == 0 ? qt0 : ks == 1 ? qt1 : ks == 2 ? gt0 : gt1);
    float* pv = (float*)((ks < 2 ? kblk : vblk) + (ks & 1) * (C::BK / 2) * D);
    if (rh == 1) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int j = dt * 4 + q4;
          *(f32x4*)(pk + (j * 64 + lane) * 4) = f32x4{dkacc[dt][4 * q4], dkacc[dt][4 * q4 + 1],
                                                       dkacc[dt][4 * q4 + 2], dkacc[dt][4 * q4 + 3]};
          *(f32x4*)(pv + (j * 64 + lane) * 4) = f32x4{dvacc[dt][4 * q4], dvacc[dt][4 * q4 + 1],
                                                       dvacc[dt][4 * q4 + 2], dvacc[dt][4 * q4 + 3]};
        }
    }
    __syncthreads();
    if (rh == 0) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int j = dt * 4 + q4;
          const f32x4 ok = *(const f32x4*)(pk + (j * 64 + lane) * 4);
          const f32x4 ov = *(const f32x4*)(pv + (j * 64 + lane) * 4);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            dkacc[dt][4 * q4 + r] += ok[r];
            dvacc[dt][4 * q4 + r] += ov[r];
          }
        }
      }
      const size_t ro = (((size_t)b * a.Lk + kw0 + l32) * a.Hkv + g) * D;
      const bool key_ok = kw0 + l32 < a.Lk;
      store_row16<TT, C::DT>((E*)a.dk + ro, dkacc, DROP ? a.scale * a.drop_scale : a.scale, hh, key_ok);
      store_row16<TT, C::DT>((E*)a.dv + ro, dvacc, DROP ? a.drop_scale : 1.f, hh, key_ok);
    }
  }
}

// ------------------------------------------------------------------ dQ

// SPLIT (grids of at most one work-group per CU): 8 waves, two 4-wave halves
// over alternate key tiles of the same 128 rows, each with its own tile
// buffers; half 1 adds its dQ partial sums into half 0's through LDS at the
// end.  Otherwise each work-group of 4 waves walks all tiles.
template <typename TT, int D, bool DROP, bool SPLIT>
__global__ __launch_bounds__(SPLIT ? 512 : 256, SPLIT ? 1 : 2) void bwd_dq_kernel(BwdArgs a) {
  using C = BwdCfg<D>;
  using E = typename TT::elem;
  using V8 = typename TT::vec8;
  using V4 = typename TT::vec4;
  constexpr int NH = SPLIT ? 2 : 1;  // key halves
  constexpr int TS = NH;             // tile stride of one half
  __shared__ __attribute__((aligned(16))) E kt0[NH * C::TILE];
  __shared__ __attribute__((aligned(16))) E kt1[NH * C::TILE];
  __shared__ __attribute__((aligned(16))) E vt0[NH * C::TILE];
  __shared__ __attribute__((aligned(16))) E vt1[NH * C::TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave = wave_id & 3;               // 32-row group of the work-group's rows
  const int hf = SPLIT ? (wave_id >> 2) : 0;  // key half
  const int hoff = hf * C::TILE;              // this half's tile buffers
  const int hh = lane >> 5, l32 = lane & 31, j16 = lane & 15, grp = lane >> 4;

  const int n_heads = a.B * a.Hq;
  const int qb_rank = blockIdx.x / n_heads, bh = blockIdx.x % n_heads;
  const int b = bh / a.Hq, hq = bh % a.Hq, g = hq / a.group;
  const int qb = a.causal ? (a.n_qblocks - 1 - qb_rank) : qb_rank;  // heaviest first when causal
  const int q0 = qb * C::BM;
  const int off = a.Lk - a.Lq;
  const int W = a.window;

  // Key tiles of the work-group and the keys this lane's row sees.
  const int row_hi = min(q0 + C::BM, a.Lq) - 1;
  int j_lo = 0, j_hi = a.Lk - 1;
  if (a.causal) j_hi = min(j_hi, row_hi + off);
  if (W >= 0) {
    j_lo = max(j_lo, q0 + off - W);
    if (!a.causal) j_hi = min(j_hi, row_hi + off + W);
  }
  const int t_lo = j_lo / C::BN;
  const int t_hi = (j_hi >= j_lo) ? j_hi / C::BN + 1 : t_lo;
  const int qi = q0 + wave * 32 + l32;
  const uint32_t drop_bh = (uint32_t)bh;  // b * Hq + hq
  int jlo_row = 0, jhi_row = a.Lk - 1;
  if (a.causal) jhi_row = min(jhi_row, qi + off);
  if (W >= 0) {
    jlo_row = max(jlo_row, qi + off - W);
    if (!a.causal) jhi_row = min(jhi_row, qi + off + W);
  }
  if (qi >= a.Lq) jhi_row = jlo_row - 1;  // rows past Lq see nothing
  const int wr_lo = q0 + wave * 32, wr_hi = min(wr_lo + 31, a.Lq - 1);

  // Q and dO of this lane's row as B operands; the row's statistics.
  V8 qf[C::DSTEPS], gf[C::DSTEPS];
  float l2 = INFINITY, dvv = 0.f;
  {
    const size_t base = (((size_t)b * a.Lq + q0) * a.Hq + hq) * D;
    const uint32_t bytes = rows_range((long long)a.Lq - q0, (size_t)a.Hq * D, D, sizeof(E));
    const rsrc_t rq = make_rsrc((const E*)a.q + base, bytes);
    const rsrc_t rg = make_rsrc((const E*)a.dout + base, bytes);
    const uint32_t o = (uint32_t)(((size_t)(wave * 32 + l32) * a.Hq * D + 8 * hh) * sizeof(E));
#pragma unroll
    for (int s = 0; s < C::DSTEPS; ++s) {
      qf[s] = __builtin_bit_cast(V8, buf_load16(rq, o + 32 * s));
      gf[s] = __builtin_bit_cast(V8, buf_load16(rg, o + 32 * s));
    }
    if (qi < a.Lq) {
      const size_t so = ((size_t)b * a.Hq + hq) * a.Lq + qi;
      l2 = a.L2[so];
      dvv = a.Dv[so];
    }
  }

  int noff[C::DSTEPS];
#pragma unroll
  for (int s = 0; s < C::DSTEPS; ++s) noff[s] = hoff + l32 * D + (((2 * s + hh) ^ bswz(l32)) << 3);
  int toff[C::DT];
  {
    const int r = 4 * hh + (j16 >> 2);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const int col = 32 * dt + 16 * (grp & 1) + 4 * (j16 & 3);
      toff[dt] = hoff + r * D + ((((col >> 3) ^ bswz(r)) << 3) + 4 * ((col >> 2) & 1));
    }
  }

  const size_t kv_rs = (size_t)a.Hkv * D;
  const E* kb = (const E*)a.k + ((size_t)b * a.Lk * a.Hkv + g) * D;
  const E* vb = (const E*)a.v + ((size_t)b * a.Lk * a.Hkv + g) * D;
  uint32_t src[C::IPW];
#pragma unroll
  for (int i = 0; i < C::IPW; ++i) {
    const int r = (wave * C::IPW + i) * C::RPI + lane / C::CPR;
    const int p = lane % C::CPR;
    src[i] = (uint32_t)(((size_t)r * kv_rs + ((p ^ bswz(r)) << 3)) * sizeof(E));
  }
  auto issue = [&](int t, auto par) {
    constexpr int P = decltype(par)::value;
    const uint32_t bytes = t < t_hi ? rows_range((long long)a.Lk - (long long)t * C::BN, kv_rs, D, sizeof(E)) : 0u;
    const rsrc_t rk = make_rsrc(kb + (size_t)t * C::BN * kv_rs, bytes);
    const rsrc_t rv = make_rsrc(vb + (size_t)t * C::BN * kv_rs, bytes);
#pragma unroll
    for (int i = 0; i < C::IPW; ++i) {
      buf_load16_lds(rk, src[i], (P ? kt1 : kt0) + hoff + (wave * C::IPW + i) * C::RPI * D);
      buf_load16_lds(rv, src[i], (P ? vt1 : vt0) + hoff + (wave * C::IPW + i) * C::RPI * D);
    }
  };

  f32x16 dqacc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) dqacc[dt] = f32x16{};
  const float sl2 = a.scale_log2;

  // (SPLIT: t+1 below is this half's next tile, t+2.  The next tile is
  // issued even past the range, where it loads zeros: half 1's last body
  // may be such a tile, and its buffer must not hold an older tile.)
  auto body = [&](int t, auto par) {
    constexpr int P = decltype(par)::value;
    if (SPLIT || t + TS < t_hi) issue(t + TS, Par<1 - P>{});
    const E* ks = P ? kt1 : kt0;
    const E* vs = P ? vt1 : vt0;
    // S^T = K Q^T and dP^T = V dO^T: 64 keys (two halves) x 32 rows.
    f32x16 st[2], pt[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      st[kh] = f32x16{};
      pt[kh] = f32x16{};
    }
    // Dropout: bit keep_bit(16*kh + r) keeps register r of half kh; registers 4g'..4g'+3
    // of half kh are the keys of the 4-key group with counter word 0 =
    // 16*t + 2*(4*kh + g') + hh, and the two rows of a pair sit in lanes l, l^1.
    // The four calls' forty rounds run between the products (round j after
    // k-step j * DSTEPS / 40), one call in flight, so the generator's vector
    // work overlaps the matrix unit.
    uint32_t kbits = 0u;
    if constexpr (DROP) {
      uint32_t c0 = (uint32_t)(16 * t + hh), row = (uint32_t)qi, k0 = a.seed_lo, k1 = a.seed_hi, dbh = drop_bh;
      asm volatile("" : "+v"(c0), "+v"(row), "+s"(k0), "+s"(k1), "+s"(dbh));
      const uint32_t thr2 = a.drop_thr | (a.drop_thr << 16);
      uint4 dc = make_uint4(0u, 0u, 0u, 0u);
      uint32_t acc_e = 0u, acc_o = 0u;
      static_for<C::DSTEPS>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          st[kh] = TT::mfma32(*(const V8*)(ks + noff[s] + kh * 32 * D), qf[s], st[kh]);
          pt[kh] = TT::mfma32(*(const V8*)(vs + noff[s] + kh * 32 * D), gf[s], pt[kh]);
        }
        static_for<40>([&](auto jc) {
          constexpr int j = decltype(jc)::value, k = j / 10, r = j % 10;
          if constexpr ((j * C::DSTEPS) / 40 == s) {
            if constexpr (r == 0) dc = keep_call(c0, row, dbh, a.drop_offset, k);
            philox_round(dc, k0 + (uint32_t)r * kPhiloxW0, k1 + (uint32_t)r * kPhiloxW1);
            if constexpr (r == 9) keep_fold(acc_e, acc_o, dc, thr2, k);
          }
        });
        __builtin_amdgcn_sched_barrier(0);
      });
      kbits = keep_finish(acc_e, acc_o, row);
    } else {
#pragma unroll
      for (int s = 0; s < C::DSTEPS; ++s) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          st[kh] = TT::mfma32(*(const V8*)(ks + noff[s] + kh * 32 * D), qf[s], st[kh]);
          pt[kh] = TT::mfma32(*(const V8*)(vs + noff[s] + kh * 32 * D), gf[s], pt[kh]);
        }
      }
    }
    // Register r of half kh is key t*BN + kh*32 + 8*(r/4) + 4*hh + r%4.
    const int jt = t * C::BN;
    const bool full = (jt + C::BN <= a.Lk) && (!a.causal || jt + C::BN - 1 <= wr_lo + off) &&
                      (W < 0 || jt >= wr_hi + off - W) && (W < 0 || a.causal || jt + C::BN - 1 <= wr_lo + off + W) &&
                      (wr_lo + 31 < a.Lq);
    uint32_t pw[4][4];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      float sv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = __builtin_fmaf(st[kh][r], sl2, -l2);
        if (!full) {
          const int j = jt + kh * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          x = (j >= jlo_row && j <= jhi_row) ? x : -INFINITY;
        }
        const float p = fast_exp2(x);
        if constexpr (DROP)
          sv[r] = p * __builtin_fmaf((float)((kbits >> keep_bit(16 * kh + r)) & 1u), pt[kh][r], -dvv);
        else
          sv[r] = p * (pt[kh][r] - dvv);
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) pw[2 * kh + (m >> 2)][m & 3] = pack2<TT>(sv[2 * m], sv[2 * m + 1]);
    }
    // dQ^T += K^T dS^T over the 4 key steps of 16.
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const V8 bs = __builtin_bit_cast(V8, make_uint4(pw[s][0], pw[s][1], pw[s][2], pw[s][3]));
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const E* k0p = ks + toff[dt] + 16 * s * D;
        dqacc[dt] = TT::mfma32(cat4<V4, V8>(TT::read_tr(k0p), TT::read_tr(k0p + 8 * D)), bs, dqacc[dt]);
      }
    }
    wait_vmem();
    __syncthreads();
  };

  if (t_lo < t_hi) {
    issue(t_lo + hf, Par<0>{});  // SPLIT: past the range (one tile) it loads zeros
    wait_vmem();
    __syncthreads();
    // Both halves run the same number of bodies (the barriers are the
    // work-group's); with an odd tile count half 1's last tile lies past the
    // range, holds zeros and is masked whole, so it adds nothing.
    const int n_it = (t_hi - t_lo + NH - 1) / NH;
    for (int i = 0; i < n_it; i += 2) {
      body(t_lo + hf + i * TS, Par<0>{});
      if (i + 1 < n_it) body(t_lo + hf + (i + 1) * TS, Par<1>{});
    }
  }

  if constexpr (SPLIT) {
    // Every load has landed and every wave passed the last barrier (or none
    // ran), so the tile buffers are free: half 1 leaves its sums in them,
    // lane for lane, and half 0 adds them.
    __syncthreads();
    float* xo[4] = {(float*)kt0, (float*)kt1, (float*)vt0, (float*)vt1};
    const int xi = wave * 64 + lane;
    if (hf == 1) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[dt][r * 256 + xi] = dqacc[dt][r];
    }
    __syncthreads();
    if (hf == 1) return;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) dqacc[dt][r] += xo[dt][r * 256 + xi];
  }
  E* dqrow = (E*)a.dq + (((size_t)b * a.Lq + qi) * a.Hq + hq) * D;
  if constexpr (DROP) {
    // The dropout instance has no registers to spare for the lane-pair swap
    // of store_row16 (its D = 128 kernel would spill): 8-byte stores.
    if (qi < a.Lq) {
      const float sc = a.scale * a.drop_scale;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(uint2*)(dqrow + 32 * dt + 8 * q4 + 4 * hh) =
              make_uint2(pack2<TT>(dqacc[dt][4 * q4] * sc, dqacc[dt][4 * q4 + 1] * sc),
                         pack2<TT>(dqacc[dt][4 * q4 + 2] * sc, dqacc[dt][4 * q4 + 3] * sc));
    }
  } else {
    store_row16<TT, C::DT>(dqrow, dqacc, a.scale, hh, qi < a.Lq);
  }
}

template <typename TT, int D, bool DROP = false>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  using C = BwdCfg<D>;
  const long long rows = (long long)a.B * a.Lq * a.Hq;
  hipError_t e = hipSuccess;
  if (rows > 0) {
    const long long pre_blocks = (rows + 256 / (D / 8) - 1) / (256 / (D / 8));
    hipLaunchKernelGGL((bwd_pre_kernel<TT, D>), dim3((unsigned)pre_blocks), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.Lk > 0) {
    const long long kblocks = (long long)((a.Lk + C::BK - 1) / C::BK) * a.B * a.Hkv;
    hipLaunchKernelGGL((bwd_dkdv_kernel<TT, D, DROP>), dim3((unsigned)kblocks), dim3(512), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long qblocks = (long long)a.n_qblocks * a.B * a.Hq;
  if (qblocks > 0) {
    if (a.kv_split)
      hipLaunchKernelGGL((bwd_dq_kernel<TT, D, DROP, true>), dim3((unsigned)qblocks), dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<TT, D, DROP, false>), dim3((unsigned)qblocks), dim3(256), 0, stream, a);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_bwd(const BwdArgs& a, int D, int dtype, hipStream_t stream) {
  if (dtype == 1) return D == 128 ? launch_bwd_t<BF16, 128>(a, stream) : launch_bwd_t<BF16, 64>(a, stream);
  return D == 128 ? launch_bwd_t<F16, 128>(a, stream) : launch_bwd_t<F16, 64>(a, stream);
}

hipError_t launch_bwd_dropout(const BwdArgs& a, int D, int dtype, hipStream_t stream) {
  if (dtype == 1)
    return D == 128 ? launch_bwd_t<BF16, 128, true>(a, stream) : launch_bwd_t<BF16, 64, true>(a, stream);
  return D == 128 ? launch_bwd_t<F16, 128, true>(a, stream) : launch_bwd_t<F16, 64, true>(a, stream);
}

}  // namespace attn
