// FP8 (e4m3) attention forward.
//
// The forward-only FP8 path of the "Flash Attention" skill page (scenario 3:
// q, k, v cast to float8_e4m3fn, forward pass only), with per-tensor descale
// factors as in that interface: out = softmax(scale * dq*dk * q k^T) * dv*v,
// computed with v_mfma_f32_32x32x64_f8f6f4 (fp8 x fp8 -> fp32), output bf16.
//
// Per work-group (4 waves x 32 query rows of one head), per 64-key tile:
//   S^T = K Q^T      A = K rows from LDS (32 bytes per lane), B = the wave's
//                    Q rows (registers); one MFMA covers 64 of the head dim;
//   P   = exp2(S^T * scale * log2(e) - m)  in fp32, packed to e4m3 straight
//                    from the S^T accumulators as the B operand of
//   O^T += V^T P^T   one MFMA per 32-wide head-dim tile covers all 64 keys.
//                    V^T comes from four ds_read_b64_tr_b8 reads; each returns
//                    8 consecutive LDS rows of one head-dim column, and the
//                    direct-to-LDS loads place the tile's keys in the LDS row
//                    order that makes those 8 rows exactly the keys the lane's
//                    accumulator registers hold.
// The exponent base m moves only when a row's maximum exceeds it by more than
// 8 (base 2), and then to 8 below the new maximum, so the probabilities fill
// e4m3's range (0, 2^8] instead of sinking into its subnormals.  The row sum
// is accumulated in fp32 from the unrounded probabilities, so the lse is that
// of the fp8 inputs' exact scores.
#include <hip/hip_runtime.h>

#include "common.h"
#include "internal.h"

namespace attn {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

template <int D>
struct F8Cfg {
  static constexpr int BM = kPrefillBlockM;  // query rows per work-group
  static constexpr int BN = 64;              // keys per tile
  static constexpr int CPR = D / 16;         // 16-byte chunks per row
  static constexpr int RPI = 1024 / D;       // rows per 1 KiB direct-to-LDS load
  static constexpr int IPW = BN / RPI / 4;   // load instructions per wave per tile
  static constexpr int KS = D / 64;          // k-steps of S^T (64 head-dim bytes each)
  static constexpr int DT = D / 32;          // 32-wide head-dim tiles of O^T
  static constexpr int TILE = BN * D;        // bytes of a K or V tile
};

// Chunk swizzle inside a row: 16 consecutive rows of a row read, and the 8
// rows x 16 bytes of a transposed read, fall on distinct LDS banks.
template <int D>
__device__ __forceinline__ constexpr int f8swz(int r) {
  if constexpr (D == 128) return (r >> 1) & 7;
  else return (r >> 2) & 3;
}

// LDS row rho of a V tile holds key sigma(rho): rows 16j + 8hh + t (t < 8)
// hold the keys 32*(j/2) + 16*(j%2) + 8*(t/4) + 4*hh + t%4 -- the keys a lane
// of half hh holds in accumulator registers 8*(j%2)..8*(j%2)+7 of key half j/2.
__device__ __forceinline__ int vkey(int rho) {
  const int j = rho >> 4, hh = (rho >> 3) & 1, t = rho & 7;
  return 32 * (j >> 1) + 16 * (j & 1) + 8 * (t >> 2) + 4 * hh + (t & 3);
}

__device__ __forceinline__ i32x8 cat8(i32x2 a, i32x2 b, i32x2 c, i32x2 d) {
  return i32x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_fp8_kernel(F8Args a) {
  using C = F8Cfg<D>;
  __shared__ __attribute__((aligned(16))) unsigned char kt0[C::TILE];
  __shared__ __attribute__((aligned(16))) unsigned char kt1[C::TILE];
  __shared__ __attribute__((aligned(16))) unsigned char vt0[C::TILE];
  __shared__ __attribute__((aligned(16))) unsigned char vt1[C::TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, l32 = lane & 31, j16 = lane & 15, grp = lane >> 4;

  const int n_heads = a.B * a.Hq;
  const int qb_rank = blockIdx.x / n_heads, bh = blockIdx.x % n_heads;
  const int b = bh / a.Hq, hq = bh % a.Hq, g = hq / a.group;
  const int qb = a.causal ? (a.n_qblocks - 1 - qb_rank) : qb_rank;  // heaviest first when causal
  const int q0 = qb * C::BM;
  const int off = a.Lk - a.Lq;  // bottom-right alignment of the causal diagonal
  const int W = a.window;

  // Key tiles of the work-group; the keys this lane's row sees.
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
  int jlo_row = 0, jhi_row = a.Lk - 1;
  if (a.causal) jhi_row = min(jhi_row, qi + off);
  if (W >= 0) {
    jlo_row = max(jlo_row, qi + off - W);
    if (!a.causal) jhi_row = min(jhi_row, qi + off + W);
  }
  const int wr_lo = q0 + wave * 32, wr_hi = min(wr_lo + 31, a.Lq - 1);

  // Q operand (B of S^T): row qi, head-dim bytes 64*s + 32*hh .. +31.  The
  // kernel keeps the base-2 scale positive, so that the row maximum can be
  // taken on the raw scores and each probability is one FMA and one exp2: a
  // negative scale moves into Q (an exact sign flip of every e4m3 byte) and
  // a zero scale zeroes Q.
  float sl2 = a.scale_log2;
  uint32_t qsign = 0u, qkeep = 0xffffffffu;
  if (sl2 < 0.f) { qsign = 0x80808080u; sl2 = -sl2; }
  if (sl2 == 0.f) { qkeep = 0u; sl2 = 1.f; }
  i32x8 qf[C::KS];
  {
    const size_t base = (((size_t)b * a.Lq + q0) * a.Hq + hq) * D;
    const rsrc_t rq = make_rsrc((const unsigned char*)a.q + base, rows_range(a.Lq - q0, (size_t)a.Hq * D, D, 1));
    const uint32_t o = (uint32_t)((size_t)(wave * 32 + l32) * a.Hq * D + 32 * hh);
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const uint4 lo = buf_load16(rq, o + 64 * s), hi = buf_load16(rq, o + 64 * s + 16);
      qf[s] = i32x8{(int)((lo.x ^ qsign) & qkeep), (int)((lo.y ^ qsign) & qkeep), (int)((lo.z ^ qsign) & qkeep),
                    (int)((lo.w ^ qsign) & qkeep), (int)((hi.x ^ qsign) & qkeep), (int)((hi.y ^ qsign) & qkeep),
                    (int)((hi.z ^ qsign) & qkeep), (int)((hi.w ^ qsign) & qkeep)};
    }
  }

  // LDS offsets.  K row read: row l32 (+32 per key half), chunks 4s+2hh, +1.
  // The swizzle only permutes the chunk bits (4..log2(D)-1) of an offset, so
  // chunk c ^ x of a row is the row's chunk-0 offset with (c << 4) XORed in:
  // one base register per read kind, the rest folded into XOR immediates and
  // the LDS instructions' offset fields.
  const int kbase = l32 * D + (((2 * hh) ^ f8swz<D>(l32)) << 4);
  auto koff = [&](int s, int u) { return kbase ^ ((4 * s + u) << 4); };
  // V^T transposed read j of head-dim tile dt: rows 16j + 8hh + j16/2,
  // logical columns 32*dt + 16*(grp&1) + 8*(j16&1) .. +7.  The swizzle of
  // rows 16j + c does not depend on j (it uses bits 1-3 of the row at D=128
  // and 2-3 at D=64), so read j is read 0 plus 16*j rows.
  static_assert(f8swz<D>(16) == f8swz<D>(0), "the V swizzle has period 16 rows");
  const int vrow = 8 * hh + (j16 >> 1);
  const int vbase = vrow * D + ((((16 * (grp & 1)) >> 4) ^ f8swz<D>(vrow)) << 4) + 8 * (j16 & 1);
  auto voff = [&](int dt, int j) { return (vbase ^ ((2 * dt) << 4)) + 16 * j * D; };

  // Direct-to-LDS staging: lane -> LDS row (wave*IPW + i)*RPI + lane/CPR,
  // physical chunk lane%CPR, which holds logical chunk (lane%CPR) ^ swizzle.
  const size_t row_bytes = (size_t)a.Hkv * D;
  const unsigned char* kb = (const unsigned char*)a.k + ((size_t)b * a.Lk * a.Hkv + g) * D;
  const unsigned char* vb = (const unsigned char*)a.v + ((size_t)b * a.Lk * a.Hkv + g) * D;
  uint32_t ksrc[C::IPW], vsrc[C::IPW];
#pragma unroll
  for (int i = 0; i < C::IPW; ++i) {
    const int r = (wave * C::IPW + i) * C::RPI + lane / C::CPR;
    const int p = lane % C::CPR;
    ksrc[i] = (uint32_t)((size_t)r * row_bytes + ((p ^ f8swz<D>(r)) << 4));
    vsrc[i] = (uint32_t)((size_t)vkey(r) * row_bytes + ((p ^ f8swz<D>(r)) << 4));
  }
  auto issue = [&](int t, auto par) {
    constexpr int P = decltype(par)::value;
    const uint32_t bytes = t < t_hi ? rows_range((long long)a.Lk - (long long)t * C::BN, row_bytes, D, 1) : 0u;
    const rsrc_t rk = make_rsrc(kb + (size_t)t * C::BN * row_bytes, bytes);
    const rsrc_t rv = make_rsrc(vb + (size_t)t * C::BN * row_bytes, bytes);
#pragma unroll
    for (int i = 0; i < C::IPW; ++i) {
      buf_load16_lds(rk, ksrc[i], (P ? kt1 : kt0) + (wave * C::IPW + i) * C::RPI * D);
      buf_load16_lds(rv, vsrc[i], (P ? vt1 : vt0) + (wave * C::IPW + i) * C::RPI * D);
    }
  };

  f32x16 oacc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) oacc[dt] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.f;

  auto body = [&](int t, auto par) {
    constexpr int P = decltype(par)::value;
    if (t + 1 < t_hi) issue(t + 1, Par<1 - P>{});
    const unsigned char* ks = P ? kt1 : kt0;
    const unsigned char* vs = P ? vt1 : vt0;
    // S^T = K Q^T: two 32-key halves.
    f32x16 st[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      st[kh] = f32x16{};
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const uint4 lo = *(const uint4*)(ks + koff(s, 0) + kh * 32 * D);
        const uint4 hi = *(const uint4*)(ks + koff(s, 1) + kh * 32 * D);
        const i32x8 ka = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        st[kh] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qf[s], st[kh], 0, 0, 0, 0, 0, 0);
      }
    }
    // Register r of half kh is key t*BN + 32*kh + 8*(r/4) + 4*hh + r%4.
    const int jt = t * C::BN;
    const bool full = (jt + C::BN <= a.Lk) && (!a.causal || jt + C::BN - 1 <= wr_lo + off) &&
                      (W < 0 || jt >= wr_hi + off - W) && (W < 0 || a.causal || jt + C::BN - 1 <= wr_lo + off + W) &&
                      (wr_lo + 31 < a.Lq);
    // Raw scores (sl2 > 0 keeps their order); edge tiles are masked in one
    // rare branch, not per element.
    if (!full) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = jt + 32 * kh + 8 * (r >> 2) + 4 * hh + (r & 3);
          st[kh][r] = (j >= jlo_row && j <= jhi_row) ? st[kh][r] : -INFINITY;
        }
    }
    float x[32];
    float mx_a = -INFINITY, mx_b = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[16 * kh + r] = st[kh][r];
        if (r & 1) mx_b = fmaxf(mx_b, st[kh][r]);
        else mx_a = fmaxf(mx_a, st[kh][r]);
      }
    const float mx = max_xor32(fmaxf(mx_a, mx_b)) * sl2;  // -inf stays -inf
    // Move the exponent base only when this row's maximum passes it by > 8,
    // and then to 8 below the maximum (probabilities stay in (0, 2^8]).
    const bool need = mx > m_ref + 8.f;
    if (__any(need)) {
      if (need) {
        const float m_new = mx - 8.f;
        const float alpha = fast_exp2(m_ref - m_new);
        m_ref = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) oacc[dt] *= alpha;
      }
    }
    const float nb = m_ref == -INFINITY ? 0.f : -m_ref;
    int pk[8];  // P^T as the B operand: byte e = probability of register e%16 of half e/16
    float rs = 0.f;
#pragma unroll
    for (int w4 = 0; w4 < 8; ++w4) {
      const float p0 = fast_exp2(__builtin_fmaf(x[4 * w4], sl2, nb));
      const float p1 = fast_exp2(__builtin_fmaf(x[4 * w4 + 1], sl2, nb));
      const float p2 = fast_exp2(__builtin_fmaf(x[4 * w4 + 2], sl2, nb));
      const float p3 = fast_exp2(__builtin_fmaf(x[4 * w4 + 3], sl2, nb));
      rs += (p0 + p1) + (p2 + p3);
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
      pk[w4] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, w, true);
    }
    l_run += rs;
    const i32x8 pb = i32x8{pk[0], pk[1], pk[2], pk[3], pk[4], pk[5], pk[6], pk[7]};
    // O^T += V^T P^T: one MFMA per head-dim tile covers the 64 keys.
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const i32x8 va = cat8(__builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(i32x2, vs + voff(dt, 0))),
                            __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(i32x2, vs + voff(dt, 1))),
                            __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(i32x2, vs + voff(dt, 2))),
                            __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(i32x2, vs + voff(dt, 3))));
      oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, oacc[dt], 0, 0, 0, 0, 0, 0);
    }
    wait_vmem();
    __syncthreads();
  };

  if (t_lo < t_hi) {
    issue(t_lo, Par<0>{});
    wait_vmem();
    __syncthreads();
    for (int t = t_lo; t < t_hi; t += 2) {
      body(t, Par<0>{});
      if (t + 1 < t_hi) body(t + 1, Par<1>{});
    }
  }

  // Epilogue: O = dv * O^T / l in bf16; lse in natural log units.
  const float lt = sum_xor32(l_run);
  const float inv = lt > 0.f ? a.v_descale / lt : 0.f;
  store_row16<BF16, C::DT>((__bf16*)a.o + (((size_t)b * a.Lq + qi) * a.Hq + hq) * D, oacc, inv, hh, qi < a.Lq);
  if (qi < a.Lq) {
    if (a.lse != nullptr && hh == 0)
      a.lse[((size_t)b * a.Hq + hq) * a.Lq + qi] = lt > 0.f ? (m_ref + log2f(lt)) * kLn2 : -INFINITY;
  }
}

hipError_t launch_fwd_fp8(const F8Args& a, int D, hipStream_t stream) {
  const long long blocks = (long long)a.n_qblocks * a.Hq * a.B;
  if (D == 128)
    hipLaunchKernelGGL((fwd_fp8_kernel<128>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<64>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
