// Shared device helpers for the gfx950 attention kernels.
//
// MFMA lane layouts used throughout (CDNA4, wave64; verified on the device):
//  v_mfma_f32_32x32x16_{bf16,f16}: lane l holds A[l%32][8*(l/32)+e] and
//    B[8*(l/32)+e][l%32] (e = 0..7); accumulator register r of lane l is
//    C[8*(r/4) + 4*(l/32) + r%4][l%32].
//  v_mfma_f32_16x16x32_{bf16,f16}: lane l holds A[l%16][8*(l/16)+e] and
//    B[8*(l/16)+e][l%16]; register r of lane l is C[4*(l/16) + r][l%16].
//  v_mfma_f32_16x16x16_{bf16,f16}: as above with 4 elements per lane:
//    A[l%16][4*(l/16)+e], B[4*(l/16)+e][l%16] (e = 0..3); same C layout.
//  ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives
//    element i%4 of the 8-byte chunk addressed by group lane 4*e + i/4, for
//    e = 0..3.  Pointing group lane j at row (r0 + j/4), columns
//    (c0 + 4*(j%4) .. +3) of a row-major 16-bit matrix hands lane i the
//    column c0 + i of rows r0..r0+3: a transposed fetch of a 4 x 16 block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ranges.h"

#include <type_traits>
#include <utility>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// Element-type traits: storage is 16 bits; arithmetic is fp32 with MFMA.
struct BF16 {
  typedef __bf16 elem;
  typedef bf16x8 vec8;
  typedef bf16x4 vec4;
  static __device__ __forceinline__ f32x16 mfma32(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16k16(vec4 a, vec4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
  }
  static __device__ __forceinline__ vec4 read_tr(const void* lds) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(vec4, lds));
  }
  static __device__ __forceinline__ elem cvt(float x) { return (elem)x; }  // RNE
  static __device__ __forceinline__ float to_f32(elem x) { return (float)x; }
};

struct F16 {
  typedef _Float16 elem;
  typedef f16x8 vec8;
  typedef f16x4 vec4;
  static __device__ __forceinline__ f32x16 mfma32(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16k16(vec4 a, vec4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ vec4 read_tr(const void* lds) {
    typedef __fp16 h4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(vec4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(LDS_PTR(h4, lds)));
  }
  static __device__ __forceinline__ elem cvt(float x) { return (elem)x; }  // RNE
  static __device__ __forceinline__ float to_f32(elem x) { return (float)x; }
};

// Cache-policy operand of the buffer intrinsics on gfx950: bit 1 is NT
// (non-temporal: streamed data that should not stay in the caches).
constexpr int kCachePolicyNT = 2;

// Raw buffer access: a 128-bit resource (base, byte range) lets a load outside
// [0, bytes) return zeros without a branch.  The third word is the gfx9-family
// default (raw, untyped, 32-bit data).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ __forceinline__ int buf_load4(rsrc_t r, uint32_t byte_off) {
  return (int)__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0);
}
// Range-checked stores: a store outside [0, bytes) of its resource is dropped,
// so a resource of size 0 turns a store into a no-op without a branch.
typedef unsigned u32x4_t __attribute__((vector_size(16)));
typedef unsigned u32x2_t __attribute__((vector_size(8)));
__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t byte_off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, byte_off, 0, 0);
}
__device__ __forceinline__ void buf_store8(rsrc_t r, uint32_t byte_off, u32x2_t v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off, 0, 0);
}
__device__ __forceinline__ void buf_store4(rsrc_t r, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, byte_off, 0, 0);
}

// Memory reads written as inline assembly.  The compiler does not see what
// they read, so it adds no memory-counter wait for direct-to-LDS loads in
// flight; the caller places that wait (wait_vm).  Each block issues its reads
// and waits for them before it ends, so its outputs are complete when the
// statement completes.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
// s_waitcnt vmcnt(N): at most N vector-memory operations of this wave remain
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}
// Four 16-byte reads (ds_read_b128).
__device__ __forceinline__ void lds_read16_x4(u32x4_t (&r)[4], const uint32_t (&addr)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3])
      : "memory");
}
__device__ __forceinline__ void lds_read16_x2(u32x4_t (&r)[2], const uint32_t (&addr)[2]) {
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1])
      : "v"(addr[0]), "v"(addr[1])
      : "memory");
}
// Transposed reads (ds_read_b64_tr_b16, lane layout at the top of this file).
__device__ __forceinline__ void lds_read_tr8_x8(u32x2_t (&r)[8], const uint32_t (&addr)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
        "=&v"(r[7])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]),
        "v"(addr[7])
      : "memory");
}
// Four (two) 16-byte buffer loads, then s_waitcnt vmcnt(0): this also waits
// for every earlier vector-memory operation of the wave.
__device__ __forceinline__ void buf_load16_x4_sync(u32x4_t (&r)[4], rsrc_t rs, const uint32_t (&off)[4]) {
  asm volatile(
      "buffer_load_dwordx4 %0, %4, %8, 0 offen\n\t"
      "buffer_load_dwordx4 %1, %5, %8, 0 offen\n\t"
      "buffer_load_dwordx4 %2, %6, %8, 0 offen\n\t"
      "buffer_load_dwordx4 %3, %7, %8, 0 offen\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(rs)
      : "memory");
}
__device__ __forceinline__ void buf_load16_x2_sync(u32x4_t (&r)[2], rsrc_t rs, const uint32_t (&off)[2]) {
  asm volatile(
      "buffer_load_dwordx4 %0, %2, %4, 0 offen\n\t"
      "buffer_load_dwordx4 %1, %3, %4, 0 offen\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1])
      : "v"(off[0]), "v"(off[1]), "s"(rs)
      : "memory");
}
__device__ __forceinline__ void lds_read_tr8_x4(u32x2_t (&r)[4], const uint32_t (&addr)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3])
      : "memory");
}

// Direct global->LDS load: each of the 64 lanes fetches 16 bytes at
// byte_off inside the resource and the wave writes them to 1 KiB of LDS
// starting at lds_dst (lane i lands at lds_dst + 16*i).  Out-of-range lanes
// write zeros.  Completion is tracked by vmcnt (see wait_vmem()).
__device__ __forceinline__ void buf_load16_lds(rsrc_t r, uint32_t byte_off, void* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, byte_off, 0,
                                           0, 0);
}
// The 4-byte form: lane i's dword lands at lds_dst + 4*i.
__device__ __forceinline__ void buf_load4_lds(rsrc_t r, uint32_t byte_off, void* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 4, byte_off, 0,
                                           0, 0);
}
// s_waitcnt vmcnt(0): every vector-memory load of this wave has landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Compile-time buffer parity of a double-buffered loop body.
template <int P>
struct Par {
  static constexpr int value = P;
};

// Two fp32 values rounded (to nearest even) to the element type and packed.
template <typename TT>
__device__ __forceinline__ uint32_t pack2(float a, float b);
template <>
__device__ __forceinline__ uint32_t pack2<BF16>(float a, float b) {
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, (v2){(__bf16)a, (__bf16)b});
}
template <>
__device__ __forceinline__ uint32_t pack2<F16>(float a, float b) {
  typedef _Float16 v2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, (v2){(_Float16)a, (_Float16)b});
}

// One output row of the 32x32 MFMA accumulator layout, scaled by inv and
// rounded to the element type.  Lane l (row l mod 32, half hh = l / 32) holds
// columns 32*d + 8*q + 4*hh + 0..3 in registers 4q..4q+3 of block d, so lanes
// l and l^32 each hold half of every 8 columns.  One v_permlane32_swap per
// packed dword gives the low half-wave the 8 columns of q = 0 and 2 and the
// high half-wave those of q = 1 and 3, and each lane stores 16-byte pieces.
// The swaps run in every lane; store selects the lanes that write.
template <typename TT, int DB>
__device__ __forceinline__ void store_row16(void* orow, const f32x16 (&acc)[DB], float inv, int hh, bool store) {
  uint16_t* o = (uint16_t*)orow;  // 16-bit elements
#pragma unroll
  for (int d = 0; d < DB; ++d) {  // one block at a time: few extra registers live
    uint4 w[2];
#pragma unroll
    for (int qp = 0; qp < 2; ++qp) {
      uint32_t e[2][2];  // [q = 2*qp + i][dword]
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int q = 2 * qp + i;
        e[i][0] = pack2<TT>(acc[d][4 * q] * inv, acc[d][4 * q + 1] * inv);
        e[i][1] = pack2<TT>(acc[d][4 * q + 2] * inv, acc[d][4 * q + 3] * inv);
      }
      const auto x = __builtin_amdgcn_permlane32_swap(e[0][0], e[1][0], false, false);
      const auto y = __builtin_amdgcn_permlane32_swap(e[0][1], e[1][1], false, false);
      w[qp] = make_uint4(x[0], y[0], x[1], y[1]);
    }
    if (store) {
#pragma unroll
      for (int qp = 0; qp < 2; ++qp) *(uint4*)(o + 32 * d + 16 * qp + 8 * hh) = w[qp];
    }
  }
}

template <typename V4, typename V8>
__device__ __forceinline__ V8 cat4(V4 lo, V4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Reductions across lane l and lane l^32 (or l^16).  v_permlane32_swap trades
// the two 32-lane halves between its operands (v_permlane16_swap trades the
// odd and even 16-lane rows); with both operands = x, one result holds x[l]
// and the other x[l^32] (x[l^16]) in every lane, so their max/sum is the
// pairwise reduction, in one VALU op and without the LDS crossbar.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr float kLn2 = 0.69314718055994530942f;

// Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
// Shaw ("Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011): ten rounds,
// each taking the 32x32->64-bit products of word 0 by 0xD2511F53 and of word
// 2 by 0xCD9E8D57, and outputting (hi(w2-product) ^ x1 ^ k0, lo(w2-product),
// hi(w0-product) ^ x3 ^ k1, lo(w0-product)); the key grows by the Weyl
// increments (0x9E3779B9, 0xBB67AE85) after every round.  The key is
// wave-uniform where it is used, so its schedule runs on the scalar unit.
// A round is two v_mad_u64_u32 and two three-input XORs (v_bitop3_b32 with
// the truth table of a ^ b ^ c).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}
// One round with the round's key (k0r, k1r).
__device__ __forceinline__ void philox_round(uint4& c, uint32_t k0r, uint32_t k1r) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
  c = make_uint4(xor3((uint32_t)(p1 >> 32), c.y, k0r), (uint32_t)p1, xor3((uint32_t)(p0 >> 32), c.w, k1r), (uint32_t)p0);
}
// The Weyl increments of the key after every round.
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    philox_round(c, k0, k1);
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return c;
}

// 4x4 transpose inside each quad of lanes: lane q (q = lane % 4) holds row q
// of a 4x4 matrix in x[0..3] and ends with column q (x[c] = row c, column q).
// Two exchange stages across lane bits 0 and 1 (DPP quad permutations): at
// stage b, the elements whose index differs from the lane in bit b trade
// places with the partner lane's element of the mirrored index.
__device__ __forceinline__ void quad_transpose(uint32_t (&x)[4], int q) {
  constexpr int kSwap1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);  // quad_perm [1,0,3,2]
  constexpr int kSwap2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);  // quad_perm [2,3,0,1]
  const bool odd = q & 1, hi = q & 2;
#pragma unroll
  for (int e = 0; e < 4; e += 2) {  // pairs (0,1), (2,3)
    const uint32_t r = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? x[e] : x[e + 1]), kSwap1, 0xF, 0xF, false);
    if (odd) x[e] = r; else x[e + 1] = r;
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) {  // pairs (0,2), (1,3)
    const uint32_t r = (uint32_t)__builtin_amdgcn_mov_dpp((int)(hi ? x[e] : x[e + 2]), kSwap2, 0xF, 0xF, false);
    if (hi) x[e] = r; else x[e + 2] = r;
  }
}

// Dropout keep decisions.  Element (row i, key j) of head bh takes word j % 4
// of Philox4x32-10 at counter (j / 4, i / 2, bh, offset) under the seed's key;
// of that word the low 16 bits for even i and the high 16 bits for odd i; it
// is kept iff that number is >= thr = floor(p * 2^16).  One call thus decides
// four keys of two neighbouring rows.
//
// Drop flags of both halves of a word w: bit 0 set iff its low 16 bits are
// below thr, bit 16 iff its high 16 bits are (thr2 holds thr in both halves,
// ones2 holds 1 in both).  The saturating packed difference thr - half is
// zero exactly when the half is kept, and its minimum with 1 is the flag.
// (Written out: the compiler turns the same packed builtins into a compare,
// a select and a permute per half.)
__device__ __forceinline__ uint32_t drop_flags2(uint32_t w, uint32_t thr2, uint32_t ones2) {
  uint32_t d;
  asm("v_pk_sub_u16 %0, %1, %2 clamp\n\t"
      "v_pk_min_u16 %0, %0, %3"
      : "=&v"(d)
      : "s"(thr2), "v"(w), "s"(ones2));
  return d;
}

// Bit of element e (e = 0..31) in a 32-element keep mask in pair order:
// elements 2m and 2m+1 at bits m and 16 + m, so that one shift and one mask
// give a packed pair's two decisions as the 16-bit halves of a word.
__host__ __device__ constexpr int keep_bit(int e) { return (e >> 1) + 16 * (e & 1); }

// Keep mask of one row over eight 4-key groups whose counter words 0 are
// c0 + 2g (g = 0..7): element 4g + (key % 4) at bit keep_bit(element), set =
// kept.  For layouts with one row per lane in which the other row of the pair
// (row ^ 1) is in lane ^ 1 (and every lane of the wave is active): each lane
// draws the four calls of the groups g with g % 2 == row % 2 and the two
// lanes trade the decisions for each other's row.  In steps, so that a caller
// can spread the calls' rounds over other work:
//   keep_call(c0, row, bh, offset, k)   counter of this lane's call k (0..3);
//   keep_fold(acc_e, acc_o, r, thr2, k) folds call k's output r;
//   keep_finish(acc_e, acc_o, row)      the mask from the folded flags.
// Folding: word w of call k (keys 4g + w, g = 2k + row % 2) has its two rows'
// drop flags at bits 0 (even row) and 16 (odd row).  The flag of element
// e = 4g + w sits at keep_bit(e) = 2g + w/2 for even w and 16 + 2g + (w-1)/2
// for odd w, so even words are shifted into acc_e by 4k + w/2 and odd words
// into acc_o by 4k + (w-1)/2; the remaining 2 * (row % 2) is added at the end.
// Each accumulator then holds the even row's flags in its low half and the
// odd row's in its high half, and two byte permutes gather this lane's row
// (low half of acc_e, low half of acc_o moved up) and the other row.
__device__ __forceinline__ uint4 keep_call(uint32_t c0, uint32_t row, uint32_t bh, uint32_t offset, int k) {
  return make_uint4(c0 + 2u * (row & 1u) + 4u * (uint32_t)k, row >> 1, bh, offset);
}
__device__ __forceinline__ void keep_fold(uint32_t& acc_e, uint32_t& acc_o, uint4 r, uint32_t thr2, int k) {
  constexpr uint32_t ones2 = 0x00010001u;
  acc_e |= drop_flags2(r.x, thr2, ones2) << (4 * k);
  acc_o |= drop_flags2(r.y, thr2, ones2) << (4 * k);
  acc_e |= drop_flags2(r.z, thr2, ones2) << (4 * k + 1);
  acc_o |= drop_flags2(r.w, thr2, ones2) << (4 * k + 1);
}
__device__ __forceinline__ uint32_t keep_finish(uint32_t acc_e, uint32_t acc_o, uint32_t row) {
  const uint32_t par = row & 1u;
  acc_e <<= 2u * par;
  acc_o <<= 2u * par;
  // Bytes 0-3 of acc_e and 4-7 of acc_o: this row's half of each, then the
  // other row's.
  const uint32_t sel_mine = par ? 0x07060302u : 0x05040100u;
  const uint32_t sel_other = par ? 0x05040100u : 0x07060302u;
  const uint32_t mine = __builtin_amdgcn_perm(acc_o, acc_e, sel_mine);
  const uint32_t other = __builtin_amdgcn_perm(acc_o, acc_e, sel_other);
  constexpr int kSwapPairs = 1 | (0 << 2) | (3 << 4) | (2 << 6);  // quad_perm [1,0,3,2]
  const uint32_t got = (uint32_t)__builtin_amdgcn_mov_dpp((int)other, kSwapPairs, 0xF, 0xF, false);
  return ~(mine | got);
}
__device__ __forceinline__ uint32_t keep_bits_row_pair(uint32_t c0, uint32_t row, uint32_t bh, uint32_t offset,
                                                       uint32_t k0, uint32_t k1, uint32_t thr) {
  const uint32_t thr2 = thr | (thr << 16);
  uint32_t acc_e = 0u, acc_o = 0u;
#pragma unroll
  for (int k = 0; k < 4; ++k) keep_fold(acc_e, acc_o, philox4x32_10(keep_call(c0, row, bh, offset, k), k0, k1), thr2, k);
  return keep_finish(acc_e, acc_o, row);
}

// f(std::integral_constant<int, i>) for i = 0..N-1, expanded at compile time,
// so that per-iteration indices (register array slots, schedule positions)
// are constants.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace attn
