// Device helpers shared by the libiskv kernels: storage-type conversion and
// RoPE angles from the precomputed tables.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

#include "iskv_internal.hpp"

namespace iskv {

// bf16 is carried as its uint16 bit pattern.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> struct Store;
template <> struct Store<float> {
  static __device__ __forceinline__ float load(const float *p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float *p, size_t i, float v) { p[i] = v; }
};
template <> struct Store<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t *p, size_t i) {
    return bf16_to_f32(p[i].bits);
  }
  static __device__ __forceinline__ void store(bf16_t *p, size_t i, float v) {
    p[i].bits = f32_to_bf16(v);
  }
};

// cos, sin of pos * theta_i for frequency i < 64, from the anchor table
// (multiples of 64 positions) and the step table (offsets 0..63), by the
// angle-addition identity.  Both tables hold float values of float64-exact
// angles, so the result is within a few float ulps for any position covered.
// the two table entries whose product is the rotation of position pos for
// frequency i, and that product
__device__ __forceinline__ void rope_load(const Shared &S, int64_t pos, int i, float2 &A, float2 &B) {
  const int64_t a = pos / kRopeAnchor;
  const int o = (int)(pos - a * kRopeAnchor);
  A = reinterpret_cast<const float2 *>(S.rope_anchor)[a * 64 + i];
  B = reinterpret_cast<const float2 *>(S.rope_step)[o * 64 + i];
}
__device__ __forceinline__ void rope_combine(float2 A, float2 B, float &c, float &s) {
  c = A.x * B.x - A.y * B.y;
  s = A.y * B.x + A.x * B.y;
}
__device__ __forceinline__ void rope_cs(const Shared &S, int64_t pos, int i, float &c, float &s) {
  float2 A, B;
  rope_load(S, pos, i, A, B);
  rope_combine(A, B, c, s);
}

__device__ __forceinline__ void set_flag(const Shared &S, int f) { atomicOr(S.flags, f); }

// MFMA operand types and wrappers (gfx950).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short short4_ __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef unsigned uint4_ __attribute__((ext_vector_type(4)));
typedef unsigned uint2_ __attribute__((ext_vector_type(2)));

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// (a, b) -> packed bf16 high parts (round to nearest even) and low parts.
__device__ __forceinline__ void split2(float a, float b, unsigned &hi, unsigned &lo) {
  const bf16x2 h = __builtin_convertvector((floatx2){a, b}, bf16x2);
  const unsigned hb = __builtin_bit_cast(unsigned, h);
  const float ha = __uint_as_float(hb << 16), hh = __uint_as_float(hb & 0xffff0000u);
  const bf16x2 l = __builtin_convertvector((floatx2){a - ha, b - hh}, bf16x2);
  hi = hb;
  lo = __builtin_bit_cast(unsigned, l);
}

// (a, b) -> three packed bf16 parts: hi + mid + lo represents each value to
// ~2^-24 relative (every float whose exponent leaves room for the low part).
__device__ __forceinline__ void split3(float a, float b, unsigned &hi, unsigned &mid, unsigned &lo) {
  const bf16x2 h = __builtin_convertvector((floatx2){a, b}, bf16x2);
  const unsigned hb = __builtin_bit_cast(unsigned, h);
  const float ra = a - __uint_as_float(hb << 16), rb = b - __uint_as_float(hb & 0xffff0000u);
  const bf16x2 m = __builtin_convertvector((floatx2){ra, rb}, bf16x2);
  const unsigned mb = __builtin_bit_cast(unsigned, m);
  const bf16x2 l = __builtin_convertvector(
      (floatx2){ra - __uint_as_float(mb << 16), rb - __uint_as_float(mb & 0xffff0000u)}, bf16x2);
  hi = hb;
  mid = mb;
  lo = __builtin_bit_cast(unsigned, l);
}

// The same split with each residual x - hi(x) from one v_dot2c_f32_bf16: the
// packed high parts dotted with bf16 (-1, 0) or (0, -1) and accumulated onto
// x (exact: the products and the sum are exact in fp32).  The two constant
// operands sit in scalar registers (SplitK, made once per kernel): written
// as immediates, these packed bf16 pairs are not encoded as intended.
struct SplitK {
  unsigned m0, m1;       // bf16 (-1, 0) and (0, -1), element 0 in the low half
};
__device__ __forceinline__ SplitK split_consts() {
  unsigned m0 = 0x0000BF80u, m1 = 0xBF800000u;
  asm volatile("" : "+s"(m0), "+s"(m1));
  return SplitK{m0, m1};
}
__device__ __forceinline__ void split2(float a, float b, unsigned &hi, unsigned &lo, SplitK k) {
  const bf16x2 h = __builtin_convertvector((floatx2){a, b}, bf16x2);
  const float la = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, k.m0), a, false);
  const float lb = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, k.m1), b, false);
  const bf16x2 l = __builtin_convertvector((floatx2){la, lb}, bf16x2);
  hi = __builtin_bit_cast(unsigned, h);
  lo = __builtin_bit_cast(unsigned, l);
}

// (a, b) -> packed fp16 (round to nearest even), and the fp16 remainder of
// each: hi + lo holds a float to ~2^-22 relative.
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ unsigned pack_f16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((floatx2){a, b}, halfx2));
}
__device__ __forceinline__ void split2_f16(float a, float b, unsigned &hi, unsigned &lo) {
  const halfx2 h = __builtin_convertvector((floatx2){a, b}, halfx2);
  hi = __builtin_bit_cast(unsigned, h);
  lo = pack_f16(a - (float)h.x, b - (float)h.y);
}
__device__ __forceinline__ floatx4 mfma32h(uint4_ a, uint4_ b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, a),
                                                __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
}
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ floatx4 mfma16h(uint2_ a, uint2_ b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(halfx4, a), __builtin_bit_cast(halfx4, b), c,
                                               0, 0, 0);
}
// two bf16 (low half first) -> two fp16: exact for |x| <= 65504 down to the
// fp16 normal range (bf16 carries 8 significant bits, fp16 11); larger
// magnitudes saturate at 65504 (round toward zero)
__device__ __forceinline__ unsigned bf16x2_to_f16x2(unsigned x) {
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(x << 16),
                                                                 __uint_as_float(x & 0xffff0000u)));
}
__device__ __forceinline__ floatx4 mfma32(uint4_ a, uint4_ b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(uint2_ a, uint2_ b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_, a),
                                                   __builtin_bit_cast(short4_, b), c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// reductions over the four lane rows (lanes l, l^16, l^32, l^48)
// v_permlane16_swap / v_permlane32_swap with both operands = v return the
// pair (v[l], v[l ^ 16]) (resp. ^ 32) in some order in every lane, without
// the LDS round trip of a lane shuffle.
// max(a, b) as the median of (a, b, +inf): no operand canonicalization
__device__ __forceinline__ float max2(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, INFINITY); }
__device__ __forceinline__ float xor16_max(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max2(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max2(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float row_max(float v) { return xor32_max(xor16_max(v)); }
__device__ __forceinline__ float row_sum(float v) { return xor32_sum(xor16_sum(v)); }

}  // namespace iskv
