// Thin wrappers over the gfx950 matrix-core builtins used by libfno, with their lane layouts.
//
// 16x16x4 f32  : A lane l holds A[l%16][l/16];            B holds B[l/16][l%16]
// 16x16x32 bf16 / f16: A lane l holds A[l%16][8*(l/16) + e];    B holds B[8*(l/16) + e][l%16]
// 16x16 result : lane l, register r holds D[4*(l/16) + r][l%16]
// (checked on the device against a host matrix product for these exact builtins)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fno {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// float -> bfloat16 round-to-nearest-even, as raw bits
__device__ __forceinline__ uint16_t bf16_bits(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));

// two floats -> packed bfloat16 pair (lo = a, hi = b), round-to-nearest-even; one
// v_cvt_pk_bf16_f32 on gfx950
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}

__device__ __forceinline__ bf16x8 to_bf16x8(float4 a, float4 b) {
  bf16x8 r;
  r[0] = (__bf16)a.x;
  r[1] = (__bf16)a.y;
  r[2] = (__bf16)a.z;
  r[3] = (__bf16)a.w;
  r[4] = (__bf16)b.x;
  r[5] = (__bf16)b.y;
  r[6] = (__bf16)b.z;
  r[7] = (__bf16)b.w;
  return r;
}

// Eight floats as a bfloat16 pair hi + lo: hi = bf16(v) and lo = bf16(v - hi), both rounded to
// nearest even.  v - hi is exact in float32 and |v - hi| <= 2^-9 |v|, so |v - (hi + lo)| <=
// 2^-18 |v|.  Three bf16 products hi*hi + hi*lo + lo*hi (exact in the float32 accumulator)
// then equal a*b up to about 3 * 2^-18 |a b|: the dropped lo*lo term and the two lo roundings.
__device__ __forceinline__ void split_bf16x8(const float (&v)[8], bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    h[k] = pack_bf16x2(v[2 * k], v[2 * k + 1]);
    const float h0 = __uint_as_float(h[k] << 16);
    const float h1 = __uint_as_float(h[k] & 0xffff0000u);
    l[k] = pack_bf16x2(v[2 * k] - h0, v[2 * k + 1] - h1);
  }
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}

// acc += a * b for split operands (three bf16 products, the small ones first)
__device__ __forceinline__ f32x4 mfma_split3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl,
                                             f32x4 acc) {
  acc = mfma_bf16(ah, bl, acc);
  acc = mfma_bf16(al, bh, acc);
  return mfma_bf16(ah, bh, acc);
}

// ---- half-precision operand formats ------------------------------------------------------
// H = 1: bfloat16 (fp32's exponent range, 8-bit significand); H = 2: IEEE half (5-bit
// exponent, 11-bit significand).  Operands travel as 16-bit patterns; an MFMA operand of 8
// values is Half<H>::v8.  Every conversion rounds to nearest even.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int H>
struct Half;

template <>
struct Half<1> {
  using elem = __bf16;
  using v8 = bf16x8;
  static __device__ __forceinline__ f32x4 mfma(v8 a, v8 b, f32x4 c) { return mfma_bf16(a, b, c); }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_bf16x2(a, b); }
  static __device__ __forceinline__ uint16_t bits(float v) { return bf16_bits(v); }
  static __device__ __forceinline__ float value(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
  }
};

template <>
struct Half<2> {
  using elem = _Float16;
  using v8 = f16x8;
  static __device__ __forceinline__ f32x4 mfma(v8 a, v8 b, f32x4 c) { return mfma_f16(a, b, c); }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    const f32x2_v v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_v));
  }
  static __device__ __forceinline__ uint16_t bits(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
  }
  static __device__ __forceinline__ float value(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
  }
};

// the format a kernel instantiated with H uses for its half operands (H = 0: fp32 kernels,
// whose half branches are never taken)
template <int H>
using HalfOf = Half<H == 0 ? 1 : H>;

// v rounded to the half format H (as a float)
template <int H>
__device__ __forceinline__ float round_half(float v) {
  return HalfOf<H>::value(HalfOf<H>::bits(v));
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// Streaming loads of a field: a kernel reads each of its elements once, so the loads carry the
// nontemporal hint and the lines are not kept for reuse, which leaves L2 and the memory-side
// cache to the data that is reused (tables, spectra, the lines other kernels write next).
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float4 load_stream4(const float* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float2 load_stream2(const float2* p) {
  const f32x2 v = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p));
  return make_float2(v[0], v[1]);
}

}  // namespace fno
