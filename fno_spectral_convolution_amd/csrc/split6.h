// Float32 products on the bfloat16 matrix cores.
//
// A float32 value v splits exactly into three bfloat16 terms, v = h + m + l: h = bf16(v),
// m = bf16(v - h), l = bf16(v - h - m), each difference exact in float32 and each term
// carrying the next 8 of v's 24 significant bits.  A product a b then expands into nine
// products of terms; the six of order <= 2 (h h, h m, m h, h l, l h, m m) are kept and the
// three dropped ones (m l, l m, l l) are below 2^-23 |a b|, with float32 accumulation in the
// matrix core: the result matches a float32 product to float32 rounding.  On gfx950 a bfloat16
// 16x16x32 MFMA does 8 times the K of a float32 16x16x4 MFMA in half the cycles, so the six
// products cost 3/8 of the float32 ones per K.
#pragma once

#include "mfma.h"

namespace fno {

__device__ __forceinline__ void split3(float v, __bf16& h, __bf16& m, __bf16& l) {
  h = (__bf16)v;
  const float r1 = v - (float)h;
  m = (__bf16)r1;
  l = (__bf16)(r1 - (float)m);
}

__device__ __forceinline__ void split3_bf16x8(const float (&v)[8], bf16x8& h, bf16x8& m,
                                              bf16x8& l) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    __bf16 a, b, c;
    split3(v[e], a, b, c);
    h[e] = a;
    m[e] = b;
    l[e] = c;
  }
}

// acc + (a b) from the split operands: smallest terms first
__device__ __forceinline__ f32x4 mfma_split6(bf16x8 ah, bf16x8 am, bf16x8 al, bf16x8 bh,
                                             bf16x8 bm, bf16x8 bl, f32x4 acc) {
  f32x4 s = mfma_bf16(am, bm, zero4());
  s = mfma_bf16(ah, bl, s);
  s = mfma_bf16(al, bh, s);
  s = mfma_bf16(ah, bm, s);
  s = mfma_bf16(am, bh, s);
  s = mfma_bf16(ah, bh, s);
  return acc + s;
}

}  // namespace fno
