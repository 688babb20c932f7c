// Shared pieces of the forward plane transforms (the matrix-core and the FFT variants): the
// launch arguments, the operand prologue and the final combine of the two real products.
#ifndef LIBFNO_PLANE_COMMON_H
#define LIBFNO_PLANE_COMMON_H

#include "fno_internal.h"
#include "pointwise.h"

namespace fno {

constexpr int kPlaneMaxModes = 32;  // m_a limit of the matrix-core plane transform

struct PlaneArgs {
  int Na, Nb, ma, mb;
  int64_t planes;
  int rows_per_chunk;
  const float* in0;
  const float* in1;
  const void* t1;        // [Nb][jpad] f32, or half bits (the plan's format)
  const void* f2;        // [4ma][Na] f32, or half bits (hi)
  const uint16_t* f2lo;  // half residual of f2 (half paths)
  const uint16_t* t1t;   // half t1 transposed, [jpad][Nb]
  float2* out;           // [nch][planes][2ma][mb]
};

template <int PIN>
__device__ __forceinline__ float prologue(float v, float w) {
  if (PIN == PLANE_TANH) return tanh_fast(v);
  if (PIN == PLANE_GELU_GRAD) return v * gelu_grad_as(w);
  if (PIN == PLANE_GELU) return gelu_as(v);
  if (PIN == PLANE_TANH_GELU) return tanh_gelu(v);
  return v;
}

__device__ __forceinline__ float cmp4(const float4& v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

// ------------------------------------------------------------------------------------------
// Combine X2 (cos rows 0..2ma-1, sin rows 2ma..4ma-1, interleaved re/im columns) held in LDS
// into the complex partial spectrum of this chunk.
__device__ __forceinline__ void combine_store(const float* s_x2, int jpad, int ma, int mb,
                                              float2* dst, int tid, int nthreads = 256) {
  for (int e = tid; e < 2 * ma * mb; e += nthreads) {
    const int sr = e / mb, k = e - sr * mb;
    const float* c = s_x2 + sr * jpad + 2 * k;
    const float* sn = s_x2 + (2 * ma + sr) * jpad + 2 * k;
    dst[e] = make_float2(c[0] + sn[1], c[1] - sn[0]);
  }
}

}  // namespace fno

#endif  // LIBFNO_PLANE_COMMON_H
