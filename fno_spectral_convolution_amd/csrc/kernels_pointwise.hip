// Pointwise lift / projection of an FNO stack on the matrix cores:
//   hidden == 0:  y[o][p] = b1[o] + sum_c W1[o][c] x[c][p]
//   hidden  > 0:  y[o][p] = b2[o] + sum_h W2[o][h] GELU(b1[h] + sum_c W1[h][c] x[c][p])
// (the lift and the two-layer projection around the spectral blocks; model-parallel FNO page,
// "Proposed method").  A work-group takes 64 consecutive points of one batch entry: the x
// tile [cin][64] is staged in LDS, the first product (M = hidden or cout, K = cin, N = 64)
// runs as 16x16x4 f32 MFMAs with bias and GELU applied to its fragments, the hidden tile goes
// to LDS and feeds the second product (M = cout, K = hidden); the output tile leaves through
// LDS as row-contiguous float4 stores.  Waves take M-tiles round-robin; weight fragments are
// read through L2.  Point tails are zero-filled on load and masked on store.
#include "fno_internal.h"
#include "mfma.h"
#include "pointwise.h"

namespace fno {

constexpr int kPwP = 64;        // points per work-group
constexpr int kPwS = kPwP + 4;  // LDS row stride (floats)

// D[M][64] += W[M rows][K] . S[K][64] over N-tiles nt0 .. nt0 + NN - 1 of M-tile mt; W
// row-major with row stride ldw.  Fragment of M-tile mt, N-tile nt: lane (m, q), register r
// <-> row 16 mt + 4 q + r, column 16 nt + m.  K-step ks uses k = 4 ks + q.
// bias[i] for i < n, else 0 (bias may be null: a uniform branch); unconditional clamped load
__device__ __forceinline__ float masked_bias(const float* __restrict__ bias, int i, int n) {
  if (!bias) return 0.f;
  const float v = bias[min(i, n - 1)];
  return __uint_as_float(__float_as_uint(v) & (i < n ? 0xffffffffu : 0u));
}

template <int NN>
__device__ __forceinline__ void pw_tile(const float* __restrict__ w, int ldw, int M, int K,
                                        const float* s_in, int mt, int nt0, int m, int q,
                                        f32x4 (&acc)[NN]) {
  const int row = 16 * mt + m;
  const bool row_ok = row < M;
  const float* wr = w + min(row, M - 1) * ldw;
  // groups of 4 K-steps: the 4 weight loads (through L2) go out together.  Loads are
  // unconditional (clamped index) and masked, so none of them can be moved into a branch;
  // K-steps past K read zero rows of s_in (it holds 16-row multiples).
  for (int ks0 = 0; ks0 < (K + 15) / 16 * 4; ks0 += 4) {
    float a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = 4 * (ks0 + j) + q;
      const float wv = wr[min(k, K - 1)];
      const uint32_t keep = (row_ok && k < K) ? 0xffffffffu : 0u;
      a[j] = __uint_as_float(__float_as_uint(wv) & keep);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = 4 * (ks0 + j) + q;
#pragma unroll
      for (int jj = 0; jj < NN; ++jj)
        acc[jj] = mfma_f32(a[j], s_in[k * kPwS + 16 * (nt0 + jj) + m], acc[jj]);
    }
  }
}

__global__ void __launch_bounds__(256)
k_pointwise_mfma(int64_t npts, int cin, int hidden, int cout, const float* __restrict__ x,
                 const float* __restrict__ w1, const float* __restrict__ b1,
                 const float* __restrict__ w2, const float* __restrict__ b2,
                 float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) float s_pw[];
  const int cin_p = (cin + 15) / 16 * 16;
  const int mid = hidden > 0 ? hidden : cout;   // rows of the first product
  const int mid_p = (mid + 15) / 16 * 16;
  const int cout_p = (cout + 15) / 16 * 16;
  float* s_x = s_pw;                             // [cin_p][kPwS], cin_p = 16-row multiple
  float* s_h = s_x + cin_p * kPwS;               // [mid_p][kPwS]  (hidden tile or output)
  float* s_y = hidden > 0 ? s_h + mid_p * kPwS : s_h;  // [cout_p][kPwS]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  const int b = blockIdx.y;
  const int64_t p0 = (int64_t)blockIdx.x * kPwP;
  const int np = (int)min((int64_t)kPwP, npts - p0);
  // x tile: rows >= cin and points past the end are zero.  Full tiles use float4 loads, four
  // per thread issued together (row c, points 4 f .. 4 f + 3 for item c * 16 + f).
  if (np == kPwP && (npts % 4) == 0) {
    const float* xb = x + (int64_t)b * cin * npts + p0;
    for (int e0 = tid; e0 < cin_p * (kPwP / 4); e0 += 4 * 256) {
      float4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = e0 + 256 * j;
        const int c = min(e / (kPwP / 4), cin - 1), f = e % (kPwP / 4);
        v[j] = *reinterpret_cast<const float4*>(xb + (int64_t)c * npts + 4 * f);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = e0 + 256 * j;
        const int c = e / (kPwP / 4), f = e % (kPwP / 4);
        if (c < cin_p) {
          const bool live = c < cin;
          *reinterpret_cast<float4*>(s_x + c * kPwS + 4 * f) =
              live ? v[j] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
  } else {
    for (int e = tid; e < cin_p * kPwP; e += 256) {
      const int c = e / kPwP, pp = e % kPwP;
      float v = 0.f;
      if (c < cin && pp < np) v = x[((int64_t)b * cin + c) * npts + p0 + pp];
      s_x[c * kPwS + pp] = v;
    }
  }
  __syncthreads();
  for (int mt = wave; mt < mid_p / 16; mt += 4) {
    f32x4 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = zero4();
    pw_tile<4>(w1, cin, mid, cin, s_x, mt, 0, m, q, acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 16 * mt + 4 * q + r;
      const float bh = masked_bias(b1, h, mid);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float v = acc[nt][r] + bh;
        const float gv = gelu_as(v);
        s_h[h * kPwS + 16 * nt + m] = hidden > 0 ? (h < mid ? gv : 0.f) : v;
      }
    }
  }
  __syncthreads();
  if (hidden > 0) {
    // (M-tile, N-tile) pairs round-robin over the waves: a narrow output (one M-tile) still
    // keeps all four waves busy
    for (int u = wave; u < (cout_p / 16) * 4; u += 4) {
      const int mt = u / 4, nt = u % 4;
      f32x4 acc[1] = {zero4()};
      pw_tile<1>(w2, hidden, cout, hidden, s_h, mt, nt, m, q, acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = 16 * mt + 4 * q + r;
        const float bo = masked_bias(b2, o, cout);
        s_y[o * kPwS + 16 * nt + m] = acc[0][r] + bo;
      }
    }
    __syncthreads();
  }
  // row-contiguous stores: 16 threads per output row of 64 points
  for (int e = tid; e < cout * (kPwP / 4); e += 256) {
    const int o = e / (kPwP / 4), c4 = e % (kPwP / 4);
    const float4 v = *reinterpret_cast<const float4*>(s_y + o * kPwS + 4 * c4);
    float* dst = y + ((int64_t)b * cout + o) * npts + p0 + 4 * c4;
    if (4 * c4 + 4 <= np && (npts % 4) == 0) {
      *reinterpret_cast<float4*>(dst) = v;
    } else {
      if (4 * c4 + 0 < np) dst[0] = v.x;
      if (4 * c4 + 1 < np) dst[1] = v.y;
      if (4 * c4 + 2 < np) dst[2] = v.z;
      if (4 * c4 + 3 < np) dst[3] = v.w;
    }
  }
}

hipError_t launch_pointwise(int64_t batch, int64_t npts, int cin, int hidden, int cout,
                            const float* x, const float* w1, const float* b1, const float* w2,
                            const float* b2, float* y, hipStream_t s) {
  const int cin_p = (cin + 15) / 16 * 16;
  const int mid = hidden > 0 ? hidden : cout;
  const int mid_p = (mid + 15) / 16 * 16;
  const int cout_p = (cout + 15) / 16 * 16;
  const size_t lds = sizeof(float) * kPwS * (cin_p + mid_p + (hidden > 0 ? cout_p : 0));
  const int64_t tiles = (npts + kPwP - 1) / kPwP;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  if (lds > 65536) {  // wide hidden layers need more than the default dynamic LDS limit
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_pointwise_mfma),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_pointwise_mfma, dim3((unsigned)tiles, (unsigned)batch), dim3(256), lds,
                     s, npts, cin, hidden, cout, x, w1, b1, w2, b2, y);
  return hipGetLastError();
}

}  // namespace fno
