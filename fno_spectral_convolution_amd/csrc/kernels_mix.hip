// Per-mode complex channel mix of the FNO block and its two gradients:
//   forward   yhat[b,o,t] = sum_i xhat[b,i,t] W[c(t),i,o,kappa(t)]
//   input     ghx[b,i,t]  = sum_o ghat[b,o,t] conj(W[c(t),i,o,kappa(t)])
//   weight    dW[c,i,o,k] = sum_b conj(xhat[b,i,t]) ghat[b,o,t]
// with ghat scaled by gamma(k_last)/Ntot (the adjoint of the inverse transform).  The mix
// streams W once and is bound by that HBM read (B complex products per weight), so it runs
// on the vector ALUs: each thread owns one mode and kMixOB channels, keeps a batch tile of
// accumulators in registers and reads consecutive modes of W (and of the spectra) with its
// neighbours, so every load is coalesced.  On the mixed path every operand is rounded to
// bfloat16 before the product (the half-precision contraction of the mixed-precision
// neural-operator page, "Tiivistelmä"); accumulation is float32.
#include "fno_internal.h"

namespace fno {

constexpr int kMixOB = 4;  // output channels per thread
constexpr int kMixBT = 8;  // batch entries per pass

__device__ __forceinline__ float mround(float v, bool bf) {
  if (!bf) return v;
  uint32_t u = __float_as_uint(v);
  u += 0x7fffu + ((u >> 16) & 1u);
  return __uint_as_float(u & 0xffff0000u);
}

__device__ __forceinline__ float mix_adj_scale(const Geom& g, int64_t t) {
  const int kb = (int)(t % g.mb);
  const bool one = (kb == 0) || (2 * kb == g.Nb);
  return (one ? 1.0f : 2.0f) * g.inv_ntot;
}

__global__ void __launch_bounds__(256)
k_mix_fwd_blk(Geom g, const int32_t* __restrict__ mode_woff, const float2* __restrict__ xhat,
              const float2* __restrict__ w, float2* __restrict__ yhat) {
  const int64_t K = g.K;
  const int nob = (g.Cout + kMixOB - 1) / kMixOB;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)nob * K) return;
  const int ob = (int)(idx / K);
  const int64_t t = idx - (int64_t)ob * K;
  const int o0 = ob * kMixOB;
  const bool bf = g.bf16;
  const int64_t wb0 = mode_woff[t] + (int64_t)o0 * g.Mprod;
  const int64_t wsi = (int64_t)g.Cout * g.Mprod;
  for (int b0 = 0; b0 < g.B; b0 += kMixBT) {
    const int nb = min(kMixBT, g.B - b0);
    float2 acc[kMixOB][kMixBT];
#pragma unroll
    for (int j = 0; j < kMixOB; ++j)
#pragma unroll
      for (int b = 0; b < kMixBT; ++b) acc[j][b] = make_float2(0.f, 0.f);
    for (int ci = 0; ci < g.Cin; ++ci) {
      float2 wv[kMixOB];
#pragma unroll
      for (int j = 0; j < kMixOB; ++j) {
        float2 v = make_float2(0.f, 0.f);
        if (o0 + j < g.Cout) v = w[wb0 + ci * wsi + (int64_t)j * g.Mprod];
        wv[j] = make_float2(mround(v.x, bf), mround(v.y, bf));
      }
#pragma unroll
      for (int b = 0; b < kMixBT; ++b) {
        if (b >= nb) break;
        const float2 xv = xhat[((int64_t)(b0 + b) * g.Cin + ci) * K + t];
        const float xr = mround(xv.x, bf), xi = mround(xv.y, bf);
#pragma unroll
        for (int j = 0; j < kMixOB; ++j) {
          acc[j][b].x += xr * wv[j].x - xi * wv[j].y;
          acc[j][b].y += xr * wv[j].y + xi * wv[j].x;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kMixOB; ++j) {
      if (o0 + j >= g.Cout) break;
#pragma unroll
      for (int b = 0; b < kMixBT; ++b) {
        if (b >= nb) break;
        yhat[((int64_t)(b0 + b) * g.Cout + o0 + j) * K + t] = acc[j][b];
      }
    }
  }
}

__global__ void __launch_bounds__(256)
k_mix_bwd_dx_blk(Geom g, const int32_t* __restrict__ mode_woff, const float2* __restrict__ ghat,
                 const float2* __restrict__ w, float2* __restrict__ ghx) {
  const int64_t K = g.K;
  const int nib = (g.Cin + kMixOB - 1) / kMixOB;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)nib * K) return;
  const int ib = (int)(idx / K);
  const int64_t t = idx - (int64_t)ib * K;
  const int i0 = ib * kMixOB;
  const bool bf = g.bf16;
  const float sc = mix_adj_scale(g, t);
  const int64_t wb0 = mode_woff[t] + (int64_t)i0 * g.Cout * g.Mprod;
  const int64_t wsi = (int64_t)g.Cout * g.Mprod;
  for (int b0 = 0; b0 < g.B; b0 += kMixBT) {
    const int nb = min(kMixBT, g.B - b0);
    float2 acc[kMixOB][kMixBT];
#pragma unroll
    for (int j = 0; j < kMixOB; ++j)
#pragma unroll
      for (int b = 0; b < kMixBT; ++b) acc[j][b] = make_float2(0.f, 0.f);
    for (int o = 0; o < g.Cout; ++o) {
      float2 wv[kMixOB];
#pragma unroll
      for (int j = 0; j < kMixOB; ++j) {
        float2 v = make_float2(0.f, 0.f);
        if (i0 + j < g.Cin) v = w[wb0 + (int64_t)j * wsi + (int64_t)o * g.Mprod];
        wv[j] = make_float2(mround(v.x, bf), mround(v.y, bf));
      }
#pragma unroll
      for (int b = 0; b < kMixBT; ++b) {
        if (b >= nb) break;
        const float2 gv = ghat[((int64_t)(b0 + b) * g.Cout + o) * K + t];
        const float gr = mround(gv.x * sc, bf), gi = mround(gv.y * sc, bf);
#pragma unroll
        for (int j = 0; j < kMixOB; ++j) {  // (gr + i gi) conj(w)
          acc[j][b].x += gr * wv[j].x + gi * wv[j].y;
          acc[j][b].y += gi * wv[j].x - gr * wv[j].y;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kMixOB; ++j) {
      if (i0 + j >= g.Cin) break;
#pragma unroll
      for (int b = 0; b < kMixBT; ++b) {
        if (b >= nb) break;
        ghx[((int64_t)(b0 + b) * g.Cin + i0 + j) * K + t] = acc[j][b];
      }
    }
  }
}

// One thread per (mode, input channel, block of kMixOB output channels).
__global__ void __launch_bounds__(256)
k_mix_bwd_dw_blk(Geom g, const int32_t* __restrict__ mode_woff, const float2* __restrict__ xhat,
                 const float2* __restrict__ ghat, float2* __restrict__ dw) {
  const int64_t K = g.K;
  const int nob = (g.Cout + kMixOB - 1) / kMixOB;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)g.Cin * nob * K) return;
  const int64_t t = idx % K;
  const int64_t r = idx / K;
  const int ob = (int)(r % nob);
  const int ci = (int)(r / nob);
  const int o0 = ob * kMixOB;
  const bool bf = g.bf16;
  const float sc = mix_adj_scale(g, t);
  float2 acc[kMixOB];
#pragma unroll
  for (int j = 0; j < kMixOB; ++j) acc[j] = make_float2(0.f, 0.f);
  for (int b = 0; b < g.B; ++b) {
    const float2 xv = xhat[((int64_t)b * g.Cin + ci) * K + t];
    const float xr = mround(xv.x, bf), xi = mround(xv.y, bf);
#pragma unroll
    for (int j = 0; j < kMixOB; ++j) {
      if (o0 + j >= g.Cout) break;
      const float2 gv = ghat[((int64_t)b * g.Cout + o0 + j) * K + t];
      const float gr = mround(gv.x * sc, bf), gi = mround(gv.y * sc, bf);
      acc[j].x += xr * gr + xi * gi;  // conj(x) g
      acc[j].y += xr * gi - xi * gr;
    }
  }
  const int64_t wbase = mode_woff[t] + ((int64_t)ci * g.Cout + o0) * g.Mprod;
#pragma unroll
  for (int j = 0; j < kMixOB; ++j) {
    if (o0 + j >= g.Cout) break;
    dw[wbase + (int64_t)j * g.Mprod] = acc[j];
  }
}

hipError_t launch_mix_fwd(const fno_plan* p, const float2* xhat, int nparts,
                          int64_t part_stride, const float2* w, float2* yhat, hipStream_t s) {
  (void)nparts;
  (void)part_stride;
  const Geom& g = p->g;
  const int64_t total = (int64_t)((g.Cout + kMixOB - 1) / kMixOB) * g.K;
  hipLaunchKernelGGL(k_mix_fwd_blk, dim3((unsigned)((total + 63) / 64)), dim3(64), 0, s, g,
                     p->t.mode_woff, xhat, w, yhat);
  return hipGetLastError();
}

hipError_t launch_mix_bwd_dx(const fno_plan* p, const float2* ghat, const float2* w,
                             float2* ghx, hipStream_t s) {
  const Geom& g = p->g;
  const int64_t total = (int64_t)((g.Cin + kMixOB - 1) / kMixOB) * g.K;
  hipLaunchKernelGGL(k_mix_bwd_dx_blk, dim3((unsigned)((total + 63) / 64)), dim3(64), 0, s, g,
                     p->t.mode_woff, ghat, w, ghx);
  return hipGetLastError();
}

hipError_t launch_mix_bwd_dw(const fno_plan* p, const float2* xhat, const float2* ghat,
                             float2* dw, hipStream_t s) {
  const Geom& g = p->g;
  const int64_t total = (int64_t)g.Cin * ((g.Cout + kMixOB - 1) / kMixOB) * g.K;
  hipLaunchKernelGGL(k_mix_bwd_dw_blk, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     g, p->t.mode_woff, xhat, ghat, dw);
  return hipGetLastError();
}

}  // namespace fno
