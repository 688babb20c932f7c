// Generic (any d = 2..4) kernels of the FNO spectral block: LDS-staged VALU versions.
//
// Every transform here is the truncated DFT of the block computed directly for the retained
// modes only ("spectral convolution from FNO's linear-algebra form" -- model-parallel FNO
// page, "Proposed method").  Twiddles come from per-axis root tables (cos, sin)(2 pi t / N)
// built on the host in float64; the index k*p is reduced modulo N in integers.
//
// Half paths (bfloat16 or IEEE-half operands, fp32 accumulation -- mixed-precision
// neural-operator page, "Tiivistelmä"): every operand of a transform or mix product
// (pre-activated input, twiddle, spectrum value, weight) is rounded to the plan's format
// (nearest-even) before the multiply; products and sums are float32.  IEEE-half plans scale each
// transform by 1/sqrt(N_j) in both directions (Geom::sc), as their tables do.
#include "fno_internal.h"
#include "pointwise.h"

#include <math.h>

namespace fno {

__device__ __forceinline__ float bf16r(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7fffu + ((u >> 16) & 1u);
  return __uint_as_float(u & 0xffff0000u);
}

// an operand in the plan's arithmetic: 0 fp32, 1 bfloat16, 2 IEEE half (nearest-even)
__device__ __forceinline__ float opnd(float v, int half) {
  return half == 2 ? (float)(_Float16)v : (half == 1 ? bf16r(v) : v);
}

__device__ __forceinline__ float gelu_f(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

__device__ __forceinline__ float gelu_grad_f(float z) {
  const float cdf = 0.5f * (1.0f + erff(z * 0.70710678118654752f));
  const float pdf = expf(-0.5f * z * z) * 0.39894228040143268f;
  return cdf + z * pdf;
}

// array index of retained position s of an outer axis (N, m): s < m -> s, else N - 2m + s
__device__ __forceinline__ int kidx(int s, int n, int m) { return s < m ? s : n - 2 * m + s; }

// ------------------------------------------------------------------------------------------
// Plane transform: rows [r_begin, r_end) of each [Na][Nb] plane -> partial spectrum
// [2ma][mb] (complex).  Grid (planes, nch), 256 threads.
constexpr int kPlaneThreads = 256;
constexpr int kPlaneRB = 8;          // rows staged per step
constexpr int kPlaneMaxAcc = 16;     // (2ma * mb) / 256 accumulators per thread

template <int PIN>
__global__ void __launch_bounds__(kPlaneThreads)
k_plane_fwd(Geom g, const float2* __restrict__ root_b, const float2* __restrict__ root_a,
            const float* __restrict__ in0, const float* __restrict__ in1,
            float2* __restrict__ out, int64_t planes, int rows_per_chunk) {
  extern __shared__ float smem[];
  const int Na = g.Na, Nb = g.Nb, ma = g.ma, mb = g.mb;
  float2* s_rb = reinterpret_cast<float2*>(smem);          // [Nb]
  float2* s_ra = s_rb + Nb;                                 // [Na]
  float2* s_R = s_ra + Na;                                  // [RB][mb]
  float* s_x = reinterpret_cast<float*>(s_R + kPlaneRB * mb);  // [RB][Nb]
  const int tid = threadIdx.x;
  const int64_t plane = blockIdx.x;
  const int chunk = blockIdx.y;
  const int bf = g.half;
  for (int t = tid; t < Nb; t += kPlaneThreads) s_rb[t] = root_b[t];
  for (int t = tid; t < Na; t += kPlaneThreads) s_ra[t] = root_a[t];
  const int r_begin = chunk * rows_per_chunk;
  const int r_end = min(Na, r_begin + rows_per_chunk);
  const int nout = 2 * ma * mb;
  float2 acc[kPlaneMaxAcc];
#pragma unroll
  for (int q = 0; q < kPlaneMaxAcc; ++q) acc[q] = make_float2(0.f, 0.f);
  const int64_t base = plane * (int64_t)Na * Nb;
  for (int r0 = r_begin; r0 < r_end; r0 += kPlaneRB) {
    const int nr = min(kPlaneRB, r_end - r0);
    __syncthreads();
    for (int e = tid; e < nr * Nb; e += kPlaneThreads) {
      const int64_t off = base + (int64_t)r0 * Nb + e;
      float v = in0[off];
      if (PIN == PLANE_GELU || PIN == PLANE_TANH_GELU) v = gelu_f(v);
      if (PIN == PLANE_TANH || PIN == PLANE_TANH_GELU) v = tanhf(v);
      if (PIN == PLANE_GELU_GRAD) v = v * gelu_grad_f(in1[off]);
      s_x[e] = opnd(v, bf);
    }
    __syncthreads();
    // last axis: R[r][k] = sum_c x[r][c] e^{-2 pi i k c / Nb}
    for (int e = tid; e < nr * mb; e += kPlaneThreads) {
      const int r = e / mb, k = e - r * mb;
      const float* xr = s_x + r * Nb;
      float re = 0.f, im = 0.f;
      int idx = 0;
      for (int c = 0; c < Nb; ++c) {
        const float2 w = s_rb[idx];
        const float xv = xr[c];
        re += xv * w.x;
        im -= xv * w.y;
        idx += k;
        if (idx >= Nb) idx -= Nb;
      }
      s_R[e] = make_float2(opnd(re, bf), opnd(im, bf));
    }
    __syncthreads();
    // axis a: X[s][k] += sum_r R[r][k] e^{-2 pi i ka(s) row / Na}
#pragma unroll
    for (int q = 0; q < kPlaneMaxAcc; ++q) {
      const int o = tid + q * kPlaneThreads;
      if (o < nout) {
        const int s = o / mb, k = o - s * mb;
        const int ka = kidx(s, Na, ma);
        float2 a = acc[q];
        for (int r = 0; r < nr; ++r) {
          const int row = r0 + r;
          const float2 w = s_ra[(int)(((int64_t)ka * row) % Na)];
          const float2 R = s_R[r * mb + k];
          a.x += R.x * w.x + R.y * w.y;
          a.y += R.y * w.x - R.x * w.y;
        }
        acc[q] = a;
      }
    }
  }
  float2* dst = out + ((int64_t)chunk * planes + plane) * nout;
#pragma unroll
  for (int q = 0; q < kPlaneMaxAcc; ++q) {
    const int o = tid + q * kPlaneThreads;
    if (o < nout) {
      const float sc = g.sc[g.d - 2] * g.sc[g.d - 1];
      dst[o] = make_float2(acc[q].x * sc, acc[q].y * sc);
    }
  }
}

hipError_t launch_plane_fwd(const fno_plan* p, int plane_in, int chans, const float* in0,
                            const float* in1, float2* out, hipStream_t s) {
  const bool al16 = ((uintptr_t)in0 % 16 == 0) && ((uintptr_t)in1 % 16 == 0);
  if (p->nch == 1 && al16 && plane_small_ok(p))
    return launch_plane_small(p, plane_in, chans, in0, in1, out, s);
  if (p->plane_fft) return launch_plane_fft(p, plane_in, chans, in0, in1, out, s);
  if (plane_fast_ok(p)) return launch_plane_fwd_fast(p, plane_in, chans, in0, in1, out, s);
  const Geom& g = p->g;
  const int64_t planes = (int64_t)g.B * chans * g.O;
  const int rows = p->plane_rows;
  dim3 grid((unsigned)planes, (unsigned)p->nch);
  const size_t lds = sizeof(float2) * (g.Nb + g.Na + kPlaneRB * g.mb) +
                     sizeof(float) * kPlaneRB * g.Nb;
  const float2* rb = g.bf16 ? p->t.root_bf[g.d - 1] : p->t.root[g.d - 1];
  const float2* ra = g.bf16 ? p->t.root_bf[g.d - 2] : p->t.root[g.d - 2];
  switch (plane_in) {
    case PLANE_X:
      hipLaunchKernelGGL(k_plane_fwd<PLANE_X>, grid, dim3(kPlaneThreads), lds, s, g, rb, ra,
                         in0, in1, out, planes, rows);
      break;
    case PLANE_TANH:
      hipLaunchKernelGGL(k_plane_fwd<PLANE_TANH>, grid, dim3(kPlaneThreads), lds, s, g, rb, ra,
                         in0, in1, out, planes, rows);
      break;
    case PLANE_GELU:
      hipLaunchKernelGGL(k_plane_fwd<PLANE_GELU>, grid, dim3(kPlaneThreads), lds, s, g, rb, ra,
                         in0, in1, out, planes, rows);
      break;
    case PLANE_TANH_GELU:
      hipLaunchKernelGGL(k_plane_fwd<PLANE_TANH_GELU>, grid, dim3(kPlaneThreads), lds, s, g, rb,
                         ra, in0, in1, out, planes, rows);
      break;
    default:
      hipLaunchKernelGGL(k_plane_fwd<PLANE_GELU_GRAD>, grid, dim3(kPlaneThreads), lds, s, g, rb,
                         ra, in0, in1, out, planes, rows);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Sum of `nparts` partial spectra (fixed order: deterministic).
__global__ void k_reduce_parts(const float2* __restrict__ in, int nparts, int64_t stride,
                               int64_t n, float2* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float2 a = in[i];
  for (int q = 1; q < nparts; ++q) {
    const float2 v = in[(int64_t)q * stride + i];
    a.x += v.x;
    a.y += v.y;
  }
  out[i] = a;
}

hipError_t launch_reduce_parts(const float2* in, int nparts, int64_t part_stride, int64_t n,
                               float2* out, hipStream_t s) {
  const int threads = 256;
  hipLaunchKernelGGL(k_reduce_parts, dim3((unsigned)((n + threads - 1) / threads)),
                     dim3(threads), 0, s, in, nparts, part_stride, n, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Truncated DFT along one outer axis j: in [pre][Lin][post] -> out [pre][Lout][post].
// Forward: Lin = N, Lout = 2m, out[s] = sum_p in[p] e^{-i 2 pi k(s) p / N}.
// Inverse: Lin = 2m, Lout = N, out[p] = sum_s in[s] e^{+i 2 pi k(s) p / N}.
template <bool INV>
__global__ void k_outer(const float2* __restrict__ root, int N, int m, int64_t pre,
                        int64_t post, const float2* __restrict__ in, float2* __restrict__ out,
                        int bf, float sc) {
  const int Lin = INV ? 2 * m : N;
  const int Lout = INV ? N : 2 * m;
  const int64_t total = pre * Lout * post;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t q = i % post;
  const int64_t r = i / post;
  const int lo = (int)(r % Lout);
  const int64_t pr = r / Lout;
  const float2* src = in + pr * Lin * post + q;
  float re = 0.f, im = 0.f;
  for (int li = 0; li < Lin; ++li) {
    const int k = INV ? kidx(li, N, m) : kidx(lo, N, m);
    const int p = INV ? lo : li;
    const float2 w = root[(int)(((int64_t)k * p) % N)];
    const float2 v = src[(int64_t)li * post];
    const float vr = opnd(v.x, bf), vi = opnd(v.y, bf);
    if (INV) {  // (vr + i vi)(c + i s)
      re += vr * w.x - vi * w.y;
      im += vi * w.x + vr * w.y;
    } else {    // (vr + i vi)(c - i s)
      re += vr * w.x + vi * w.y;
      im += vi * w.x - vr * w.y;
    }
  }
  out[i] = make_float2(re * sc, im * sc);
}

static void outer_shape(const fno_plan* p, int axis, int chans, bool inv, int64_t* pre,
                        int64_t* post) {
  const Geom& g = p->g;
  int64_t a = (int64_t)g.B * chans;
  for (int i = 0; i < axis; ++i) a *= g.N[i];
  int64_t b = g.mb;
  // forward transforms axes d-3..0 after the plane kernel: axes > axis are already 2m;
  // inverse transforms axes 0..d-2: axes > axis are still 2m.
  for (int i = axis + 1; i <= g.d - 2; ++i) b *= 2 * g.M[i];
  (void)inv;
  *pre = a;
  *post = b;
}

hipError_t launch_outer_fwd(const fno_plan* p, int axis, int chans, const float2* in,
                            int nparts, int64_t part_stride, float2* out, hipStream_t s) {
  (void)nparts;
  (void)part_stride;
  if (outer_fast_ok(p, axis, false)) return launch_outer_mfma(p, axis, chans, false, in, out, s);
  const Geom& g = p->g;
  int64_t pre, post;
  outer_shape(p, axis, chans, false, &pre, &post);
  const int64_t total = pre * 2 * g.M[axis] * post;
  const float2* root = g.bf16 ? p->t.root_bf[axis] : p->t.root[axis];
  hipLaunchKernelGGL(k_outer<false>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     root, g.N[axis], g.M[axis], pre, post, in, out, g.half, g.sc[axis]);
  return hipGetLastError();
}

hipError_t launch_outer_inv(const fno_plan* p, int axis, int chans, const float2* in,
                            float2* out, hipStream_t s) {
  if (outer_fast_ok(p, axis, true)) return launch_outer_mfma(p, axis, chans, true, in, out, s);
  const Geom& g = p->g;
  int64_t pre, post;
  outer_shape(p, axis, chans, true, &pre, &post);
  const int64_t total = pre * (int64_t)g.N[axis] * post;
  const float2* root = g.bf16 ? p->t.root_bf[axis] : p->t.root[axis];
  hipLaunchKernelGGL(k_outer<true>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     root, g.N[axis], g.M[axis], pre, post, in, out, g.half, g.sc[axis]);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Forward epilogue: y_spec from T [B][C][lines][mb] by the last-axis inverse (gamma/Ntot),
// then (EPI_BLOCK) + Wb x + bias and GELU.  One thread per point, 256 points per group.
constexpr int kEpiThreads = 128;

__global__ void __launch_bounds__(kEpiThreads)
k_epilogue_fwd(Geom g, int mode, bool gelu, bool ig, const float2* __restrict__ root_b,
               const float2* __restrict__ T, const float* __restrict__ x,
               const float* __restrict__ wb, const float* __restrict__ bias,
               float* __restrict__ y, float* __restrict__ zsave) {
  extern __shared__ float smem[];
  const int Cin = g.Cin, Cout = g.Cout, Nb = g.Nb, mb = g.mb;
  float2* s_rb = reinterpret_cast<float2*>(smem);            // [Nb]
  float* s_wb = reinterpret_cast<float*>(s_rb + Nb);         // [Cout][Cin]
  float* s_bias = s_wb + Cout * Cin;                         // [Cout]
  float* s_x = s_bias + Cout;                                // [Cin][256]
  const int tid = threadIdx.x;
  const int b = blockIdx.y;
  const int64_t P = g.P;
  const int64_t p = (int64_t)blockIdx.x * kEpiThreads + tid;
  const bool block = (mode == EPI_BLOCK);
  for (int t = tid; t < Nb; t += kEpiThreads) s_rb[t] = root_b[t];
  if (block) {
    for (int t = tid; t < Cout * Cin; t += kEpiThreads) s_wb[t] = wb[t];
    for (int t = tid; t < Cout; t += kEpiThreads) s_bias[t] = bias ? bias[t] : 0.f;
    for (int ci = 0; ci < Cin; ++ci) {
      const float xv = (p < P) ? x[((int64_t)b * Cin + ci) * P + p] : 0.f;
      s_x[ci * kEpiThreads + tid] = ig ? gelu_f(xv) : xv;  // the block's input
    }
  }
  __syncthreads();
  if (p >= P) return;
  const int64_t line = p / Nb;
  const int pb = (int)(p - line * Nb);
  const int64_t lines = P / Nb;
  const int bf = g.half;
  for (int o = 0; o < Cout; ++o) {
    const float2* tr = T + (((int64_t)b * Cout + o) * lines + line) * mb;
    float ys = 0.f;
    int idx = 0;
    for (int k = 0; k < mb; ++k) {
      const float2 tv = tr[k];
      const float2 w = s_rb[idx];
      const float gk = (k == 0 || 2 * k == Nb) ? 1.f : 2.f;
      ys += gk * (opnd(tv.x, bf) * w.x - opnd(tv.y, bf) * w.y);
      idx += pb;
      if (idx >= Nb) idx -= Nb;
    }
    float z = ys * (g.half == 2 ? g.sc[g.d - 1] * g.inv_gain[0] : g.inv_ntot);
    if (block) {
      float acc = s_bias[o];
      const float* wr = s_wb + o * Cin;
      for (int ci = 0; ci < Cin; ++ci) acc += wr[ci] * s_x[ci * kEpiThreads + tid];
      z += acc;
    }
    const int64_t off = ((int64_t)b * Cout + o) * P + p;
    if (zsave) zsave[off] = z;
    const float yv = (block && gelu) ? gelu_f(z) : z;
    raise_half_flag(g.half_flag, !__builtin_isfinite(yv));
    y[off] = yv;
  }
}

hipError_t launch_epilogue_fwd(const fno_plan* p, int mode, const float2* T, const float* x,
                               const float* wb, const float* bias, float* y, float* zsave,
                               hipStream_t s) {
  if (epilogue_fast_ok(p, mode, true))
    return launch_epilogue_fwd_fast(p, mode, T, x, wb, bias, y, zsave, s);
  const Geom& g = p->g;
  const bool gelu = mode == EPI_BLOCK && (p->desc.flags & FNO_FLAG_GELU) != 0;
  if (mode == EPI_BLOCK_PREACT) mode = EPI_BLOCK;  // the same kernel, without the GELU
  const size_t lds = sizeof(float2) * g.Nb +
                     sizeof(float) * ((size_t)g.Cout * g.Cin + g.Cout +
                                      (mode == EPI_BLOCK ? (size_t)g.Cin * kEpiThreads : 0));
  dim3 grid((unsigned)((g.P + kEpiThreads - 1) / kEpiThreads), (unsigned)g.B);
  const bool ig = (p->desc.flags & FNO_FLAG_INPUT_GELU) != 0;
  const float2* rb = g.bf16 ? p->t.root_bf[g.d - 1] : p->t.root[g.d - 1];
  hipLaunchKernelGGL(k_epilogue_fwd, grid, dim3(kEpiThreads), lds, s, g, mode, gelu, ig, rb, T, x,
                     wb, (p->desc.flags & FNO_FLAG_BIAS) ? bias : nullptr, y, zsave);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Backward epilogue.  grad_x[i] = sum_o Wb[o,i] g_z[o] (EPI_BLOCK) + s(x_i) gxs_i with
// gxs from Tg [B][Cin][lines][mb] by the unit-scale last-axis inverse; per-group partial
// sums of g_z x^T and g_z for the bypass gradients.  64 points per tile, one wave.
constexpr int kEbThreads = 64;
constexpr int kEbPairs = (64 * 64 + 64 + kEbThreads - 1) / kEbThreads;

__global__ void __launch_bounds__(kEbThreads)
k_epilogue_bwd(Geom g, int mode, bool gelu, bool tanh_pre, bool ig,
               const float2* __restrict__ root_b,
               const float2* __restrict__ Tg, const float* __restrict__ x,
               const float* __restrict__ wb, const float* __restrict__ gy,
               const float* __restrict__ z, float* __restrict__ grad_x,
               float* __restrict__ red_part, int64_t tiles_per_group) {
  extern __shared__ float smem[];
  const int Cin = g.Cin, Cout = g.Cout, Nb = g.Nb, mb = g.mb;
  float2* s_rb = reinterpret_cast<float2*>(smem);      // [Nb]
  float* s_wb = reinterpret_cast<float*>(s_rb + Nb);   // [Cout][Cin]
  float* s_gz = s_wb + Cout * Cin;                     // [Cout][128]
  float* s_x = s_gz + Cout * kEbThreads;               // [Cin][128]
  const int tid = threadIdx.x;
  const int b = blockIdx.y;
  const int64_t P = g.P;
  const bool block = (mode == EPI_BLOCK);
  const int bf = g.half;
  for (int t = tid; t < Nb; t += kEbThreads) s_rb[t] = root_b[t];
  if (block)
    for (int t = tid; t < Cout * Cin; t += kEbThreads) s_wb[t] = wb[t];
  const int npair = Cout * Cin + Cout;
  // per-thread partial sums of the bypass gradients: pairs tid, tid+128, ...
  float pacc[kEbPairs];
  const int my_pairs = block ? (npair + kEbThreads - 1) / kEbThreads : 0;
#pragma unroll
  for (int q = 0; q < kEbPairs; ++q) pacc[q] = 0.f;
  const int64_t lines = P / Nb;
  const int64_t t_begin = (int64_t)blockIdx.x * tiles_per_group;
  const int64_t t_end = min((P + kEbThreads - 1) / kEbThreads, t_begin + tiles_per_group);
  for (int64_t tile = t_begin; tile < t_end; ++tile) {
    const int64_t p = tile * kEbThreads + tid;
    const bool live = p < P;
    __syncthreads();
    if (block) {
      for (int o = 0; o < Cout; ++o) {
        float v = 0.f;
        if (live) {
          const int64_t off = ((int64_t)b * Cout + o) * P + p;
          v = gy[off];
          if (gelu) v *= gelu_grad_f(z[off]);
        }
        s_gz[o * kEbThreads + tid] = v;
      }
      for (int ci = 0; ci < Cin; ++ci) {
        const float xv = live ? x[((int64_t)b * Cin + ci) * P + p] : 0.f;
        s_x[ci * kEbThreads + tid] = ig ? gelu_f(xv) : xv;  // the block's input
      }
    }
    __syncthreads();
    if (live && grad_x) {
      const int64_t line = p / Nb;
      const int pb = (int)(p - line * Nb);
      for (int ci = 0; ci < Cin; ++ci) {
        const float2* tr = Tg + (((int64_t)b * Cin + ci) * lines + line) * mb;
        float gs = 0.f;
        int idx = 0;
        for (int k = 0; k < mb; ++k) {
          const float2 tv = tr[k];
          const float2 w = s_rb[idx];
          gs += opnd(tv.x, bf) * w.x - opnd(tv.y, bf) * w.y;
          idx += pb;
          if (idx >= Nb) idx -= Nb;
        }
        gs *= g.sc[g.d - 1] * g.inv_gain[1];  // 1 except on IEEE-half plans
        const int64_t off = ((int64_t)b * Cin + ci) * P + p;
        if (tanh_pre) {
          const float xv = block ? s_x[ci * kEbThreads + tid] : (ig ? gelu_f(x[off]) : x[off]);
          const float th = tanhf(xv);
          gs *= (1.f - th * th);
        }
        if (block) {
          float acc = 0.f;
          for (int o = 0; o < Cout; ++o) acc += s_wb[o * Cin + ci] * s_gz[o * kEbThreads + tid];
          gs += acc;
        }
        if (ig) gs *= gelu_grad_f(x[off]);  // the input was GELU(x)
        raise_half_flag(g.half_flag, !__builtin_isfinite(gs));
        grad_x[off] = gs;
      }
    }
    if (block) {
      for (int q = 0; q < my_pairs; ++q) {
        const int pr = tid + q * kEbThreads;
        if (pr < npair) {
          float a = 0.f;
          if (pr < Cout * Cin) {
            const int o = pr / Cin, ci = pr - o * Cin;
            const float* gz = s_gz + o * kEbThreads;
            const float* xv = s_x + ci * kEbThreads;
            for (int e = 0; e < kEbThreads; ++e) a += gz[e] * xv[e];
          } else {
            const float* gz = s_gz + (pr - Cout * Cin) * kEbThreads;
            for (int e = 0; e < kEbThreads; ++e) a += gz[e];
          }
          pacc[q] += a;
        }
      }
    }
  }
  if (block && red_part) {
    float* dst = red_part + ((int64_t)b * gridDim.x + blockIdx.x) * npair;
    for (int q = 0; q < my_pairs; ++q) {
      const int pr = tid + q * kEbThreads;
      if (pr < npair) dst[pr] = pacc[q];
    }
  }
}

hipError_t launch_epilogue_bwd(const fno_plan* p, int mode, const float2* Tg, const float* x,
                               const float* wb, const float* gy, const float* z,
                               float* grad_x, float* red_part, hipStream_t s) {
  if (epilogue_bwd_fast(p, mode, grad_x))
    return launch_epilogue_bwd_fast(p, mode, Tg, x, wb, gy, z, grad_x, red_part, s);
  const Geom& g = p->g;
  const int64_t tiles = (g.P + kEbThreads - 1) / kEbThreads;
  const int groups = p->nred / g.B;
  const int64_t tpg = (tiles + groups - 1) / groups;
  const size_t lds = sizeof(float2) * g.Nb +
                     sizeof(float) * ((size_t)g.Cout * g.Cin +
                                      (mode == EPI_BLOCK ? (size_t)(g.Cout + g.Cin) * kEbThreads
                                                         : 0));
  const bool gelu = z != nullptr;  // the caller passes z exactly when GELU' applies
  const bool tanh_pre = (p->desc.flags & FNO_FLAG_TANH_PREACT) != 0;
  const bool ig = (p->desc.flags & FNO_FLAG_INPUT_GELU) != 0;
  const float2* rb = g.bf16 ? p->t.root_bf[g.d - 1] : p->t.root[g.d - 1];
  hipLaunchKernelGGL(k_epilogue_bwd, dim3((unsigned)groups, (unsigned)g.B), dim3(kEbThreads),
                     lds, s, g, mode, gelu, tanh_pre, ig, rb, Tg, x, wb, gy, z, grad_x, red_part,
                     tpg);
  return hipGetLastError();
}

// Sum of the per-work-group bypass-gradient partials.  A group of 256 threads owns E
// consecutive entries; thread slice k (0..256/E-1) sums partials k, k+256/E, ... with 8 loads
// in flight, and the slice sums are added in the fixed order 0, 1, .. (deterministic).  E = 16
// reads 64-byte row segments where the grid still has at least 128 work-groups, else E = 8.
template <int E>
__global__ void __launch_bounds__(256)
k_bypass_finish(const float* __restrict__ part, int nparts, int cout, int cin,
                float* __restrict__ dwb, float* __restrict__ dbias) {
  constexpr int S = 256 / E;
  __shared__ float s_sum[S][E];
  const int npair = cout * cin + cout;
  const int el = threadIdx.x % E, slice = threadIdx.x / E;
  const int e = blockIdx.x * E + el;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (e < npair) {
    int q = slice;
    for (; q + 7 * S < nparts; q += 8 * S) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += part[(int64_t)(q + j * S) * npair + e];
    }
    for (; q < nparts; q += S) acc[0] += part[(int64_t)q * npair + e];
  }
  s_sum[slice][el] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  __syncthreads();
  if (slice == 0 && e < npair) {
    float v = 0.f;
    for (int k = 0; k < S; ++k) v += s_sum[k][el];
    if (e < cout * cin) {
      if (dwb) dwb[e] = v;
    } else if (dbias) {
      dbias[e - cout * cin] = v;
    }
  }
}

hipError_t launch_bypass_grad_finish(const fno_plan* p, const float* red_part, float* dwb,
                                     float* dbias, const float* grad_x, hipStream_t s) {
  const Geom& g = p->g;
  const int npair = g.Cout * g.Cin + g.Cout;
  const int nparts = epilogue_bwd_fast(p, EPI_BLOCK, grad_x) ? epilogue_bwd_fast_groups(p) : p->nred;
  if (npair >= 128 * 16)
    hipLaunchKernelGGL(k_bypass_finish<16>, dim3((npair + 15) / 16), dim3(256), 0, s, red_part,
                       nparts, g.Cout, g.Cin, dwb, dbias);
  else
    hipLaunchKernelGGL(k_bypass_finish<8>, dim3((npair + 7) / 8), dim3(256), 0, s, red_part,
                       nparts, g.Cout, g.Cin, dwb, dbias);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// MSE: g = 2 (y - t) / n; per-group partial sums in double, then one fixed-order finish.
__global__ void k_mse_part(int64_t n, const float* __restrict__ y, const float* __restrict__ t,
                           float* __restrict__ g, float grad_scale, double* __restrict__ part) {
  __shared__ double s_red[256];
  const int tid = threadIdx.x;
  const float sc = (float)(2.0 * (double)grad_scale / (double)n);
  double a = 0.0;
  const int64_t n4 = n / 4;
  const float4* y4 = reinterpret_cast<const float4*>(y);
  const float4* t4 = reinterpret_cast<const float4*>(t);
  float4* g4 = reinterpret_cast<float4*>(g);
  for (int64_t i = (int64_t)blockIdx.x * 256 + tid; i < n4; i += (int64_t)gridDim.x * 256) {
    const float4 yv = y4[i], tv = t4[i];
    const float4 d = make_float4(yv.x - tv.x, yv.y - tv.y, yv.z - tv.z, yv.w - tv.w);
    g4[i] = make_float4(sc * d.x, sc * d.y, sc * d.z, sc * d.w);
    a += (double)(d.x * d.x + d.y * d.y) + (double)(d.z * d.z + d.w * d.w);
  }
  for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * 256 + tid; i < n; i += (int64_t)gridDim.x * 256) {
    const float d = y[i] - t[i];
    g[i] = sc * d;
    a += (double)d * (double)d;
  }
  s_red[tid] = a;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) s_red[tid] += s_red[tid + w];
    __syncthreads();
  }
  if (tid == 0) part[blockIdx.x] = s_red[0];
}

__global__ void k_mse_finish(int64_t n, int nparts, const double* __restrict__ part,
                             float* __restrict__ loss) {
  __shared__ double s_red[256];
  const int tid = threadIdx.x;
  double a = 0.0;
  for (int i = tid; i < nparts; i += 256) a += part[i];
  s_red[tid] = a;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) s_red[tid] += s_red[tid + w];
    __syncthreads();
  }
  if (tid == 0) *loss = (float)(s_red[0] / (double)n);
}

hipError_t launch_mse(int64_t n, const float* y, const float* t, float* g, float* loss,
                      float grad_scale, double* part, int nparts, hipStream_t s) {
  hipLaunchKernelGGL(k_mse_part, dim3(nparts), dim3(256), 0, s, n, y, t, g, grad_scale, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !loss) return e;
  hipLaunchKernelGGL(k_mse_finish, dim3(1), dim3(256), 0, s, n, nparts, part, loss);
  return hipGetLastError();
}

// The loss through the output GELU: gz holds z on entry; y = GELU(z) (or z), and
// gz = sc (y - t) GELU'(z) on exit, the gradient of grad_scale * mean((y - t)^2) at z.
__global__ void k_mse_preact_part(int64_t n, const float* __restrict__ t, float* __restrict__ gz,
                                  bool gelu, float grad_scale, double* __restrict__ part) {
  __shared__ double s_red[256];
  const int tid = threadIdx.x;
  const float sc = (float)(2.0 * (double)grad_scale / (double)n);
  double a = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + tid; i < n; i += (int64_t)gridDim.x * 256) {
    const float z = gz[i];
    float y = z, gp = 1.f;
    if (gelu) {
      y = gelu_f(z);
      gp = gelu_grad_f(z);
    }
    const float d = y - t[i];
    gz[i] = sc * d * gp;
    a += (double)d * (double)d;
  }
  s_red[tid] = a;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) s_red[tid] += s_red[tid + w];
    __syncthreads();
  }
  if (tid == 0) part[blockIdx.x] = s_red[0];
}

hipError_t launch_mse_preact(int64_t n, const float* t, float* gz, bool gelu, float grad_scale,
                             double* part, int nparts, hipStream_t s) {
  hipLaunchKernelGGL(k_mse_preact_part, dim3(nparts), dim3(256), 0, s, n, t, gz, gelu,
                     grad_scale, part);
  return hipGetLastError();
}

hipError_t launch_mse_finish(int64_t n, int nparts, const double* part, float* loss,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_mse_finish, dim3(1), dim3(256), 0, s, n, nparts, part, loss);
  return hipGetLastError();
}

}  // namespace fno
