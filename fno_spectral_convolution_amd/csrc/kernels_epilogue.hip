// Matrix-core epilogues of the FNO block (the two kernels that stream the activation fields).
//
// Forward, per point p of a line of the contiguous axis and every output channel o:
//   z[o,p] = sum_k GT[p,k] Tcat[o,k] + sum_i Wb[o,i] x[i,p] + bias[o],   y = GELU(z)
// where Tcat[o, 2kb] / Tcat[o, 2kb+1] are the real / imaginary parts of the spectrum after
// the outer-axis inverses, and GT[p, 2kb] = g(kb) cos(2 pi kb p / Nb) / Ntot,
// GT[p, 2kb+1] = -g(kb) sin(2 pi kb p / Nb) / Ntot (g = 1 at DC / Nyquist, else 2): the
// last-axis inverse of the zero-padded half spectrum taking the real part.
// Backward, per point:
//   grad_x[i,p] = s(x_i) sum_k GU[p,k] Tgcat[i,k] + sum_o Wb[o,i] g_z[o,p],
//   g_z = g_y GELU'(z),   dWb[o,i] += sum_p g_z[o,p] x[i,p],   dbias[o] += sum_p g_z[o,p]
// with GU the unit-scale table (the adjoint of the forward transform) and s = 1 - tanh^2.
//
// Work split: one wave per group of 16*TM consecutive points of one line (TM = 4 forward,
// 2 backward) and all channels.  Results are computed transposed (points x channels) so that
// every lane reads and writes whole float4s of one channel's contiguous points:
//   spectral part : 16x16x32 bf16 (mixed path) or 16x16x4 f32 MFMA, K = 2 mb (padded)
//   bypass / grads: 16x16x4 f32 MFMA, K = channels (4 per step) or points (backward dWb)
// The last-axis table is read through L2 (it is shared by every wave); Wb lives in LDS.
#include "fno_internal.h"
#include "mfma.h"

#include <math.h>

namespace fno {

struct EpiArgs {
  int B, C;            // batch, channels (Cin = Cout = C)
  int64_t P;           // points per field
  int Nb, mb, kpad;    // contiguous axis, its retained bins, padded 2*mb
  int64_t lines;       // P / Nb
  int64_t npg;         // point groups over the whole batch
  int64_t pg_per_wg;   // contiguous point groups handled by one work-group
  const float* x;
  const float2* T;     // [B][C][lines][mb]
  const float* wb;     // [C][C] (o, i)
  const float* bias;   // [C] or null
  const void* gt;      // [Nb][kpad] f32 or bf16 bits
  float* y;            // forward output (or grad_x backward)
  float* z;            // forward z save (nullable)
  const float* gy;     // backward incoming gradient
  const float* zin;    // backward saved z
  float* part;         // backward per-group partials [grid][C*C + C]
  int block;           // bypass/bias/GELU present (else spectral only)
  int gelu;
};

__device__ __forceinline__ float gelu_fast(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

__device__ __forceinline__ float gelu_grad_fast(float z) {
  const float cdf = 0.5f * (1.0f + erff(z * 0.70710678118654752f));
  const float pdf = __expf(-0.5f * z * z) * 0.39894228040143268f;
  return cdf + z * pdf;
}

__device__ __forceinline__ float comp(const float4& v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

// Spectral part of one point group: acc[t][nt] (+)= GT^T x Tcat^T.
//   M-tile t, row m  <-> point p0 + TM*m + t  (A operand: GT row)
//   N-tile nt, col n <-> channel 16*nt + n    (B operand: Tcat row of that channel)
template <int C, int TM, bool BF>
__device__ __forceinline__ void spectral_part(const EpiArgs& a, const float2* Trow0,
                                              int pb0, int m, int q,
                                              f32x4 (&acc)[TM][(C + 15) / 16]) {
  constexpr int NT = (C + 15) / 16;
  const int kf_end = 2 * a.mb;
  const int64_t cstride = a.lines * a.mb;  // complex elements between channels
  if (BF) {
    const uint16_t* gt = static_cast<const uint16_t*>(a.gt);
    for (int s = 0; s < a.kpad / 32; ++s) {
      const int kf = 32 * s + 8 * q;
      bf16x8 A[TM];
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const int p = pb0 + TM * m + t;
        A[t] = *reinterpret_cast<const bf16x8*>(gt + (int64_t)p * a.kpad + kf);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int o = 16 * nt + m;
        float4 u0 = make_float4(0.f, 0.f, 0.f, 0.f), u1 = u0;
        if (o < C) {
          const float* tr = reinterpret_cast<const float*>(Trow0 + (int64_t)o * cstride);
          if (kf < kf_end) u0 = *reinterpret_cast<const float4*>(tr + kf);
          if (kf + 4 < kf_end) u1 = *reinterpret_cast<const float4*>(tr + kf + 4);
        }
        const bf16x8 Bv = to_bf16x8(u0, u1);
#pragma unroll
        for (int t = 0; t < TM; ++t) acc[t][nt] = mfma_bf16(A[t], Bv, acc[t][nt]);
      }
    }
  } else {
    const float* gt = static_cast<const float*>(a.gt);
    for (int g = 0; g < a.kpad / 16; ++g) {
      const int kf = 16 * g + 4 * q;
      float4 A4[TM];
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const int p = pb0 + TM * m + t;
        A4[t] = *reinterpret_cast<const float4*>(gt + (int64_t)p * a.kpad + kf);
      }
      float4 B4[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int o = 16 * nt + m;
        B4[nt] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (o < C && kf < kf_end)
          B4[nt] = *reinterpret_cast<const float4*>(
              reinterpret_cast<const float*>(Trow0 + (int64_t)o * cstride) + kf);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int t = 0; t < TM; ++t)
            acc[t][nt] = mfma_f32(comp(A4[t], j), comp(B4[nt], j), acc[t][nt]);
    }
  }
}

// ------------------------------------------------------------------------------------------
template <int C, bool BF>
__global__ void __launch_bounds__(256) k_epi_fwd_fast(EpiArgs a) {
  constexpr int TM = 4;
  constexpr int CP = (C + 15) / 16 * 16;
  constexpr int NT = CP / 16;
  __shared__ float s_wbt[C * CP];  // Wb^T[i][o], o padded with zeros
  __shared__ float s_bias[CP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  if (a.block) {
    for (int e = tid; e < C * CP; e += 256) {
      const int i = e / CP, o = e - i * CP;
      s_wbt[e] = (o < C) ? a.wb[o * C + i] : 0.f;
    }
    for (int o = tid; o < CP; o += 256) s_bias[o] = (o < C && a.bias) ? a.bias[o] : 0.f;
  }
  __syncthreads();
  const int64_t pg_per_b = a.P / (16 * TM);
  const int64_t g_begin = (int64_t)blockIdx.x * a.pg_per_wg;
  const int64_t g_end = min(a.npg, g_begin + a.pg_per_wg);
  for (int64_t pg = g_begin + wave; pg < g_end; pg += 4) {
    const int b = (int)(pg / pg_per_b);
    const int64_t p0 = (pg - (int64_t)b * pg_per_b) * (16 * TM);
    const int64_t line = p0 / a.Nb;
    const int pb0 = (int)(p0 - line * a.Nb);
    f32x4 acc[TM][NT];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[t][nt] = zero4();
    const float2* Trow0 = a.T + ((int64_t)b * C * a.lines + line) * a.mb;
    spectral_part<C, TM, BF>(a, Trow0, pb0, m, q, acc);
    if (a.block) {
      const float* xb = a.x + (int64_t)b * C * a.P + p0 + TM * m;
      float4 X[C / 4];
#pragma unroll
      for (int kb = 0; kb < C / 4; ++kb)
        X[kb] = *reinterpret_cast<const float4*>(xb + (int64_t)(4 * kb + q) * a.P);
#pragma unroll
      for (int kb = 0; kb < C / 4; ++kb) {
        float bw[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) bw[nt] = s_wbt[(4 * kb + q) * CP + 16 * nt + m];
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[t][nt] = mfma_f32(comp(X[kb], t), bw[nt], acc[t][nt]);
      }
    }
    // lane (n = m, q): channel o = 16 nt + m, points p0 + 16 q + 4 r + t
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int o = 16 * nt + m;
      if (o >= C) continue;
      const float bo = a.block ? s_bias[o] : 0.f;
      const int64_t base = ((int64_t)b * C + o) * a.P + p0 + 16 * q;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float4 v = make_float4(acc[0][nt][r] + bo, acc[1][nt][r] + bo, acc[2][nt][r] + bo,
                               acc[3][nt][r] + bo);
        if (a.z) *reinterpret_cast<float4*>(a.z + base + 4 * r) = v;
        if (a.block && a.gelu) {
          v.x = gelu_fast(v.x);
          v.y = gelu_fast(v.y);
          v.z = gelu_fast(v.z);
          v.w = gelu_fast(v.w);
        }
        *reinterpret_cast<float4*>(a.y + base + 4 * r) = v;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Backward.  Channel-major register tiles: lane (m, q) holds channel 16*ct + m at the 4*TM
// consecutive points p0 + 4*TM*q + u, u = 0 .. 4*TM-1 (TM float4s).
template <int C, bool BF, bool TANH>
__global__ void __launch_bounds__(256) k_epi_bwd_fast(EpiArgs a) {
  constexpr int TM = 2;
  constexpr int PG = 16 * TM;      // points per group
  constexpr int PPL = 4 * TM;      // points per lane
  constexpr int CP = (C + 15) / 16 * 16;
  constexpr int NT = CP / 16;
  constexpr int GZS = PG + 4;      // row stride of the transpose buffer (floats)
  constexpr int kGz = 4 * C * GZS;         // per-wave g_z[o][point] transpose tiles
  constexpr int kRed = C * CP + 16 * CP;   // work-group reduction (reuses the same LDS)
  __shared__ float s_wb[C * CP];           // Wb[o][i], i padded with zeros
  __shared__ float s_buf[kGz > kRed ? kGz : kRed];
  float* s_red = s_buf;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  if (a.block)
    for (int e = tid; e < C * CP; e += 256) {
      const int o = e / CP, i = e - o * CP;
      s_wb[e] = (i < C) ? a.wb[o * C + i] : 0.f;
    }
  __syncthreads();
  f32x4 dwb[NT][NT];
  float dbl[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    dbl[u] = 0.f;
#pragma unroll
    for (int v = 0; v < NT; ++v) dwb[u][v] = zero4();
  }
  float* gzw = s_buf + wave * C * GZS;
  const bool want_gx = a.y != nullptr;
  const int64_t pg_per_b = a.P / PG;
  const int64_t g_begin = (int64_t)blockIdx.x * a.pg_per_wg;
  const int64_t g_end = min(a.npg, g_begin + a.pg_per_wg);
  for (int64_t pg = g_begin + wave; pg < g_end; pg += 4) {
    const int b = (int)(pg / pg_per_b);
    const int64_t p0 = (pg - (int64_t)b * pg_per_b) * PG;
    const int64_t line = p0 / a.Nb;
    const int pb0 = (int)(p0 - line * a.Nb);
    f32x4 acc[TM][NT];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[t][nt] = zero4();
    if (want_gx) {
      const float2* Trow0 = a.T + ((int64_t)b * C * a.lines + line) * a.mb;
      spectral_part<C, TM, BF>(a, Trow0, pb0, m, q, acc);
    }
    // x, channel-major: X[ct][h] = x[16 ct + m][p0 + PPL q + 4 h .. +3]
    float4 X[NT][TM];
    const int64_t fb = (int64_t)b * C * a.P + p0 + PPL * q;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      const int c = 16 * ct + m;
#pragma unroll
      for (int h = 0; h < TM; ++h)
        X[ct][h] = (c < C && (TANH || a.block))
                       ? *reinterpret_cast<const float4*>(a.x + fb + (int64_t)c * a.P + 4 * h)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (TANH) {
      // acc[t][nt][r] is channel 16 nt + m at point p0 + PPL q + TM r + t
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int t = 0; t < TM; ++t) {
            const int u = TM * r + t;
            const float th = tanhf(comp(X[nt][u >> 2], u & 3));
            acc[t][nt][r] *= (1.f - th * th);
          }
    }
    if (a.block) {
      // g_z channel-major, then the bypass-weight gradient straight from registers
      float4 GZ[NT][TM];
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        const int o = 16 * ct + m;
#pragma unroll
        for (int h = 0; h < TM; ++h) {
          float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
          if (o < C) {
            const int64_t off = fb + (int64_t)o * a.P + 4 * h;
            g = *reinterpret_cast<const float4*>(a.gy + off);
            if (a.gelu) {
              const float4 zz = *reinterpret_cast<const float4*>(a.zin + off);
              g.x *= gelu_grad_fast(zz.x);
              g.y *= gelu_grad_fast(zz.y);
              g.z *= gelu_grad_fast(zz.z);
              g.w *= gelu_grad_fast(zz.w);
            }
            *reinterpret_cast<float4*>(gzw + o * GZS + PPL * q + 4 * h) = g;
          }
          GZ[ct][h] = g;
          dbl[ct] += (g.x + g.y) + (g.z + g.w);
        }
      }
      // dWb[o][i] += sum_u GZ(o, u) X(i, u): K-step u takes point p0 + PPL q + u
#pragma unroll
      for (int u = 0; u < PPL; ++u)
#pragma unroll
        for (int mo = 0; mo < NT; ++mo)
#pragma unroll
          for (int ni = 0; ni < NT; ++ni)
            dwb[mo][ni] = mfma_f32(comp(GZ[mo][u >> 2], u & 3), comp(X[ni][u >> 2], u & 3),
                                   dwb[mo][ni]);
      // the transposed g_z tile must be complete before this wave reads it back
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // grad_x^T[p][i] += sum_o g_z^T[p][o] Wb[o][i]; A: lane (m, q) = g_z[4kb+q][TM m + t]
#pragma unroll
      for (int kb = 0; kb < C / 4 && want_gx; ++kb) {
        const int o = 4 * kb + q;
        float At[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) At[t] = gzw[o * GZS + TM * m + t];
        float bw[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) bw[nt] = s_wb[o * CP + 16 * nt + m];
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[t][nt] = mfma_f32(At[t], bw[nt], acc[t][nt]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // grad_x: lane (m, q), channel 16 nt + m, points p0 + PPL q + TM r + t
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int i = 16 * nt + m;
      if (i >= C || !want_gx) continue;
      float v[PPL];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < TM; ++t) v[TM * r + t] = acc[t][nt][r];
      float* dst = a.y + fb + (int64_t)i * a.P;
#pragma unroll
      for (int h = 0; h < TM; ++h)
        *reinterpret_cast<float4*>(dst + 4 * h) =
            make_float4(v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]);
    }
  }
  if (!a.block || !a.part) return;
  __syncthreads();  // every wave is done with its transpose tile before s_red reuses it
  // Deterministic work-group reduction: waves add their partials in order 0..3.
  // dwb[mo][ni][r] is dWb[16 mo + 4 q + r][16 ni + m]; dbl[ct] is a partial of dbias[16 ct + m].
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int mo = 0; mo < NT; ++mo)
#pragma unroll
        for (int ni = 0; ni < NT; ++ni)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = (16 * mo + 4 * q + r) * CP + 16 * ni + m;
            if (16 * mo + 4 * q + r < C)
              s_red[e] = (w == 0 ? 0.f : s_red[e]) + dwb[mo][ni][r];
          }
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) s_red[C * CP + (w * 4 + q) * CP + 16 * ct + m] = dbl[ct];
    }
    __syncthreads();
  }
  float* dst = a.part + (int64_t)blockIdx.x * (C * C + C);
  for (int e = tid; e < C * C + C; e += 256) {
    float v;
    if (e < C * C) {
      const int o = e / C, i = e - o * C;
      v = s_red[o * CP + i];
    } else {
      const int o = e - C * C;
      v = 0.f;
      for (int k = 0; k < 16; ++k) v += s_red[C * CP + k * CP + o];
    }
    dst[e] = v;
  }
}

// ------------------------------------------------------------------------------------------
template <int C>
static hipError_t launch_fwd_c(const EpiArgs& a, bool bf, int wgs, hipStream_t s) {
  if (bf)
    hipLaunchKernelGGL((k_epi_fwd_fast<C, true>), dim3(wgs), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_epi_fwd_fast<C, false>), dim3(wgs), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int C>
static hipError_t launch_bwd_c(const EpiArgs& a, bool bf, bool tanh_pre, int wgs, hipStream_t s) {
  if (bf) {
    if (tanh_pre)
      hipLaunchKernelGGL((k_epi_bwd_fast<C, true, true>), dim3(wgs), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_epi_bwd_fast<C, true, false>), dim3(wgs), dim3(256), 0, s, a);
  } else {
    if (tanh_pre)
      hipLaunchKernelGGL((k_epi_bwd_fast<C, false, true>), dim3(wgs), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_epi_bwd_fast<C, false, false>), dim3(wgs), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

bool epilogue_fast_ok(const fno_plan* p, int mode, bool fwd) {
  const Geom& g = p->g;
  const int C = fwd ? g.Cout : g.Cin;
  if (mode == EPI_BLOCK && g.Cin != g.Cout) return false;
  if (!(C == 16 || C == 20 || C == 32 || C == 48 || C == 64)) return false;
  if (g.Nb % 64 != 0 || g.mb % 2 != 0) return false;
  return true;
}

static EpiArgs make_args(const fno_plan* p, int C, int pg_points, int wgs_cap, int* wgs) {
  const Geom& g = p->g;
  EpiArgs a{};
  a.B = g.B;
  a.C = C;
  a.P = g.P;
  a.Nb = g.Nb;
  a.mb = g.mb;
  a.kpad = p->kpad;
  a.lines = g.P / g.Nb;
  a.npg = (int64_t)g.B * (g.P / pg_points);
  int64_t w = (a.npg + 3) / 4;
  if (w > wgs_cap) w = wgs_cap;
  if (w < 1) w = 1;
  a.pg_per_wg = (a.npg + w - 1) / w;
  a.pg_per_wg = (a.pg_per_wg + 3) / 4 * 4;
  *wgs = (int)((a.npg + a.pg_per_wg - 1) / a.pg_per_wg);
  return a;
}

hipError_t launch_epilogue_fwd_fast(const fno_plan* p, int mode, const float2* T, const float* x,
                                    const float* wb, const float* bias, float* y, float* zsave,
                                    hipStream_t s) {
  const Geom& g = p->g;
  int wgs = 0;
  EpiArgs a = make_args(p, g.Cout, 64, 1024, &wgs);
  a.x = x;
  a.T = T;
  a.wb = wb;
  a.bias = (p->desc.flags & FNO_FLAG_BIAS) ? bias : nullptr;
  a.gt = g.bf16 ? (const void*)p->t.gt_fwd_bf : (const void*)p->t.gt_fwd;
  a.y = y;
  a.z = zsave;
  a.block = mode == EPI_BLOCK;
  a.gelu = (p->desc.flags & FNO_FLAG_GELU) != 0;
  switch (g.Cout) {
    case 16: return launch_fwd_c<16>(a, g.bf16, wgs, s);
    case 20: return launch_fwd_c<20>(a, g.bf16, wgs, s);
    case 32: return launch_fwd_c<32>(a, g.bf16, wgs, s);
    case 48: return launch_fwd_c<48>(a, g.bf16, wgs, s);
    default: return launch_fwd_c<64>(a, g.bf16, wgs, s);
  }
}

int epilogue_bwd_fast_groups(const fno_plan* p) {
  int wgs = 0;
  (void)make_args(p, p->g.Cin, 32, 512, &wgs);
  return wgs;
}

hipError_t launch_epilogue_bwd_fast(const fno_plan* p, int mode, const float2* Tg,
                                    const float* x, const float* wb, const float* gy,
                                    const float* z, float* grad_x, float* red_part,
                                    hipStream_t s) {
  const Geom& g = p->g;
  int wgs = 0;
  EpiArgs a = make_args(p, g.Cin, 32, 512, &wgs);
  a.x = x;
  a.T = Tg;
  a.wb = wb;
  a.gt = g.bf16 ? (const void*)p->t.gt_unit_bf : (const void*)p->t.gt_unit;
  a.y = grad_x;
  a.gy = gy;
  a.zin = z;
  a.part = red_part;
  a.block = mode == EPI_BLOCK;
  a.gelu = (p->desc.flags & FNO_FLAG_GELU) != 0;
  const bool tanh_pre = (p->desc.flags & FNO_FLAG_TANH_PREACT) != 0;
  switch (g.Cin) {
    case 16: return launch_bwd_c<16>(a, g.bf16, tanh_pre, wgs, s);
    case 20: return launch_bwd_c<20>(a, g.bf16, tanh_pre, wgs, s);
    case 32: return launch_bwd_c<32>(a, g.bf16, tanh_pre, wgs, s);
    case 48: return launch_bwd_c<48>(a, g.bf16, tanh_pre, wgs, s);
    default: return launch_bwd_c<64>(a, g.bf16, tanh_pre, wgs, s);
  }
}

}  // namespace fno
