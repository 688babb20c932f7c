// Per-mode complex channel mix of the FNO block and its two gradients, on the matrix cores:
//   forward   yhat[b,o,t] = sum_i xhat[b,i,t] W[c(t),i,o,kappa(t)]
//   input     ghx[b,i,t]  = sum_o g[b,o,t] conj(W[c(t),i,o,kappa(t)])
//   weight    dW[c,i,o,k] = sum_b conj(xhat[b,i,t]) g[b,o,t]
// with g = ghat scaled by gamma(k_last)/Ntot (the adjoint of the inverse transform; gamma alone
// when the plan's transform tables carry 1/sqrt(N_j) in both directions).  IEEE-half plans
// multiply yhat and ghx by a power-of-two gain that the last inverse stage divides out.  This is
// the per-mode contraction of the FNO spectral layer (model-parallel FNO page, "Proposed
// method"); on the half paths every operand is rounded to bfloat16 or IEEE half and products
// accumulate in float32 (mixed-precision neural-operator page, "Tiivistelmä").
//
// Each mode's complex product is one real GEMM with the real and imaginary parts stacked:
//   rows  = 2 x 8 (re / im part x 8 batch entries, or x 8 input channels for dW)
//   K     = 2 x (contracted channels or batch entries), pairs (re, im)
//   cols  = 16 output (or input) channels
// e.g. forward: A[b][2i] = xr, A[b][2i+1] = -xi, A[8+b][2i] = xi, A[8+b][2i+1] = xr,
//               B[2i][o] = wr, B[2i+1][o] = wi   ->   D[b][o] = Re y, D[8+b][o] = Im y.
// A work-group owns 16 consecutive modes (their weights are 128-byte runs of W) and one
// 16-column tile; it streams K-chunks through LDS in fragment order (16 B per lane per
// fragment), prefetching the next chunk into registers.  bf16 path: 16x16x32 MFMA, chunk K =
// 32; fp32 path: 16x16x4 MFMA, chunk K = 16 (k-slot q of step s <-> k = 4 q + s).  Results
// pass through LDS so the stores are 128-byte runs of modes as well.  The mix streams W once
// and is bound by that read (or, for dW, by its write).
#include "fno_internal.h"
#include "mfma.h"
#include "pointwise.h"

namespace fno {

constexpr int kMT = 16;                 // modes per work-group
constexpr int kRowB = 64;               // bytes per LDS fragment row (32 bf16 or 16 f32)
constexpr int kTB = 16 * kRowB + 16;    // bytes per mode of a [16 rows][K chunk] LDS tile
constexpr int kOutTB = 8 * 16 * 8 + 16;  // bytes per mode of the [8][16] complex output tile

__device__ __forceinline__ float mix_scale(const Geom& g, int64_t t) {
  const int kb = (int)(t % g.mb);
  const bool one = (kb == 0) || (2 * kb == g.Nb);
  return (one ? 1.0f : 2.0f) * g.adj_scale;
}

// (v0, v1) into K slots (k, k + 1) of row r of mode tile t
template <int H>
__device__ __forceinline__ void put_pair(unsigned char* tile, int t, int r, int k, float v0,
                                         float v1) {
  constexpr bool BF = H != 0;
  unsigned char* p = tile + t * kTB + r * kRowB + k * (BF ? 2 : 4);
  if constexpr (BF) {
    *reinterpret_cast<uint32_t*>(p) = HalfOf<H>::pack2(v0, v1);
  } else {
    *reinterpret_cast<float2*>(p) = make_float2(v0, v1);
  }
}

// acc += A_t x B_t over one LDS chunk (lane (m, q) reads 16 B of row m of both tiles)
template <int H>
__device__ __forceinline__ f32x4 chunk_product(const unsigned char* ta, const unsigned char* tb,
                                               int t, int m, int q, f32x4 acc) {
  const int off = t * kTB + m * kRowB + 16 * q;
  if constexpr (H != 0) {
    using V = typename HalfOf<H>::v8;
    const V av = *reinterpret_cast<const V*>(ta + off);
    const V bv = *reinterpret_cast<const V*>(tb + off);
    return HalfOf<H>::mfma(av, bv, acc);
  } else {
    const float4 av = *reinterpret_cast<const float4*>(ta + off);
    const float4 bv = *reinterpret_cast<const float4*>(tb + off);
    acc = mfma_f32(av.x, bv.x, acc);
    acc = mfma_f32(av.y, bv.y, acc);
    acc = mfma_f32(av.z, bv.z, acc);
    return mfma_f32(av.w, bv.w, acc);
  }
}

// D fragment of mode tile t (rows 4 q + r: part (4q+r) / 8, entry (4q+r) % 8; column m) into
// the complex output tile [t][entry][column]
__device__ __forceinline__ void put_out(unsigned char* out, int t, int m, int q, const f32x4& d) {
  float* base = reinterpret_cast<float*>(out + t * kOutTB) + (q >> 1);  // re or im half
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = 4 * (q & 1) + r;
    base[2 * (e * 16 + m)] = d[r];
  }
}

// ------------------------------------------------------------------------------------------
// Forward (DX = false) and input gradient (DX = true).  Grid: (mode groups, 16-column tiles of
// the output channels, 8-entry batch tiles).  Contracted channels: Cin (forward) or Cout.
template <int H, bool DX>
__device__ __forceinline__ void mix_body(const Geom& g, const int32_t* __restrict__ mode_woff,
                                         const float2* __restrict__ spec,
                                         const float2* __restrict__ w, float2* __restrict__ out,
                                         uint3 bid, unsigned char* s_a, unsigned char* s_b) {
  constexpr bool BF = H != 0;       // half operands (bfloat16 or IEEE half)
  constexpr int IC = BF ? 16 : 8;  // contracted channels per chunk (K = 2 IC)
  constexpr int NW = 16 * IC / 16;  // weight complex values per thread per chunk (16 modes x IC x 16 cols / 256)
  constexpr int NS = 8 * IC / 16;   // spectrum values per thread per chunk (16 modes x 8 x IC / 256)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  const int64_t K = g.K;
  const int ncon = DX ? g.Cout : g.Cin;  // contracted
  const int nout = DX ? g.Cin : g.Cout;  // columns
  const int64_t t0 = (int64_t)bid.x * kMT;
  const int n0 = bid.y * 16;
  const int b0 = bid.z * 8;
  // every load of this thread is for mode t0 + (tid & 15); offsets fit in 32 bits (fields and
  // weights are limited to 2^31 elements)
  const int tl = tid & 15;
  const int tm = (int)min(t0 + tl, K - 1);
  const int Ki = (int)K;
  const float sc = DX ? mix_scale(g, tm) : 1.0f;
  // weight u of this thread: contracted channel c0 + u, column n0 + (tid >> 4)
  const int ncol = min(n0 + (tid >> 4), nout - 1);
  const int wbase = mode_woff[tm] + ncol * (DX ? g.w_si : g.w_so);
  const int wstep = DX ? g.w_so : g.w_si;
  float2 pw[NW], ps[NS];
  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int u = 0; u < NW; ++u) pw[u] = w[wbase + min(c0 + u, ncon - 1) * wstep];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int pr = (tid >> 4) + 16 * u;
      const int b = min(b0 + pr / IC, g.B - 1), cc = min(c0 + pr % IC, ncon - 1);
      ps[u] = spec[(b * ncon + cc) * Ki + tm];
    }
  };
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = zero4();
  load_chunk(0);
  for (int c0 = 0; c0 < ncon; c0 += IC) {
    __syncthreads();  // previous chunk's fragments consumed
#pragma unroll
    for (int u = 0; u < NW; ++u) {
      const int pr = (tid >> 4) + 16 * u;
      const int kc = pr / 16, n = pr % 16;
      const bool ok = c0 + kc < ncon && n0 + n < nout;
      // B[2 kc][n] = wr, B[2 kc + 1][n] = wi (conj(W) is taken by the A layout of DX)
      put_pair<H>(s_b, tl, n, 2 * kc, ok ? pw[u].x : 0.f, ok ? pw[u].y : 0.f);
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int pr = (tid >> 4) + 16 * u;
      const int bb = pr / IC, kc = pr % IC;
      const bool ok = c0 + kc < ncon && b0 + bb < g.B;
      const float vr = ok ? ps[u].x * sc : 0.f, vi = ok ? ps[u].y * sc : 0.f;
      if (DX) {  // (gr + i gi) conj(w): rows b: (gr, gi); rows 8 + b: (gi, -gr)
        put_pair<H>(s_a, tl, bb, 2 * kc, vr, vi);
        put_pair<H>(s_a, tl, 8 + bb, 2 * kc, vi, -vr);
      } else {   // (xr + i xi) w: rows b: (xr, -xi); rows 8 + b: (xi, xr)
        put_pair<H>(s_a, tl, bb, 2 * kc, vr, -vi);
        put_pair<H>(s_a, tl, 8 + bb, 2 * kc, vi, vr);
      }
    }
    load_chunk(min(c0 + IC, ncon - 1));
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = chunk_product<H>(s_a, s_b, 4 * wave + j, m, q, acc[j]);
  }
  __syncthreads();
  unsigned char* s_out = s_a;  // [16 modes][8 entries][16 columns] complex
#pragma unroll
  for (int j = 0; j < 4; ++j) put_out(s_out, 4 * wave + j, m, q, acc[j]);
  __syncthreads();
  // out[b][n][t]: thread -> mode tl, (entry, column) pairs (tid >> 4) + 16 u
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int pr = (tid >> 4) + 16 * u;
    const int bb = pr / 16, n = pr % 16;
    const int64_t t = t0 + tl;
    if (t < K && b0 + bb < g.B && n0 + n < nout) {
      float2 v = *reinterpret_cast<const float2*>(s_out + tl * kOutTB + (bb * 16 + n) * 8);
      if constexpr (H == 2) {  // IEEE half: the mix gain (a power of two)
        v.x *= g.mix_gain[DX];
        v.y *= g.mix_gain[DX];
      }
      out[((int64_t)(b0 + bb) * nout + n0 + n) * K + t] = v;
    }
  }
}

template <int H, bool DX>
__global__ void __launch_bounds__(256) k_mix_mfma(Geom g, const int32_t* __restrict__ mode_woff,
                                                  const float2* __restrict__ spec,
                                                  const float2* __restrict__ w,
                                                  float2* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) unsigned char s_a[kMT * kTB];
  __shared__ __attribute__((aligned(16))) unsigned char s_b[kMT * kTB];
  mix_body<H, DX>(g, mode_woff, spec, w, out, make_uint3(blockIdx.x, blockIdx.y, blockIdx.z),
                  s_a, s_b);
}

// ------------------------------------------------------------------------------------------
// Weight gradient.  Grid: (mode groups, gridDim.y parts of the 8-channel tiles of Cin, 16-column
// tiles of Cout): a work-group walks the Cin tiles y, y + gridDim.y, ..., and the first batch
// chunk of the next tile is loaded while the current one is computed and stored.
// Rows 0..7: Re, rows 8..15: Im of the 8 input channels; K = (batch entry, re / im).
template <int H>
__device__ __forceinline__ void mix_dw_body(const Geom& g, const int32_t* __restrict__ mode_woff,
                                            const float2* __restrict__ xhat,
                                            const float2* __restrict__ ghat,
                                            float2* __restrict__ dw, uint3 bid, int nparts,
                                            unsigned char* s_a, unsigned char* s_b) {
  constexpr bool BF = H != 0;
  constexpr int BC = BF ? 16 : 8;  // batch entries per chunk (K = 2 BC)
  constexpr int NX = 8 * BC / 16;   // x values per thread per chunk (16 modes x 8 ch x BC / 256)
  constexpr int NG = 16 * BC / 16;  // g values per thread per chunk (16 modes x 16 ch x BC / 256)
  bool bad = false;  // IEEE-half plans: a non-finite weight gradient was written
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  const int64_t K = g.K;
  const int64_t t0 = (int64_t)bid.x * kMT;
  const int istride = nparts * 8;
  const int o0 = bid.z * 16;
  const int tl = tid & 15;
  const int tm = (int)min(t0 + tl, K - 1);
  const int Ki = (int)K;
  const float sc = mix_scale(g, tm);
  const int64_t wmode = mode_woff[tm];
  float2 px[NX], pg[NG];
  // x value u: batch c0 + pr / 8, channel i0 + pr % 8; g value u: batch c0 + u, channel
  // o0 + (tid >> 4)   (pr = (tid >> 4) + 16 u)
  const int ocol = min(o0 + (tid >> 4), g.Cout - 1);
  auto load_chunk = [&](int i0, int c0) {
#pragma unroll
    for (int u = 0; u < NX; ++u) {
      const int pr = (tid >> 4) + 16 * u;
      const int b = min(c0 + pr / 8, g.B - 1), i = min(i0 + pr % 8, g.Cin - 1);
      px[u] = xhat[(b * g.Cin + i) * Ki + tm];
    }
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      const int b = min(c0 + u, g.B - 1);
      pg[u] = ghat[(b * g.Cout + ocol) * Ki + tm];
    }
  };
  load_chunk(bid.y * 8, 0);
  for (int i0 = bid.y * 8; i0 < g.Cin; i0 += istride) {
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = zero4();
    for (int c0 = 0; c0 < g.B; c0 += BC) {
      __syncthreads();  // the previous chunk's fragments and output tile are consumed
#pragma unroll
      for (int u = 0; u < NX; ++u) {
        const int pr = (tid >> 4) + 16 * u;
        const int bb = pr / 8, ii = pr % 8;
        const bool ok = c0 + bb < g.B && i0 + ii < g.Cin;
        const float xr = ok ? px[u].x : 0.f, xi = ok ? px[u].y : 0.f;
        // conj(x) g: rows i: (xr, xi); rows 8 + i: (-xi, xr)
        put_pair<H>(s_a, tl, ii, 2 * bb, xr, xi);
        put_pair<H>(s_a, tl, 8 + ii, 2 * bb, -xi, xr);
      }
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        const int pr = (tid >> 4) + 16 * u;
        const int bb = pr / 16, oo = pr % 16;
        const bool ok = c0 + bb < g.B && o0 + oo < g.Cout;
        put_pair<H>(s_b, tl, oo, 2 * bb, ok ? pg[u].x * sc : 0.f, ok ? pg[u].y * sc : 0.f);
      }
      // the next chunk: this tile's next batch chunk, else the next tile's first (clamped
      // copies past the end)
      const bool more = c0 + BC < g.B;
      load_chunk(more ? i0 : min(i0 + istride, g.Cin - 1), more ? c0 + BC : 0);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = chunk_product<H>(s_a, s_b, 4 * wave + j, m, q, acc[j]);
    }
    __syncthreads();
    unsigned char* s_out = s_a;  // [16 modes][8 input channels][16 output channels] complex
#pragma unroll
    for (int j = 0; j < 4; ++j) put_out(s_out, 4 * wave + j, m, q, acc[j]);
    __syncthreads();
    const int64_t t = t0 + tl;
    if (t < K) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int pr = (tid >> 4) + 16 * u;
        const int ii = pr / 16, oo = pr % 16;
        if (i0 + ii < g.Cin && o0 + oo < g.Cout) {
          const float2 v =
              *reinterpret_cast<const float2*>(s_out + tl * kOutTB + (ii * 16 + oo) * 8);
          if constexpr (H == 2) bad |= !(__builtin_isfinite(v.x) & __builtin_isfinite(v.y));
          dw[wmode + (int64_t)(i0 + ii) * g.w_si + (int64_t)(o0 + oo) * g.w_so] = v;
        }
      }
    }
  }
  if constexpr (H == 2) raise_half_flag(g.half_flag, bad);
}

template <int H>
__global__ void __launch_bounds__(256) k_mix_mfma_dw(Geom g, const int32_t* __restrict__ mode_woff,
                                                     const float2* __restrict__ xhat,
                                                     const float2* __restrict__ ghat,
                                                     float2* __restrict__ dw) {
  __shared__ __attribute__((aligned(16))) unsigned char s_a[kMT * kTB];
  __shared__ __attribute__((aligned(16))) unsigned char s_b[kMT * kTB];
  mix_dw_body<H>(g, mode_woff, xhat, ghat, dw, make_uint3(blockIdx.x, blockIdx.y, blockIdx.z),
                 gridDim.y, s_a, s_b);
}

// Both gradients of the mix in one launch: the first ndx work-groups take the input gradient
// (grid gdx), the rest the weight gradient (grid gdw).  The two read the same incoming spectrum
// and are otherwise independent; in one grid each fills the other's ramp and tail.
template <int H>
__global__ void __launch_bounds__(256) k_mix_mfma_bwd(Geom g, const int32_t* __restrict__ mode_woff,
                                                      const float2* __restrict__ xhat,
                                                      const float2* __restrict__ ghat,
                                                      const float2* __restrict__ w,
                                                      float2* __restrict__ ghx,
                                                      float2* __restrict__ dw, uint3 gdx,
                                                      uint3 gdw) {
  __shared__ __attribute__((aligned(16))) unsigned char s_a[kMT * kTB];
  __shared__ __attribute__((aligned(16))) unsigned char s_b[kMT * kTB];
  const uint32_t ndx = gdx.x * gdx.y * gdx.z;
  uint32_t i = blockIdx.x;
  if (i < ndx) {
    const uint3 bid = make_uint3(i % gdx.x, (i / gdx.x) % gdx.y, i / (gdx.x * gdx.y));
    mix_body<H, true>(g, mode_woff, ghat, w, ghx, bid, s_a, s_b);
  } else {
    i -= ndx;
    const uint3 bid = make_uint3(i % gdw.x, (i / gdw.x) % gdw.y, i / (gdw.x * gdw.y));
    mix_dw_body<H>(g, mode_woff, xhat, ghat, dw, bid, (int)gdw.y, s_a, s_b);
  }
}

// ------------------------------------------------------------------------------------------
// ------------------------------------------------------------------------------------------
// Forward mix for one or two batch entries, on the vector units.  The matrix-core tiles above
// hold eight batch entries per fragment, so with one or two most of each product is padding
// and the kernel streams W well below the memory rate.  Here lane l of a work-group owns mode
// 64 blockIdx.x + l and wave v owns output channels OPT v .. OPT v + OPT - 1: every W load of a
// wave is a run of 64 consecutive modes, and the waves of a work-group read the same input
// spectrum (through L1 / L2).  Half plans round both operands to their format, whose products
// are exact in float32, as the matrix cores take them.
template <int H, int NB, int OPT>
__global__ void __launch_bounds__(1024) k_mix_valu_fwd(Geom g, const int32_t* __restrict__ mode_woff,
                                                       const float2* __restrict__ spec,
                                                       const float2* __restrict__ w,
                                                       float2* __restrict__ out) {
  const int64_t K = g.K;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 64 + lane;
  const int64_t tm = t < K ? t : K - 1;
  const int o0 = wave * OPT;
  const int wb = mode_woff[tm];
  int wo[OPT];
#pragma unroll
  for (int j = 0; j < OPT; ++j) wo[j] = wb + min(o0 + j, g.Cout - 1) * g.w_so;
  float ar[NB][OPT], ai[NB][OPT];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < OPT; ++j) ar[b][j] = ai[b][j] = 0.f;
#pragma unroll 4
  for (int i = 0; i < g.Cin; ++i) {
    float2 xv[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      xv[b] = spec[((int64_t)b * g.Cin + i) * K + tm];
      if constexpr (H != 0) xv[b] = make_float2(round_half<H>(xv[b].x), round_half<H>(xv[b].y));
    }
#pragma unroll
    for (int j = 0; j < OPT; ++j) {
      float2 wv = w[wo[j] + i * g.w_si];
      if constexpr (H != 0) wv = make_float2(round_half<H>(wv.x), round_half<H>(wv.y));
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        ar[b][j] = fmaf(xv[b].x, wv.x, ar[b][j]);
        ar[b][j] = fmaf(-xv[b].y, wv.y, ar[b][j]);
        ai[b][j] = fmaf(xv[b].x, wv.y, ai[b][j]);
        ai[b][j] = fmaf(xv[b].y, wv.x, ai[b][j]);
      }
    }
  }
  if (t >= K) return;
  const float gain = H == 2 ? g.mix_gain[0] : 1.0f;  // IEEE half: the mix gain (a power of two)
#pragma unroll
  for (int j = 0; j < OPT; ++j) {
    if (o0 + j >= g.Cout) break;
#pragma unroll
    for (int b = 0; b < NB; ++b)
      out[((int64_t)b * g.Cout + o0 + j) * K + t] = make_float2(ar[b][j] * gain, ai[b][j] * gain);
  }
}

// Both gradients of the mix for one or two batch entries, on the vector units: lane l owns mode
// 64 blockIdx.x + l and wave v input channels OPT v .. OPT v + OPT - 1.  For each output
// channel o the wave loads g[b, o] (shared by the work-group's waves) and, per input channel,
//   ghx[b, i] += g[b, o] sc conj(W[i, o])          (when ghx is wanted)
//   dW[i, o]   = sum_b conj(xhat[b, i]) g[b, o] sc  (when dw is wanted; xhat held in registers)
// so that W loads and dW stores are runs of 64 consecutive modes.  Operands are rounded as the
// matrix-core kernels round them (g after its scale).
template <int H, int NB, int OPT>
__global__ void __launch_bounds__(1024) k_mix_valu_bwd(Geom g, const int32_t* __restrict__ mode_woff,
                                                       const float2* __restrict__ xhat,
                                                       const float2* __restrict__ ghat,
                                                       const float2* __restrict__ w,
                                                       float2* __restrict__ ghx,
                                                       float2* __restrict__ dw) {
  const int64_t K = g.K;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 64 + lane;
  const int64_t tm = t < K ? t : K - 1;
  const bool live = t < K;
  const int i0 = wave * OPT;
  const int wb = mode_woff[tm];
  const float sc = mix_scale(g, tm);
  auto rnd = [](float2 v) {
    if constexpr (H != 0) v = make_float2(round_half<H>(v.x), round_half<H>(v.y));
    return v;
  };
  int wi[OPT];
  float2 xv[NB][OPT];
#pragma unroll
  for (int j = 0; j < OPT; ++j) {
    const int i = min(i0 + j, g.Cin - 1);
    wi[j] = wb + i * g.w_si;
#pragma unroll
    for (int b = 0; b < NB; ++b)
      xv[b][j] = dw ? rnd(xhat[((int64_t)b * g.Cin + i) * K + tm]) : make_float2(0.f, 0.f);
  }
  float ar[NB][OPT], ai[NB][OPT];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < OPT; ++j) ar[b][j] = ai[b][j] = 0.f;
  bool bad = false;  // IEEE-half plans: a non-finite weight gradient was written
#pragma unroll 2
  for (int o = 0; o < g.Cout; ++o) {
    float2 gv[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float2 v = ghat[((int64_t)b * g.Cout + o) * K + tm];
      gv[b] = rnd(make_float2(v.x * sc, v.y * sc));
    }
    if (ghx) {
#pragma unroll
      for (int j = 0; j < OPT; ++j) {
        const float2 wv = rnd(w[wi[j] + o * g.w_so]);
#pragma unroll
        for (int b = 0; b < NB; ++b) {  // g conj(w)
          ar[b][j] = fmaf(gv[b].x, wv.x, ar[b][j]);
          ar[b][j] = fmaf(gv[b].y, wv.y, ar[b][j]);
          ai[b][j] = fmaf(gv[b].y, wv.x, ai[b][j]);
          ai[b][j] = fmaf(-gv[b].x, wv.y, ai[b][j]);
        }
      }
    }
    if (dw) {
#pragma unroll
      for (int j = 0; j < OPT; ++j) {
        float re = 0.f, im = 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b) {  // conj(x) g
          re = fmaf(xv[b][j].x, gv[b].x, re);
          re = fmaf(xv[b][j].y, gv[b].y, re);
          im = fmaf(xv[b][j].x, gv[b].y, im);
          im = fmaf(-xv[b][j].y, gv[b].x, im);
        }
        if (live && i0 + j < g.Cin) {
          if constexpr (H == 2) bad |= !(__builtin_isfinite(re) & __builtin_isfinite(im));
          dw[wi[j] + o * g.w_so] = make_float2(re, im);
        }
      }
    }
  }
  if (ghx && live) {
    const float gain = H == 2 ? g.mix_gain[1] : 1.0f;
#pragma unroll
    for (int j = 0; j < OPT; ++j) {
      if (i0 + j >= g.Cin) break;
#pragma unroll
      for (int b = 0; b < NB; ++b)
        ghx[((int64_t)b * g.Cin + i0 + j) * K + t] = make_float2(ar[b][j] * gain, ai[b][j] * gain);
    }
  }
  if constexpr (H == 2) raise_half_flag(g.half_flag, bad);
}

// the vector-unit mixes apply to one or two batch entries and at most 16 x 4 channels on the
// side a work-group's waves split (plans hold at most 64)
static bool mix_valu_ok(const Geom& g) { return g.B >= 1 && g.B <= 2 && g.Cout <= 64; }
static bool mix_valu_bwd_ok(const Geom& g) { return g.B >= 1 && g.B <= 2 && g.Cin <= 64; }

// channels per wave of the vector-unit mixes: two where four would leave fewer than 4096 waves
// in the grid (the work-group keeps at most 16 waves), else four
static int mix_valu_opt(int64_t blocks, int chans) {
  return chans <= 32 && blocks * ((chans + 3) / 4) < 4096 ? 2 : 4;
}

template <int H, int NB>
static void launch_mix_valu_bwd_nb(const Geom& g, const int32_t* woff, const float2* xhat,
                                   const float2* ghat, const float2* w, float2* ghx, float2* dw,
                                   hipStream_t s) {
  const unsigned blocks = (unsigned)((g.K + 63) / 64);
  const int opt = mix_valu_opt(blocks, g.Cin);
  if (opt == 2) {
    const int waves = (g.Cin + 1) / 2;
    hipLaunchKernelGGL((k_mix_valu_bwd<H, NB, 2>), dim3(blocks), dim3(64 * waves), 0, s, g, woff,
                       xhat, ghat, w, ghx, dw);
  } else {
    const int waves = (g.Cin + 3) / 4;
    hipLaunchKernelGGL((k_mix_valu_bwd<H, NB, 4>), dim3(blocks), dim3(64 * waves), 0, s, g, woff,
                       xhat, ghat, w, ghx, dw);
  }
}

static hipError_t launch_mix_valu_bwd(const Geom& g, const int32_t* woff, const float2* xhat,
                                      const float2* ghat, const float2* w, float2* ghx,
                                      float2* dw, hipStream_t s) {
  if (g.half == 2) {
    if (g.B == 1) launch_mix_valu_bwd_nb<2, 1>(g, woff, xhat, ghat, w, ghx, dw, s);
    else launch_mix_valu_bwd_nb<2, 2>(g, woff, xhat, ghat, w, ghx, dw, s);
  } else if (g.half == 1) {
    if (g.B == 1) launch_mix_valu_bwd_nb<1, 1>(g, woff, xhat, ghat, w, ghx, dw, s);
    else launch_mix_valu_bwd_nb<1, 2>(g, woff, xhat, ghat, w, ghx, dw, s);
  } else {
    if (g.B == 1) launch_mix_valu_bwd_nb<0, 1>(g, woff, xhat, ghat, w, ghx, dw, s);
    else launch_mix_valu_bwd_nb<0, 2>(g, woff, xhat, ghat, w, ghx, dw, s);
  }
  return hipGetLastError();
}

template <int H, int NB>
static void launch_mix_valu_nb(const Geom& g, const int32_t* woff, const float2* xhat,
                               const float2* w, float2* yhat, hipStream_t s) {
  const unsigned blocks = (unsigned)((g.K + 63) / 64);
  const int opt = mix_valu_opt(blocks, g.Cout);
  if (opt == 2) {
    const int waves = (g.Cout + 1) / 2;
    hipLaunchKernelGGL((k_mix_valu_fwd<H, NB, 2>), dim3(blocks), dim3(64 * waves), 0, s, g, woff,
                       xhat, w, yhat);
  } else {
    const int waves = (g.Cout + 3) / 4;
    hipLaunchKernelGGL((k_mix_valu_fwd<H, NB, 4>), dim3(blocks), dim3(64 * waves), 0, s, g, woff,
                       xhat, w, yhat);
  }
}

template <int H>
static void launch_mix_valu(const Geom& g, const int32_t* woff, const float2* xhat,
                            const float2* w, float2* yhat, hipStream_t s) {
  if (g.B == 1)
    launch_mix_valu_nb<H, 1>(g, woff, xhat, w, yhat, s);
  else
    launch_mix_valu_nb<H, 2>(g, woff, xhat, w, yhat, s);
}

static dim3 mix_grid(const Geom& g, int cols) {
  return dim3((unsigned)((g.K + kMT - 1) / kMT), (unsigned)((cols + 15) / 16),
              (unsigned)((g.B + 7) / 8));
}

hipError_t launch_mix_fwd_g(const Geom& g, const int32_t* woff, const float2* xhat,
                            const float2* w, float2* yhat, hipStream_t s) {
  if (mix_valu_ok(g)) {
    if (g.half == 2)
      launch_mix_valu<2>(g, woff, xhat, w, yhat, s);
    else if (g.half == 1)
      launch_mix_valu<1>(g, woff, xhat, w, yhat, s);
    else
      launch_mix_valu<0>(g, woff, xhat, w, yhat, s);
    return hipGetLastError();
  }
  if (g.half == 2)
    hipLaunchKernelGGL((k_mix_mfma<2, false>), mix_grid(g, g.Cout), dim3(256), 0, s, g, woff,
                       xhat, w, yhat);
  else if (g.half == 1)
    hipLaunchKernelGGL((k_mix_mfma<1, false>), mix_grid(g, g.Cout), dim3(256), 0, s, g, woff,
                       xhat, w, yhat);
  else
    hipLaunchKernelGGL((k_mix_mfma<0, false>), mix_grid(g, g.Cout), dim3(256), 0, s, g, woff,
                       xhat, w, yhat);
  return hipGetLastError();
}

hipError_t launch_mix_bwd_dx_g(const Geom& g, const int32_t* woff, const float2* ghat,
                               const float2* w, float2* ghx, hipStream_t s) {
  if (mix_valu_bwd_ok(g)) return launch_mix_valu_bwd(g, woff, nullptr, ghat, w, ghx, nullptr, s);
  if (g.half == 2)
    hipLaunchKernelGGL((k_mix_mfma<2, true>), mix_grid(g, g.Cin), dim3(256), 0, s, g, woff,
                       ghat, w, ghx);
  else if (g.half == 1)
    hipLaunchKernelGGL((k_mix_mfma<1, true>), mix_grid(g, g.Cin), dim3(256), 0, s, g, woff,
                       ghat, w, ghx);
  else
    hipLaunchKernelGGL((k_mix_mfma<0, true>), mix_grid(g, g.Cin), dim3(256), 0, s, g, woff,
                       ghat, w, ghx);
  return hipGetLastError();
}

// weight-gradient grid: (mode groups, parts of the Cin tiles, Cout tiles); Cin tiles per
// work-group: about 1024 work-groups in all, at most every tile in one
static dim3 mix_dw_grid(const Geom& g) {
  const int64_t mg = (g.K + kMT - 1) / kMT, ot = (g.Cout + 15) / 16, itiles = (g.Cin + 7) / 8;
  int64_t parts = (1024 + mg * ot - 1) / (mg * ot);
  if (parts > itiles) parts = itiles;
  if (parts < 1) parts = 1;
  return dim3((unsigned)mg, (unsigned)parts, (unsigned)ot);
}

hipError_t launch_mix_bwd_dw_g(const Geom& g, const int32_t* woff, const float2* xhat,
                               const float2* ghat, float2* dw, hipStream_t s) {
  if (mix_valu_bwd_ok(g)) return launch_mix_valu_bwd(g, woff, xhat, ghat, nullptr, nullptr, dw, s);
  const dim3 grid = mix_dw_grid(g);
  if (g.half == 2)
    hipLaunchKernelGGL((k_mix_mfma_dw<2>), grid, dim3(256), 0, s, g, woff, xhat, ghat, dw);
  else if (g.half == 1)
    hipLaunchKernelGGL((k_mix_mfma_dw<1>), grid, dim3(256), 0, s, g, woff, xhat, ghat, dw);
  else
    hipLaunchKernelGGL((k_mix_mfma_dw<0>), grid, dim3(256), 0, s, g, woff, xhat, ghat, dw);
  return hipGetLastError();
}

hipError_t launch_mix_fwd(const fno_plan* p, const float2* xhat, int nparts,
                          int64_t part_stride, const float2* w, float2* yhat, hipStream_t s) {
  (void)nparts;
  (void)part_stride;
  return launch_mix_fwd_g(p->g, p->t.mode_woff, xhat, w, yhat, s);
}

hipError_t launch_mix_bwd_dx(const fno_plan* p, const float2* ghat, const float2* w,
                             float2* ghx, hipStream_t s) {
  return launch_mix_bwd_dx_g(p->g, p->t.mode_woff, ghat, w, ghx, s);
}

hipError_t launch_mix_bwd_dw(const fno_plan* p, const float2* xhat, const float2* ghat,
                             float2* dw, hipStream_t s) {
  return launch_mix_bwd_dw_g(p->g, p->t.mode_woff, xhat, ghat, dw, s);
}

hipError_t launch_mix_bwd_both(const fno_plan* p, const float2* xhat, const float2* ghat,
                               const float2* w, float2* ghx, float2* dw, hipStream_t s) {
  const Geom& g = p->g;
  if (mix_valu_bwd_ok(g))
    return launch_mix_valu_bwd(g, p->t.mode_woff, xhat, ghat, w, ghx, dw, s);
  const dim3 gx = mix_grid(g, g.Cin), gw = mix_dw_grid(g);
  const uint64_t n = (uint64_t)gx.x * gx.y * gx.z + (uint64_t)gw.x * gw.y * gw.z;
  if (n > 0x7fffffffu) return hipErrorInvalidValue;
  const uint3 ux = make_uint3(gx.x, gx.y, gx.z), uw = make_uint3(gw.x, gw.y, gw.z);
  const int32_t* woff = p->t.mode_woff;
  if (g.half == 2)
    hipLaunchKernelGGL((k_mix_mfma_bwd<2>), dim3((unsigned)n), dim3(256), 0, s, g, woff, xhat,
                       ghat, w, ghx, dw, ux, uw);
  else if (g.half == 1)
    hipLaunchKernelGGL((k_mix_mfma_bwd<1>), dim3((unsigned)n), dim3(256), 0, s, g, woff, xhat,
                       ghat, w, ghx, dw, ux, uw);
  else
    hipLaunchKernelGGL((k_mix_mfma_bwd<0>), dim3((unsigned)n), dim3(256), 0, s, g, woff, xhat,
                       ghat, w, ghx, dw, ux, uw);
  return hipGetLastError();
}

}  // namespace fno
