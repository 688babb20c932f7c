// Pointwise lift / projection of an FNO stack on the matrix cores:
//   hidden == 0:  y[o][p] = b1[o] + sum_c W1[o][c] x[c][p]
//   hidden  > 0:  y[o][p] = b2[o] + sum_h W2[o][h] GELU(b1[h] + sum_c W1[h][c] x[c][p])
// (the lift and the two-layer projection around the spectral blocks; model-parallel FNO page,
// "Proposed method").  A work-group takes 64 consecutive points of one batch entry: the x
// tile [cin][64] is staged in LDS, the first product (M = hidden or cout, K = cin, N = 64)
// runs as 16x16x4 f32 MFMAs with bias and GELU applied to its fragments, the hidden tile goes
// to LDS and feeds the second product (M = cout, K = hidden); the output tile leaves through
// LDS as row-contiguous float4 stores.  Waves take M-tiles round-robin; weight fragments are
// read through L2.  Point tails are zero-filled on load and masked on store.  A projection to
// at most kPwSmallOut channels does its second product on the VALU instead (see below); on whole
// tiles with cin <= 32 and hidden <= 128 it runs as a grid-stride walk (k_proj_narrow).  A lift
// from at most four channels runs on the VALU altogether (k_lift_valu).
#include "fno_internal.h"
#include "mfma.h"
#include "pointwise.h"

namespace fno {

constexpr int kPwP = 64;        // points per work-group
constexpr int kPwS = kPwP + 4;  // LDS row stride (floats)
constexpr int kPwSmallOut = 4;  // projections to at most this many channels skip the hidden tile

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

// NOUT = 1 .. kPwSmallOut: a projection to exactly NOUT channels (the narrow path below);
// NOUT = 0: every other shape
template <int NOUT>
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
        v[j] = load_stream4(xb + (int64_t)c * npts + 4 * f);
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
  if constexpr (NOUT > 0) {
    // narrow output (the projection to a few channels): the second product runs on the
    // VALU from the GELU'd fragments of the first, without the hidden tile.  Lane (m, q) adds
    // W2[o][h] GELU(.)[h][p] over its rows h = 16 mt + 4 q + r for points p = 16 nt + m; the
    // four lane quarters are then summed by two xor butterflies and the four waves in order
    // (a fixed order: deterministic).
    float part[NOUT][4];
#pragma unroll
    for (int o = 0; o < NOUT; ++o)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) part[o][nt] = 0.f;
    for (int mt = wave; mt < mid_p / 16; mt += 4) {
      f32x4 acc[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[nt] = zero4();
      pw_tile<4>(w1, cin, mid, cin, s_x, mt, 0, m, q, acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 16 * mt + 4 * q + r;
        const float bh = masked_bias(b1, h, mid);
        float w2v[NOUT];
#pragma unroll
        for (int o = 0; o < NOUT; ++o) {
          const float wv = w2[o * hidden + min(h, hidden - 1)];
          w2v[o] = __uint_as_float(__float_as_uint(wv) & (h < hidden ? 0xffffffffu : 0u));
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const float gv = gelu_as(acc[nt][r] + bh);
#pragma unroll
          for (int o = 0; o < NOUT; ++o) part[o][nt] = fmaf(w2v[o], gv, part[o][nt]);
        }
      }
    }
    float* s_red = s_h;  // [4 waves][NOUT][kPwP]
#pragma unroll
    for (int o = 0; o < NOUT; ++o)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        float v = part[o][nt];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (q == 0) s_red[(wave * NOUT + o) * kPwP + 16 * nt + m] = v;
      }
    __syncthreads();
    for (int e = tid; e < NOUT * (kPwP / 4); e += 256) {
      const int o = e / (kPwP / 4), c4 = e % (kPwP / 4);
      const float bo = masked_bias(b2, o, cout);
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int pp = 4 * c4 + j;
        v[j] = bo + (((s_red[(0 * NOUT + o) * kPwP + pp] +
                       s_red[(1 * NOUT + o) * kPwP + pp]) +
                      s_red[(2 * NOUT + o) * kPwP + pp]) +
                     s_red[(3 * NOUT + o) * kPwP + pp]);
      }
      float* dst = y + ((int64_t)b * cout + o) * npts + p0 + 4 * c4;
      if (4 * c4 + 4 <= np && (npts % 4) == 0) {
        *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (4 * c4 + j < np) dst[j] = v[j];
      }
    }
    return;
  }
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

// v = h + m + l exactly for eight floats: h = bf16(v), m = bf16(v - h), l = bf16(v - h - m),
// each rounded to nearest even (two values per conversion); every remainder is exact in
// float32 and carries the next 8 of v's 24 significant bits, so l is exact too.
__device__ __forceinline__ void split3_x8(const float (&v)[8], bf16x8& h, bf16x8& m,
                                          bf16x8& l) {
  uint32_t hh[4], mm[4], ll[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    hh[k] = pack_bf16x2(v[2 * k], v[2 * k + 1]);
    const float r0 = v[2 * k] - __uint_as_float(hh[k] << 16);
    const float r1 = v[2 * k + 1] - __uint_as_float(hh[k] & 0xffff0000u);
    mm[k] = pack_bf16x2(r0, r1);
    ll[k] = pack_bf16x2(r0 - __uint_as_float(mm[k] << 16),
                        r1 - __uint_as_float(mm[k] & 0xffff0000u));
  }
  h = __builtin_bit_cast(bf16x8, make_uint4(hh[0], hh[1], hh[2], hh[3]));
  m = __builtin_bit_cast(bf16x8, make_uint4(mm[0], mm[1], mm[2], mm[3]));
  l = __builtin_bit_cast(bf16x8, make_uint4(ll[0], ll[1], ll[2], ll[3]));
}

// The narrow projection (NOUT <= kPwSmallOut outputs) for cin <= 32, hidden <= 64 MPW and a point
// count that is a multiple of kPwP, as a grid-stride walk over the 64-point tiles of all batch
// entries.  What k_pointwise_mfma<NOUT> loads per tile stays in registers for the whole walk:
// wave w's W1 fragments (M-tiles w + 4 j, j < MPW; K padded to 32 with zero weights and zero
// x rows), b1 (the accumulators start from it) and W2 / 2 (GELU's factor 1/2 is exact there).
// The next tile's x rows are loaded into registers while the current one is multiplied.
// The first product runs in float32 precision on the bfloat16 matrix cores: both operands are
// split exactly into three bfloat16 terms and the six term products of order <= 2 are
// accumulated in float32 (the dropped three are below 2^-23 |a b|), one 16x16x32 MFMA per term
// product over the whole K, 96 cycles per 16x16 tile against 256 for eight float32 16x16x4
// MFMAs.  The x tile is staged as the three term planes [point][32 channels] (64-byte point
// rows of four 16-byte channel chunks, chunk c of point p at c ^ ((p >> 1) & 3), so that eight
// consecutive lanes of a 16-byte access cover every bank).  Same summation order over the
// hidden rows and waves as the tile kernel, except that the bias enters the products first.
template <int NOUT, int MPW>
__global__ void __launch_bounds__(256)
    __attribute__((amdgpu_waves_per_eu(NOUT * MPW < 6 ? 4 : 3)))
k_proj_narrow(int64_t ntiles, int64_t tiles_per_entry, int64_t npts, int cin, int hidden,
              const float* __restrict__ x, const float* __restrict__ w1,
              const float* __restrict__ b1, const float* __restrict__ w2,
              const float* __restrict__ b2, float* __restrict__ y) {
  __shared__ uint4 s_xs[3 * kPwP * 4];                                   // [term][point][chunk]
  __shared__ __attribute__((aligned(16))) float s_red[4 * NOUT * kPwP];  // [wave][o][point]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  bf16x8 wh[MPW], wm[MPW], wl[MPW];
  float w2h[MPW][4][NOUT];
  f32x4 bias0[MPW];
#pragma unroll
  for (int j = 0; j < MPW; ++j) {
    // A operand: lane (m, q) holds W1[16 mt + m][8 q + e], e = 0..7
    const int row = 16 * (wave + 4 * j) + m;
    const float* wr = w1 + (int64_t)min(row, hidden - 1) * cin;
    float wv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = 8 * q + e;
      const float v = wr[min(k, cin - 1)];
      wv[e] = __uint_as_float(__float_as_uint(v) & (row < hidden && k < cin ? ~0u : 0u));
    }
    split3_x8(wv, wh[j], wm[j], wl[j]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 16 * (wave + 4 * j) + 4 * q + r;
      bias0[j][r] = masked_bias(b1, h, hidden);
#pragma unroll
      for (int o = 0; o < NOUT; ++o) {
        const float wv2 = w2[o * hidden + min(h, hidden - 1)];
        w2h[j][r][o] = 0.5f * __uint_as_float(__float_as_uint(wv2) & (h < hidden ? ~0u : 0u));
      }
    }
  }
  // the output bias of the channel this thread stores (threads below NOUT * 16), loaded once:
  // a load in the store phase would wait for the next tile's loads as well
  const float bo = masked_bias(b2, tid / (kPwP / 4), NOUT);
  // x: thread (point p = tid % 64, channel chunk cg = tid / 64) loads channels 8 cg .. 8 cg + 7
  // of its point (clamped into the input; channels >= cin are zeroed when staged)
  const int p = tid & (kPwP - 1), cg = tid / kPwP;
  float xv[8];
  auto load_tile = [&](int64_t i) {
    const int64_t b = i / tiles_per_entry, t = i - b * tiles_per_entry;
    const float* xb = x + b * cin * npts + t * kPwP + p;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      xv[e] = __builtin_nontemporal_load(xb + (int64_t)min(8 * cg + e, cin - 1) * npts);
  };
  const int64_t G = gridDim.x;
  int64_t i = blockIdx.x;
  load_tile(i);
  for (; i < ntiles; i += G) {
    {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = __uint_as_float(__float_as_uint(xv[e]) & (8 * cg + e < cin ? ~0u : 0u));
      bf16x8 h, mm, l;
      split3_x8(v, h, mm, l);
      const int slot = 4 * p + (cg ^ ((p >> 1) & 3));
      s_xs[slot] = __builtin_bit_cast(uint4, h);
      s_xs[4 * kPwP + slot] = __builtin_bit_cast(uint4, mm);
      s_xs[8 * kPwP + slot] = __builtin_bit_cast(uint4, l);
    }
    __syncthreads();
    // the next tile of this work-group (the last walk reloads its own tile, unused): its loads
    // are in flight while this tile is multiplied
    load_tile(min(i + G, ntiles - 1));
    float part[NOUT][4];
#pragma unroll
    for (int o = 0; o < NOUT; ++o)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) part[o][nt] = 0.f;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      // B operand: lane (m, q) holds x[8 q + e][point 16 nt + m]
      const int pp = 16 * nt + m;
      const int slot = 4 * pp + (q ^ ((pp >> 1) & 3));
      const bf16x8 bh = __builtin_bit_cast(bf16x8, s_xs[slot]);
      const bf16x8 bm = __builtin_bit_cast(bf16x8, s_xs[4 * kPwP + slot]);
      const bf16x8 bl = __builtin_bit_cast(bf16x8, s_xs[8 * kPwP + slot]);
#pragma unroll
      for (int j = 0; j < MPW; ++j) {
        f32x4 acc = bias0[j];  // the six term products, smallest first
        acc = mfma_bf16(wm[j], bm, acc);
        acc = mfma_bf16(wh[j], bl, acc);
        acc = mfma_bf16(wl[j], bh, acc);
        acc = mfma_bf16(wh[j], bm, acc);
        acc = mfma_bf16(wm[j], bh, acc);
        acc = mfma_bf16(wh[j], bh, acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = acc[r];
          const float g2 = fmaf(fabsf(v), normal_erf(v).erf_abs, v);  // 2 GELU(v)
#pragma unroll
          for (int o = 0; o < NOUT; ++o) part[o][nt] = fmaf(w2h[j][r][o], g2, part[o][nt]);
        }
      }
    }
#pragma unroll
    for (int o = 0; o < NOUT; ++o)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        float v = part[o][nt];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (q == 0) s_red[(wave * NOUT + o) * kPwP + 16 * nt + m] = v;
      }
    __syncthreads();
    // one float4 of 4 points per thread of the first NOUT * 16; s_x and s_red are next written
    // after the following tile's first barrier, which these reads precede
    if (tid < NOUT * (kPwP / 4)) {
      const int o = tid / (kPwP / 4), c4 = tid % (kPwP / 4);
      float v[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int pp = 4 * c4 + jj;
        v[jj] = bo + (((s_red[(0 * NOUT + o) * kPwP + pp] + s_red[(1 * NOUT + o) * kPwP + pp]) +
                       s_red[(2 * NOUT + o) * kPwP + pp]) +
                      s_red[(3 * NOUT + o) * kPwP + pp]);
      }
      const int64_t b = i / tiles_per_entry, t = i - b * tiles_per_entry;
      *reinterpret_cast<float4*>(y + (b * NOUT + o) * npts + t * kPwP + 4 * c4) =
          make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// A lift from at most four input channels does 2 cin flops per output value, too little for the
// matrix cores: a thread takes 4 consecutive points of one batch entry and writes them for
// every output channel (each output row leaves as float4 stores, contiguous over the threads),
// so the kernel is bound by its output stream.
template <int CIN>
__global__ void __launch_bounds__(256)
k_lift_valu(int64_t npts, int cout, const float* __restrict__ x, const float* __restrict__ w1,
            const float* __restrict__ b1, float* __restrict__ y) {
  const int b = blockIdx.y;
  const int64_t p = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (p >= npts) return;  // npts % 4 == 0: a thread's four points are all present or all absent
  float4 xv[CIN];
#pragma unroll
  for (int c = 0; c < CIN; ++c) xv[c] = load_stream4(x + ((int64_t)b * CIN + c) * npts + p);
  float* yb = y + (int64_t)b * cout * npts + p;
  for (int o = 0; o < cout; ++o) {
    const float bo = b1 ? b1[o] : 0.f;
    float4 v = make_float4(bo, bo, bo, bo);
#pragma unroll
    for (int c = 0; c < CIN; ++c) {
      const float wc = w1[o * CIN + c];
      v.x = fmaf(wc, xv[c].x, v.x);
      v.y = fmaf(wc, xv[c].y, v.y);
      v.z = fmaf(wc, xv[c].z, v.z);
      v.w = fmaf(wc, xv[c].w, v.w);
    }
    *reinterpret_cast<float4*>(yb + (int64_t)o * npts) = v;
  }
}

hipError_t launch_pointwise(int64_t batch, int64_t npts, int cin, int hidden, int cout,
                            const float* x, const float* w1, const float* b1, const float* w2,
                            const float* b2, float* y, hipStream_t s) {
  auto al16 = [](const void* v) { return ((uintptr_t)v & 15u) == 0; };
  if (hidden == 0 && cin <= 4 && npts % 4 == 0 && al16(x) && al16(y)) {
    const int64_t groups = (npts / 4 + 255) / 256;
    if (groups > 0x7fffffff || batch > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)groups, (unsigned)batch);
    switch (cin) {
      case 1: hipLaunchKernelGGL(k_lift_valu<1>, grid, dim3(256), 0, s, npts, cout, x, w1, b1, y);
              break;
      case 2: hipLaunchKernelGGL(k_lift_valu<2>, grid, dim3(256), 0, s, npts, cout, x, w1, b1, y);
              break;
      case 3: hipLaunchKernelGGL(k_lift_valu<3>, grid, dim3(256), 0, s, npts, cout, x, w1, b1, y);
              break;
      default: hipLaunchKernelGGL(k_lift_valu<4>, grid, dim3(256), 0, s, npts, cout, x, w1, b1, y);
               break;
    }
    return hipGetLastError();
  }
  if (hidden > 0 && cout <= kPwSmallOut && cin <= 32 && hidden <= 128 && npts % kPwP == 0 &&
      al16(x) && al16(y)) {
    const int64_t tpe = npts / kPwP, ntiles = batch * tpe;
    // eight work-groups per compute unit; each walks about ntiles / 2048 tiles
    const unsigned grid = (unsigned)min(ntiles, (int64_t)2048);
    const bool two = hidden > 64;
#define FNO_PROJ_NARROW(NO)                                                                     \
  if (two)                                                                                    \
    hipLaunchKernelGGL((k_proj_narrow<NO, 2>), dim3(grid), dim3(256), 0, s, ntiles, tpe, npts, \
                       cin, hidden, x, w1, b1, w2, b2, y);                                    \
  else                                                                                        \
    hipLaunchKernelGGL((k_proj_narrow<NO, 1>), dim3(grid), dim3(256), 0, s, ntiles, tpe, npts, \
                       cin, hidden, x, w1, b1, w2, b2, y);
    switch (cout) {
      case 1: FNO_PROJ_NARROW(1) break;
      case 2: FNO_PROJ_NARROW(2) break;
      case 3: FNO_PROJ_NARROW(3) break;
      default: FNO_PROJ_NARROW(4) break;
    }
#undef FNO_PROJ_NARROW
    return hipGetLastError();
  }
  const int cin_p = (cin + 15) / 16 * 16;
  const int mid = hidden > 0 ? hidden : cout;
  const int mid_p = (mid + 15) / 16 * 16;
  const int cout_p = (cout + 15) / 16 * 16;
  // a narrow projection keeps only the x tile and the per-wave partial sums (in s_h's place)
  const size_t lds = (hidden > 0 && cout <= kPwSmallOut)
                         ? sizeof(float) * ((size_t)kPwS * cin_p + 4 * kPwSmallOut * kPwP)
                         : sizeof(float) * kPwS * (cin_p + mid_p + (hidden > 0 ? cout_p : 0));
  const int64_t tiles = (npts + kPwP - 1) / kPwP;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  if (lds > 65536) {  // wide hidden layers need more than the default dynamic LDS limit
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_pointwise_mfma<0>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)tiles, (unsigned)batch);
  const int nout = (hidden > 0 && cout <= kPwSmallOut) ? cout : 0;
  switch (nout) {
    case 1: hipLaunchKernelGGL((k_pointwise_mfma<1>), grid, dim3(256), lds, s, npts, cin, hidden,
                               cout, x, w1, b1, w2, b2, y); break;
    case 2: hipLaunchKernelGGL((k_pointwise_mfma<2>), grid, dim3(256), lds, s, npts, cin, hidden,
                               cout, x, w1, b1, w2, b2, y); break;
    case 3: hipLaunchKernelGGL((k_pointwise_mfma<3>), grid, dim3(256), lds, s, npts, cin, hidden,
                               cout, x, w1, b1, w2, b2, y); break;
    case 4: hipLaunchKernelGGL((k_pointwise_mfma<4>), grid, dim3(256), lds, s, npts, cin, hidden,
                               cout, x, w1, b1, w2, b2, y); break;
    default: hipLaunchKernelGGL((k_pointwise_mfma<0>), grid, dim3(256), lds, s, npts, cin,
                                hidden, cout, x, w1, b1, w2, b2, y); break;
  }
  return hipGetLastError();
}

}  // namespace fno
