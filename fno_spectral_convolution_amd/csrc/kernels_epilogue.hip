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
// Work split: a work-group walks a contiguous range of 64-point groups (whole lines of the
// contiguous axis).  All 256 threads load the group's channel rows with float4 (prefetched one
// group ahead) into [channel][point] LDS tiles; the spectrum rows of the current line are
// staged in LDS once per line.  The 4 waves then split the 16x16 output tiles.  Products are
// computed transposed (points x channels):
//   spectral part : 16x16x32 bf16 (mixed path) or 16x16x4 f32 MFMA, K = 2 mb (padded)
//   bypass / grads: 16x16x4 f32 MFMA, K = channels (4 per step) or points (backward dWb)
// The last-axis table is read through L2 (shared by every wave); Wb slices sit in registers.
#include "fno_internal.h"
#include "mfma.h"
#include "pointwise.h"

#include <math.h>
#include <type_traits>

namespace fno {

struct EpiArgs {
  int B, C;            // batch, channels (Cin = Cout = C)
  int64_t P;           // points per field
  int Nb, mb, kpad;    // contiguous axis, its retained bins, padded 2*mb
  int64_t lines;       // P / Nb
  int lpw;             // consecutive lines of one batch entry per work-group
  int gpl_log2;        // log2 of the point groups per line (Nb / 64)
  const float* x;
  const void* T;       // [B][C][lines][mb] complex: float32, or the plan's half format (TH)
  const float* wb;     // [C][C] (o, i)
  const float* bias;   // [C] or null
  const void* gt;      // [Nb][kpad] f32 or half bits (the plan's format)
  float* y;            // forward output (or grad_x backward)
  float* z;            // forward z save (nullable)
  const float* gy;     // backward incoming gradient
  const float* zin;    // backward saved z
  float* part;         // backward per-group partials [grid][C*C + C]
  double* lpart;       // forward with the fused loss: per-group sums of (y - t)^2 [grid]
  float msc;           // its gradient scale (grad_scale 2 / n); the target is gy
  int block;           // bypass/bias/GELU present (else spectral only)
  int gelu;
  int* flag;           // IEEE-half plans: set to 1 when a non-finite output is written
};

__device__ __forceinline__ float comp(const float4& v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

constexpr int PG = 64;        // points per group (one line of the contiguous axis holds Nb/PG)
constexpr int XS = PG + 4;    // LDS row stride (floats) of the [channel][point] tiles
constexpr int kMaxKpad = 64;  // 2*mb padded; larger spectra take the generic kernels

// Stage the spectrum rows of one line (every channel, 2*mb floats) into LDS as the B operand
// of the spectral product: bf16 [CP][kpad + 8] or f32 [CP][kpad + 4], zero padded.
// T0: complex index of channel 0's row of the line; TH: T holds the half format already (the
// outer inverse rounded it as this staging would), so its bits are copied.
template <int C, int H, bool TH>
__device__ __forceinline__ void stage_line(const EpiArgs& a, int64_t T0, unsigned char* tl,
                                           int tid) {
  constexpr bool BF = H != 0;
  constexpr int CP = (C + 15) / 16 * 16;
  constexpr int kst = kMaxKpad + (BF ? 8 : 4);
  const int64_t cstride = a.lines * a.mb;
  const int kf_end = 2 * a.mb;
  constexpr int g4 = kMaxKpad / 4;  // columns kf_end .. kMaxKpad - 1 are written as zeros
  for (int e = tid; e < CP * g4; e += 256) {
    const int c = e / g4, k4 = 4 * (e - c * g4);
    const int64_t off = 2 * (T0 + (int64_t)c * cstride) + k4;  // float (or half) units
    if constexpr (TH) {
      uint2 raw = make_uint2(0u, 0u);
      if (c < C && k4 < kf_end) raw = *reinterpret_cast<const uint2*>(
                                    static_cast<const uint16_t*>(a.T) + off);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(tl) + c * kst + k4) = raw;
      continue;
    }
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < C && k4 < kf_end)
      v = *reinterpret_cast<const float4*>(static_cast<const float*>(a.T) + off);
    if (BF) {
      uint2 pk;
      pk.x = HalfOf<H>::pack2(v.x, v.y);
      pk.y = HalfOf<H>::pack2(v.z, v.w);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(tl) + c * kst + k4) = pk;
    } else {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(tl) + c * kst + k4) = v;
    }
  }
}

// The same staging split in two, so that a line's spectrum rows can be loaded while the
// previous line is computed: float4 e = tid + 256 i is channel e / 16, columns 4 (e % 16) ..;
// outside the spectrum (channel >= C or column >= 2 mb) a clamped address is loaded and zeros
// are written.
template <int C, bool TH>
struct LineT {
  static constexpr int CP = (C + 15) / 16 * 16;
  static constexpr int N = (CP * (kMaxKpad / 4) + 255) / 256;
  std::conditional_t<TH, uint2, float4> v[N];  // 4 columns: half bits, or float32
};

template <int C, bool TH>
__device__ __forceinline__ void load_line(const EpiArgs& a, int64_t T0, LineT<C, TH>& t,
                                          int tid) {
  const int64_t cstride = a.lines * a.mb;
#pragma unroll
  for (int i = 0; i < LineT<C, TH>::N; ++i) {
    const int e = tid + 256 * i;
    const int c = min(e >> 4, C - 1), k4 = min(4 * (e & 15), 2 * a.mb - 4);
    const int64_t off = 2 * (T0 + (int64_t)c * cstride) + k4;
    if constexpr (TH)
      t.v[i] = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.T) + off);
    else
      t.v[i] = *reinterpret_cast<const float4*>(static_cast<const float*>(a.T) + off);
  }
}

template <int C, int H, bool TH>
__device__ __forceinline__ void write_line(const EpiArgs& a, const LineT<C, TH>& t,
                                           unsigned char* tl, int tid) {
  constexpr bool BF = H != 0;
  constexpr int kst = kMaxKpad + (BF ? 8 : 4);
#pragma unroll
  for (int i = 0; i < LineT<C, TH>::N; ++i) {
    const int e = tid + 256 * i;
    if (e >= LineT<C, TH>::CP * (kMaxKpad / 4)) break;
    const int c = e >> 4, k4 = 4 * (e & 15);
    const bool live = c < C && k4 < 2 * a.mb;
    if constexpr (TH) {
      const uint2 raw = live ? t.v[i] : make_uint2(0u, 0u);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(tl) + c * kst + k4) = raw;
      continue;
    } else {
    const float4 v = live ? t.v[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    if (BF) {
      uint2 pk;
      pk.x = HalfOf<H>::pack2(v.x, v.y);
      pk.y = HalfOf<H>::pack2(v.z, v.w);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(tl) + c * kst + k4) = pk;
    } else {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(tl) + c * kst + k4) = v;
    }
    }
  }
}

// Fragments of the last-axis table for one point group of this wave: A operand rows
// pb0 + 16 (tbase + j) + m, all K-steps (kpad <= 64).  Loaded one group ahead.
template <int TMW, int H>
struct GtFrag {
  typename HalfOf<H>::v8 v[TMW][2];  // K-steps of 32
};
template <int TMW>
struct GtFrag<TMW, 0> {
  float4 v[TMW][4];  // K-groups of 16
};

// Point of a 64-point step held by row i of M-tile t (one tile per wave, one 64-point group
// per step): 16 (i % 4) + 4 t + i / 4.  Result row 4 q + r of a tile is then point
// 16 r + 4 t + q, so the 64 lanes writing (or reading) one register of a tile in a
// [channel][point] LDS tile of row stride 68 floats (16 channel rows m, 4 q) hit 64 distinct
// banks, and row m of the A operand (point 16 (m % 4) + 4 t + m / 4) spreads a lane quarter's
// reads of 8 channel rows over two bank halves.
__device__ __forceinline__ int step_point1(int i, int t) {
  return 16 * (i & 3) + 4 * t + (i >> 2);
}

template <int TMW, int H, bool IL = false, int MT = 4>
__device__ __forceinline__ void load_gt(const EpiArgs& a, int pb0, int tbase, int m, int q,
                                        GtFrag<TMW, H>& f) {
  constexpr bool BF = H != 0;
  using V8 = typename HalfOf<H>::v8;
#pragma unroll
  for (int j = 0; j < TMW; ++j) {
    // row m of M-tile t: point MT m + t (interleaved over the MT tiles of the step) or
    // 16 t + m of the group
    const int pt = IL ? (TMW == 1 ? step_point1(m, tbase) : MT * m + tbase + j)
                      : 16 * (tbase + j) + m;
    const int64_t row = (int64_t)(pb0 + pt) * a.kpad;
    if constexpr (BF) {
      const uint16_t* gt = static_cast<const uint16_t*>(a.gt) + row;
#pragma unroll
      for (int s = 0; s < 2; ++s) f.v[j][s] = *reinterpret_cast<const V8*>(gt + 32 * s + 8 * q);
    } else {
      const float* gt = static_cast<const float*>(a.gt) + row;
#pragma unroll
      for (int g = 0; g < 4; ++g) f.v[j][g] = *reinterpret_cast<const float4*>(gt + 16 * g + 4 * q);
    }
  }
}

// 1, 2 or 4 adjacent floats from / to LDS in one access (the pointer is aligned to the run)
template <int N>
__device__ __forceinline__ void load_lds_run(float (&v)[N], const float* p) {
  if constexpr (N == 4) {
    const float4 t = *reinterpret_cast<const float4*>(p);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  } else if constexpr (N == 2) {
    const float2 t = *reinterpret_cast<const float2*>(p);
    v[0] = t.x; v[1] = t.y;
  } else {
    v[0] = *p;
  }
}

template <int N>
__device__ __forceinline__ void store_lds_run(float* p, const float (&v)[N]) {
  if constexpr (N == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  } else if constexpr (N == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  } else {
    *p = v[0];
  }
}

// Row loads of a [C][64 G] tile (NF4 = 16 G C float4): thread t takes float4 t + 256 u, i.e.
// channel t / (16 G) + u (256 / 16 G), points 4 (t % 16 G) .. + 3, from base (already offset to
// this thread's first row and point).
template <int NF4, int NPT>
__device__ __forceinline__ void load_rows(float4 (&v)[NPT], const float* base, int64_t ustride,
                                          int tid) {
#pragma unroll
  for (int u = 0; u < NPT; ++u) {
    if constexpr (NF4 % 256 == 0) {
      v[u] = *reinterpret_cast<const float4*>(base + u * ustride);
    } else {
      if (tid + 256 * u < NF4) v[u] = *reinterpret_cast<const float4*>(base + u * ustride);
    }
  }
}

// ------------------------------------------------------------------------------------------
// Forward.  A work-group owns lpw consecutive lines of one batch entry: a contiguous range of
// points, walked in steps of G 64-point groups (G = 2 for narrow fields).  The spectrum rows of
// a line are staged in LDS when the line starts (narrow fields: loaded one line ahead); the
// step loop itself is straight-line code, so the compiler can keep the prefetches in flight
// across it: the x rows of step f + 1 are loaded while step f is computed, then the table
// fragments of step f + 1 (the last step re-loads itself instead of branching).  Wave w owns
// the M-tiles (16 points each) w G .. w G + G - 1 of the step for every channel tile, so each
// table fragment is loaded once per work-group and each x operand feeds NT products.  With
// G = 2, row m of M-tile t is point MT m + t of the step (MT = 4 G tiles), so a lane's A
// operands of its two tiles are adjacent in the [channel][point] LDS tile; with G = 1 it is
// point 16 (m % 4) + 4 t + m / 4 (step_point1), which keeps the LDS accesses of the result
// layout free of bank conflicts.  The z tile goes through LDS and the
// stores are row-contiguous: 16 G threads write one channel's 64 G points.
// MODE: 0 spectral part only, 1 block (bypass, bias, optional GELU), 2 block + z save; plus 8
// when x is a pre-activation (the bypass takes GELU(x), applied as the x tile is staged); plus
// 16 (with 1) for the fused MSE loss: the target rows of a step are loaded at its start and
// the store phase writes msc (y - t) GELU'(z) in place of y, and adds (y - t)^2 to a per-thread
// sum, reduced over the work-group in a fixed order into one partial at the end.
template <int C, int H, int MODE, int G, bool TH, int GPL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(C == 64 ? 3 : 4)))
k_epi_fwd_line(EpiArgs a) {
  constexpr bool BF = H != 0;  // half operands (bfloat16 or IEEE half)
  using V8 = typename HalfOf<H>::v8;
  constexpr int CP = (C + 15) / 16 * 16;
  constexpr int NT = CP / 16;
  constexpr int PI = PG * G;        // points per step
  constexpr int XSG = PI + 4;       // LDS row stride (floats)
  constexpr int MT = 4 * G;         // M-tiles per step; wave w owns tiles w G .. w G + G - 1
  constexpr int FPC = 16 * G;       // float4 per channel row of a step
  constexpr int NF4 = FPC * C;      // float4 of an x / z tile
  constexpr int NPT = (NF4 + 255) / 256;
  constexpr bool BLK = (MODE & 3) >= 1;
  constexpr bool ZS = (MODE & 3) == 2;
  constexpr bool IG = (MODE & 8) != 0;
  constexpr bool MS = (MODE & 16) != 0;
  static_assert(G == 1 || G == 2, "LDS runs of 1 or 2 floats");
  static_assert(!MS || (MODE & 3) == 1, "the fused loss replaces y and takes no z save");
  __shared__ __attribute__((aligned(16))) float s_x[BLK ? CP * XSG : 4];
  __shared__ __attribute__((aligned(16))) float s_o[CP * XSG];
  __shared__ double s_loss[MS ? 4 : 1];
  __shared__ __attribute__((aligned(16))) unsigned char s_tl[CP * (kMaxKpad + 8) * (BF ? 2 : 4)];
  __shared__ float s_bias[CP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  const int tbase = wave * G;
  // step point of row i of this wave's first tile (G = 2: tiles tbase, tbase + 1 interleaved,
  // so the two tiles' points are adjacent)
  auto lp = [&](int i) { return G == 1 ? step_point1(i, tbase) : MT * i + tbase; };
  const int64_t wg_per_b = a.lines / a.lpw;
  const int b = (int)(blockIdx.x / wg_per_b);
  const int64_t l0 = (int64_t)(blockIdx.x - (int64_t)b * wg_per_b) * a.lpw;
  const int gpl = 1 << a.gpl_log2;  // steps per line
  const int nf = a.lpw << a.gpl_log2;
  // S3: on half plans with a multiple of 32 channels the bypass runs as three bf16 products
  // of hi / lo split operands (float32 accumulation), K-steps of 32 channels
  constexpr bool S3 = BF && (C % 32 == 0);
  constexpr int KS = S3 ? C / 32 : 1;
  // Wb^T slices: B operand of channel tile ct, K-step kb, lane (n = m, q): Wb[16 ct + m][4 kb + q]
  float wbr[BLK && !S3 ? NT : 1][BLK && !S3 ? C / 4 : 1];
  // S3: K-step s, lane (n = m, q) holds Wb[16 ct + m][32 s + 8 q + e], e = 0..7, split
  bf16x8 wbh[BLK && S3 ? NT : 1][KS], wbl[BLK && S3 ? NT : 1][KS];
  if (BLK) {
    if constexpr (S3) {
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const float* row = a.wb + (16 * ct + m) * C + 32 * s + 8 * q;
          const float4 w0 = *reinterpret_cast<const float4*>(row);
          const float4 w1 = *reinterpret_cast<const float4*>(row + 4);
          const float v[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
          split_bf16x8(v, wbh[ct][s], wbl[ct][s]);
        }
    } else {
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        const int o = 16 * ct + m;
#pragma unroll
        for (int kb = 0; kb < C / 4; ++kb) {
          const float w = a.wb[min(o, C - 1) * C + 4 * kb + q];
          wbr[ct][kb] = o < C ? w : 0.f;
        }
      }
    }
  }
  for (int o = tid; o < CP; o += 256) s_bias[o] = (BLK && o < C && a.bias) ? a.bias[o] : 0.f;
  // float4 e = tid + 256 u of a tile: channel e / FPC, points 4 (e % FPC) .. + 3.  Past the
  // tile (e >= NF4) a thread loads and stores a copy of the last float4 (identical data) and
  // writes its x into the padding rows C .. CP - 1, which nothing reads: no branch anywhere.
  static_assert(256 * NPT <= FPC * CP, "tail float4 land in the padding rows");
  const int64_t pbase = l0 * a.Nb;
  int64_t goff[NPT];
  int xl[NPT], ol[NPT];
#pragma unroll
  for (int u = 0; u < NPT; ++u) {
    const int e = tid + 256 * u, ec = min(e, NF4 - 1);
    goff[u] = ((int64_t)b * C + ec / FPC) * a.P + pbase + 4 * (ec % FPC);
    xl[u] = (e / FPC) * XSG + 4 * (e % FPC);
    ol[u] = (ec / FPC) * XSG + 4 * (ec % FPC);
  }
  float4 pre[NPT];
#pragma unroll
  for (int u = 0; u < NPT; ++u) pre[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  // fused loss: target rows of the current step; the copies past the tile add nothing
  float4 ptg[MS ? NPT : 1];
  double lsum = 0.0;
  bool bad = false;  // IEEE-half plans: a non-finite output was written
  // table fragments: GPL == 0 reloads fragment 0 for every step; GPL = 1 or 2 (the steps of a
  // line) keeps the fragment of each step of a line in registers for the whole work-group
  GtFrag<G, H> gts[GPL > 0 ? GPL : 1];
  if (BLK) {
#pragma unroll
    for (int u = 0; u < NPT; ++u) pre[u] = load_stream4(a.x + goff[u]);
  }
#pragma unroll
  for (int gg = 0; gg < (GPL > 0 ? GPL : 1); ++gg)
    load_gt<G, H, true, MT>(a, gg * PI, tbase, m, q, gts[gg]);
  // narrow fields have few steps per line: the next line's spectrum rows stream in while
  // this one is computed (the last line re-loads itself); wide ones stage each line directly
  constexpr bool LPF = C < 64;
  const int64_t Tb = ((int64_t)b * C * a.lines + l0) * a.mb;  // complex index of this range
  LineT<LPF ? C : 16, TH> tln;
  if constexpr (LPF) load_line<C, TH>(a, Tb, tln, tid);
  constexpr int kst = kMaxKpad + (BF ? 8 : 4);
  for (int lf = 0; lf < a.lpw; ++lf) {
    // every reader of the previous line's spectrum is past that line's last barrier
    if constexpr (LPF) {
      write_line<C, H, TH>(a, tln, s_tl, tid);
      load_line<C, TH>(a, Tb + (int64_t)min(lf + 1, a.lpw - 1) * a.mb, tln, tid);
    } else {
      stage_line<C, H, TH>(a, Tb + (int64_t)lf * a.mb, s_tl, tid);
    }
#pragma unroll(GPL > 0 ? GPL : 1)
    for (int g = 0; g < (GPL > 0 ? GPL : gpl); ++g) {
      const GtFrag<G, H>& gtf = gts[GPL > 0 ? g : 0];
      const int f = (lf << a.gpl_log2) + g;
      const int fn = min(f + 1, nf - 1);
      if (BLK) {
#pragma unroll
        for (int u = 0; u < NPT; ++u) {
          float4 xv = pre[u];
          if constexpr (IG) {
            xv.x = gelu_as(xv.x);
            xv.y = gelu_as(xv.y);
            xv.z = gelu_as(xv.z);
            xv.w = gelu_as(xv.w);
          }
          *reinterpret_cast<float4*>(s_x + xl[u]) = xv;
        }
        // this step's target rows go out before the next step's x rows: the store phase
        // waits only for them
        if constexpr (MS) {
#pragma unroll
          for (int u = 0; u < NPT; ++u)
            ptg[u] = load_stream4(a.gy + goff[u] + PI * f);
        }
#pragma unroll
        for (int u = 0; u < NPT; ++u)
          pre[u] = load_stream4(a.x + goff[u] + PI * fn);
      }
      __syncthreads();  // x tile and spectrum rows visible; previous z tile consumed
      f32x4 acc[G][NT];
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) acc[j][ct] = zero4();
      // spectral part: A = table rows of this wave's tiles, B = spectrum row of channel 16 ct + m
      if constexpr (BF) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          if (32 * s2 >= a.kpad) break;
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) {
            const V8 B = *reinterpret_cast<const V8*>(
                reinterpret_cast<const uint16_t*>(s_tl) + (16 * ct + m) * kst + 32 * s2 + 8 * q);
#pragma unroll
            for (int j = 0; j < G; ++j) acc[j][ct] = HalfOf<H>::mfma(gtf.v[j][s2], B, acc[j][ct]);
          }
        }
      } else {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          if (16 * g4 >= a.kpad) break;
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) {
            const float4 B4 = *reinterpret_cast<const float4*>(
                reinterpret_cast<const float*>(s_tl) + (16 * ct + m) * kst + 16 * g4 + 4 * q);
#pragma unroll
            for (int j = 0; j < G; ++j) {
              acc[j][ct] = mfma_f32(gtf.v[j][g4].x, B4.x, acc[j][ct]);
              acc[j][ct] = mfma_f32(gtf.v[j][g4].y, B4.y, acc[j][ct]);
              acc[j][ct] = mfma_f32(gtf.v[j][g4].z, B4.z, acc[j][ct]);
              acc[j][ct] = mfma_f32(gtf.v[j][g4].w, B4.w, acc[j][ct]);
            }
          }
        }
      }
      if constexpr (GPL == 0) load_gt<G, H, true, MT>(a, (fn & (gpl - 1)) * PI, tbase, m, q, gts[0]);
      if (BLK) {
        if constexpr (S3) {
          // A: lane (m, q) holds x[32 s + 8 q + e][point MT m + tbase + j], split
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            float xv[8][G];
#pragma unroll
            for (int e = 0; e < 8; ++e)
              load_lds_run<G>(xv[e], s_x + (32 * s + 8 * q + e) * XSG + lp(m));
#pragma unroll
            for (int j = 0; j < G; ++j) {
              float v[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] = xv[e][j];
              bf16x8 ah, al;
              split_bf16x8(v, ah, al);
#pragma unroll
              for (int ct = 0; ct < NT; ++ct)
                acc[j][ct] = mfma_split3(ah, al, wbh[ct][s], wbl[ct][s], acc[j][ct]);
            }
          }
        } else {
#pragma unroll
          for (int kb = 0; kb < C / 4; ++kb) {
            float av[G];
            load_lds_run<G>(av, s_x + (4 * kb + q) * XSG + lp(m));
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
              for (int j = 0; j < G; ++j) acc[j][ct] = mfma_f32(av[j], wbr[ct][kb], acc[j][ct]);
          }
        }
      }
      // lane (n = m, q), tile tbase + j, register r: channel 16 ct + m, point
      // lp(4 q + r) + j
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        const int o = 16 * ct + m;
        const float bo = s_bias[o];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v[G];
#pragma unroll
          for (int j = 0; j < G; ++j) v[j] = acc[j][ct][r] + bo;
          store_lds_run<G>(s_o + o * XSG + lp(4 * q + r), v);
        }
      }
      __syncthreads();  // z tile complete; x tile free
#pragma unroll
      for (int u = 0; u < NPT; ++u) {
        float4 v = *reinterpret_cast<const float4*>(s_o + ol[u]);
        const int64_t off = goff[u] + PI * f;
        if constexpr (MS) {
          float4 yv = v, gp = make_float4(1.f, 1.f, 1.f, 1.f);
          if (a.gelu) {
            gelu_and_grad(v.x, yv.x, gp.x);
            gelu_and_grad(v.y, yv.y, gp.y);
            gelu_and_grad(v.z, yv.z, gp.z);
            gelu_and_grad(v.w, yv.w, gp.w);
          }
          const float4 d = make_float4(yv.x - ptg[u].x, yv.y - ptg[u].y, yv.z - ptg[u].z,
                                       yv.w - ptg[u].w);
          const double sq = (double)(d.x * d.x + d.y * d.y) + (double)(d.z * d.z + d.w * d.w);
          if constexpr (256 * NPT == NF4) {
            lsum += sq;
          } else {
            lsum += (tid + 256 * u < NF4) ? sq : 0.0;
          }
          const float4 gzv = make_float4(a.msc * d.x * gp.x, a.msc * d.y * gp.y,
                                         a.msc * d.z * gp.z, a.msc * d.w * gp.w);
          if constexpr (H == 2) bad |= !finite4(gzv);
          *reinterpret_cast<float4*>(a.y + off) = gzv;
          continue;
        }
        if (ZS) *reinterpret_cast<float4*>(a.z + off) = v;
        if (BLK && a.gelu) {
          v.x = gelu_as(v.x);
          v.y = gelu_as(v.y);
          v.z = gelu_as(v.z);
          v.w = gelu_as(v.w);
        }
        if constexpr (H == 2) bad |= !finite4(v);
        *reinterpret_cast<float4*>(a.y + off) = v;
      }
    }
  }
  if constexpr (H == 2) raise_half_flag(a.flag, bad);
  if constexpr (MS) {
    // fixed order: xor butterflies within each wave, then the four waves in turn
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o);
    if (lane == 0) s_loss[wave] = lsum;
    __syncthreads();
    if (tid == 0) a.lpart[blockIdx.x] = ((s_loss[0] + s_loss[1]) + s_loss[2]) + s_loss[3];
  }
}

// ------------------------------------------------------------------------------------------
// Backward.  Same line ownership and straight-line step pipeline as the forward (steps of G
// 64-point groups, wave w owning M-tiles w G .. w G + G - 1 for every channel tile): the g_y, z
// and x rows of step f + 1 and its table fragments are in flight while step f is computed.
//   grad_x tile : spectral product with the unit-scale table, times s(x) = 1 - tanh^2 on the
//                 tanh path, plus Wb^T g_z (A operand g_z in the interleaved point mapping);
//                 stored through LDS with row-contiguous float4 stores
//   dWb, dbias  : dWb[o][i] += sum_p g_z[o][p] x[i][p] (16x16x4 f32, K = points), reduced over
//                 the work-group in a fixed order into one partial row per work-group
// Wave w's dWb tiles: NT = 4: o-tile w, all 4 i-tiles; NT = 2: o-tile w >> 1, i-tile w & 1;
// NT = 1: the single tile over its quarter of the step's points.
// MODE: 1 spectral part only (grad_x = s(x) * spectral), 3 block, 7 block with GELU' (z read);
// plus 8 when x is a pre-activation: the x tile holds the block's input GELU(x) (for dWb and
// the tanh factor), a second tile GELU'(x), which multiplies the grad tile as it is stored.
template <int C, int H, bool TANH, int MODE, int G, bool TH, int GPL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(C == 64 ? 2 : 3)))
k_epi_bwd_line(EpiArgs a) {
  constexpr bool BF = H != 0;  // half operands (bfloat16 or IEEE half)
  using V8 = typename HalfOf<H>::v8;
  constexpr int CP = (C + 15) / 16 * 16;
  constexpr int NT = CP / 16;
  constexpr int PI = PG * G;        // points per step
  constexpr int XSG = PI + 4;       // LDS row stride (floats)
  constexpr int MT = 4 * G;         // M-tiles per step
  constexpr int FPC = 16 * G;       // float4 per channel row of a step
  constexpr int NF4 = FPC * C;
  constexpr int NPT = (NF4 + 255) / 256;
  constexpr bool BLK = (MODE & 2) != 0;
  constexpr bool GL = (MODE & 4) != 0;
  constexpr bool IG = (MODE & 8) != 0;
  constexpr bool NX = BLK || TANH || IG;  // x rows needed
  constexpr int DT = (NT == 4) ? 4 : 1;  // dWb tiles per wave
  static_assert(G == 1 || G == 2, "LDS runs of 1 or 2 floats");
  static_assert(256 * NPT <= FPC * CP, "tail float4 land in the padding rows");
  __shared__ __attribute__((aligned(16))) float s_gz[BLK ? CP * XSG : 4];
  __shared__ __attribute__((aligned(16))) float s_x[NX ? CP * XSG : 4];
  __shared__ __attribute__((aligned(16))) float s_o[CP * XSG];
  __shared__ __attribute__((aligned(16))) float s_gp[IG ? CP * XSG : 4];
  __shared__ __attribute__((aligned(16))) unsigned char s_tl[CP * (kMaxKpad + 8) * (BF ? 2 : 4)];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  const int tbase = wave * G;
  // step point of row i of this wave's first tile (G = 2: tiles tbase, tbase + 1 interleaved,
  // so the two tiles' points are adjacent)
  auto lp = [&](int i) { return G == 1 ? step_point1(i, tbase) : MT * i + tbase; };
  const int64_t wg_per_b = a.lines / a.lpw;
  const int b = (int)(blockIdx.x / wg_per_b);
  const int64_t l0 = (int64_t)(blockIdx.x - (int64_t)b * wg_per_b) * a.lpw;
  const int gpl = 1 << a.gpl_log2;
  const int nf = a.lpw << a.gpl_log2;
  // S3: on half plans with a multiple of 32 channels the bypass and dWb products run as three
  // bf16 products of hi / lo split operands (float32 accumulation), K-steps of 32
  constexpr bool S3 = BF && (C % 32 == 0);
  constexpr int KS = S3 ? C / 32 : 1;
  // bypass B operand of channel tile ct, K-step kb, lane (n = m, q): Wb[o = 4 kb + q][i = 16 ct + m]
  float wbr[BLK && !S3 ? NT : 1][BLK && !S3 ? C / 4 : 1];
  // S3: K-step s, lane (n = m, q) holds Wb[o = 32 s + 8 q + e][i = 16 ct + m], e = 0..7, split
  bf16x8 wbh[BLK && S3 ? NT : 1][KS], wbl[BLK && S3 ? NT : 1][KS];
  if (BLK) {
    if constexpr (S3) {
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = a.wb[(32 * s + 8 * q + e) * C + 16 * ct + m];
          split_bf16x8(v, wbh[ct][s], wbl[ct][s]);
        }
    } else {
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        const int i = 16 * ct + m;
#pragma unroll
        for (int kb = 0; kb < C / 4; ++kb) {
          const float w = a.wb[(4 * kb + q) * C + min(i, C - 1)];
          wbr[ct][kb] = i < C ? w : 0.f;
        }
      }
    }
  }
  // dWb tiles of this wave: S3 with NT = 4: o-tiles 2 (w >> 1) + oo, i-tiles 2 (w & 1) + ii
  // (oo, ii < 2); otherwise as described above
  constexpr int OT = (S3 && NT == 4) ? 2 : 1;
  const int mo = S3 ? (NT == 4 ? 2 * (wave >> 1) : (wave >> 1))
                    : ((NT == 4) ? wave : (NT == 2 ? (wave >> 1) : 0));
  const int ni0 = S3 ? (NT == 4 ? 2 * (wave & 1) : (wave & 1)) : ((NT == 2) ? (wave & 1) : 0);
  const bool count_db = (!S3 && NT != 2) || ((wave & 1) == 0);
  f32x4 dwb[DT];
#pragma unroll
  for (int u = 0; u < DT; ++u) dwb[u] = zero4();
  f32x4 dw3[S3 ? OT : 1][S3 ? OT : 1];
#pragma unroll
  for (int oo = 0; oo < (S3 ? OT : 1); ++oo)
#pragma unroll
    for (int ii = 0; ii < (S3 ? OT : 1); ++ii) dw3[oo][ii] = zero4();
  float dbl = 0.f, dbl3[OT];
#pragma unroll
  for (int oo = 0; oo < OT; ++oo) dbl3[oo] = 0.f;
  // float4 e = tid + 256 u of a tile: channel e / FPC, points 4 (e % FPC) .. + 3 (tails as in
  // the forward: clamped copies, padding rows)
  const int64_t pbase = l0 * a.Nb;
  int64_t goff[NPT];
  int xl[NPT], ol[NPT];
#pragma unroll
  for (int u = 0; u < NPT; ++u) {
    const int e = tid + 256 * u, ec = min(e, NF4 - 1);
    goff[u] = ((int64_t)b * C + ec / FPC) * a.P + pbase + 4 * (ec % FPC);
    xl[u] = (e / FPC) * XSG + 4 * (e % FPC);
    ol[u] = (ec / FPC) * XSG + 4 * (ec % FPC);
  }
  bool bad = false;  // IEEE-half plans: a non-finite output was written
  float4 pg_y[NPT], pz[NPT], px[NPT];
#pragma unroll
  for (int u = 0; u < NPT; ++u) {
    pg_y[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    pz[u] = pg_y[u];
    px[u] = pg_y[u];
  }
  // table fragments: GPL == 0 reloads fragment 0 for every step; GPL = 1 or 2 (the steps of a
  // line) keeps the fragment of each step of a line in registers for the whole work-group
  GtFrag<G, H> gts[GPL > 0 ? GPL : 1];
#pragma unroll
  for (int u = 0; u < NPT; ++u) {
    if (BLK) pg_y[u] = load_stream4(a.gy + goff[u]);
    if (GL) pz[u] = load_stream4(a.zin + goff[u]);
    if (NX) px[u] = load_stream4(a.x + goff[u]);
  }
#pragma unroll
  for (int gg = 0; gg < (GPL > 0 ? GPL : 1); ++gg)
    load_gt<G, H, true, MT>(a, gg * PI, tbase, m, q, gts[gg]);
  constexpr bool LPF = C < 64;
  const int64_t Tb = ((int64_t)b * C * a.lines + l0) * a.mb;  // complex index of this range
  LineT<LPF ? C : 16, TH> tln;
  if constexpr (LPF) load_line<C, TH>(a, Tb, tln, tid);
  constexpr int kst = kMaxKpad + (BF ? 8 : 4);
  for (int lf = 0; lf < a.lpw; ++lf) {
    // every reader of the previous line's spectrum is past that line's last barrier
    if constexpr (LPF) {
      write_line<C, H, TH>(a, tln, s_tl, tid);
      load_line<C, TH>(a, Tb + (int64_t)min(lf + 1, a.lpw - 1) * a.mb, tln, tid);
    } else {
      stage_line<C, H, TH>(a, Tb + (int64_t)lf * a.mb, s_tl, tid);
    }
#pragma unroll(GPL > 0 ? GPL : 1)
    for (int g = 0; g < (GPL > 0 ? GPL : gpl); ++g) {
      const GtFrag<G, H>& gtf = gts[GPL > 0 ? g : 0];
      const int f = (lf << a.gpl_log2) + g;
      const int fn = min(f + 1, nf - 1);
#pragma unroll
      for (int u = 0; u < NPT; ++u) {
        if (BLK) {
          float4 gz = pg_y[u];
          if (GL) {
            gz.x *= gelu_grad_as(pz[u].x);
            gz.y *= gelu_grad_as(pz[u].y);
            gz.z *= gelu_grad_as(pz[u].z);
            gz.w *= gelu_grad_as(pz[u].w);
          }
          *reinterpret_cast<float4*>(s_gz + xl[u]) = gz;
        }
        if constexpr (IG) {
          float4 xin, gp;
          gelu_and_grad(px[u].x, xin.x, gp.x);
          gelu_and_grad(px[u].y, xin.y, gp.y);
          gelu_and_grad(px[u].z, xin.z, gp.z);
          gelu_and_grad(px[u].w, xin.w, gp.w);
          *reinterpret_cast<float4*>(s_x + xl[u]) = xin;
          *reinterpret_cast<float4*>(s_gp + xl[u]) = gp;
        } else if (NX) {
          *reinterpret_cast<float4*>(s_x + xl[u]) = px[u];
        }
      }
#pragma unroll
      for (int u = 0; u < NPT; ++u) {
        if (BLK) pg_y[u] = load_stream4(a.gy + goff[u] + PI * fn);
        if (GL) pz[u] = load_stream4(a.zin + goff[u] + PI * fn);
        if (NX) px[u] = load_stream4(a.x + goff[u] + PI * fn);
      }
      __syncthreads();  // g_z / x tiles and spectrum rows visible; previous grad tile consumed
      f32x4 acc[G][NT];
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) acc[j][ct] = zero4();
      if constexpr (BF) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          if (32 * s2 >= a.kpad) break;
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) {
            const V8 B = *reinterpret_cast<const V8*>(
                reinterpret_cast<const uint16_t*>(s_tl) + (16 * ct + m) * kst + 32 * s2 + 8 * q);
#pragma unroll
            for (int j = 0; j < G; ++j) acc[j][ct] = HalfOf<H>::mfma(gtf.v[j][s2], B, acc[j][ct]);
          }
        }
      } else {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          if (16 * g4 >= a.kpad) break;
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) {
            const float4 B4 = *reinterpret_cast<const float4*>(
                reinterpret_cast<const float*>(s_tl) + (16 * ct + m) * kst + 16 * g4 + 4 * q);
#pragma unroll
            for (int j = 0; j < G; ++j) {
              acc[j][ct] = mfma_f32(gtf.v[j][g4].x, B4.x, acc[j][ct]);
              acc[j][ct] = mfma_f32(gtf.v[j][g4].y, B4.y, acc[j][ct]);
              acc[j][ct] = mfma_f32(gtf.v[j][g4].z, B4.z, acc[j][ct]);
              acc[j][ct] = mfma_f32(gtf.v[j][g4].w, B4.w, acc[j][ct]);
            }
          }
        }
      }
      if constexpr (GPL == 0) load_gt<G, H, true, MT>(a, (fn & (gpl - 1)) * PI, tbase, m, q, gts[0]);
      if (TANH) {
        // lane (n = m, q), tile tbase + j, register r: channel 16 ct + m, point
        // lp(4 q + r) + j
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float xv[G];
            load_lds_run<G>(xv, s_x + (16 * ct + m) * XSG + lp(4 * q + r));
#pragma unroll
            for (int j = 0; j < G; ++j) {
              const float t = tanh_fast(xv[j]);
              acc[j][ct][r] *= 1.f - t * t;
            }
          }
      }
      if (BLK) {
        if constexpr (S3) {
          // A: lane (m, q) holds g_z[o = 32 s + 8 q + e][point MT m + tbase + j], split
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            float gv[8][G];
#pragma unroll
            for (int e = 0; e < 8; ++e)
              load_lds_run<G>(gv[e], s_gz + (32 * s + 8 * q + e) * XSG + lp(m));
#pragma unroll
            for (int j = 0; j < G; ++j) {
              float v[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] = gv[e][j];
              bf16x8 ah, al;
              split_bf16x8(v, ah, al);
#pragma unroll
              for (int ct = 0; ct < NT; ++ct)
                acc[j][ct] = mfma_split3(ah, al, wbh[ct][s], wbl[ct][s], acc[j][ct]);
            }
          }
        } else {
#pragma unroll
          for (int kb = 0; kb < C / 4; ++kb) {
            float av[G];
            load_lds_run<G>(av, s_gz + (4 * kb + q) * XSG + lp(m));
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
              for (int j = 0; j < G; ++j) acc[j][ct] = mfma_f32(av[j], wbr[ct][kb], acc[j][ct]);
          }
        }
      }
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v[G];
#pragma unroll
          for (int j = 0; j < G; ++j) v[j] = acc[j][ct][r];
          store_lds_run<G>(s_o + (16 * ct + m) * XSG + lp(4 * q + r), v);
        }
      if (BLK && S3) {
        // dWb[o][i] += sum_points g_z[o][p] x[i][p] over 32-point chunks h: A lane (m, q) holds
        // g_z[16 mo' + m][32 h + 8 q + e], B lane (m, q) holds x[16 ni' + m][32 h + 8 q + e]
#pragma unroll
        for (int h = 0; h < PI / 32; ++h) {
          bf16x8 gh[OT], gl[OT];
#pragma unroll
          for (int oo = 0; oo < OT; ++oo) {
            const float* r = s_gz + (16 * (mo + oo) + m) * XSG + 32 * h + 8 * q;
            const float4 a0 = *reinterpret_cast<const float4*>(r);
            const float4 a1 = *reinterpret_cast<const float4*>(r + 4);
            if (count_db) dbl3[oo] += ((a0.x + a0.y) + (a0.z + a0.w)) + ((a1.x + a1.y) + (a1.z + a1.w));
            const float v[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            split_bf16x8(v, gh[oo], gl[oo]);
          }
#pragma unroll
          for (int ii = 0; ii < OT; ++ii) {
            const float* r = s_x + (16 * (ni0 + ii) + m) * XSG + 32 * h + 8 * q;
            const float4 b0 = *reinterpret_cast<const float4*>(r);
            const float4 b1 = *reinterpret_cast<const float4*>(r + 4);
            const float v[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
            bf16x8 xh, xl8;
            split_bf16x8(v, xh, xl8);
#pragma unroll
            for (int oo = 0; oo < OT; ++oo)
              dw3[oo][ii] = mfma_split3(gh[oo], gl[oo], xh, xl8, dw3[oo][ii]);
          }
        }
      } else if (BLK) {
        // dWb[o][i] += sum_points g_z[o][p] x[i][p]; k-slot q of MFMA jj <-> point 16 h + 4 q + jj
        constexpr int NH = PI / 16;  // 16-point chunks of the step
        const int h_lo = (NT == 1) ? wave * (NH / 4) : 0;
        const int h_hi = (NT == 1) ? (wave + 1) * (NH / 4) : NH;
        for (int h = h_lo; h < h_hi; ++h) {
          const float4 av = *reinterpret_cast<const float4*>(s_gz + (16 * mo + m) * XSG + 16 * h + 4 * q);
          if (count_db) dbl += (av.x + av.y) + (av.z + av.w);
#pragma unroll
          for (int u = 0; u < DT; ++u) {
            const int ni = (NT == 4) ? u : ni0;
            const float4 bv = *reinterpret_cast<const float4*>(s_x + (16 * ni + m) * XSG + 16 * h + 4 * q);
            dwb[u] = mfma_f32(av.x, bv.x, dwb[u]);
            dwb[u] = mfma_f32(av.y, bv.y, dwb[u]);
            dwb[u] = mfma_f32(av.z, bv.z, dwb[u]);
            dwb[u] = mfma_f32(av.w, bv.w, dwb[u]);
          }
        }
      }
      __syncthreads();  // grad tile complete; g_z / x tiles free
#pragma unroll
      for (int u = 0; u < NPT; ++u) {
        float4 v = *reinterpret_cast<const float4*>(s_o + ol[u]);
        if constexpr (IG) {
          const float4 gp = *reinterpret_cast<const float4*>(s_gp + ol[u]);
          v.x *= gp.x;
          v.y *= gp.y;
          v.z *= gp.z;
          v.w *= gp.w;
        }
        if constexpr (H == 2) bad |= !finite4(v);
        *reinterpret_cast<float4*>(a.y + goff[u] + PI * f) = v;
      }
    }
  }
  if constexpr (H == 2) raise_half_flag(a.flag, bad);
  if (!BLK || !a.part) return;
  // Deterministic work-group reduction (fixed wave order) into LDS, then one partial row.
  float* s_red = s_gz;  // [C][CP] dWb
  float* s_db = s_x;    // [4 waves][4 q][CP] dbias partials
  __syncthreads();
  for (int e = tid; e < C * CP; e += 256) s_red[e] = 0.f;
  for (int e = tid; e < 16 * CP; e += 256) s_db[e] = 0.f;
  __syncthreads();
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
      if constexpr (S3) {
#pragma unroll
        for (int oo = 0; oo < OT; ++oo) {
#pragma unroll
          for (int ii = 0; ii < OT; ++ii)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              s_red[(16 * (mo + oo) + 4 * q + r) * CP + 16 * (ni0 + ii) + m] += dw3[oo][ii][r];
          s_db[(w * 4 + q) * CP + 16 * (mo + oo) + m] += dbl3[oo];
        }
      } else {
#pragma unroll
        for (int u = 0; u < DT; ++u) {
          const int ni = (NT == 4) ? u : ni0;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int o = 16 * mo + 4 * q + r, ii = 16 * ni + m;
            if (o < C) s_red[o * CP + ii] += dwb[u][r];
          }
        }
        s_db[(w * 4 + q) * CP + 16 * mo + m] += dbl;
      }
    }
    __syncthreads();
  }
  float* dst = a.part + (int64_t)blockIdx.x * (C * C + C);
  for (int e = tid; e < C * C + C; e += 256) {
    float v;
    if (e < C * C) {
      const int o = e / C, ii = e - o * C;
      v = s_red[o * CP + ii];
    } else {
      const int o = e - C * C;
      v = 0.f;
      for (int k = 0; k < 16; ++k) v += s_db[k * CP + o];
    }
    dst[e] = v;
  }
}

// ------------------------------------------------------------------------------------------
// th: T arrives in the half format (width 64 with half operands only)
template <int C, int G>
static hipError_t launch_fwd_c(const EpiArgs& a, int half, int mode, int wgs, hipStream_t s,
                               bool th = false) {
  if constexpr (C == 64 && G == 1) {
    if (th && half != 0) {
#define FNO_EPI_FWD(HV, MV) \
  hipLaunchKernelGGL((k_epi_fwd_line<C, HV, MV, G, true, 0>), dim3(wgs), dim3(256), 0, s, a)
#define FNO_EPI_FWD_M(HV)                   \
  do {                                      \
    if (mode == 0) FNO_EPI_FWD(HV, 0);        \
    else if (mode == 1) FNO_EPI_FWD(HV, 1);   \
    else if (mode == 2) FNO_EPI_FWD(HV, 2);   \
    else if (mode == 9) FNO_EPI_FWD(HV, 9);   \
    else if (mode == 10) FNO_EPI_FWD(HV, 10); \
    else if (mode == 17) FNO_EPI_FWD(HV, 17); \
    else FNO_EPI_FWD(HV, 25);                 \
  } while (0)
      if (half == 2) FNO_EPI_FWD_M(2);
      else FNO_EPI_FWD_M(1);
#undef FNO_EPI_FWD_M
#undef FNO_EPI_FWD
      return hipGetLastError();
    }
  }
  if (th) return hipErrorInvalidValue;
#define FNO_EPI_FWD(HV, MV, GP) \
  hipLaunchKernelGGL((k_epi_fwd_line<C, HV, MV, G, false, GP>), dim3(wgs), dim3(256), 0, s, a)
#define FNO_EPI_FWD_M(HV, GP)                   \
  do {                                          \
    if (mode == 0) FNO_EPI_FWD(HV, 0, GP);        \
    else if (mode == 1) FNO_EPI_FWD(HV, 1, GP);   \
    else if (mode == 2) FNO_EPI_FWD(HV, 2, GP);   \
    else if (mode == 9) FNO_EPI_FWD(HV, 9, GP);   \
    else if (mode == 10) FNO_EPI_FWD(HV, 10, GP); \
    else if (mode == 17) FNO_EPI_FWD(HV, 17, GP); \
    else FNO_EPI_FWD(HV, 25, GP);                 \
  } while (0)
  // float32 plans keep the table fragments of lines of one or two steps in registers
  const int gpl = 1 << a.gpl_log2;
  if (half == 2) FNO_EPI_FWD_M(2, 0);
  else if (half == 1) FNO_EPI_FWD_M(1, 0);
  else if (gpl == 1) FNO_EPI_FWD_M(0, 1);
  else if (gpl == 2) FNO_EPI_FWD_M(0, 2);
  else FNO_EPI_FWD_M(0, 0);
#undef FNO_EPI_FWD_M
#undef FNO_EPI_FWD
  return hipGetLastError();
}

template <int C, int G>
static hipError_t launch_bwd_c(const EpiArgs& a, int half, bool tanh_pre, int mode, int wgs,
                               hipStream_t s, bool th = false) {
  if constexpr (C == 64 && G == 1) {
    if (th && half != 0) {
#define FNO_EPI_BWD(BFV, TV, MV) \
  hipLaunchKernelGGL((k_epi_bwd_line<C, BFV, TV, MV, G, true, 0>), dim3(wgs), dim3(256), 0, s, a)
#define FNO_EPI_BWD_M(BFV, TV)                   \
  do {                                           \
    if (mode == 1) FNO_EPI_BWD(BFV, TV, 1);        \
    else if (mode == 3) FNO_EPI_BWD(BFV, TV, 3);   \
    else if (mode == 7) FNO_EPI_BWD(BFV, TV, 7);   \
    else if (mode == 9) FNO_EPI_BWD(BFV, TV, 9);   \
    else if (mode == 11) FNO_EPI_BWD(BFV, TV, 11); \
    else FNO_EPI_BWD(BFV, TV, 15);                 \
  } while (0)
      if (half == 2) {
        if (tanh_pre) FNO_EPI_BWD_M(2, true);
        else FNO_EPI_BWD_M(2, false);
      } else {
        if (tanh_pre) FNO_EPI_BWD_M(1, true);
        else FNO_EPI_BWD_M(1, false);
      }
#undef FNO_EPI_BWD_M
#undef FNO_EPI_BWD
      return hipGetLastError();
    }
  }
  if (th) return hipErrorInvalidValue;
#define FNO_EPI_BWD(BFV, TV, MV, GP) \
  hipLaunchKernelGGL((k_epi_bwd_line<C, BFV, TV, MV, G, false, GP>), dim3(wgs), dim3(256), 0, s, a)
#define FNO_EPI_BWD_M(BFV, TV, GP)                  \
  do {                                              \
    if (mode == 1) FNO_EPI_BWD(BFV, TV, 1, GP);       \
    else if (mode == 3) FNO_EPI_BWD(BFV, TV, 3, GP);  \
    else if (mode == 7) FNO_EPI_BWD(BFV, TV, 7, GP);  \
    else if (mode == 9) FNO_EPI_BWD(BFV, TV, 9, GP);  \
    else if (mode == 11) FNO_EPI_BWD(BFV, TV, 11, GP); \
    else FNO_EPI_BWD(BFV, TV, 15, GP);                \
  } while (0)
  // float32 plans keep the table fragments of lines of one or two steps in registers
  const int gpl = 1 << a.gpl_log2;
  if (half == 2) {
    if (tanh_pre) FNO_EPI_BWD_M(2, true, 0);
    else FNO_EPI_BWD_M(2, false, 0);
  } else if (half == 1) {
    if (tanh_pre) FNO_EPI_BWD_M(1, true, 0);
    else FNO_EPI_BWD_M(1, false, 0);
  } else if (gpl == 1) {
    if (tanh_pre) FNO_EPI_BWD_M(0, true, 1);
    else FNO_EPI_BWD_M(0, false, 1);
  } else if (gpl == 2) {
    if (tanh_pre) FNO_EPI_BWD_M(0, true, 2);
    else FNO_EPI_BWD_M(0, false, 2);
  } else {
    if (tanh_pre) FNO_EPI_BWD_M(0, true, 0);
    else FNO_EPI_BWD_M(0, false, 0);
  }
#undef FNO_EPI_BWD_M
#undef FNO_EPI_BWD
  return hipGetLastError();
}

bool epilogue_fast_ok(const fno_plan* p, int mode, bool fwd) {
  const Geom& g = p->g;
  const int C = fwd ? g.Cout : g.Cin;
  if (mode != EPI_SPECTRAL && g.Cin != g.Cout) return false;
  if (!(C == 16 || C == 20 || C == 32 || C == 64)) return false;
  if (g.Nb % 64 != 0 || g.mb % 2 != 0 || p->kpad > kMaxKpad) return false;
  const int gpl = g.Nb / 64;  // point groups per line: a power of two (shift / mask indexing)
  if ((gpl & (gpl - 1)) != 0) return false;
  return true;
}

// Lines per work-group: the largest power of two dividing the lines of a batch entry that still
// leaves at least min_wgs work-groups.  Measured: fields of up to 20 channels (little work per
// line) keep 2048 work-groups in both directions; wider ones do best with 1024 (forward at 32
// and 64 channels: 78 -> 75 and 230 -> 217 us per launch against 2048; backward at 64: 333
// against 350 us with 2048, whose partials also double the gradient finish).
static int64_t epi_min_wgs(int channels) { return channels <= 20 ? 2048 : 1024; }

static int lines_per_wg(int64_t lines, int64_t batch, int64_t min_wgs) {
  int lpw = 1;
  while (lines % (2 * lpw) == 0 && batch * lines / (2 * lpw) >= min_wgs) lpw *= 2;
  return lpw;
}

static int fwd_lines_per_wg(int64_t lines, int64_t batch, int channels) {
  return lines_per_wg(lines, batch, epi_min_wgs(channels));
}

// Arguments of the forward line kernel; kmode bits as the kernel's MODE (without its width).
static EpiArgs fwd_args(const fno_plan* p, int* G, int64_t* wgs) {
  const Geom& g = p->g;
  EpiArgs a{};
  a.B = g.B;
  a.C = g.Cout;
  a.P = g.P;
  a.Nb = g.Nb;
  a.mb = g.mb;
  a.kpad = p->kpad;
  a.lines = g.P / g.Nb;
  a.lpw = fwd_lines_per_wg(a.lines, g.B, g.Cout);
  // fields of up to 20 channels take two 64-point groups per step when a line holds them (at
  // 32 channels one group per step keeps more waves resident and is faster)
  *G = (g.Cout <= 20 && g.Nb >= 2 * PG) ? 2 : 1;
  int gl = 0;
  while ((PG * *G << gl) < g.Nb) ++gl;
  a.gpl_log2 = gl;
  a.gt = g.bf16 ? (const void*)p->t.gt_fwd_bf : (const void*)p->t.gt_fwd;
  a.flag = g.half_flag;
  *wgs = (int64_t)g.B * a.lines / a.lpw;
  return a;
}

static hipError_t launch_fwd_any(const fno_plan* p, const EpiArgs& a, int G, int kmode,
                                 int64_t wgs, hipStream_t s, bool th = false) {
  const Geom& g = p->g;
  if (wgs > 0x7fffffff) return hipErrorInvalidValue;
  if (G == 2) {
    switch (g.Cout) {
      case 16: if (th) return hipErrorInvalidValue;
             return launch_fwd_c<16, 2>(a, g.half, kmode, (int)wgs, s);
      case 20: return launch_fwd_c<20, 2>(a, g.half, kmode, (int)wgs, s);
      default: return launch_fwd_c<32, 2>(a, g.half, kmode, (int)wgs, s);
    }
  }
  switch (g.Cout) {
    case 16: if (th) return hipErrorInvalidValue;
             return launch_fwd_c<16, 1>(a, g.half, kmode, (int)wgs, s);
    case 20: return launch_fwd_c<20, 1>(a, g.half, kmode, (int)wgs, s);
    case 32: return launch_fwd_c<32, 1>(a, g.half, kmode, (int)wgs, s);
    default: return launch_fwd_c<64, 1>(a, g.half, kmode, (int)wgs, s, th);
  }
}

int epilogue_fwd_fast_groups(const fno_plan* p) {
  if (!epilogue_fast_ok(p, EPI_BLOCK, true)) return 0;
  int G = 1;
  int64_t wgs = 0;
  (void)fwd_args(p, &G, &wgs);
  return wgs > 0x7fffffff ? 0 : (int)wgs;
}

hipError_t launch_epilogue_fwd_fast(const fno_plan* p, int mode, const void* T, const float* x,
                                    const float* wb, const float* bias, float* y, float* zsave,
                                    hipStream_t s, bool t_half) {
  int G = 1;
  int64_t wgs = 0;
  EpiArgs a = fwd_args(p, &G, &wgs);
  a.x = x;
  a.T = T;
  a.wb = wb;
  a.bias = (p->desc.flags & FNO_FLAG_BIAS) ? bias : nullptr;
  a.y = y;
  a.z = zsave;
  a.gelu = mode == EPI_BLOCK && (p->desc.flags & FNO_FLAG_GELU) != 0;
  const bool ig = (p->desc.flags & FNO_FLAG_INPUT_GELU) != 0;
  const int kmode = mode == EPI_SPECTRAL ? 0 : ((zsave ? 2 : 1) | (ig ? 8 : 0));
  a.block = kmode != 0;
  return launch_fwd_any(p, a, G, kmode, wgs, s, t_half);
}

hipError_t launch_epilogue_fwd_mse(const fno_plan* p, const void* T, const float* x,
                                   const float* wb, const float* bias, const float* tgt,
                                   float msc, float* gz, double* lpart, hipStream_t s,
                                   bool t_half) {
  int G = 1;
  int64_t wgs = 0;
  EpiArgs a = fwd_args(p, &G, &wgs);
  a.x = x;
  a.T = T;
  a.wb = wb;
  a.bias = (p->desc.flags & FNO_FLAG_BIAS) ? bias : nullptr;
  a.y = gz;
  a.gy = tgt;
  a.msc = msc;
  a.lpart = lpart;
  a.gelu = (p->desc.flags & FNO_FLAG_GELU) != 0;
  const bool ig = (p->desc.flags & FNO_FLAG_INPUT_GELU) != 0;
  const int kmode = 1 | 16 | (ig ? 8 : 0);
  a.block = 1;
  return launch_fwd_any(p, a, G, kmode, wgs, s, t_half);
}

// Lines per backward work-group (each writes one row of bypass-gradient partials, so fewer
// work-groups also mean a shorter finish): as the forward's.
static int bwd_lines_per_wg(int64_t lines, int64_t batch, int channels) {
  return lines_per_wg(lines, batch, epi_min_wgs(channels));
}

int epilogue_bwd_fast_groups(const fno_plan* p) {
  if (!epilogue_fast_ok(p, EPI_BLOCK, false)) return 0;
  const int64_t lines = p->g.P / p->g.Nb;
  return (int)((int64_t)p->g.B * lines / bwd_lines_per_wg(lines, p->g.B, p->g.Cin));
}

hipError_t launch_epilogue_bwd_fast(const fno_plan* p, int mode, const void* Tg,
                                    const float* x, const float* wb, const float* gy,
                                    const float* z, float* grad_x, float* red_part,
                                    hipStream_t s, bool t_half) {
  const Geom& g = p->g;
  EpiArgs a{};
  a.B = g.B;
  a.C = g.Cin;
  a.P = g.P;
  a.Nb = g.Nb;
  a.mb = g.mb;
  a.kpad = p->kpad;
  a.lines = g.P / g.Nb;
  a.lpw = bwd_lines_per_wg(a.lines, g.B, g.Cin);
  // one 64-point group per step: with three input tiles in flight, larger steps cost more in
  // occupancy than they save in barriers (measured on the 128^3 width-20 backward)
  int gl = 0;
  while ((PG << gl) < g.Nb) ++gl;
  a.gpl_log2 = gl;
  a.x = x;
  a.T = Tg;
  a.wb = wb;
  a.gt = g.bf16 ? (const void*)p->t.gt_unit_bf : (const void*)p->t.gt_unit;
  a.y = grad_x;
  a.gy = gy;
  a.zin = z;
  a.part = red_part;
  a.flag = g.half_flag;
  a.block = mode == EPI_BLOCK;
  a.gelu = z != nullptr;
  const bool tanh_pre = (p->desc.flags & FNO_FLAG_TANH_PREACT) != 0;
  const int kmode = (mode != EPI_BLOCK ? 1 : (z ? 7 : 3)) |
                    ((p->desc.flags & FNO_FLAG_INPUT_GELU) ? 8 : 0);
  const int64_t wgs = (int64_t)g.B * a.lines / a.lpw;
  if (wgs > 0x7fffffff) return hipErrorInvalidValue;
  switch (g.Cin) {
    case 16: if (t_half) return hipErrorInvalidValue;
             return launch_bwd_c<16, 1>(a, g.half, tanh_pre, kmode, (int)wgs, s);
    case 20: if (t_half) return hipErrorInvalidValue;
             return launch_bwd_c<20, 1>(a, g.half, tanh_pre, kmode, (int)wgs, s);
    case 32: if (t_half) return hipErrorInvalidValue;
             return launch_bwd_c<32, 1>(a, g.half, tanh_pre, kmode, (int)wgs, s);
    default: return launch_bwd_c<64, 1>(a, g.half, tanh_pre, kmode, (int)wgs, s, t_half);
  }
}

}  // namespace fno
