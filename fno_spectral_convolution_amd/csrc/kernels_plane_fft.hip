// Forward plane transform with a fast Fourier transform along the contiguous axis (float32
// plans).
//
// It computes what the matrix-core plane transform computes -- the truncated real DFT of
// every row (bins k < m_b), then the truncated DFT of the next axis for the retained modes --
// but takes the row transform by an FFT instead of a dense product: the spectral convolution
// is defined on the FFT of the field (model-parallel FNO page, "Proposed method"), and the
// FFT needs O(log Nb) operations per value where the dense product needs 4 m_b.
//
// Row transform.  A row of Nb = 2M real values is read as M complex values
// z[n] = x[2n] + i x[2n+1] and transformed by a two-pass Stockham (self-sorting) FFT, with
// L = M / 16 lanes per row:
//   pass 1, radix 16, in registers: lane g loads z[g + L s] for s < 16 straight from HBM
//          (for each s the row's L lanes read L consecutive float2) and writes its 16-point
//          DFT to the row's LDS buffer at 16 g + t;
//   pass 2, radix L, through LDS: butterfly i < 16 reads y[i + 16 t] for t < L, multiplies
//          by e^{-2 pi i t i / M} and takes the L-point DFT, which is Z[i + 16 t] in natural
//          order.
// Only Z[k] and Z[M - k] of the kept bins are needed, and the real spectrum follows from the
// even/odd split of the packing:
//   X[k] = (Z[k] + conj Z[M-k]) / 2 - (i/2) e^{-2 pi i k / Nb} (Z[k] - conj Z[M-k]).
// X goes to LDS transposed, [re/im column][row], and every 64 rows it feeds the next-axis
// product on the matrix cores as in the dense kernel.  Twiddles come from the plan's float64-
// built root table of the axis, rounded once to float32.
#include "fno_internal.h"
#include "mfma.h"
#include "plane_common.h"
#include "pointwise.h"

#include <type_traits>

namespace fno {
namespace {

__device__ __forceinline__ float2 c_add(float2 a, float2 b) {
  return make_float2(a.x + b.x, a.y + b.y);
}
__device__ __forceinline__ float2 c_sub(float2 a, float2 b) {
  return make_float2(a.x - b.x, a.y - b.y);
}
__device__ __forceinline__ float2 c_mul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

// v * e^{-2 pi i e / 16}; e is a compile-time constant after unrolling, so the switch folds.
__device__ __forceinline__ float2 w16_mul(float2 v, int e) {
  constexpr float C1 = 0.92387953251128674f;  // cos(pi/8)
  constexpr float S1 = 0.38268343236508978f;  // sin(pi/8)
  constexpr float R = 0.70710678118654752f;   // sqrt(1/2)
  float c, s;
  switch (e & 15) {
    case 0: return v;
    case 4: return make_float2(v.y, -v.x);
    case 8: return make_float2(-v.x, -v.y);
    case 12: return make_float2(-v.y, v.x);
    case 2: return make_float2(R * (v.x + v.y), R * (v.y - v.x));
    case 6: return make_float2(R * (v.y - v.x), -R * (v.x + v.y));
    case 10: return make_float2(-R * (v.x + v.y), R * (v.x - v.y));
    case 14: return make_float2(R * (v.x - v.y), R * (v.x + v.y));
    case 1: c = C1; s = S1; break;
    case 3: c = S1; s = C1; break;
    case 5: c = -S1; s = C1; break;
    case 7: c = -C1; s = S1; break;
    case 9: c = -C1; s = -S1; break;
    case 11: c = -S1; s = -C1; break;
    case 13: c = S1; s = -C1; break;
    default: c = C1; s = -S1; break;  // 15
  }
  // (c - i s) v
  return make_float2(v.x * c + v.y * s, v.y * c - v.x * s);
}

// 4-point DFT, y_k = sum_n a_n e^{-2 pi i n k / 4}
__device__ __forceinline__ void dft4(float2 a0, float2 a1, float2 a2, float2 a3, float2& y0,
                                     float2& y1, float2& y2, float2& y3) {
  const float2 s02 = c_add(a0, a2), d02 = c_sub(a0, a2);
  const float2 s13 = c_add(a1, a3), d13 = c_sub(a1, a3);
  y0 = c_add(s02, s13);
  y2 = c_sub(s02, s13);
  y1 = make_float2(d02.x + d13.y, d02.y - d13.x);  // d02 - i d13
  y3 = make_float2(d02.x - d13.y, d02.y + d13.x);  // d02 + i d13
}

// R-point DFT in registers, natural order in and out (R = 4, 8, 16).  With n = n1 + P n2 and
// k = k1 + Q k2 (P Q = R, Q = 4): an inner 4-point DFT over n2, the twiddle e^{-2 pi i n1 k1/R},
// then a P-point DFT over n1.
template <int R>
__device__ __forceinline__ void dft(const float2 (&in)[R], float2 (&out)[R]) {
  if constexpr (R == 4) {
    dft4(in[0], in[1], in[2], in[3], out[0], out[1], out[2], out[3]);
  } else if constexpr (R == 8) {
    float2 A[2][4];
#pragma unroll
    for (int n1 = 0; n1 < 2; ++n1)
      dft4(in[n1], in[n1 + 2], in[n1 + 4], in[n1 + 6], A[n1][0], A[n1][1], A[n1][2], A[n1][3]);
#pragma unroll
    for (int k1 = 0; k1 < 4; ++k1) {
      const float2 b = w16_mul(A[1][k1], 2 * k1);
      out[k1] = c_add(A[0][k1], b);
      out[k1 + 4] = c_sub(A[0][k1], b);
    }
  } else {
    static_assert(R == 16, "radix 4, 8 or 16");
    float2 A[4][4];
#pragma unroll
    for (int n1 = 0; n1 < 4; ++n1) {
      dft4(in[n1], in[n1 + 4], in[n1 + 8], in[n1 + 12], A[n1][0], A[n1][1], A[n1][2],
           A[n1][3]);
#pragma unroll
      for (int k1 = 1; k1 < 4; ++k1) A[n1][k1] = w16_mul(A[n1][k1], n1 * k1);
    }
#pragma unroll
    for (int k1 = 0; k1 < 4; ++k1)
      dft4(A[0][k1], A[1][k1], A[2][k1], A[3][k1], out[k1], out[k1 + 4], out[k1 + 8],
           out[k1 + 12]);
  }
}

// NB = Nb in {128, 256, 512}; NTJ = jpad / 16 column tiles of the row spectra.
template <int PIN, int NB, int NTJ>
__global__ void __launch_bounds__(256) k_plane_fft(PlaneArgs a, const float2* __restrict__ root) {
  constexpr int M = NB / 2;                  // complex points per row
  constexpr int L = M / 16;                  // lanes per row = radix of pass 2
  constexpr int U2 = 16 / L;                 // pass-2 butterflies per lane
  constexpr int RPW = 64 / L;                // rows per wave and pass
  constexpr int RPP = 4 * RPW;               // rows per pass
  constexpr int PASSES = 64 / RPP;           // passes per 64-row block
  constexpr int JP = 16 * NTJ;
  constexpr int JP2 = JP / 2;                // bins held per row (k < m_b, the rest zero)
  constexpr int TN = JP2 > 16 ? 4 : 2;       // pass-2 outputs kept per butterfly
  constexpr int KPL = (JP2 + L - 1) / L;     // bins per lane in the half-spectrum step
  // row buffer stride (complex): 18 per lane (16 values, 16-byte aligned) plus a pad that
  // puts consecutive rows 2L dwords apart in the banks, so a half-wave's pass-2 reads over
  // its rows hit distinct banks
  constexpr int RST = 18 * L + ((64 - (34 * L) % 64) % 64) / 2;
  constexpr int RS = 64 + 4;                 // row stride of the transposed spectra (floats)
  constexpr int FFT_BYTES = 4 * RPW * RST * 8;
  constexpr int LOOP_BYTES = FFT_BYTES + JP * RS * 4;
  constexpr int END_BYTES = 4 * kPlaneMaxModes * JP * 4;
  static_assert(L >= 4 && L <= 16 && M == 16 * L, "rows of 128, 256 or 512 points");
  static_assert(PASSES * RPP == 64, "passes must tile 64 rows");
  __shared__ __attribute__((aligned(16)))
  unsigned char s_raw[LOOP_BYTES > END_BYTES ? LOOP_BYTES : END_BYTES];
  float2* s_fft = reinterpret_cast<float2*>(s_raw);
  float* s_rt = reinterpret_cast<float*>(s_raw + FFT_BYTES);
  float* s_x2 = reinterpret_cast<float*>(s_raw);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gi = lane % L, rw = lane / L;  // lane within the row, row within the wave
  const int m = lane & 15, q = lane >> 4;  // matrix-core lane coordinates
  const int IT = a.ma / 4;
  const int64_t plane = blockIdx.x;
  const int chunk = blockIdx.y;
  const int r_begin = chunk * a.rows_per_chunk;
  const int r_end = min(a.Na, r_begin + a.rows_per_chunk);
  float2* row_buf = s_fft + (wave * RPW + rw) * RST;

  // pass-2 twiddles e^{-2 pi i t i2 / M} of this lane's butterflies i2 = gi + L u
  float2 tw[U2][L];
#pragma unroll
  for (int u = 0; u < U2; ++u) {
    tw[u][0] = make_float2(1.f, 0.f);
#pragma unroll
    for (int t = 1; t < L; ++t) {
      const float2 r = root[(2 * t * (gi + L * u)) % NB];  // (cos, sin)(2 pi e / Nb)
      tw[u][t] = make_float2(r.x, -r.y);
    }
  }
  // (cos, sin)(2 pi k / Nb) of this lane's bins k = gi + L v
  float2 hw[KPL];
#pragma unroll
  for (int v = 0; v < KPL; ++v) hw[v] = root[(gi + L * v) % NB];

  f32x4 x2[2][NTJ];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < NTJ; ++v) x2[u][v] = zero4();

  const float2* base0 = reinterpret_cast<const float2*>(a.in0 + plane * (int64_t)a.Na * NB);
  const float2* base1 = (PIN == PLANE_GELU_GRAD)
                            ? reinterpret_cast<const float2*>(a.in1 + plane * (int64_t)a.Na * NB)
                            : nullptr;
  const float* f2 = static_cast<const float*>(a.f2);
  const int nblk = (r_end - r_begin + 63) / 64;  // 64-row blocks of the chunk
  // row of this lane in global pass pi (PASSES passes per 64-row block)
  auto pass_row = [&](int pi) {
    return r_begin + 64 * (pi / PASSES) + (pi % PASSES) * RPP + wave * RPW + rw;
  };
  // rows past the chunk load its last row again (an L2 hit) and their spectra are written as
  // zeros: a branch around the loads would make the compiler wait for every load in flight
  auto load_to = [&](float2 (&d0)[16], float2 (&d1)[16], int pi) {
    const int64_t off = (int64_t)min(pass_row(pi), r_end - 1) * M + gi;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      d0[s] = load_stream2(base0 + off + L * s);
      if (PIN == PLANE_GELU_GRAD) d1[s] = load_stream2(base1 + off + L * s);
    }
  };
  // F2 fragments of a 64-row block (kg, u): rows 16 it + m, columns r0 + 16 kg + 4 q + jj;
  // columns past the chunk are clamped into the table and masked to zero
  float4 fa[4][2];
  auto load_f2 = [&](int r0) {
#pragma unroll
    for (int kg = 0; kg < 4; ++kg)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int it = min(wave + 4 * u, IT - 1);
        const int row0 = r0 + 16 * kg + 4 * q;
        const int64_t fo = (int64_t)(16 * it + m) * a.Na + min(row0, a.Na - 4);
        const float4 v = *reinterpret_cast<const float4*>(f2 + fo);
        auto keep = [&](float x, int j) {
          return __uint_as_float(__float_as_uint(x) & (row0 + j < r_end ? 0xffffffffu : 0u));
        };
        fa[kg][u] = make_float4(keep(v.x, 0), keep(v.y, 1), keep(v.z, 2), keep(v.w, 3));
      }
  };
  // one pass over RPP rows from the register set (d0, d1): the prologue, the next loads of
  // the set (dist passes ahead; with the block's F2 fragments first when F2LOAD), the FFT
  // and the half spectrum into s_rt
  auto pass = [&](float2 (&d0)[16], float2 (&d1)[16], int pi, int dist, auto f2_tag) {
    float2 v[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const float2 w = (PIN == PLANE_GELU_GRAD) ? d1[s] : make_float2(0.f, 0.f);
      v[s] = make_float2(prologue<PIN>(d0[s].x, w.x), prologue<PIN>(d0[s].y, w.y));
    }
    const bool ok = pass_row(pi) < r_end;
    if constexpr (decltype(f2_tag)::value) load_f2(r_begin + 64 * (pi / PASSES));
    load_to(d0, d1, pi + dist);

    // pass 1: radix 16 in registers, output at 16 gi + t (padded index 18 gi + t)
    float2 y[16];
    dft<16>(v, y);
#pragma unroll
    for (int t = 0; t < 16; t += 2)
      *reinterpret_cast<float4*>(row_buf + 18 * gi + t) =
          make_float4(y[t].x, y[t].y, y[t + 1].x, y[t + 1].y);
    // a row's lanes are one wave's: LDS operations of a wave complete in order, so a
    // scheduling barrier is all that the exchange needs
    __builtin_amdgcn_wave_barrier();

    // pass 2: radix L; keep Z[i2 + 16 t] for t in {0, 1, L-2, L-1} (TN = 4) or {0, L-1}
    float2 zs[U2][TN];
#pragma unroll
    for (int u = 0; u < U2; ++u) {
      const int i2 = gi + L * u;
      float2 w[L], Z[L];
#pragma unroll
      for (int t = 0; t < L; ++t) {
        const float2 e = row_buf[i2 + 18 * t];
        w[t] = t == 0 ? e : c_mul(e, tw[u][t]);
      }
      dft<L>(w, Z);
#pragma unroll
      for (int sl = 0; sl < TN; ++sl) zs[u][sl] = Z[sl < TN / 2 ? sl : L - TN + sl];
    }
    __builtin_amdgcn_wave_barrier();
    // kept outputs, slot sl at 16 sl + i2: Z[k] for k < 16 TN / 2 sits at index k
#pragma unroll
    for (int u = 0; u < U2; ++u)
#pragma unroll
      for (int sl = 0; sl < TN; ++sl) row_buf[16 * sl + gi + L * u] = zs[u][sl];
    __builtin_amdgcn_wave_barrier();

    // half spectrum of the real row, written transposed for the next-axis product
    const int rin = (pi % PASSES) * RPP + wave * RPW + rw;
#pragma unroll
    for (int vv = 0; vv < KPL; ++vv) {
      const int k = gi + L * vv;
      if (k < JP2) {
        float re = 0.f, im = 0.f;
        if (k < a.mb) {
          const float2 zk = row_buf[k];
          // Z[M - k]: slot TN-1 holds Z[M-16 .. M-1], slot TN-2 (TN = 4) Z[M-32 .. M-17]
          const int km = k == 0 ? 0 : (k <= 16 ? 16 * (TN - 1) + 16 - k : 16 * (TN - 2) + 32 - k);
          const float2 zm = row_buf[km];
          const float sr = zk.x + zm.x, si = zk.y - zm.y;  // Z[k] + conj Z[M-k]
          const float dr = zk.x - zm.x, di = zk.y + zm.y;  // Z[k] - conj Z[M-k]
          const float c = hw[vv].x, sn = hw[vv].y;
          re = ok ? 0.5f * (sr + c * di - sn * dr) : 0.f;
          im = ok ? 0.5f * (si - c * dr - sn * di) : 0.f;
        }
        s_rt[(2 * k) * RS + rin] = re;
        s_rt[(2 * k + 1) * RS + rin] = im;
      }
    }
  };
  // next-axis product of a 64-row block: K-groups of 16 rows; MFMA jj uses row 16 kg + 4 q + jj
  auto second = [&]() {
    __syncthreads();
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      float4 bv[NTJ];
#pragma unroll
      for (int v = 0; v < NTJ; ++v)
        bv[v] = *reinterpret_cast<const float4*>(s_rt + (16 * v + m) * RS + 16 * kg + 4 * q);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (wave + 4 * u >= IT) break;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int v = 0; v < NTJ; ++v)
            x2[u][v] = mfma_f32(cmp4(fa[kg][u], jj), cmp4(bv[v], jj), x2[u][v]);
      }
    }
    __syncthreads();
  };

  constexpr std::integral_constant<bool, true> kF2{};
  constexpr std::integral_constant<bool, false> kNoF2{};
  float2 pa0[16], pa1[16];
  // (the gradient prologue reads two fields: two register sets of both would not fit)
  if constexpr (PASSES >= 2 && PIN != PLANE_GELU_GRAD) {
    // two register sets alternate over the passes, each reloaded two passes ahead, so one
    // pass of rows is always in flight while another is transformed; a block's F2 fragments
    // are loaded in its last pass ahead of that pass's row loads, so waiting for them does
    // not wait for the rows
    float2 pb0[16], pb1[16];
    load_to(pa0, pa1, 0);
    load_to(pb0, pb1, 1);
    for (int blk = 0; blk < nblk; ++blk) {
      const int p0 = blk * PASSES;
#pragma unroll
      for (int ps = 0; ps + 2 < PASSES; ps += 2) {
        pass(pa0, pa1, p0 + ps, 2, kNoF2);
        pass(pb0, pb1, p0 + ps + 1, 2, kNoF2);
      }
      pass(pa0, pa1, p0 + PASSES - 2, 2, kNoF2);
      pass(pb0, pb1, p0 + PASSES - 1, 2, kF2);
      second();
    }
  } else {
    load_to(pa0, pa1, 0);
    for (int blk = 0; blk < nblk; ++blk) {
#pragma unroll
      for (int ps = 0; ps + 1 < PASSES; ++ps) pass(pa0, pa1, blk * PASSES + ps, 1, kNoF2);
      pass(pa0, pa1, blk * PASSES + PASSES - 1, 1, kF2);
      second();
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int it = wave + 4 * u;
    if (it >= IT) break;
#pragma unroll
    for (int v = 0; v < NTJ; ++v)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_x2[(16 * it + 4 * q + r) * JP + 16 * v + m] = x2[u][v][r];
  }
  __syncthreads();
  combine_store(s_x2, JP, a.ma, a.mb,
                a.out + ((int64_t)chunk * a.planes + plane) * (2 * a.ma * a.mb), tid);
}

template <int PIN, int NB>
void launch_fft_nb(const fno_plan* p, const PlaneArgs& a, const float2* root, dim3 grid,
                   hipStream_t s) {
  switch (p->jpad) {
    case 16: hipLaunchKernelGGL((k_plane_fft<PIN, NB, 1>), grid, dim3(256), 0, s, a, root); break;
    case 32: hipLaunchKernelGGL((k_plane_fft<PIN, NB, 2>), grid, dim3(256), 0, s, a, root); break;
    default: hipLaunchKernelGGL((k_plane_fft<PIN, NB, 4>), grid, dim3(256), 0, s, a, root); break;
  }
}

template <int PIN>
void launch_fft_pin(const fno_plan* p, const PlaneArgs& a, const float2* root, dim3 grid,
                    hipStream_t s) {
  switch (p->g.Nb) {
    case 128: launch_fft_nb<PIN, 128>(p, a, root, grid, s); break;
    case 256: launch_fft_nb<PIN, 256>(p, a, root, grid, s); break;
    default: launch_fft_nb<PIN, 512>(p, a, root, grid, s); break;
  }
}

}  // namespace

bool plane_fft_ok(const fno_plan* p) {
  const Geom& g = p->g;
  if (g.bf16) return false;  // the half paths keep the dense products at the half rate
  if (!(g.Nb == 128 || g.Nb == 256 || g.Nb == 512)) return false;
  if (!(p->jpad == 16 || p->jpad == 32 || p->jpad == 64)) return false;
  if (g.ma % 4 != 0 || g.ma > kPlaneMaxModes) return false;  // F2: <= 2 tiles of 16 rows/wave
  // vector loads of F2 rows need 8-aligned row offsets
  if (g.Na % 8 != 0 || (p->plane_rows % 64 != 0 && p->plane_rows != g.Na)) return false;
  return true;
}

// Measured on float32 plans (per launch, same inputs): rows of 512 points with 32 bins,
// 135 us against 195 us for the dense product; rows of 256 with 16 bins, 34 us against 37 us;
// rows of 128 with 16 bins, 111 us against 101 us (there four lanes share a row and the
// loads of a wave spread over 16 rows in 32-byte pieces).
bool plane_fft_default(const fno_plan* p) { return p->g.Nb >= 256; }

hipError_t launch_plane_fft(const fno_plan* p, int plane_in, int chans, const float* in0,
                            const float* in1, float2* out, hipStream_t s) {
  const Geom& g = p->g;
  PlaneArgs a{};
  a.Na = g.Na;
  a.Nb = g.Nb;
  a.ma = g.ma;
  a.mb = g.mb;
  a.planes = (int64_t)g.B * chans * g.O;
  a.rows_per_chunk = p->plane_rows;
  a.in0 = in0;
  a.in1 = in1;
  a.f2 = p->t.f2;
  a.out = out;
  const float2* root = p->t.root[g.d - 1];
  dim3 grid((unsigned)a.planes, (unsigned)p->nch);
  switch (plane_in) {
    case PLANE_X: launch_fft_pin<PLANE_X>(p, a, root, grid, s); break;
    case PLANE_TANH: launch_fft_pin<PLANE_TANH>(p, a, root, grid, s); break;
    case PLANE_GELU: launch_fft_pin<PLANE_GELU>(p, a, root, grid, s); break;
    case PLANE_TANH_GELU: launch_fft_pin<PLANE_TANH_GELU>(p, a, root, grid, s); break;
    default: launch_fft_pin<PLANE_GELU_GRAD>(p, a, root, grid, s); break;
  }
  return hipGetLastError();
}

}  // namespace fno
