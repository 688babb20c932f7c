// Matrix-core forward transform of one [Na][Nb] plane (the last two axes of a field).
//
//   R[row][j]  = sum_c x'[row][c] T1[c][j]            (j < jpad = 16*NTJ; T1[c][2k] = cos,
//                                                     T1[c][2k+1] = -sin of 2 pi k c / Nb)
//   X2[i][j]  += sum_row F2[i][row] R[row][j]          (F2[i] = cos rows i < 2ma, sin rows
//                                                     i >= 2ma of 2 pi ka(i) row / Na)
//   X[s][k]    = (X2[s][2k] + X2[2ma+s][2k+1]) + i (X2[s][2k+1] - X2[2ma+s][2k])
// i.e. the truncated real DFT of the contiguous axis followed by the truncated DFT of the
// next axis, for the retained modes only (the FNO spectral transform computed from its
// linear-algebra form -- model-parallel FNO page, "Proposed method").
//
// One work-group (4 waves) handles a chunk of rows of one plane.  Rows are streamed with
// coalesced float4 loads (prefetched one sub-round ahead), pre-activated (tanh, GELU') and
// staged in LDS; wave w owns N-tile (w % NTJ) of R and keeps its slice of T1 in registers,
// so the table is never re-read.  R goes to LDS transposed and feeds the second product,
// whose M-tiles (rows of F2, read through L2) are split over the waves.  Each chunk writes
// its partial spectrum; chunks are summed by the next kernel in a fixed order.
#include "fno_internal.h"
#include "mfma.h"
#include "plane_common.h"
#include "pointwise.h"

#include <math.h>
#include <type_traits>

namespace fno {

// bf16 operands, fp32 accumulation.  NB = Nb (multiple of 32, <= 512), NTJ = jpad / 16.
template <int PIN, int NB, int NTJ, int H>
__global__ void __launch_bounds__(256) k_plane_bf16(PlaneArgs a) {
  using HT = Half<H>;  // the plan's half format (bfloat16 or IEEE half)
  using V8 = typename HT::v8;
  using E = typename HT::elem;
  constexpr int SUB = 16 * (4 / NTJ);   // rows per sub-round (one M-tile per wave)
  constexpr int XS = NB + 8;            // LDS row stride (bf16 elements)
  constexpr int RS = 64 + 8;            // Rt row stride (bf16 elements)
  constexpr int KS = NB / 32;           // K-steps of the first product
  constexpr int LPR = NB / 4;           // float4 per row
  constexpr int NLD = SUB * LPR / 256;  // float4 loads per thread per sub-round
  constexpr int JP = 16 * NTJ;
  static_assert(SUB * LPR % 256 == 0, "sub-round must split evenly");
  constexpr int LOOP_BYTES = SUB * XS * 2 + JP * RS * 2;
  constexpr int END_BYTES = 4 * kPlaneMaxModes * JP * 4;
  __shared__ __attribute__((aligned(16)))
  unsigned char s_raw[LOOP_BYTES > END_BYTES ? LOOP_BYTES : END_BYTES];
  uint16_t* s_x = reinterpret_cast<uint16_t*>(s_raw);
  uint16_t* s_rt = s_x + SUB * XS;
  float* s_x2 = reinterpret_cast<float*>(s_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  const int jt = wave % NTJ, mt = wave / NTJ;
  const int IT = a.ma / 4;  // 16-row tiles of F2 (4 ma rows)
  const int64_t plane = blockIdx.x;
  const int chunk = blockIdx.y;
  const int r_begin = chunk * a.rows_per_chunk;
  const int r_end = min(a.Na, r_begin + a.rows_per_chunk);

  // this wave's slice of T1: B[k][n] = T1[32 s + 8 q + e][16 jt + m]
  V8 tb[KS];
  {
    const uint16_t* t1 = static_cast<const uint16_t*>(a.t1);
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        tb[s][e] = __builtin_bit_cast(E, t1[(32 * s + 8 * q + e) * JP + 16 * jt + m]);
  }
  f32x4 x2[2][NTJ];  // i-tiles wave and wave + 4
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < NTJ; ++v) x2[u][v] = zero4();

  const float* base0 = a.in0 + plane * (int64_t)a.Na * NB;
  const float* base1 = (PIN == PLANE_GELU_GRAD) ? a.in1 + plane * (int64_t)a.Na * NB : nullptr;
  float4 pre0[NLD], pre1[NLD];
  // rows at or beyond r_end are zero (no memory access)
  auto load_sub = [&](int r0) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int e = tid + 256 * u;
      const int row = r0 + e / LPR, c4 = e % LPR;
      pre0[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      pre1[u] = pre0[u];
      if (row < r_end) {
        pre0[u] = load_stream4(base0 + (int64_t)row * NB + 4 * c4);
        if (PIN == PLANE_GELU_GRAD)
          pre1[u] = load_stream4(base1 + (int64_t)row * NB + 4 * c4);
      }
    }
  };
  auto stage_sub = [&]() {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int e = tid + 256 * u;
      const int r = e / LPR, c4 = e % LPR;
      const float4 v = pre0[u], w = pre1[u];
      uint2 packed;
      packed.x = HT::pack2(prologue<PIN>(v.x, w.x), prologue<PIN>(v.y, w.y));
      packed.y = HT::pack2(prologue<PIN>(v.z, w.z), prologue<PIN>(v.w, w.w));
      *reinterpret_cast<uint2*>(s_x + r * XS + 4 * c4) = packed;
    }
  };

  const uint16_t* f2 = static_cast<const uint16_t*>(a.f2);
  load_sub(r_begin);
  for (int r0 = r_begin; r0 < r_end; r0 += 64) {
    // 64 rows of R per stage, SUB rows per sub-round
    for (int sub = 0; sub < 64; sub += SUB) {
      __syncthreads();  // previous readers of s_x / s_rt are done
      stage_sub();
      load_sub(r0 + sub + SUB);  // prefetch the next sub-round
      __syncthreads();
      f32x4 d = zero4();
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const V8 av =
            *reinterpret_cast<const V8*>(s_x + (16 * mt + m) * XS + 32 * s + 8 * q);
        d = HT::mfma(av, tb[s], d);
      }
      // D rows 16 mt + 4 q + r, column 16 jt + m  ->  Rt[column][stage row]
      uint2 pk;
      pk.x = HT::pack2(d[0], d[1]);
      pk.y = HT::pack2(d[2], d[3]);
      *reinterpret_cast<uint2*>(s_rt + (16 * jt + m) * RS + sub + 16 * mt + 4 * q) = pk;
    }
    __syncthreads();
    // second product over these 64 rows, K-steps of 32 rows (slot e <-> row krow + e)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int krow = 32 * ks + 8 * q;
      V8 bv[NTJ];
#pragma unroll
      for (int v = 0; v < NTJ; ++v)
        bv[v] = *reinterpret_cast<const V8*>(s_rt + (16 * v + m) * RS + krow);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int it = wave + 4 * u;
        if (it >= IT) break;
        const int64_t fo = (int64_t)(16 * it + m) * a.Na + r0 + krow;
        V8 ah, al;
        if (r0 + krow + 8 <= r_end) {
          ah = *reinterpret_cast<const V8*>(f2 + fo);
          al = *reinterpret_cast<const V8*>(a.f2lo + fo);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const bool in = r0 + krow + e < r_end;
            ah[e] = __builtin_bit_cast(E, in ? f2[fo + e] : (uint16_t)0);
            al[e] = __builtin_bit_cast(E, in ? a.f2lo[fo + e] : (uint16_t)0);
          }
        }
#pragma unroll
        for (int v = 0; v < NTJ; ++v) {
          x2[u][v] = HT::mfma(ah, bv[v], x2[u][v]);
          x2[u][v] = HT::mfma(al, bv[v], x2[u][v]);
        }
      }
    }
  }
  __syncthreads();  // the loop buffers are reused for X2
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

// fp32 operands.  First product with 16x16x4 MFMAs: lane (m, q) reads xs[row][16 g + 4 q ..]
// and MFMA jj uses component jj (k-slot q <-> column 16 g + 4 q + jj).
template <int PIN, int NB, int NTJ>
__global__ void __launch_bounds__(256) k_plane_f32(PlaneArgs a) {
  constexpr int SUB = 16 * (4 / NTJ);
  constexpr int XS = NB + 4;
  constexpr int RS = 64 + 4;
  constexpr int KG = NB / 16;
  constexpr int LPR = NB / 4;
  constexpr int NLD = SUB * LPR / 256;
  constexpr int JP = 16 * NTJ;
  static_assert(SUB * LPR % 256 == 0, "sub-round must split evenly");
  constexpr int LOOP_BYTES = SUB * XS * 4 + JP * RS * 4;
  constexpr int END_BYTES = 4 * kPlaneMaxModes * JP * 4;
  __shared__ __attribute__((aligned(16)))
  unsigned char s_raw[LOOP_BYTES > END_BYTES ? LOOP_BYTES : END_BYTES];
  float* s_x = reinterpret_cast<float*>(s_raw);
  float* s_rt = s_x + SUB * XS;
  float* s_x2 = reinterpret_cast<float*>(s_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  const int jt = wave % NTJ, mt = wave / NTJ;
  const int IT = a.ma / 4;
  const int64_t plane = blockIdx.x;
  const int chunk = blockIdx.y;
  const int r_begin = chunk * a.rows_per_chunk;
  const int r_end = min(a.Na, r_begin + a.rows_per_chunk);

  // T1 slice: for group g, MFMA jj: B[q][n] = T1[16 g + 4 q + jj][16 jt + m]
  float4 tb[KG];
  {
    const float* t1 = static_cast<const float*>(a.t1);
#pragma unroll
    for (int g = 0; g < KG; ++g)
      tb[g] = make_float4(t1[(16 * g + 4 * q + 0) * JP + 16 * jt + m],
                          t1[(16 * g + 4 * q + 1) * JP + 16 * jt + m],
                          t1[(16 * g + 4 * q + 2) * JP + 16 * jt + m],
                          t1[(16 * g + 4 * q + 3) * JP + 16 * jt + m]);
  }
  f32x4 x2[2][NTJ];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < NTJ; ++v) x2[u][v] = zero4();

  const float* base0 = a.in0 + plane * (int64_t)a.Na * NB;
  const float* base1 = (PIN == PLANE_GELU_GRAD) ? a.in1 + plane * (int64_t)a.Na * NB : nullptr;
  float4 pre0[NLD], pre1[NLD];
  auto load_sub = [&](int r0) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int e = tid + 256 * u;
      const int row = r0 + e / LPR, c4 = e % LPR;
      pre0[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      pre1[u] = pre0[u];
      if (row < r_end) {
        pre0[u] = load_stream4(base0 + (int64_t)row * NB + 4 * c4);
        if (PIN == PLANE_GELU_GRAD)
          pre1[u] = load_stream4(base1 + (int64_t)row * NB + 4 * c4);
      }
    }
  };
  auto stage_sub = [&]() {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int e = tid + 256 * u;
      const int r = e / LPR, c4 = e % LPR;
      const float4 v = pre0[u], w = pre1[u];
      *reinterpret_cast<float4*>(s_x + r * XS + 4 * c4) =
          make_float4(prologue<PIN>(v.x, w.x), prologue<PIN>(v.y, w.y), prologue<PIN>(v.z, w.z),
                      prologue<PIN>(v.w, w.w));
    }
  };

  const float* f2 = static_cast<const float*>(a.f2);
  load_sub(r_begin);
  for (int r0 = r_begin; r0 < r_end; r0 += 64) {
    for (int sub = 0; sub < 64; sub += SUB) {
      __syncthreads();
      stage_sub();
      load_sub(r0 + sub + SUB);
      __syncthreads();
      f32x4 d = zero4();
#pragma unroll
      for (int g = 0; g < KG; ++g) {
        const float4 av =
            *reinterpret_cast<const float4*>(s_x + (16 * mt + m) * XS + 16 * g + 4 * q);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) d = mfma_f32(cmp4(av, jj), cmp4(tb[g], jj), d);
      }
      *reinterpret_cast<float4*>(s_rt + (16 * jt + m) * RS + sub + 16 * mt + 4 * q) =
          make_float4(d[0], d[1], d[2], d[3]);
    }
    __syncthreads();
    // second product: K-groups of 16 rows; MFMA jj uses row 16 kg + 4 q + jj
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      float4 bv[NTJ];
#pragma unroll
      for (int v = 0; v < NTJ; ++v)
        bv[v] = *reinterpret_cast<const float4*>(s_rt + (16 * v + m) * RS + 16 * kg + 4 * q);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int it = wave + 4 * u;
        if (it >= IT) break;
        const int row0 = r0 + 16 * kg + 4 * q;
        const int64_t fo = (int64_t)(16 * it + m) * a.Na + row0;
        float4 av;
        if (row0 + 4 <= r_end) {
          av = *reinterpret_cast<const float4*>(f2 + fo);
        } else {
          av.x = (row0 + 0 < r_end) ? f2[fo + 0] : 0.f;
          av.y = (row0 + 1 < r_end) ? f2[fo + 1] : 0.f;
          av.z = (row0 + 2 < r_end) ? f2[fo + 2] : 0.f;
          av.w = (row0 + 3 < r_end) ? f2[fo + 3] : 0.f;
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int v = 0; v < NTJ; ++v)
            x2[u][v] = mfma_f32(cmp4(av, jj), cmp4(bv[v], jj), x2[u][v]);
      }
    }
  }
  __syncthreads();
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

// ------------------------------------------------------------------------------------------
// bf16 operands, 4 column tiles (jpad = 64), 512 threads.  The contiguous-axis table sits in
// LDS, shared by the 8 waves, instead of in registers; this leaves room for twice the rows in
// flight per CU.  Each sub-round stages 32 rows (double-buffered LDS tile, one barrier per
// sub-round); wave w computes column tile w % 4 of M-tile w / 4.  Every 64 rows the outer-
// axis product runs, its tiles (F2 M-tile, column tile) spread over the 8 waves.  The loop is
// straight-line: rows past the chunk are loaded from a clamped row and staged as zeros, and
// the F2 fragments of a stage are loaded at its start.
template <int PIN, int NB, int H>
__global__ void __launch_bounds__(512) k_plane_bf16_lds(PlaneArgs a) {
  using HT = Half<H>;  // the plan's half format (bfloat16 or IEEE half)
  using V8 = typename HT::v8;
  constexpr int NTJ = 4;
  constexpr int JP = 16 * NTJ;
  constexpr int SUB = 32;               // rows per sub-round (2 M-tiles)
  constexpr int SPS = 64 / SUB;         // sub-rounds per 64-row stage
  constexpr int XS = NB + 8;            // bf16 row stride of the table and row tiles
  constexpr int RS = 64 + 8;            // Rt row stride (bf16)
  constexpr int KS = NB / 32;           // K-steps of the first product
  constexpr int LPR = NB / 4;           // float4 per row
  constexpr int NLD = SUB * LPR / 512;  // float4 per thread per sub-round and input
  constexpr int NT2 = NTJ;              // second product: wave w owns F2 row tile w, all column tiles
  static_assert(SUB * LPR % 512 == 0, "sub-round must split evenly");
  static_assert(SPS == 2, "the loops below handle a 64-row stage as two sub-rounds");
  constexpr std::integral_constant<bool, true> kTrue{};
  constexpr std::integral_constant<bool, false> kFalse{};
  constexpr int T1_B = JP * XS * 2, X_B = SUB * XS * 2, RT_B = JP * RS * 2;
  constexpr int LOOP_B = T1_B + 2 * X_B + RT_B;
  constexpr int END_B = 4 * kPlaneMaxModes * JP * 4;
  __shared__ __attribute__((aligned(16))) unsigned char s_raw[LOOP_B > END_B ? LOOP_B : END_B];
  uint16_t* s_t1 = reinterpret_cast<uint16_t*>(s_raw);
  uint16_t* s_xb = reinterpret_cast<uint16_t*>(s_raw + T1_B);  // two [SUB][XS] tiles
  uint16_t* s_rt = reinterpret_cast<uint16_t*>(s_raw + T1_B + 2 * X_B);
  float* s_x2 = reinterpret_cast<float*>(s_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  const int jt = wave % NTJ, mt = wave / NTJ;
  const int IT = a.ma / 4;  // 16-row tiles of F2 (4 ma rows)
  const int64_t plane = blockIdx.x;
  const int chunk = blockIdx.y;
  const int r_begin = chunk * a.rows_per_chunk;
  const int r_end = min(a.Na, r_begin + a.rows_per_chunk);
  const int nsub = (r_end - r_begin + 63) / 64 * SPS;

  // table -> LDS, [JP][XS] (row j = output column, K along the row)
  for (int e = tid; e < JP * NB / 8; e += 512) {
    const int j = e / (NB / 8), c8 = e % (NB / 8);
    *reinterpret_cast<uint4*>(s_t1 + j * XS + 8 * c8) =
        *reinterpret_cast<const uint4*>(a.t1t + (int64_t)j * NB + 8 * c8);
  }
  const float* base0 = a.in0 + plane * (int64_t)a.Na * NB;
  const float* base1 = (PIN == PLANE_GELU_GRAD) ? a.in1 + plane * (int64_t)a.Na * NB : base0;
  // thread's float4 u of sub-round n: row SUB n + (tid + 512 u) / LPR, column 4 ((tid + 512 u) % LPR)
  const uint16_t* f2 = static_cast<const uint16_t*>(a.f2);
  f32x4 x2[NT2];
#pragma unroll
  for (int k = 0; k < NT2; ++k) x2[k] = zero4();
  V8 fh[2], fl[2];  // this wave's F2 row tile, both K-steps of a stage (hi, lo)
  auto load_sub = [&](int n, float4 (&d0)[NLD], float4 (&d1)[NLD]) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int e = tid + 512 * u;
      const int row = min(r_begin + SUB * n + e / LPR, r_end - 1);
      const int64_t off = (int64_t)row * NB + 4 * (e % LPR);
      d0[u] = load_stream4(base0 + off);
      if (PIN == PLANE_GELU_GRAD) d1[u] = load_stream4(base1 + off);
    }
  };
  // stage sub-round n's rows (tanh / GELU' prologue, bf16); rows past the chunk are zero.
  // Even sub-rounds (the first of a 64-row stage) also load the stage's F2 fragments; the
  // choice is a compile-time tag so that the loop has no branch around memory operations.
  auto stage = [&](auto first_tag, int n, const float4 (&c0)[NLD], const float4 (&c1)[NLD]) {
    uint16_t* s_x = s_xb + (n & 1) * (SUB * XS);
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int e = tid + 512 * u;
      const int r = e / LPR, c4 = e % LPR;
      const bool live = r_begin + SUB * n + r < r_end;
      const float4 v = c0[u], w = c1[u];
      // a bit mask, not a branch: divergent control flow here would make the compiler wait
      // for every load in flight at the top of the loop
      const uint32_t keep = live ? 0xffffffffu : 0u;
      const float o0 = __uint_as_float(__float_as_uint(prologue<PIN>(v.x, w.x)) & keep);
      const float o1 = __uint_as_float(__float_as_uint(prologue<PIN>(v.y, w.y)) & keep);
      const float o2 = __uint_as_float(__float_as_uint(prologue<PIN>(v.z, w.z)) & keep);
      const float o3 = __uint_as_float(__float_as_uint(prologue<PIN>(v.w, w.w)) & keep);
      uint2 packed;
      packed.x = HT::pack2(o0, o1);
      packed.y = HT::pack2(o2, o3);
      *reinterpret_cast<uint2*>(s_x + r * XS + 4 * c4) = packed;
    }
    if constexpr (decltype(first_tag)::value) {
      // F2 fragments of this stage (columns r0 .. r0 + 63; a block past the rows only meets
      // zero rows of R, so its column is clamped into the table)
      const int r0 = r_begin + 64 * (n / SPS);
      const int it = min(wave, IT - 1);  // waves past IT repeat the last tile (dropped)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int col = min(r0 + 32 * ks + 8 * q, a.Na - 8);
        const int64_t fo = (int64_t)(16 * it + m) * a.Na + col;
        fh[ks] = *reinterpret_cast<const V8*>(f2 + fo);
        fl[ks] = *reinterpret_cast<const V8*>(a.f2lo + fo);
      }
    }
  };
  // products of sub-round n (after its rows are staged and the next loads are issued).  The
  // next sub-round writes the other row buffer and, after its barrier, Rt: every wave reaches
  // that barrier only after finishing this sub-round's reads.
  auto compute = [&](auto last_tag, int n) {
    constexpr int sr = decltype(last_tag)::value ? 1 : 0;
    const uint16_t* s_x = s_xb + (n & 1) * (SUB * XS);
    __syncthreads();  // row tile visible
    f32x4 d = zero4();
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      const V8 av = *reinterpret_cast<const V8*>(s_x + (16 * mt + m) * XS + 32 * s2 + 8 * q);
      const V8 bv = *reinterpret_cast<const V8*>(s_t1 + (16 * jt + m) * XS + 32 * s2 + 8 * q);
      d = HT::mfma(av, bv, d);
    }
    // D rows 16 mt + 4 q + r (stage row SUB sr + ..), column 16 jt + m  ->  Rt[column][row]
    uint2 pk;
    pk.x = HT::pack2(d[0], d[1]);
    pk.y = HT::pack2(d[2], d[3]);
    *reinterpret_cast<uint2*>(s_rt + (16 * jt + m) * RS + SUB * sr + 16 * mt + 4 * q) = pk;
    if constexpr (decltype(last_tag)::value) {
      __syncthreads();  // Rt of the 64-row stage complete
      // every wave runs its products (a wave past IT repeats the last F2 tile and its result
      // is dropped at the end), so no branch separates the F2 loads from their use
#pragma unroll
      for (int v = 0; v < NT2; ++v) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const V8 bv = *reinterpret_cast<const V8*>(s_rt + (16 * v + m) * RS + 32 * ks + 8 * q);
          x2[v] = HT::mfma(fh[ks], bv, x2[v]);
          x2[v] = HT::mfma(fl[ks], bv, x2[v]);
        }
      }
    }
  };
  // Two register sets alternate: each is staged and then reloaded two sub-rounds ahead, so
  // one sub-round's rows are always in flight while another is staged (nsub is even: whole
  // 64-row stages of 32-row sub-rounds).  The scheduling barrier keeps set A's loads ahead
  // of set B's, the order in which the loop waits for them.
  float4 a0[NLD], a1[NLD], b0[NLD], b1[NLD];
#pragma unroll
  for (int u = 0; u < NLD; ++u) {
    a1[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    b1[u] = a1[u];
  }
  load_sub(0, a0, a1);
  __builtin_amdgcn_sched_barrier(0);
  load_sub(min(1, nsub - 1), b0, b1);
  for (int n = 0; n < nsub; n += 2) {
    stage(kTrue, n, a0, a1);
    load_sub(min(n + 2, nsub - 1), a0, a1);
    compute(kFalse, n);
    stage(kFalse, n + 1, b0, b1);
    load_sub(min(n + 3, nsub - 1), b0, b1);
    compute(kTrue, n + 1);
  }
  __syncthreads();  // the loop buffers are reused for X2
  if (wave < IT) {
#pragma unroll
    for (int v = 0; v < NT2; ++v)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_x2[(16 * wave + 4 * q + r) * JP + 16 * v + m] = x2[v][r];
  }
  __syncthreads();
  combine_store(s_x2, JP, a.ma, a.mb,
                a.out + ((int64_t)chunk * a.planes + plane) * (2 * a.ma * a.mb), tid, 512);
}

// ------------------------------------------------------------------------------------------
bool plane_fast_ok(const fno_plan* p) {
  const Geom& g = p->g;
  const int jpad = p->jpad;
  if (!(g.Nb == 64 || g.Nb == 128 || g.Nb == 256 || g.Nb == 512)) return false;
  if (!(jpad == 16 || jpad == 32 || jpad == 64)) return false;
  if (g.ma % 4 != 0 || g.ma > kPlaneMaxModes) return false;  // F2: <= 2 tiles of 16 rows/wave
  // vector loads of F2 rows need 8-aligned row offsets
  if (g.Na % 8 != 0 || (p->plane_rows % 64 != 0 && p->plane_rows != g.Na)) return false;
  if (!g.bf16) {
    const int sub = 16 * (4 / (jpad / 16));
    if (sub * (g.Nb + 4) * 4 > 48 * 1024) return false;  // LDS of the staged rows
  }
  return true;
}

template <int PIN, int NB, int NTJ>
static void launch_plane_t(const fno_plan* p, const PlaneArgs& a, dim3 grid, hipStream_t s) {
  if (p->g.half == 2 && NTJ == 4)
    hipLaunchKernelGGL((k_plane_bf16_lds<PIN, NB, 2>), grid, dim3(512), 0, s, a);
  else if (p->g.half == 2)
    hipLaunchKernelGGL((k_plane_bf16<PIN, NB, NTJ, 2>), grid, dim3(256), 0, s, a);
  else if (p->g.bf16 && NTJ == 4)
    hipLaunchKernelGGL((k_plane_bf16_lds<PIN, NB, 1>), grid, dim3(512), 0, s, a);
  else if (p->g.bf16)
    hipLaunchKernelGGL((k_plane_bf16<PIN, NB, NTJ, 1>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_plane_f32<PIN, NB, NTJ>), grid, dim3(256), 0, s, a);
}

template <int PIN, int NB>
static void launch_plane_nb(const fno_plan* p, const PlaneArgs& a, dim3 grid, hipStream_t s) {
  switch (p->jpad) {
    case 16: launch_plane_t<PIN, NB, 1>(p, a, grid, s); break;
    case 32: launch_plane_t<PIN, NB, 2>(p, a, grid, s); break;
    default: launch_plane_t<PIN, NB, 4>(p, a, grid, s); break;
  }
}

template <int PIN>
static void launch_plane_pin(const fno_plan* p, const PlaneArgs& a, dim3 grid, hipStream_t s) {
  switch (p->g.Nb) {
    case 64: launch_plane_nb<PIN, 64>(p, a, grid, s); break;
    case 128: launch_plane_nb<PIN, 128>(p, a, grid, s); break;
    case 256: launch_plane_nb<PIN, 256>(p, a, grid, s); break;
    default: launch_plane_nb<PIN, 512>(p, a, grid, s); break;
  }
}

hipError_t launch_plane_fwd_fast(const fno_plan* p, int plane_in, int chans, const float* in0,
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
  a.t1 = g.bf16 ? (const void*)p->t.t1_bf : (const void*)p->t.t1;
  a.f2 = g.bf16 ? (const void*)p->t.f2_bf : (const void*)p->t.f2;
  a.f2lo = p->t.f2_bf_lo;
  a.t1t = p->t.t1t_bf;
  a.out = out;
  dim3 grid((unsigned)a.planes, (unsigned)p->nch);
  switch (plane_in) {
    case PLANE_X: launch_plane_pin<PLANE_X>(p, a, grid, s); break;
    case PLANE_TANH: launch_plane_pin<PLANE_TANH>(p, a, grid, s); break;
    case PLANE_GELU: launch_plane_pin<PLANE_GELU>(p, a, grid, s); break;
    case PLANE_TANH_GELU: launch_plane_pin<PLANE_TANH_GELU>(p, a, grid, s); break;
    default: launch_plane_pin<PLANE_GELU_GRAD>(p, a, grid, s); break;
  }
  return hipGetLastError();
}

}  // namespace fno
