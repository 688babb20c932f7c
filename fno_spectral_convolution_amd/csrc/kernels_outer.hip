// Matrix-core truncated DFT along one outer axis of a spectrum tensor [pre][Lin][post]
// (complex) -> [pre][Lout][post]:
//   forward:  out[s] = sum_p in[p] e^{-2 pi i k(s) p / N}   (Lin = N, Lout = 2m)
//   inverse:  out[p] = sum_s in[s] e^{+2 pi i k(s) p / N}   (Lin = 2m, Lout = N: the
//             zero-padded inverse, evaluated only from the retained rows)
// As a real product with interleaved (re, im) columns:
//   out = [Mr | Mi] . [X ; Xs],  Xs[l][2c] = -X[l][2c+1],  Xs[l][2c+1] = X[l][2c]
// so K = 2 Lin.  The twiddle matrix A = [Mr | Mi] ([Lout_pad][2 Lin_pad], zero padded) is
// built on the host in float64 and read through L2; a work-group stages its column tile of
// the input, transposed and with the swapped copy, in LDS and its waves split the M-tiles.
// Column n of N-tile t is column NT n + t of the work-group's tile, so a lane holds NT
// adjacent output columns of a row and 16 lanes store 16 NT adjacent floats at once.
#include "fno_internal.h"
#include "mfma.h"

namespace fno {

// v where keep, else zeros, by masking the bits
__device__ __forceinline__ float4 mask4(const float4& v, bool keep) {
  const uint32_t k = keep ? 0xffffffffu : 0u;
  return make_float4(__uint_as_float(__float_as_uint(v.x) & k), __uint_as_float(__float_as_uint(v.y) & k),
                     __uint_as_float(__float_as_uint(v.z) & k), __uint_as_float(__float_as_uint(v.w) & k));
}

struct OuterArgs {
  int Lin, Lout, Lin_pad, Lout_pad;
  int64_t post2;         // floats per row (2 * post)
  const float* in;       // [pre][Lin][post2]
  float* out;            // [pre][Lout][post2]
  const void* A;         // [Lout_pad][2 Lin_pad] f32, or bf16 bits (hi)
  const uint16_t* Alo;   // bf16 residual (bf16 path)
  int64_t pre;           // slabs
  int msplit, mt_per;    // k_outer_mfma: work-groups per slab, output row tiles of each
  uint16_t* outh;        // k_outer_mfma: the output in the plan's half format instead, or null
};

template <int H, int NT>
__global__ void __launch_bounds__(256) k_outer_mfma(OuterArgs a) {
  constexpr bool BF = H != 0;  // half operands (bfloat16 or IEEE half)
  using V8 = typename HalfOf<H>::v8;
  constexpr int CT = 16 * NT;  // columns per work-group
  extern __shared__ __attribute__((aligned(16))) unsigned char s_raw[];
  const int K = 2 * a.Lin_pad;
  const int KS = K + (BF ? 8 : 4);  // row stride of Bt (elements)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  // With msplit > 1 the output row tiles of a slab are split over msplit work-groups, which
  // the numbering keeps on one XCD (work-group x runs on XCD x % 8) so that they share the
  // slab's input in its L2: x = 8 msplit grp + 8 ms + i is slab 8 grp + i, part ms.
  int64_t pre = blockIdx.x;
  int ms = 0;
  if (a.msplit > 1) {
    const int64_t x = blockIdx.x;
    const int64_t grp = x / (8 * a.msplit);
    const int r = (int)(x - grp * 8 * a.msplit);
    ms = r / 8;
    pre = grp * 8 + (r & 7);
    if (pre >= a.pre) return;  // the whole work-group: past the last slab
  }
  const int mt_begin = ms * a.mt_per;
  const int mt_end = min(a.Lout_pad / 16, mt_begin + a.mt_per);
  const int64_t c0 = (int64_t)blockIdx.y * CT;
  const float* src = a.in + pre * a.Lin * a.post2;
  // Bt[c][k]: k < Lin_pad -> X[k][c0 + c]; k >= Lin_pad -> Xs[k - Lin_pad][c0 + c]
  // staged row of column c (local): 16 (c % NT) + c / NT
  auto brow = [](int c) { return 16 * (c % NT) + c / NT; };
  // 8 loads per thread in flight at a time: clamped addresses and a mask, no branch around
  // the loads (which would make each wait for the one before it)
  constexpr int SU = 8;
  const int nel = a.Lin_pad * CT;
  if (NT == 4 && (a.post2 & 3) == 0) {
    // rows of whole float4: thread f = tid + 256 u loads columns 4 (f % 16) .. + 3 of input row
    // f / 16 (zero past the slab's rows or columns); staged row of column 4 c4 + j is
    // 16 j + c4, and the swapped copy of column c goes to the row of column c ^ 1
    constexpr int FU = 4;
    const int nf = a.Lin_pad * (CT / 4);
    for (int f0 = 0; f0 < nf; f0 += 256 * FU) {
      float4 v[FU];
#pragma unroll
      for (int u = 0; u < FU; ++u) {
        const int f = f0 + tid + 256 * u;
        const int li = f >> 4, c4 = f & 15;
        const int64_t col = c0 + 4 * c4;
        const bool ok = f < nf && li < a.Lin && col < a.post2;
        const int64_t off = (int64_t)min(li, a.Lin - 1) * a.post2 + min(col, a.post2 - 4);
        const float4 x = *reinterpret_cast<const float4*>(src + off);
        v[u] = ok ? x : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the LDS writes
#pragma unroll
      for (int u = 0; u < FU; ++u) {
        const int f = f0 + tid + 256 * u;
        if (f >= nf) continue;
        const int li = f >> 4, c4 = f & 15;
        const float w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float vs = (j & 1) ? -w[j] : w[j];  // Xs[li][(4 c4 + j) ^ 1]
          const int rj = 16 * j + c4, rs = 16 * (j ^ 1) + c4;
          if (BF) {
            uint16_t* bt = reinterpret_cast<uint16_t*>(s_raw);
            bt[rj * KS + li] = HalfOf<H>::bits(w[j]);
            bt[rs * KS + a.Lin_pad + li] = HalfOf<H>::bits(vs);
          } else {
            float* bt = reinterpret_cast<float*>(s_raw);
            bt[rj * KS + li] = w[j];
            bt[rs * KS + a.Lin_pad + li] = vs;
          }
        }
      }
    }
  } else
  for (int e0 = 0; e0 < nel; e0 += 256 * SU) {
    float v[SU];
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int e = e0 + tid + 256 * u;
      const int li = e / CT, c = e - li * CT;
      const int64_t col = c0 + c;
      const bool ok = e < nel && li < a.Lin && col < a.post2;
      const int64_t off = (int64_t)min(li, a.Lin - 1) * a.post2 + min(col, a.post2 - 1);
      const float x = src[off];
      v[u] = ok ? x : 0.f;
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the LDS writes
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int e = e0 + tid + 256 * u;
      if (e >= nel) continue;
      const int li = e / CT, c = e - li * CT;
      const int cp = c ^ 1;
      const float vs = (c & 1) ? -v[u] : v[u];  // Xs[li][c^1]
      if (BF) {
        uint16_t* bt = reinterpret_cast<uint16_t*>(s_raw);
        bt[brow(c) * KS + li] = HalfOf<H>::bits(v[u]);
        bt[brow(cp) * KS + a.Lin_pad + li] = HalfOf<H>::bits(vs);
      } else {
        float* bt = reinterpret_cast<float*>(s_raw);
        bt[brow(c) * KS + li] = v[u];
        bt[brow(cp) * KS + a.Lin_pad + li] = vs;
      }
    }
  }
  __syncthreads();
  float* dst = a.out + pre * a.Lout * a.post2;
  for (int mt = mt_begin + wave; mt < mt_end; mt += 4) {
    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = zero4();
    const int prow = 16 * mt + m;
    if (BF) {
      const uint16_t* A = static_cast<const uint16_t*>(a.A) + (int64_t)prow * K;
      const uint16_t* Al = a.Alo + (int64_t)prow * K;
      const uint16_t* bt = reinterpret_cast<const uint16_t*>(s_raw);
      for (int k0 = 0; k0 < K; k0 += 32) {
        const V8 ah = *reinterpret_cast<const V8*>(A + k0 + 8 * q);
        const V8 al = *reinterpret_cast<const V8*>(Al + k0 + 8 * q);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const V8 bv = *reinterpret_cast<const V8*>(bt + (16 * nt + m) * KS + k0 + 8 * q);
          acc[nt] = HalfOf<H>::mfma(ah, bv, acc[nt]);
          acc[nt] = HalfOf<H>::mfma(al, bv, acc[nt]);
        }
      }
    } else {
      const float* A = static_cast<const float*>(a.A) + (int64_t)prow * K;
      const float* bt = reinterpret_cast<const float*>(s_raw);
      for (int k0 = 0; k0 < K; k0 += 16) {
        const float4 av = *reinterpret_cast<const float4*>(A + k0 + 4 * q);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float4 bv = *reinterpret_cast<const float4*>(bt + (16 * nt + m) * KS + k0 + 4 * q);
          acc[nt] = mfma_f32(av.x, bv.x, acc[nt]);
          acc[nt] = mfma_f32(av.y, bv.y, acc[nt]);
          acc[nt] = mfma_f32(av.z, bv.z, acc[nt]);
          acc[nt] = mfma_f32(av.w, bv.w, acc[nt]);
        }
      }
    }
    // lane (n = m, q): rows 16 mt + 4 q + r, columns c0 + NT m + nt (nt = 0 .. NT-1)
    const int64_t col = c0 + NT * m;
    if constexpr (BF && NT == 4) {
      if (a.outh) {
        // rounded to the half format here (nearest even), as its consumer would round it
        uint16_t* dh = a.outh + pre * a.Lout * a.post2;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int p = 16 * mt + 4 * q + r;
          if (p >= a.Lout) continue;
          uint16_t* d = dh + (int64_t)p * a.post2 + col;
          if (col + 4 <= a.post2 && (a.post2 % 4) == 0) {
            *reinterpret_cast<uint2*>(d) = make_uint2(HalfOf<H>::pack2(acc[0][r], acc[1][r]),
                                                      HalfOf<H>::pack2(acc[2][r], acc[3][r]));
          } else {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
              if (col + nt < a.post2) d[nt] = HalfOf<H>::bits(acc[nt][r]);
          }
        }
        continue;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = 16 * mt + 4 * q + r;
      if (p >= a.Lout) continue;
      float* d = dst + (int64_t)p * a.post2 + col;
      if (col + NT <= a.post2 && (a.post2 % NT) == 0) {
        if constexpr (NT == 4) {
          *reinterpret_cast<float4*>(d) = make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
        } else if constexpr (NT == 2) {
          *reinterpret_cast<float2*>(d) = make_float2(acc[0][r], acc[1][r]);
        } else {
          d[0] = acc[0][r];
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          if (col + nt < a.post2) d[nt] = acc[nt][r];
      }
    }
  }
}

// Forward transform of an outer axis when few rows are kept (Lout <= 64): the product
// out[o][c] = sum_k Mr[o][k] X[k][c] + Mi[o][k] Xs[k][c] has a short M and a long K, so a
// work-group owns a block of CB = 64 NTW columns of one slab and streams the slab's rows through
// LDS in 16-row chunks (float4 rows, prefetched one chunk ahead in registers) while every output
// tile stays in registers: wave w owns N-tiles w NTW .. w NTW + NTW - 1 for all MT row tiles.
// K-step ks, k-slot q is row k0 + 4 q + ks, so a lane's table operands for a chunk are one float4
// per table half and row tile.  Xs needs no copy: it is X at the partner column c ^ 1, negated
// for even c (a lane constant).  fp32 operands.
template <int MT, int NTW>
__global__ void __launch_bounds__(256) k_outer_fwd_stream(OuterArgs a) {
  constexpr int CB = 64 * NTW;   // columns per work-group
  constexpr int CBS = CB + 4;    // LDS row stride: the four k-slot groups on distinct banks
  constexpr int F4R = CB / 4;    // float4 per chunk row
  __shared__ __attribute__((aligned(16))) float s_x[16 * CBS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  const int64_t pre = blockIdx.y;
  const int c0 = blockIdx.x * CB;
  const float* src = a.in + pre * a.Lin * a.post2;
  float* dst = a.out + pre * a.Lout * a.post2;
  const int K2 = 2 * a.Lin_pad;  // table row stride
  const float* A = static_cast<const float*>(a.A);
  // chunk element i of this thread: float4 e = tid + 256 i -> row e / F4R, columns 4 (e % F4R)
  int xrow[NTW], xcol[NTW];
  bool xcol_ok[NTW];
#pragma unroll
  for (int i = 0; i < NTW; ++i) {
    const int e = tid + 256 * i;
    xrow[i] = e / F4R;
    const int col = c0 + 4 * (e % F4R);
    xcol_ok[i] = col < a.post2;
    xcol[i] = min(col, a.post2 - 4);
  }
  // the raw rows (clamped, valid addresses) and a bit per element telling whether it lies in
  // the slab; the mask is applied when the chunk is staged, so that no instruction uses a load
  // before then (a select or mask right after each load made the compiler wait for it before
  // issuing the next)
  auto load_chunk = [&](int k0, float4 (&v)[NTW], uint32_t& okm) {
    okm = 0u;
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
      const int row = k0 + xrow[i];
      v[i] = *reinterpret_cast<const float4*>(src + (int64_t)min(row, a.Lin - 1) * a.post2 + xcol[i]);
      okm |= (row < a.Lin && xcol_ok[i]) ? (1u << i) : 0u;
    }
  };
  auto load_tab = [&](int k0, float4 (&r)[MT], float4 (&im)[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float* row = A + (int64_t)(16 * mt + m) * K2 + k0 + 4 * q;
      r[mt] = *reinterpret_cast<const float4*>(row);
      im[mt] = *reinterpret_cast<const float4*>(row + a.Lin_pad);
    }
  };
  f32x4 acc[MT][NTW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[mt][j] = zero4();
  float4 xv[NTW], tr[MT], ti[MT];
  uint32_t xok;
  load_chunk(0, xv, xok);
  load_tab(0, tr, ti);
  const float sgn = (m & 1) ? 1.f : -1.f;  // Xs[k][c] = sgn * X[k][c ^ 1]
  const int nchunk = a.Lin_pad / 16;
  for (int ch = 0; ch < nchunk; ++ch) {
#pragma unroll
    for (int i = 0; i < NTW; ++i)
      *reinterpret_cast<float4*>(s_x + xrow[i] * CBS + 4 * ((tid + 256 * i) % F4R)) =
          mask4(xv[i], (xok >> i) & 1u);
    float4 cr[MT], ci[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      cr[mt] = tr[mt];
      ci[mt] = ti[mt];
    }
    // the next chunk (the last one loads itself again: no branch around the loads)
    const int kn = 16 * min(ch + 1, nchunk - 1);
    load_chunk(kn, xv, xok);
    load_tab(kn, tr, ti);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const float* xr = s_x + (4 * q + ks) * CBS + 16 * wave * NTW + m;
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const float bx = xr[16 * j];
        const float bs = sgn * xr[16 * j + ((m & 1) ? -1 : 1)];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const float ar = ks == 0 ? cr[mt].x : ks == 1 ? cr[mt].y : ks == 2 ? cr[mt].z : cr[mt].w;
          const float ai = ks == 0 ? ci[mt].x : ks == 1 ? ci[mt].y : ks == 2 ? ci[mt].z : ci[mt].w;
          acc[mt][j] = mfma_f32(ar, bx, acc[mt][j]);
          acc[mt][j] = mfma_f32(ai, bs, acc[mt][j]);
        }
      }
    }
    __syncthreads();
  }
  // lane (n = m, q), register r: output row 16 mt + 4 q + r, column c0 + 16 (w NTW + j) + m
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int o = 16 * mt + 4 * q + r;
      if (o >= a.Lout) continue;
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int col = c0 + 16 * (wave * NTW + j) + m;
        if (col < a.post2) dst[(int64_t)o * a.post2 + col] = acc[mt][j][r];
      }
    }
}

// The same streaming transform on the mixed path: 32-row chunks, one 16x16x32 bf16 MFMA K-step
// per chunk and term, the table as its bf16 hi + lo pair (two products per term).  K-slot (q, e)
// is row k0 + 8 q + e; a lane reads the column pair (c & ~1) of each of its 8 rows as one float2,
// which gives both X[k][c] and the partner for Xs, rounded to bf16 as operands.
template <int H, int MT, int NTW>
__global__ void __launch_bounds__(256) k_outer_fwd_stream_bf(OuterArgs a) {
  using HT = Half<H>;
  using V8 = typename HT::v8;
  constexpr int CB = 64 * NTW;
  constexpr int CBS = CB + 4;
  constexpr int F4R = CB / 4;
  constexpr int NL = 2 * NTW;  // float4 of a 32-row chunk per thread
  __shared__ __attribute__((aligned(16))) float s_x[32 * CBS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  const int64_t pre = blockIdx.y;
  const int c0 = blockIdx.x * CB;
  const float* src = a.in + pre * a.Lin * a.post2;
  float* dst = a.out + pre * a.Lout * a.post2;
  const int K2 = 2 * a.Lin_pad;
  const uint16_t* Ah = static_cast<const uint16_t*>(a.A);
  const uint16_t* Al = a.Alo;
  int xrow[NL], xcol[NL];
  bool xcol_ok[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int e = tid + 256 * i;
    xrow[i] = e / F4R;
    const int col = c0 + 4 * (e % F4R);
    xcol_ok[i] = col < a.post2;
    xcol[i] = min(col, a.post2 - 4);
  }
  // raw rows and an in-slab bit per element, masked when staged (as in k_outer_fwd_stream)
  auto load_chunk = [&](int k0, float4 (&v)[NL], uint32_t& okm) {
    okm = 0u;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int row = k0 + xrow[i];
      v[i] = *reinterpret_cast<const float4*>(src + (int64_t)min(row, a.Lin - 1) * a.post2 + xcol[i]);
      okm |= (row < a.Lin && xcol_ok[i]) ? (1u << i) : 0u;
    }
  };
  // table fragments of a K-step: [row tile][Mr hi, Mr lo, Mi hi, Mi lo], columns k0 + 8 q ..
  auto load_tab = [&](int k0, V8 (&t)[MT][4]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int64_t row = (int64_t)(16 * mt + m) * K2 + min(k0 + 8 * q, a.Lin_pad - 8);
      t[mt][0] = *reinterpret_cast<const V8*>(Ah + row);
      t[mt][1] = *reinterpret_cast<const V8*>(Al + row);
      t[mt][2] = *reinterpret_cast<const V8*>(Ah + row + a.Lin_pad);
      t[mt][3] = *reinterpret_cast<const V8*>(Al + row + a.Lin_pad);
    }
  };
  f32x4 acc[MT][NTW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[mt][j] = zero4();
  float4 xv[NL];
  uint32_t xok;
  V8 tb[MT][4];
  load_chunk(0, xv, xok);
  load_tab(0, tb);
  const bool odd = (m & 1) != 0;
  const int nchunk = (a.Lin_pad + 31) / 32;
  for (int ch = 0; ch < nchunk; ++ch) {
#pragma unroll
    for (int i = 0; i < NL; ++i)
      *reinterpret_cast<float4*>(s_x + xrow[i] * CBS + 4 * ((tid + 256 * i) % F4R)) =
          mask4(xv[i], (xok >> i) & 1u);
    V8 ct[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 4; ++h) ct[mt][h] = tb[mt][h];
    // rows past Lin in a chunk are loaded as zeros, so the (clamped) table operands of K-slots
    // past Lin_pad multiply zeros
    const int kn = 32 * min(ch + 1, nchunk - 1);
    load_chunk(kn, xv, xok);
    load_tab(kn, tb);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const float* xr = s_x + 8 * q * CBS + 16 * (wave * NTW + j) + (m & ~1);
      float xe[8], xs[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 pr = *reinterpret_cast<const float2*>(xr + e * CBS);
        xe[e] = odd ? pr.y : pr.x;
        xs[e] = odd ? pr.x : -pr.y;
      }
      const V8 bx = __builtin_bit_cast(
          V8, make_uint4(HT::pack2(xe[0], xe[1]), HT::pack2(xe[2], xe[3]),
                         HT::pack2(xe[4], xe[5]), HT::pack2(xe[6], xe[7])));
      const V8 bs = __builtin_bit_cast(
          V8, make_uint4(HT::pack2(xs[0], xs[1]), HT::pack2(xs[2], xs[3]),
                         HT::pack2(xs[4], xs[5]), HT::pack2(xs[6], xs[7])));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt][j] = HT::mfma(ct[mt][0], bx, acc[mt][j]);
        acc[mt][j] = HT::mfma(ct[mt][1], bx, acc[mt][j]);
        acc[mt][j] = HT::mfma(ct[mt][2], bs, acc[mt][j]);
        acc[mt][j] = HT::mfma(ct[mt][3], bs, acc[mt][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int o = 16 * mt + 4 * q + r;
      if (o >= a.Lout) continue;
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int col = c0 + 16 * (wave * NTW + j) + m;
        if (col < a.post2) dst[(int64_t)o * a.post2 + col] = acc[mt][j][r];
      }
    }
}

// Inverse transform of an outer axis from few kept rows (Lin <= 64) to N rows: a short K and a
// long M.  A work-group owns a block of CB = 64 NTW columns of one slab: the kept rows of the block
// are staged once in LDS (row-major, float4 loads), then wave w walks all output row tiles for its
// N-tiles w NTW .. w NTW + NTW - 1 and stores each finished tile.  Operands as in the streaming
// forward transform (fp32 16x16x4 with K-slot q <-> row 4 q + ks of a 16-row group; bf16
// 16x16x32 with K-slot (q, e) <-> row 8 q + e, the table as its hi + lo pair).
template <int H, int NTW>
__global__ void __launch_bounds__(256) k_outer_inv_stream(OuterArgs a) {
  constexpr bool BF = H != 0;  // half operands (bfloat16 or IEEE half)
  using HT = HalfOf<H>;
  using V8 = typename HT::v8;
  constexpr int CB = 64 * NTW;
  constexpr int CBS = CB + 4;
  constexpr int F4R = CB / 4;
  extern __shared__ __attribute__((aligned(16))) float s_xi[];  // [Lin_pad][CBS]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  const int64_t pre = blockIdx.y;
  const int c0 = blockIdx.x * CB;
  const float* src = a.in + pre * a.Lin * a.post2;
  float* dst = a.out + pre * a.Lout * a.post2;
  const int K2 = 2 * a.Lin_pad;
  // stage the kept rows (rows past Lin and columns past the slab as zeros)
  for (int e = tid; e < a.Lin_pad * F4R; e += 256) {
    const int row = e / F4R, col = c0 + 4 * (e - row * F4R);
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row < a.Lin && col < a.post2)
      v = *reinterpret_cast<const float4*>(src + (int64_t)row * a.post2 + col);
    *reinterpret_cast<float4*>(s_xi + row * CBS + 4 * (e - row * F4R)) = v;
  }
  __syncthreads();
  const bool odd = (m & 1) != 0;
  const float sgn = odd ? 1.f : -1.f;  // Xs[k][c] = sgn * X[k][c ^ 1]
  const int colw = 16 * wave * NTW + m;
  for (int mt = 0; mt < a.Lout_pad / 16; ++mt) {
    f32x4 acc[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[j] = zero4();
    const int orow = 16 * mt + m;
    if constexpr (!BF) {
      const float* A = static_cast<const float*>(a.A) + (int64_t)orow * K2;
      for (int g = 0; g < a.Lin_pad / 16; ++g) {
        const float4 ar = *reinterpret_cast<const float4*>(A + 16 * g + 4 * q);
        const float4 ai = *reinterpret_cast<const float4*>(A + a.Lin_pad + 16 * g + 4 * q);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const float* xr = s_xi + (16 * g + 4 * q + ks) * CBS + colw;
          const float tr = ks == 0 ? ar.x : ks == 1 ? ar.y : ks == 2 ? ar.z : ar.w;
          const float ti = ks == 0 ? ai.x : ks == 1 ? ai.y : ks == 2 ? ai.z : ai.w;
#pragma unroll
          for (int j = 0; j < NTW; ++j) {
            const float bx = xr[16 * j];
            const float bs = sgn * xr[16 * j + (odd ? -1 : 1)];
            acc[j] = mfma_f32(tr, bx, acc[j]);
            acc[j] = mfma_f32(ti, bs, acc[j]);
          }
        }
      }
    } else {
      const uint16_t* Ah = static_cast<const uint16_t*>(a.A) + (int64_t)orow * K2;
      const uint16_t* Al = a.Alo + (int64_t)orow * K2;
      for (int k0 = 0; k0 < a.Lin_pad; k0 += 32) {
        // K-slots past Lin_pad (a 16-row remainder) read zero rows of the staged block: the
        // table columns are clamped into the row
        const int tc = min(k0 + 8 * q, a.Lin_pad - 8);
        const uint32_t km = k0 + 8 * q < a.Lin_pad ? 0xffffffffu : 0u;  // mask, not a branch
        auto ld = [&](const uint16_t* p) {
          uint4 v = *reinterpret_cast<const uint4*>(p);
          v.x &= km; v.y &= km; v.z &= km; v.w &= km;
          return __builtin_bit_cast(V8, v);
        };
        const V8 rh = ld(Ah + tc), rl = ld(Al + tc);
        const V8 ih = ld(Ah + a.Lin_pad + tc), il = ld(Al + a.Lin_pad + tc);
        const int xr0 = min(k0 + 8 * q, a.Lin_pad - 8);
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const float* xr = s_xi + xr0 * CBS + 16 * (wave * NTW + j) + (m & ~1);
          float xe[8], xs[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float2 pr = *reinterpret_cast<const float2*>(xr + e * CBS);
            xe[e] = odd ? pr.y : pr.x;
            xs[e] = odd ? pr.x : -pr.y;
          }
          const V8 bx = __builtin_bit_cast(
              V8, make_uint4(HT::pack2(xe[0], xe[1]), HT::pack2(xe[2], xe[3]),
                             HT::pack2(xe[4], xe[5]), HT::pack2(xe[6], xe[7])));
          const V8 bs = __builtin_bit_cast(
              V8, make_uint4(HT::pack2(xs[0], xs[1]), HT::pack2(xs[2], xs[3]),
                             HT::pack2(xs[4], xs[5]), HT::pack2(xs[6], xs[7])));
          acc[j] = HT::mfma(rh, bx, acc[j]);
          acc[j] = HT::mfma(rl, bx, acc[j]);
          acc[j] = HT::mfma(ih, bs, acc[j]);
          acc[j] = HT::mfma(il, bs, acc[j]);
        }
      }
    }
    // lane (n = m, q), register r: output row 16 mt + 4 q + r, column c0 + 16 (w NTW + j) + m
    if constexpr (BF) {
      if (a.outh) {
        // the plan's half format (nearest even), as its consumer would round it: an even lane
        // (real part) stores its value with its odd neighbour's (imaginary part, swapped in by
        // a DPP quad permutation) as one 32-bit pair
        uint16_t* dh = a.outh + pre * a.Lout * a.post2;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int o = 16 * mt + 4 * q + r;
#pragma unroll
          for (int j = 0; j < NTW; ++j) {
            const float v = acc[j][r];
            const float pv = __int_as_float(
                __builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
            const int col = c0 + 16 * (wave * NTW + j) + m;
            if (o < a.Lout && !odd && col < a.post2)
              *reinterpret_cast<uint32_t*>(dh + (int64_t)o * a.post2 + col) =
                  HT::pack2(v, pv);
          }
        }
        continue;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int o = 16 * mt + 4 * q + r;
      if (o >= a.Lout) continue;
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int col = c0 + 16 * (wave * NTW + j) + m;
        if (col < a.post2) dst[(int64_t)o * a.post2 + col] = acc[j][r];
      }
    }
  }
}

// Inverse transform of an outer axis for many narrow slabs (float32; at most 32 kept rows in,
// at most 128 rows out, one column tile of 16 NT columns): a work-group walks spw consecutive
// slabs.  Wave w owns output row tiles w and w + 4 for every slab and keeps their table
// fragments (K-groups of 16) in registers, so the table is read from L2 once per work-group
// rather than once per slab; the next slab's input is loaded into registers while the current
// one is staged in LDS (transposed, with the swapped copy, as in k_outer_mfma) and multiplied.
template <int NT>
__global__ void __launch_bounds__(256) k_outer_inv_slabs(OuterArgs a, int spw) {
  constexpr int CT = 16 * NT;
  constexpr int KMAX = 64;             // 2 Lin_pad <= 64
  constexpr int KSM = KMAX + 4;        // LDS row stride
  constexpr int EU = 32 * CT / 256;    // input elements per thread (Lin_pad <= 32 rows)
  __shared__ __attribute__((aligned(16))) float s_bt[CT * KSM];
  const int K = 2 * a.Lin_pad;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  const int mtiles = a.Lout_pad / 16;
  const int64_t c0 = (int64_t)blockIdx.y * CT;
  const int64_t p0 = (int64_t)blockIdx.x * spw;
  const int64_t p_end = min(p0 + spw, a.pre);
  if (p0 >= a.pre) return;  // the whole work-group
  const float* A = static_cast<const float*>(a.A);
  // table fragments of row tiles wave + 4 t: lane (m, q), K-group g holds A[16 mt + m][16 g +
  // 4 q .. + 3]; tiles past the table and groups past K load clamped copies, never used
  float4 af[2][KMAX / 16];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int mt = min(wave + 4 * t, mtiles - 1);
#pragma unroll
    for (int g = 0; g < KMAX / 16; ++g)
      af[t][g] = *reinterpret_cast<const float4*>(A + (int64_t)(16 * mt + m) * K +
                                                  min(16 * g, K - 16) + 4 * q);
  }
  // input element e = tid + 256 u: row e / CT, column c0 + e % CT (zero past the slab)
  float xv[EU];
  auto load_slab = [&](int64_t pre) {
    const float* src = a.in + pre * a.Lin * a.post2;
#pragma unroll
    for (int u = 0; u < EU; ++u) {
      const int e = tid + 256 * u;
      const int li = e / CT, c = e - li * CT;
      const int64_t col = c0 + c;
      const bool ok = li < a.Lin && col < a.post2;
      const float x = src[(int64_t)min(li, a.Lin - 1) * a.post2 + min(col, a.post2 - 1)];
      xv[u] = ok ? x : 0.f;
    }
  };
  // Bt[c][k]: k < Lin_pad -> X[k][c0 + c]; k >= Lin_pad -> Xs[k - Lin_pad][c0 + c]; staged row
  // of column c: 16 (c % NT) + c / NT
  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < EU; ++u) {
      const int e = tid + 256 * u;
      const int li = e / CT, c = e - li * CT;
      if (li >= a.Lin_pad) continue;
      const int cp = c ^ 1;
      s_bt[(16 * (c % NT) + c / NT) * KSM + li] = xv[u];
      s_bt[(16 * (cp % NT) + cp / NT) * KSM + a.Lin_pad + li] = (c & 1) ? -xv[u] : xv[u];
    }
  };
  load_slab(p0);
  for (int64_t pre = p0; pre < p_end; ++pre) {
    __syncthreads();  // the previous slab's products are done with s_bt
    stage();
    load_slab(min(pre + 1, p_end - 1));  // in flight during the products (the last reloads)
    __syncthreads();
    float* dst = a.out + pre * a.Lout * a.post2;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int mt = wave + 4 * t;
      if (mt >= mtiles) break;
      f32x4 acc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = zero4();
#pragma unroll
      for (int g = 0; g < KMAX / 16; ++g) {
        if (16 * g >= K) break;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float4 bv =
              *reinterpret_cast<const float4*>(s_bt + (16 * nt + m) * KSM + 16 * g + 4 * q);
          acc[nt] = mfma_f32(af[t][g].x, bv.x, acc[nt]);
          acc[nt] = mfma_f32(af[t][g].y, bv.y, acc[nt]);
          acc[nt] = mfma_f32(af[t][g].z, bv.z, acc[nt]);
          acc[nt] = mfma_f32(af[t][g].w, bv.w, acc[nt]);
        }
      }
      // lane (n = m, q): rows 16 mt + 4 q + r, columns c0 + NT m + nt
      const int64_t col = c0 + NT * m;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pr = 16 * mt + 4 * q + r;
        if (pr >= a.Lout) continue;
        float* d = dst + (int64_t)pr * a.post2 + col;
        if (col + NT <= a.post2 && (a.post2 % NT) == 0) {
          if constexpr (NT == 4) {
            *reinterpret_cast<float4*>(d) =
                make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
          } else if constexpr (NT == 2) {
            *reinterpret_cast<float2*>(d) = make_float2(acc[0][r], acc[1][r]);
          } else {
            d[0] = acc[0][r];
          }
        } else {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            if (col + nt < a.post2) d[nt] = acc[nt][r];
        }
      }
    }
  }
}

template <int H>
static hipError_t launch_inv_stream(int ntw, dim3 grid, size_t lds, const OuterArgs& a,
                                    hipStream_t s) {
  switch (ntw) {
    case 1: hipLaunchKernelGGL((k_outer_inv_stream<H, 1>), grid, dim3(256), lds, s, a); break;
    case 2: hipLaunchKernelGGL((k_outer_inv_stream<H, 2>), grid, dim3(256), lds, s, a); break;
    case 3: hipLaunchKernelGGL((k_outer_inv_stream<H, 3>), grid, dim3(256), lds, s, a); break;
    case 4: hipLaunchKernelGGL((k_outer_inv_stream<H, 4>), grid, dim3(256), lds, s, a); break;
    case 5: hipLaunchKernelGGL((k_outer_inv_stream<H, 5>), grid, dim3(256), lds, s, a); break;
    default: hipLaunchKernelGGL((k_outer_inv_stream<H, 6>), grid, dim3(256), lds, s, a); break;
  }
  return hipGetLastError();
}

template <int MT, int NTW>
static hipError_t launch_stream_t(dim3 grid, const OuterArgs& a, int half, hipStream_t s) {
  if (half) {
    if constexpr (NTW <= 6) {
      if (half == 2)
        hipLaunchKernelGGL((k_outer_fwd_stream_bf<2, MT, NTW>), grid, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((k_outer_fwd_stream_bf<1, MT, NTW>), grid, dim3(256), 0, s, a);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    hipLaunchKernelGGL((k_outer_fwd_stream<MT, NTW>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <int MT>
static hipError_t launch_stream_mt(int ntw, dim3 grid, const OuterArgs& a, int bf,
                                   hipStream_t s) {
  switch (ntw) {
    case 1: return launch_stream_t<MT, 1>(grid, a, bf, s);
    case 2: return launch_stream_t<MT, 2>(grid, a, bf, s);
    case 3: return launch_stream_t<MT, 3>(grid, a, bf, s);
    case 4: return launch_stream_t<MT, 4>(grid, a, bf, s);
  }
  if constexpr (MT <= 2) {
    switch (ntw) {
      case 5: return launch_stream_t<MT, 5>(grid, a, bf, s);
      case 6: return launch_stream_t<MT, 6>(grid, a, bf, s);
      case 7: return launch_stream_t<MT, 7>(grid, a, bf, s);
      case 8: return launch_stream_t<MT, 8>(grid, a, bf, s);
    }
  }
  return hipErrorInvalidValue;
}

static hipError_t launch_outer_stream(int mt, int ntw, dim3 grid, const OuterArgs& a, int bf,
                                      hipStream_t s) {
  switch (mt) {
    case 1: return launch_stream_mt<1>(ntw, grid, a, bf, s);
    case 2: return launch_stream_mt<2>(ntw, grid, a, bf, s);
    case 3: return launch_stream_mt<3>(ntw, grid, a, bf, s);
    default: return launch_stream_mt<4>(ntw, grid, a, bf, s);
  }
}

static int pad16(int v) { return (v + 15) / 16 * 16; }

// the inverse from few kept rows streams column blocks of many wide slabs (k_outer_inv_stream)
static bool inv_stream_ok(const OuterArgs& a, int64_t pre) {
  return a.Lin_pad <= 64 && a.post2 % 4 == 0 && a.post2 >= 256 && pre >= 1024 && pre <= 65535;
}

// launch of k_outer_inv_stream for the shape in a (column blocks as wide as the row needs, up
// to 6 N-tiles per wave, narrower while that leaves fewer than ~1024 work-groups)
static hipError_t launch_inv_stream_any(const OuterArgs& a, int64_t pre, int half,
                                        hipStream_t s);

static hipError_t launch_outer_generic(const fno_plan* p, OuterArgs a, int64_t pre,
                                       hipStream_t s);
// work-groups the multi-slab inverse aims for (each walks ceil(slabs / this) slabs)
constexpr int64_t kSlabWgs = 1024;

// pre/post of the transform of axis j (see the generic kernel) and the launch
hipError_t launch_outer_mfma(const fno_plan* p, int axis, int chans, bool inv, const float2* in,
                             float2* out, hipStream_t s) {
  const Geom& g = p->g;
  int64_t pre = (int64_t)g.B * chans;
  for (int i = 0; i < axis; ++i) pre *= g.N[i];
  int64_t post = g.mb;
  for (int i = axis + 1; i <= g.d - 2; ++i) post *= 2 * g.M[i];
  OuterArgs a{};
  const int N = g.N[axis], m2 = 2 * g.M[axis];
  a.Lin = inv ? m2 : N;
  a.Lout = inv ? N : m2;
  a.Lin_pad = pad16(a.Lin);
  a.Lout_pad = pad16(a.Lout);
  a.post2 = 2 * post;
  a.in = reinterpret_cast<const float*>(in);
  a.out = reinterpret_cast<float*>(out);
  const bool bf = g.bf16;
  if (inv) {
    a.A = bf ? (const void*)p->t.oinv_bf[axis] : (const void*)p->t.oinv[axis];
    a.Alo = p->t.oinv_bf_lo[axis];
  } else {
    a.A = bf ? (const void*)p->t.ofwd_bf[axis] : (const void*)p->t.ofwd[axis];
    a.Alo = p->t.ofwd_bf_lo[axis];
  }
  if (inv && inv_stream_ok(a, pre)) {
    // few kept rows in, N rows out, many wide slabs: stage the kept rows of a column block once
    // and walk the output row tiles.  Narrow or few slabs keep the generic kernel, whose waves
    // split the output rows instead.
    return launch_inv_stream_any(a, pre, g.half, s);
  }
  if (inv && !bf && a.Lin_pad <= 32 && a.Lout_pad <= 128 && a.post2 <= 64 && pre >= 4096) {
    // many narrow float32 slabs: work-groups walk several slabs with the table in registers
    const int nt = a.post2 > 32 ? 4 : (a.post2 > 16 ? 2 : 1);
    const int64_t ctiles = (a.post2 + 16 * nt - 1) / (16 * nt);
    const int spw = (int)((pre * ctiles + kSlabWgs - 1) / kSlabWgs);
    const int64_t wgx = (pre + spw - 1) / spw;
    a.pre = pre;
    if (wgx > 0x7fffffff || ctiles > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgx, (unsigned)ctiles);
    if (nt == 4) hipLaunchKernelGGL((k_outer_inv_slabs<4>), grid, dim3(256), 0, s, a, spw);
    else if (nt == 2) hipLaunchKernelGGL((k_outer_inv_slabs<2>), grid, dim3(256), 0, s, a, spw);
    else hipLaunchKernelGGL((k_outer_inv_slabs<1>), grid, dim3(256), 0, s, a, spw);
    return hipGetLastError();
  }
  if (!inv && a.Lout_pad <= 64 && a.post2 % 4 == 0 && pre <= 65535) {
    // few kept rows, long K: stream the slab in column blocks of 64 NTW (as wide as the row
    // needs, narrower while that leaves fewer than ~1024 work-groups)
    const int mt = a.Lout_pad / 16;
    const int ntw_max = mt > 2 ? 4 : (bf ? 6 : 8);
    int ntw = (int)((a.post2 + 63) / 64);
    if (ntw > ntw_max) ntw = ntw_max;
    while (ntw > 1 && pre * ((a.post2 + 64 * ntw - 1) / (64 * ntw)) < 1024) --ntw;
    const int cb = 64 * ntw;
    dim3 grid((unsigned)((a.post2 + cb - 1) / cb), (unsigned)pre);
    return launch_outer_stream(mt, ntw, grid, a, g.half, s);
  }
  return launch_outer_generic(p, a, pre, s);
}

static hipError_t launch_inv_stream_any(const OuterArgs& a, int64_t pre, int half,
                                        hipStream_t s) {
  int ntw = (int)((a.post2 + 63) / 64);
  if (ntw > 6) ntw = 6;
  while (ntw > 1 && pre * ((a.post2 + 64 * ntw - 1) / (64 * ntw)) < 1024) --ntw;
  while (ntw > 1 && sizeof(float) * (size_t)a.Lin_pad * (64 * ntw + 4) > 65536) --ntw;
  const int cb = 64 * ntw;
  const size_t lds = sizeof(float) * (size_t)a.Lin_pad * (cb + 4);
  dim3 grid((unsigned)((a.post2 + cb - 1) / cb), (unsigned)pre);
  return half == 2 ? launch_inv_stream<2>(ntw, grid, lds, a, s)
         : half == 1 ? launch_inv_stream<1>(ntw, grid, lds, a, s)
                     : launch_inv_stream<0>(ntw, grid, lds, a, s);
}

// k_outer_mfma for the arguments of launch_outer_mfma: column tiles of 64, 32 or 16, and the
// output rows of few slabs split over up to msplit work-groups
static hipError_t launch_outer_generic(const fno_plan* p, OuterArgs a, int64_t pre,
                                       hipStream_t s) {
  const Geom& g = p->g;
  const bool bf = g.bf16;
  const int KS = 2 * a.Lin_pad + (bf ? 8 : 4);
  const size_t col_bytes = (size_t)KS * (bf ? 2 : 4);
  int nt = a.post2 >= 64 ? 4 : (a.post2 >= 32 ? 2 : 1);
  while (nt > 1 && (size_t)16 * nt * col_bytes > 64 * 1024) nt /= 2;
  if (a.outh && nt != 4) return hipErrorInvalidValue;  // the half output needs 4-column lanes
  const int ct = 16 * nt;
  const size_t lds = (size_t)ct * col_bytes;
  const int64_t ctiles = (a.post2 + ct - 1) / ct;
  // few slabs: split each slab's output row tiles over up to msplit work-groups (at least
  // four tiles, one per wave, each) until about 1024 work-groups are in flight
  const int mtiles = a.Lout_pad / 16;
  a.pre = pre;
  a.msplit = 1;
  while (2 * a.msplit * 4 <= mtiles && pre * ctiles * a.msplit < 1024) a.msplit *= 2;
  a.mt_per = (mtiles + a.msplit - 1) / a.msplit;
  const int64_t gx = a.msplit == 1 ? pre : (pre + 7) / 8 * 8 * a.msplit;
  if (gx > 0x7fffffff || ctiles > 65535) return hipErrorInvalidValue;
  dim3 grid((unsigned)gx, (unsigned)ctiles);
  if (g.half == 2) {
    if (nt == 4) hipLaunchKernelGGL((k_outer_mfma<2, 4>), grid, dim3(256), lds, s, a);
    else if (nt == 2) hipLaunchKernelGGL((k_outer_mfma<2, 2>), grid, dim3(256), lds, s, a);
    else hipLaunchKernelGGL((k_outer_mfma<2, 1>), grid, dim3(256), lds, s, a);
  } else if (bf) {
    if (nt == 4) hipLaunchKernelGGL((k_outer_mfma<1, 4>), grid, dim3(256), lds, s, a);
    else if (nt == 2) hipLaunchKernelGGL((k_outer_mfma<1, 2>), grid, dim3(256), lds, s, a);
    else hipLaunchKernelGGL((k_outer_mfma<1, 1>), grid, dim3(256), lds, s, a);
  } else {
    if (nt == 4) hipLaunchKernelGGL((k_outer_mfma<0, 4>), grid, dim3(256), lds, s, a);
    else if (nt == 2) hipLaunchKernelGGL((k_outer_mfma<0, 2>), grid, dim3(256), lds, s, a);
    else hipLaunchKernelGGL((k_outer_mfma<0, 1>), grid, dim3(256), lds, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_outer_mfma_half(const fno_plan* p, int axis, int chans, const float2* in,
                                  uint16_t* out, hipStream_t s) {
  const Geom& g = p->g;
  if (!g.bf16) return hipErrorInvalidValue;
  int64_t pre = (int64_t)g.B * chans;
  for (int i = 0; i < axis; ++i) pre *= g.N[i];
  int64_t post = g.mb;
  for (int i = axis + 1; i <= g.d - 2; ++i) post *= 2 * g.M[i];
  OuterArgs a{};
  const int N = g.N[axis], m2 = 2 * g.M[axis];
  a.Lin = m2;
  a.Lout = N;
  a.Lin_pad = pad16(a.Lin);
  a.Lout_pad = pad16(a.Lout);
  a.post2 = 2 * post;
  a.in = reinterpret_cast<const float*>(in);
  a.out = nullptr;
  a.outh = out;
  a.A = (const void*)p->t.oinv_bf[axis];
  a.Alo = p->t.oinv_bf_lo[axis];
  if (inv_stream_ok(a, pre)) return launch_inv_stream_any(a, pre, g.half, s);
  if (a.post2 < 64) return hipErrorInvalidValue;
  return launch_outer_generic(p, a, pre, s);
}

bool outer_inv_half_ok(const fno_plan* p, int axis) {
  const Geom& g = p->g;
  if (!g.bf16 || !outer_fast_ok(p, axis, true)) return false;
  int64_t pre = (int64_t)g.B * g.Cout;
  for (int i = 0; i < axis; ++i) pre *= g.N[i];
  int64_t post = g.mb;
  for (int i = axis + 1; i <= g.d - 2; ++i) post *= 2 * g.M[i];
  OuterArgs a{};
  a.Lin = 2 * g.M[axis];
  a.Lin_pad = pad16(a.Lin);
  a.post2 = 2 * post;
  return inv_stream_ok(a, pre);
}

bool outer_fast_ok(const fno_plan* p, int axis, bool inv) {
  const Geom& g = p->g;
  const int N = g.N[axis], m2 = 2 * g.M[axis];
  const int lin = pad16(inv ? m2 : N);
  // one 16-column tile of the staged input must fit the LDS budget
  if ((size_t)16 * (2 * lin + 8) * 4 > 64 * 1024) return false;
  int64_t post = g.mb;
  for (int i = axis + 1; i <= g.d - 2; ++i) post *= 2 * g.M[i];
  return (2 * post + 15) / 16 <= 65535;
}

}  // namespace fno
