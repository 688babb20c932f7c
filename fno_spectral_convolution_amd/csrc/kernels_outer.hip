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

struct OuterArgs {
  int Lin, Lout, Lin_pad, Lout_pad;
  int64_t post2;         // floats per row (2 * post)
  const float* in;       // [pre][Lin][post2]
  float* out;            // [pre][Lout][post2]
  const void* A;         // [Lout_pad][2 Lin_pad] f32, or bf16 bits (hi)
  const uint16_t* Alo;   // bf16 residual (bf16 path)
};

template <bool BF, int NT>
__global__ void __launch_bounds__(256) k_outer_mfma(OuterArgs a) {
  constexpr int CT = 16 * NT;  // columns per work-group
  extern __shared__ __attribute__((aligned(16))) unsigned char s_raw[];
  const int K = 2 * a.Lin_pad;
  const int KS = K + (BF ? 8 : 4);  // row stride of Bt (elements)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  const int64_t pre = blockIdx.x;
  const int64_t c0 = (int64_t)blockIdx.y * CT;
  const float* src = a.in + pre * a.Lin * a.post2;
  // Bt[c][k]: k < Lin_pad -> X[k][c0 + c]; k >= Lin_pad -> Xs[k - Lin_pad][c0 + c]
  // staged row of column c (local): 16 (c % NT) + c / NT
  auto brow = [](int c) { return 16 * (c % NT) + c / NT; };
  for (int e = tid; e < a.Lin_pad * CT; e += 256) {
    const int li = e / CT, c = e - li * CT;
    const int64_t col = c0 + c;
    float v = 0.f;
    if (li < a.Lin && col < a.post2) v = src[(int64_t)li * a.post2 + col];
    const int cp = c ^ 1;
    const float vs = (c & 1) ? -v : v;  // Xs[li][c^1]
    if (BF) {
      uint16_t* bt = reinterpret_cast<uint16_t*>(s_raw);
      bt[brow(c) * KS + li] = bf16_bits(v);
      bt[brow(cp) * KS + a.Lin_pad + li] = bf16_bits(vs);
    } else {
      float* bt = reinterpret_cast<float*>(s_raw);
      bt[brow(c) * KS + li] = v;
      bt[brow(cp) * KS + a.Lin_pad + li] = vs;
    }
  }
  __syncthreads();
  float* dst = a.out + pre * a.Lout * a.post2;
  for (int mt = wave; mt < a.Lout_pad / 16; mt += 4) {
    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = zero4();
    const int prow = 16 * mt + m;
    if (BF) {
      const uint16_t* A = static_cast<const uint16_t*>(a.A) + (int64_t)prow * K;
      const uint16_t* Al = a.Alo + (int64_t)prow * K;
      const uint16_t* bt = reinterpret_cast<const uint16_t*>(s_raw);
      for (int k0 = 0; k0 < K; k0 += 32) {
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(A + k0 + 8 * q);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(Al + k0 + 8 * q);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const bf16x8 bv = *reinterpret_cast<const bf16x8*>(bt + (16 * nt + m) * KS + k0 + 8 * q);
          acc[nt] = mfma_bf16(ah, bv, acc[nt]);
          acc[nt] = mfma_bf16(al, bv, acc[nt]);
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

static int pad16(int v) { return (v + 15) / 16 * 16; }

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
  const int KS = 2 * a.Lin_pad + (bf ? 8 : 4);
  const size_t col_bytes = (size_t)KS * (bf ? 2 : 4);
  int nt = a.post2 >= 64 ? 4 : (a.post2 >= 32 ? 2 : 1);
  while (nt > 1 && (size_t)16 * nt * col_bytes > 64 * 1024) nt /= 2;
  const int ct = 16 * nt;
  const size_t lds = (size_t)ct * col_bytes;
  dim3 grid((unsigned)pre, (unsigned)((a.post2 + ct - 1) / ct));
  if (bf) {
    if (nt == 4) hipLaunchKernelGGL((k_outer_mfma<true, 4>), grid, dim3(256), lds, s, a);
    else if (nt == 2) hipLaunchKernelGGL((k_outer_mfma<true, 2>), grid, dim3(256), lds, s, a);
    else hipLaunchKernelGGL((k_outer_mfma<true, 1>), grid, dim3(256), lds, s, a);
  } else {
    if (nt == 4) hipLaunchKernelGGL((k_outer_mfma<false, 4>), grid, dim3(256), lds, s, a);
    else if (nt == 2) hipLaunchKernelGGL((k_outer_mfma<false, 2>), grid, dim3(256), lds, s, a);
    else hipLaunchKernelGGL((k_outer_mfma<false, 1>), grid, dim3(256), lds, s, a);
  }
  return hipGetLastError();
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
