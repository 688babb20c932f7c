// Forward transform of [Na][Nb] planes whose contiguous axis is short (Nb <= 32, e.g. the
// 20-point time axis of a space-time field): the truncated real DFT of the contiguous axis
// followed by the truncated DFT of the row axis, for the retained modes only (the FNO spectral
// transform from its linear-algebra form -- model-parallel FNO page, "Proposed method"):
//   R[row][j]  = sum_c x'[row][c] T1[c][j]               (j < 16 NTJ: cos / -sin columns)
//   X2[i][j]   = sum_row F2[i][row] R[row][j]            (F2: cos rows, then sin rows)
//   X[s][k]    = (X2[s][2k] + X2[2ma+s][2k+1]) + i (X2[s][2k+1] - X2[2ma+s][2k])
//
// One wave owns one plane at a time (no barriers between waves) and walks planes with a
// stride of the whole grid, loading the next plane while it computes the current one.
//   first product : M = rows (16 MT), K = 32 (columns c = 8 q + slot, masked past Nb), one
//                   16x16x32 bf16 MFMA per tile (mixed path) or 8 16x16x4 f32 MFMAs; each
//                   lane loads its own A operand, two float4 of its row, straight from HBM.
//   second product: 16x16x4 f32 MFMAs whose K order is chosen so that K-step s, k-slot q is
//                   row 16 (s / 4) + 4 q + s % 4: exactly the first product's D fragment held
//                   by the same lane, so R never leaves the registers.  F2 sits in LDS.  On the
//                   mixed path: 16x16x32 bf16 MFMAs taking two row tiles' fragments per K-step,
//                   F2 as its bf16 hi + lo pair (two products).
//   combine       : X2 goes to a per-wave LDS tile and is folded into the complex spectrum.
// On the half paths the pre-activated input, T1 and R are rounded to bfloat16 or IEEE half
// (the half-precision transform of the mixed-precision neural-operator page, "Tiivistelmä").
#include "fno_internal.h"
#include "mfma.h"
#include "pointwise.h"
#include "split6.h"

namespace fno {

struct SmallPlaneArgs {
  int Na, Nb, ma, mb;
  int64_t planes;
  const float* in0;
  const float* in1;
  const float* t1;       // [Nb][jpad] f32
  const uint16_t* t1bf;  // [Nb][jpad] half bits (the plan's format)
  const float* f2;       // [4 ma][Na] f32
  const uint16_t* f2bf;  // [4 ma][Na] half bits of f2, and of its residual
  const uint16_t* f2lo;
  float2* out;           // [planes][2 ma][mb]
};

template <int PIN>
__device__ __forceinline__ float small_prologue(float v, float w) {
  if (PIN == PLANE_TANH) return tanh_fast(v);
  if (PIN == PLANE_GELU_GRAD) return v * gelu_grad_as(w);
  if (PIN == PLANE_GELU) return gelu_as(v);
  if (PIN == PLANE_TANH_GELU) return tanh_gelu(v);
  return v;
}

// MT = Na / 16 row tiles, NTJ = jpad / 16 column tiles.  E6 (float32 plans): both products
// as six bfloat16 products of three-way split operands (split6.h), float32 to its rounding.
template <int PIN, int H, int MT, int NTJ, bool E6 = false>
__global__ void __launch_bounds__(256) k_plane_small(SmallPlaneArgs a) {
  static_assert(!E6 || H == 0, "the split products stand in for float32 ones");
  constexpr bool BF = H != 0;  // half operands (bfloat16 or IEEE half)
  using HT = HalfOf<H>;
  using V8 = typename HT::v8;
  using E = typename HT::elem;
  constexpr int JP = 16 * NTJ;
  constexpr bool TWO = PIN == PLANE_GELU_GRAD;
  extern __shared__ __attribute__((aligned(16))) float s_sp[];
  const int Na = 16 * MT;
  const int F2S = Na + 4;                    // F2 row stride (floats; f32 path)
  const int F2H = Na + 8;                    // F2 row stride (16-bit elements; half and E6)
  const int ROWS2 = 4 * a.ma;                // F2 rows
  const int MT2 = ROWS2 / 16;                // F2 row tiles (ma % 4 == 0)
  // F2 in LDS: f32 [4 ma][F2S]; the half pair hi [4 ma][F2H], lo [4 ma][F2H]; or (E6) the
  // bfloat16 split terms hi, mid, lo, each [4 ma][F2H]
  float* s_f2 = s_sp;
  uint16_t* s_f2h = reinterpret_cast<uint16_t*>(s_sp);
  uint16_t* s_f2l = s_f2h + ROWS2 * F2H;
  uint16_t* s_f2m = s_f2l + ROWS2 * F2H;     // E6: the middle term (after hi and lo)
  const int f2_floats = E6 ? (3 * ROWS2 * F2H + 3) / 4 * 2
                           : (BF ? ROWS2 * F2H : ROWS2 * F2S);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  float* s_w = s_sp + f2_floats + wave * (ROWS2 * JP);  // this wave's X2 tile [4 ma][JP]
  for (int e = tid; e < ROWS2 * Na; e += 256) {
    const int i = e / Na, r = e - i * Na;
    if constexpr (E6) {
      __bf16 h, mi, lo;
      split3(a.f2[e], h, mi, lo);
      s_f2h[i * F2H + r] = __builtin_bit_cast(uint16_t, h);
      s_f2m[i * F2H + r] = __builtin_bit_cast(uint16_t, mi);
      s_f2l[i * F2H + r] = __builtin_bit_cast(uint16_t, lo);
    } else if (BF) {
      s_f2h[i * F2H + r] = a.f2bf[e];
      s_f2l[i * F2H + r] = a.f2lo[e];
    } else {
      s_f2[i * F2S + r] = a.f2[e];
    }
  }
  // T1 fragments: B[k = 8 q + slot][n = 16 nt + m]; zero past Nb
  float t1r[NTJ][8];
  V8 t1b[NTJ];
  bf16x8 t1h[E6 ? NTJ : 1], t1m[E6 ? NTJ : 1], t1l[E6 ? NTJ : 1];
#pragma unroll
  for (int nt = 0; nt < NTJ; ++nt) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = 8 * q + s;
      const int cc = min(c, a.Nb - 1);
      const float v = BF ? HT::value(a.t1bf[cc * JP + 16 * nt + m])
                         : a.t1[cc * JP + 16 * nt + m];
      t1r[nt][s] = c < a.Nb ? v : 0.f;
      t1b[nt][s] = (E)t1r[nt][s];  // exact: t1r holds a half value (or zero)
    }
    if constexpr (E6) split3_bf16x8(t1r[nt], t1h[nt], t1m[nt], t1l[nt]);
  }
  __syncthreads();
  const int64_t gw = (int64_t)blockIdx.x * 4 + wave;
  const int64_t nw = (int64_t)gridDim.x * 4;
  // this lane's row of tile t is 16 t + m; its columns 8 q .. 8 q + 7 (two float4; columns
  // past Nb are read from a clamped address and masked; Nb % 4 == 0 keeps float4 alignment)
  const int c0 = min(8 * q, a.Nb - 4), c1 = min(8 * q + 4, a.Nb - 4);
  const bool live0 = 8 * q < a.Nb, live1 = 8 * q + 4 < a.Nb;
  float4 p0[MT][2], p1[TWO ? MT : 1][2];
  auto load_plane = [&](int64_t pl) {
    const float* b0 = a.in0 + pl * (int64_t)Na * a.Nb;
    const float* b1 = TWO ? a.in1 + pl * (int64_t)Na * a.Nb : b0;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int ro = (16 * t + m) * a.Nb;
      p0[t][0] = load_stream4(b0 + ro + c0);
      p0[t][1] = load_stream4(b0 + ro + c1);
      if constexpr (TWO) {
        p1[t][0] = load_stream4(b1 + ro + c0);
        p1[t][1] = load_stream4(b1 + ro + c1);
      }
    }
  };
  int64_t pl = min(gw, a.planes - 1);
  load_plane(pl);
  for (int64_t it = gw; it < a.planes; it += nw) {
    // first product, tile by tile straight from the load registers: operands pre-activated
    // and masked; R tiles (t, nt), lane (m, q) register r = R[16 t + 4 q + r][16 nt + m]
    f32x4 d[MT][NTJ];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const float4 u0 = p0[t][0], u1 = p0[t][1];
      const float4 w0 = TWO ? p1[t][0] : u0, w1 = TWO ? p1[t][1] : u1;
      const float raw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
      const float rw[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      float xv[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bool live = s < 4 ? live0 : live1;
        float v = small_prologue<PIN>(raw[s], rw[s]);
        if (BF) v = round_half<H>(v);
        xv[s] = __uint_as_float(__float_as_uint(v) & (live ? 0xffffffffu : 0u));
      }
      bf16x8 xh, xm, xl;
      if constexpr (E6) split3_bf16x8(xv, xh, xm, xl);
#pragma unroll
      for (int nt = 0; nt < NTJ; ++nt) {
        f32x4 acc = zero4();
        if constexpr (E6) {
          acc = mfma_split6(xh, xm, xl, t1h[nt], t1m[nt], t1l[nt], acc);
        } else if constexpr (BF) {
          V8 av;
#pragma unroll
          for (int s = 0; s < 8; ++s) av[s] = (E)xv[s];  // exact: already rounded
          acc = HT::mfma(av, t1b[nt], acc);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] = round_half<H>(acc[r]);
        } else {
#pragma unroll
          for (int s = 0; s < 8; ++s) acc = mfma_f32(xv[s], t1r[nt][s], acc);
        }
        d[t][nt] = acc;
      }
    }
    // the next plane's rows go out now, in flight during the second product and the combine
    const int64_t nxt = min(it + nw, a.planes - 1);
    load_plane(nxt);
    for (int mt2 = 0; mt2 < MT2; ++mt2) {
      f32x4 x2[NTJ];
#pragma unroll
      for (int nt = 0; nt < NTJ; ++nt) x2[nt] = zero4();
      if constexpr (E6) {
        // second product as the half path orders it (K-step p, slot (q, e) <-> row
        // 16 (2 p + e / 4) + 4 q + e % 4), on the split terms of F2 and of R
        const uint16_t* fh = s_f2h + (16 * mt2 + m) * F2H + 4 * q;
        const uint16_t* fm = s_f2m + (16 * mt2 + m) * F2H + 4 * q;
        const uint16_t* fl = s_f2l + (16 * mt2 + m) * F2H + 4 * q;
        auto frag = [&](const uint16_t* f, int pp) {
          const uint2 v0 = *reinterpret_cast<const uint2*>(f + 32 * pp);
          uint2 v1 = make_uint2(0u, 0u);
          if (2 * pp + 1 < MT) v1 = *reinterpret_cast<const uint2*>(f + 32 * pp + 16);
          return __builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
        };
#pragma unroll
        for (int pp = 0; pp < (MT + 1) / 2; ++pp) {
          const int t0 = 2 * pp, t1 = min(2 * pp + 1, MT - 1);
          const bf16x8 ah = frag(fh, pp), am = frag(fm, pp), al = frag(fl, pp);
#pragma unroll
          for (int nt = 0; nt < NTJ; ++nt) {
            const bool two = 2 * pp + 1 < MT;  // compile-time after unrolling
            const float bvals[8] = {d[t0][nt][0], d[t0][nt][1], d[t0][nt][2], d[t0][nt][3],
                                    two ? d[t1][nt][0] : 0.f, two ? d[t1][nt][1] : 0.f,
                                    two ? d[t1][nt][2] : 0.f, two ? d[t1][nt][3] : 0.f};
            bf16x8 bh, bm, bl;
            split3_bf16x8(bvals, bh, bm, bl);
            x2[nt] = mfma_split6(ah, am, al, bh, bm, bl, x2[nt]);
          }
        }
      } else if constexpr (!BF) {
        // second product: K-step 4 t + r, k-slot q <-> row 16 t + 4 q + r
        const float* fr = s_f2 + (16 * mt2 + m) * F2S + 4 * q;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const float4 f = *reinterpret_cast<const float4*>(fr + 16 * t);
#pragma unroll
          for (int nt = 0; nt < NTJ; ++nt) {
            x2[nt] = mfma_f32(f.x, d[t][nt][0], x2[nt]);
            x2[nt] = mfma_f32(f.y, d[t][nt][1], x2[nt]);
            x2[nt] = mfma_f32(f.z, d[t][nt][2], x2[nt]);
            x2[nt] = mfma_f32(f.w, d[t][nt][3], x2[nt]);
          }
        }
      } else {
        // second product on bf16 MFMAs (R is already rounded to bf16; F2 as its hi + lo
        // pair): K-step p, slot (q, e) <-> row 16 (2 p + e / 4) + 4 q + e % 4, so the B
        // operand is this lane's fragments of row tiles 2 p and 2 p + 1
        const uint16_t* fh = s_f2h + (16 * mt2 + m) * F2H + 4 * q;
        const uint16_t* fl = s_f2l + (16 * mt2 + m) * F2H + 4 * q;
#pragma unroll
        for (int pp = 0; pp < (MT + 1) / 2; ++pp) {
          const int t0 = 2 * pp, t1 = min(2 * pp + 1, MT - 1);
          const uint2 h0 = *reinterpret_cast<const uint2*>(fh + 32 * pp);
          const uint2 l0 = *reinterpret_cast<const uint2*>(fl + 32 * pp);
          uint2 h1 = make_uint2(0u, 0u), l1 = make_uint2(0u, 0u);
          if (2 * pp + 1 < MT) {  // compile-time after unrolling
            h1 = *reinterpret_cast<const uint2*>(fh + 32 * pp + 16);
            l1 = *reinterpret_cast<const uint2*>(fl + 32 * pp + 16);
          }
          const V8 ah = __builtin_bit_cast(V8, make_uint4(h0.x, h0.y, h1.x, h1.y));
          const V8 al = __builtin_bit_cast(V8, make_uint4(l0.x, l0.y, l1.x, l1.y));
#pragma unroll
          for (int nt = 0; nt < NTJ; ++nt) {
            const uint32_t b0 = HT::pack2(d[t0][nt][0], d[t0][nt][1]);
            const uint32_t b1 = HT::pack2(d[t0][nt][2], d[t0][nt][3]);
            const uint32_t b2 = 2 * pp + 1 < MT ? HT::pack2(d[t1][nt][0], d[t1][nt][1]) : 0u;
            const uint32_t b3 = 2 * pp + 1 < MT ? HT::pack2(d[t1][nt][2], d[t1][nt][3]) : 0u;
            const V8 bv = __builtin_bit_cast(V8, make_uint4(b0, b1, b2, b3));
            x2[nt] = HT::mfma(ah, bv, x2[nt]);
            x2[nt] = HT::mfma(al, bv, x2[nt]);
          }
        }
      }
#pragma unroll
      for (int nt = 0; nt < NTJ; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_w[(16 * mt2 + 4 * q + r) * JP + 16 * nt + m] = x2[nt][r];
    }
    // combine into the complex spectrum [2 ma][mb] (same wave: LDS ops complete in order)
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's X2 writes are done
    __builtin_amdgcn_wave_barrier();
    float2* dst = a.out + it * (int64_t)(2 * a.ma * a.mb);
    for (int e = lane; e < 2 * a.ma * a.mb; e += 64) {
      const int s = e / a.mb, k = e - s * a.mb;
      const float* c = s_w + s * JP + 2 * k;
      const float* sn = s_w + (2 * a.ma + s) * JP + 2 * k;
      dst[e] = make_float2(c[0] + sn[1], c[1] - sn[0]);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // reads of s_w done before the next plane rewrites it
    __builtin_amdgcn_wave_barrier();
  }
}

// The small-plane transform applies when the contiguous axis is short and the row axis fits
// the register-resident first product.
bool plane_small_ok(const fno_plan* p) {
  const Geom& g = p->g;
  if (g.Nb > 32 || g.Nb % 4 != 0) return false;
  if (!(g.Na == 16 || g.Na == 32 || g.Na == 64 || g.Na == 128)) return false;
  if (!(p->jpad == 16 || p->jpad == 32)) return false;
  if (g.ma % 4 != 0 || 4 * g.ma > 128) return false;
  return true;
}

template <int PIN, int H, int MT>
static void launch_small_t(const fno_plan* p, const SmallPlaneArgs& a, hipStream_t s) {
  const int jp = p->jpad;
  const int rows2 = 4 * a.ma;
  const int64_t want = (a.planes + 3) / 4;
  const unsigned grid = (unsigned)(want < 2048 ? want : 2048);
  const size_t xw = 4 * (size_t)rows2 * jp;  // the waves' X2 tiles (floats)
  // wide row spectra need more than the default dynamic LDS limit
  auto lds_limit = [](const void* k, size_t bytes) {
    if (bytes > 65536)
      (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  };
  if (jp == 16) {
    // float32 plans with one column tile: the split bfloat16 products (with two tiles, or
    // the gradient prologue's second field, the split operands would cost the kernel half
    // its occupancy)
    constexpr bool E6 = H == 0 && PIN != PLANE_GELU_GRAD;
    const size_t f2 = E6 ? (size_t)(3 * rows2 * (a.Na + 8) + 3) / 4 * 2
                         : (size_t)rows2 * (a.Na + (H != 0 ? 8 : 4));
    const size_t lds = sizeof(float) * (f2 + xw);
    lds_limit(reinterpret_cast<const void*>(k_plane_small<PIN, H, MT, 1, E6>), lds);
    hipLaunchKernelGGL((k_plane_small<PIN, H, MT, 1, E6>), dim3(grid), dim3(256), lds, s, a);
  } else {
    const size_t lds = sizeof(float) * ((size_t)rows2 * (a.Na + (H != 0 ? 8 : 4)) + xw);
    lds_limit(reinterpret_cast<const void*>(k_plane_small<PIN, H, MT, 2, false>), lds);
    hipLaunchKernelGGL((k_plane_small<PIN, H, MT, 2, false>), dim3(grid), dim3(256), lds, s, a);
  }
}

template <int PIN, int H>
static void launch_small_mt(const fno_plan* p, const SmallPlaneArgs& a, hipStream_t s) {
  switch (a.Na) {
    case 16: launch_small_t<PIN, H, 1>(p, a, s); break;
    case 32: launch_small_t<PIN, H, 2>(p, a, s); break;
    case 64: launch_small_t<PIN, H, 4>(p, a, s); break;
    default: launch_small_t<PIN, H, 8>(p, a, s); break;
  }
}

template <int PIN>
static void launch_small_pin(const fno_plan* p, const SmallPlaneArgs& a, hipStream_t s) {
  if (p->g.half == 2)
    launch_small_mt<PIN, 2>(p, a, s);
  else if (p->g.half == 1)
    launch_small_mt<PIN, 1>(p, a, s);
  else
    launch_small_mt<PIN, 0>(p, a, s);
}

hipError_t launch_plane_small(const fno_plan* p, int plane_in, int chans, const float* in0,
                              const float* in1, float2* out, hipStream_t s) {
  const Geom& g = p->g;
  SmallPlaneArgs a{};
  a.Na = g.Na;
  a.Nb = g.Nb;
  a.ma = g.ma;
  a.mb = g.mb;
  a.planes = (int64_t)g.B * chans * g.O;
  a.in0 = in0;
  a.in1 = in1;
  a.t1 = p->t.t1;
  a.t1bf = p->t.t1_bf;
  a.f2 = p->t.f2;
  a.f2bf = p->t.f2_bf;
  a.f2lo = p->t.f2_bf_lo;
  a.out = out;
  switch (plane_in) {
    case PLANE_X: launch_small_pin<PLANE_X>(p, a, s); break;
    case PLANE_TANH: launch_small_pin<PLANE_TANH>(p, a, s); break;
    case PLANE_GELU: launch_small_pin<PLANE_GELU>(p, a, s); break;
    case PLANE_TANH_GELU: launch_small_pin<PLANE_TANH_GELU>(p, a, s); break;
    default: launch_small_pin<PLANE_GELU_GRAD>(p, a, s); break;
  }
  return hipGetLastError();
}

}  // namespace fno
