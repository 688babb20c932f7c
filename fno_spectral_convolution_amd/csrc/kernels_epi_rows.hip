// Forward epilogue for fields whose contiguous axis is short (Nb <= 32, e.g. the 20-step time
// axis of a space-time field), fused with the zero-padded inverse of the row axis a:
//   U[row][k]    = sum_s T[s][k] e^{+2 pi i ka(s) row / Na}          (retained rows s < 2 ma)
//   y_spec[row][c] = sum_k g(k)/Ntot Re(U[row][k] e^{+2 pi i k c / Nb})
//   z = y_spec + Wb x + bias,  y = GELU(z)
// (the inverse half of the FNO spectral transform and its pointwise bypass: model-parallel FNO
// page, "Proposed method"; the half-precision variants (bfloat16 or IEEE half operands) of the
// mixed-precision neural-operator page, "Tiivistelmä").  T = [B][Cout][O][2 ma][mb] is the spectrum after the inverse of the
// outer axes only, so the full-size last-axis spectrum [B][Cout][O][Na][mb] never exists.
//
// A work-group owns one outer position o of one batch entry (all channels, all Na rows) and
// walks the rows in chunks of 16.  Per output channel the two inverse products chain in
// registers on the matrix cores:
//   first : U^T[k'][row] = sum_s' B'[s'][k'] A[row][s']        (k' = 2 k + re/im, s' = cos|sin
//           block + s; B' is T with the signs of the complex product folded in)
//   second: y[row][c]    = sum_k' U[row][k'] G[k'][c]           (G: the last-axis table)
// The second product takes the first's result fragment as its A operand by ordering its K so
// that K-step r, k-slot q is k' = 4 q + r.  The bypass runs on the matrix cores from the x
// chunk staged in LDS; the chunk of every channel leaves through LDS as float4 row stores.
#include "fno_internal.h"
#include "mfma.h"
#include "pointwise.h"

namespace fno {

constexpr int kErRows = 16;  // rows of axis a per chunk
constexpr int kErMA = 12;    // max modes per corner on axis a (f32 K-steps of the first product)
constexpr int kErCPW = 5;    // output channels per wave (Cout <= 20)
constexpr int kErKB = 5;     // bypass K-steps (Cin <= 20)
constexpr int kErXPT = 7;    // float4 of a chunk per thread (C * Nb <= 448)
static_assert(kErXPT == 7, "the store pass reads seven float4 per thread in one statement");
constexpr int kErRS = 36;    // s_y row stride: 32 columns + 4 (rows 4 q + r on distinct banks)
constexpr int kErYC = kErRows * kErRS;  // s_y channel stride

struct RowsEpiArgs {
  int Na, Nb, ma, mb, Cin, Cout;
  int SO, KA;      // row-axis table: offset of the sin block, row stride (elements)
  int kpad;        // last-axis table row stride
  int O;
  int gelu;
  const float2* T;          // [B][Cout][O][2 ma][mb]
  const uint16_t* Th;       // the same in the plan's half format (re, im pairs), or null
  const float* x;           // [B][Cin][O][Na][Nb]
  const float* wb;          // [Cout][Cin]
  const float* bias;        // [Cout] or null
  float* y;                 // [B][Cout][O][Na][Nb]
  float* zsave;             // [B][Cout][O][Na][Nb] or null
  const float* ainv;        // [Na][KA]: (cos | sin)(2 pi ka(s) row / Na), zero padded
  const uint16_t* ainv_bf;  // bfloat16 of ainv, and of its residual
  const uint16_t* ainv_lo;
  const float* gt;          // [Nb][kpad]: g(k)/Ntot (cos, -sin)(2 pi k c / Nb)
  const uint16_t* gt_bf;
  int* flag;                // IEEE-half plans: set to 1 when a non-finite output is written
};

// float4 e of a chunk -> (channel, float4 within the channel's 4 Nb); exact float division
// for these small integers
__device__ __forceinline__ int2 chunk_split(int e, float inv4nb, int nb4) {
  const int ch = (int)(((float)e + 0.5f) * inv4nb);
  return make_int2(ch, e - ch * nb4);
}

__device__ __forceinline__ float keep_if(float v, bool keep) {
  return __uint_as_float(__float_as_uint(v) & (keep ? 0xffffffffu : 0u));
}

// gfx950 direct global -> LDS copy of 16 bytes per lane: lane l's data lands at
// lds_wave_base + 16 l (lds_wave_base must be uniform over the wave)
__device__ __forceinline__ void copy16_to_lds(const float* src, float* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(
      (const void*)src, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

constexpr int kWaitVm0 = 0x0F70;   // s_waitcnt vmcnt(0)
// s_waitcnt vmcnt(n) for n < 16 (expcnt and lgkmcnt left free)
constexpr int wait_vm(int n) { return 0x0F70 | (n & 15); }

__device__ __forceinline__ uint32_t lds_addr(const float* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) float*)p;
}

// Seven float4 reads of s_y for the store pass, waited for inside the same statement.  Written
// out because the compiler, unable to tell s_y from the region the next chunk's x is being
// copied into, would otherwise wait for those copies before any LDS read.
__device__ __forceinline__ void lds_read7_f4(const uint32_t (&ad)[7], float4 (&v)[7]) {
  asm volatile(
      "ds_read_b128 %0, %7\n\t"
      "ds_read_b128 %1, %8\n\t"
      "ds_read_b128 %2, %9\n\t"
      "ds_read_b128 %3, %10\n\t"
      "ds_read_b128 %4, %11\n\t"
      "ds_read_b128 %5, %12\n\t"
      "ds_read_b128 %6, %13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
        "=&v"(v[6])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6])
      : "memory");
}
constexpr int kWaitLgkm0 = 0xC07F; // s_waitcnt lgkmcnt(0)

// Work-group barrier that orders LDS accesses only: unlike __syncthreads() it does not wait for
// global loads still in flight (the next chunk's copies into another LDS region).  The signal
// fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// MODE 0: y = y_spec;  1: y = act(y_spec + Wb x + bias);  2: the same and z saved.
// G: act is GELU (else the identity).  A compile-time choice: a run-time branch in the store
// pass splits its stores over two paths, and the compiler then waits for some of them to be
// acknowledged before the next chunk's products.
template <int H, int MODE, bool G>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
k_epi_rows(RowsEpiArgs a) {
  constexpr bool BF = H != 0;  // half operands (bfloat16 or IEEE half)
  using HT = HalfOf<H>;
  using V8 = typename HT::v8;
  using E = typename HT::elem;
  constexpr bool BLK = MODE >= 1;
  extern __shared__ __attribute__((aligned(16))) float s_er[];
  const int Nb = a.Nb;
  const int RP = kErRows * Nb;  // points of one channel in a chunk
  // s_y: [Cout + 1][16 rows][kErRS] (channel Cout takes the writes of absent channels, columns
  // Nb .. 31 those of absent columns); s_x: the x chunk, dense [channel][RP] (block modes)
  float* s_y = s_er;
  float* s_x = s_y + (a.Cout + 1) * kErYC;
  bool bad = false;  // IEEE-half plans: a non-finite output was written
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 15, q = lane >> 4;
  const int o = blockIdx.x, b = blockIdx.y;
  const int64_t plane = (int64_t)a.Na * Nb;
  const int nchunk = a.Na / kErRows;
  const int chs = a.O * (int)plane;  // one channel of one batch entry (32-bit offsets)
  const float inv4nb = 1.0f / (float)(4 * Nb), inv_nb = 1.0f / (float)Nb;
  const float* xb = a.x + (int64_t)b * a.Cin * chs + (int64_t)o * plane;
  const int xtot = a.Cin * 4 * Nb, ytot = a.Cout * 4 * Nb;

  // chunk c of x -> s_x: float4 e = 256 i + tid (channel e / (4 Nb)); lanes past the chunk
  // copy a clamped (valid) address into the unused tail of s_x
  auto load_x = [&](int c) {
#pragma unroll
    for (int i = 0; i < kErXPT; ++i) {
      const int2 cf = chunk_split(min(256 * i + tid, xtot - 1), inv4nb, 4 * Nb);
      copy16_to_lds(xb + cf.x * chs + 4 * cf.y + c * RP, s_x + 4 * (256 * i + 64 * wave));
    }
  };
  if constexpr (BLK) {
    // bypass rows past the copied region must hold finite values (their weights are zero)
    for (int e = 4 * 256 * kErXPT + tid; e < 4 * kErKB * RP; e += 256) s_x[e] = 0.f;
    load_x(0);
  }
  // first-product B fragments: A[row][s'] for this lane's row of chunk c
  float bfr[BF ? 1 : kErMA];
  V8 bhi[2], blo[2];
  auto load_rowtab = [&](int c) {
    const int row = kErRows * c + m;
    if constexpr (!BF) {
#pragma unroll
      for (int i = 0; i < kErMA / 4; ++i) {
        const int col = min((q >> 1) * a.SO + (q & 1) * a.ma + 4 * i, a.KA - 4);
        const float4 v = *reinterpret_cast<const float4*>(a.ainv + row * a.KA + col);
        bfr[4 * i + 0] = v.x;
        bfr[4 * i + 1] = v.y;
        bfr[4 * i + 2] = v.z;
        bfr[4 * i + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int col = min(32 * jj + 8 * q, a.KA - 8);
        bhi[jj] = *reinterpret_cast<const V8*>(a.ainv_bf + row * a.KA + col);
        blo[jj] = *reinterpret_cast<const V8*>(a.ainv_lo + row * a.KA + col);
      }
    }
  };
  // the first chunk's row table is loaded before the set-up loads below, whose waits then cover
  // it: as the kernel's last loads before the loop, the compiler would wait for every store of
  // the previous chunk before each chunk's products
  load_rowtab(0);

  // T of this (b, o): one contiguous block of 2 ma mb values per output channel.  The blocks
  // are staged in LDS (in the s_y region, unused until the first chunk's bypass) with
  // coalesced float4 loads, and the fragments below read them there: as per-lane gathers from
  // global memory they kept some eighty loads and their registers in flight at once.
  const int k = m >> 1, ri = m & 1;
  const int twoma = 2 * a.ma;
  const int tblk = twoma * a.mb;  // float2 per channel; even (ma % 4 == 0)
  float2* s_t = reinterpret_cast<float2*>(s_y);
  {
    const int tf4 = tblk >> 1;
    const int64_t tb0 = ((int64_t)b * a.Cout * a.O + o) * (int64_t)tblk;  // complex index
    const int64_t cstride = (int64_t)a.O * tblk;
    for (int e = tid; e < a.Cout * tf4; e += 256) {
      const int ch = e / tf4, r = e - ch * tf4;
      const int64_t ci = tb0 + ch * cstride + 2 * r;  // two complex values
      float4 v;
      if constexpr (BF) {
        if (a.Th) {  // exact: the half values as floats
          const uint2 u = *reinterpret_cast<const uint2*>(a.Th + 2 * ci);
          v = make_float4(HT::value((uint16_t)(u.x & 0xffffu)), HT::value((uint16_t)(u.x >> 16)),
                          HT::value((uint16_t)(u.y & 0xffffu)), HT::value((uint16_t)(u.y >> 16)));
        } else {
          v = *reinterpret_cast<const float4*>(a.T + ci);
        }
      } else {
        v = *reinterpret_cast<const float4*>(a.T + ci);
      }
      *reinterpret_cast<float4*>(s_t + ch * tblk + 2 * r) = v;
    }
  }
  __syncthreads();
  // first-product A fragments from T: lane (m, q) is k' = m (k = m / 2, re/im = m % 2)
  float afr[BF ? 1 : kErCPW][BF ? 1 : kErMA];
  V8 afb[BF ? kErCPW : 1][2];
#pragma unroll
  for (int j = 0; j < kErCPW; ++j) {
    const int cor = wave + 4 * j;
    const bool co_ok = cor < a.Cout;
    const float2* tb = s_t + min(cor, a.Cout - 1) * tblk;
    const int kc = min(k, a.mb - 1);
    if constexpr (!BF) {
      // K-step ks, slot q <-> s' = (q / 2) block, s = (q % 2) ma + ks.  The component is
      // chosen by lane-constant factors (exact), so that both halves are always loaded.
      const int part = q >> 1;
      const float fx = (ri == part) ? 1.f : 0.f;
      const float fy = (ri == part) ? 0.f : (ri ? 1.f : -1.f);
#pragma unroll
      for (int ks = 0; ks < kErMA; ++ks) {
        const int s = (q & 1) * a.ma + ks;
        const float2 t = tb[min(s, twoma - 1) * a.mb + kc];
        afr[j][ks] = keep_if(t.x * fx + t.y * fy, co_ok && ks < a.ma && k < a.mb);
      }
    } else {
      // K-step jj, slot (q, e) <-> table column 32 jj + 8 q + e
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tcol = 32 * jj + 8 * q + e;
          const int part = tcol >= a.SO ? 1 : 0;
          const int s = tcol - part * a.SO;
          const float2 t = tb[min(s, twoma - 1) * a.mb + kc];
          const float fx = (ri == part) ? 1.f : 0.f;
          const float fy = (ri == part) ? 0.f : (ri ? 1.f : -1.f);
          afb[j][jj][e] =
              (E)keep_if(t.x * fx + t.y * fy, co_ok && s < twoma && tcol < a.KA && k < a.mb);
        }
    }
    // one channel's LDS reads at a time: scheduled together, all of them and their registers
    // would be live at once
    __builtin_amdgcn_sched_barrier(0);
  }
  // second-product B fragments (G[k' = 4 q + r][c]), c = 16 ct + m
  float gfr[BF ? 1 : 2][4];
  V8 gfb[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int c = 16 * ct + m;
    const int cc = min(c, Nb - 1);
    if constexpr (!BF) {
      const float4 g4 = *reinterpret_cast<const float4*>(a.gt + cc * a.kpad + 4 * q);
      gfr[ct][0] = keep_if(g4.x, c < Nb);
      gfr[ct][1] = keep_if(g4.y, c < Nb);
      gfr[ct][2] = keep_if(g4.z, c < Nb);
      gfr[ct][3] = keep_if(g4.w, c < Nb);
    } else {
      const uint2 g2 = *reinterpret_cast<const uint2*>(a.gt_bf + cc * a.kpad + 4 * q);
      const uint32_t w0 = c < Nb ? g2.x : 0u, w1 = c < Nb ? g2.y : 0u;
      gfb[ct] = __builtin_bit_cast(V8, make_uint4(w0, w1, 0u, 0u));
    }
  }
  // bypass A fragments Wb[16 mt + m][4 kb + q] and the bias of rows 16 mt + 4 q + r
  float wbf[2][kErKB], bia[2][4];
  if constexpr (BLK) {
    // no bias: read Wb in its place (an unconditional load) and mask it
    const bool has_bias = a.bias != nullptr;
    const float* bsrc = has_bias ? a.bias : a.wb;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int co = 16 * mt + m;
#pragma unroll
      for (int kb = 0; kb < kErKB; ++kb) {
        const int ci = 4 * kb + q;
        const float w = a.wb[min(co, a.Cout - 1) * a.Cin + min(ci, a.Cin - 1)];
        wbf[mt][kb] = keep_if(w, co < a.Cout && ci < a.Cin);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int cb = 16 * mt + 4 * q + r;
        bia[mt][r] = keep_if(bsrc[min(cb, a.Cout - 1)], has_bias && cb < a.Cout);
      }
    }
  }
  const int64_t ybase = (int64_t)b * a.Cout * chs + (int64_t)o * plane;

  // global stores per thread in a chunk's store pass; vector-memory operations retire in issue
  // order, so waiting until at most that many are outstanding leaves the previous chunk's
  // stores in flight while guaranteeing this chunk's x copy and row table
  constexpr int kStores = (MODE == 2 ? 2 : 1) * kErXPT;
  static_assert(kStores < 16, "vmcnt field");
  // set-up loads done before the loop, so that the loop's own waits are those of its steady
  // state (the compiler merges the first iteration's state with the later ones).  The half
  // variants run out of registers with this wait; the load order above gives them the same.
  if constexpr (!BF) __builtin_amdgcn_s_waitcnt(kWaitVm0);
  for (int c = 0; c < nchunk; ++c) {
    // x chunk c in s_x, the row table of chunk c in registers; s_y free (previous stores read)
    __builtin_amdgcn_s_waitcnt(wait_vm(kStores));
    __syncthreads();
    if constexpr (BLK) {
      // bypass: D[co][point] = sum_ci Wb[co][ci] x[ci][point] + bias[co]
      for (int nt = wave; nt < Nb; nt += 4) {
        f32x4 d0 = zero4(), d1 = zero4();
#pragma unroll
        for (int kb = 0; kb < kErKB; ++kb) {
          const float bv = s_x[(4 * kb + q) * RP + 16 * nt + m];
          d0 = mfma_f32(wbf[0][kb], bv, d0);
          d1 = mfma_f32(wbf[1][kb], bv, d1);
        }
        // point 16 nt + m of the chunk is (row, column) = divmod(point, Nb)
        const int pt = 16 * nt + m;
        const int prow = (int)(((float)pt + 0.5f) * inv_nb);
        float* py = s_y + prow * kErRS + (pt - prow * Nb);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c0 = 4 * q + r, c1 = 16 + 4 * q + r;
          py[min(c0, a.Cout) * kErYC] = d0[r] + bia[0][r];
          py[min(c1, a.Cout) * kErYC] = d1[r] + bia[1][r];
        }
      }
      __syncthreads();
      // s_x has been read: the next chunk's x streams in during the spectral part (the last
      // chunk copies itself again, unread: a branch here would make the compiler drain every
      // load before the spectral products)
      load_x(min(c + 1, nchunk - 1));
    }
    // spectral part, one output channel at a time
#pragma unroll
    for (int j = 0; j < kErCPW; ++j) {
      const int cor = wave + 4 * j;
      f32x4 u = zero4();
      if constexpr (!BF) {
#pragma unroll
        for (int ks = 0; ks < kErMA; ++ks) u = mfma_f32(afr[j][ks], bfr[ks], u);
      } else {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          u = HT::mfma(afb[j][jj], bhi[jj], u);
          u = HT::mfma(afb[j][jj], blo[jj], u);
        }
      }
      V8 ub;
      if constexpr (BF)
        ub = __builtin_bit_cast(V8, make_uint4(HT::pack2(u[0], u[1]), HT::pack2(u[2], u[3]), 0u, 0u));
      // U (A operand, K-step r slot q <-> k' = 4 q + r) times G (B operand)
      float* py = s_y + min(cor, a.Cout) * kErYC + 4 * q * kErRS + m;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        f32x4 w = zero4();
        if constexpr (!BF) {
#pragma unroll
          for (int r = 0; r < 4; ++r) w = mfma_f32(u[r], gfr[ct][r], w);
        } else {
          w = HT::mfma(ub, gfb[ct], w);
        }
        // w[r] = y_spec[chunk row 4 q + r][column 16 ct + m]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (BLK)
            py[r * kErRS + 16 * ct] += w[r];
          else
            py[r * kErRS + 16 * ct] = w[r];
        }
      }
    }
    load_rowtab(min(c + 1, nchunk - 1));
    lds_barrier();  // s_y complete; the next chunk's x and row table may still be in flight
    const int coff = c * RP;
    // all reads first, then the stores, with no branch: threads past the chunk write a copy of
    // its last float4 (identical data)
    float4 zv[kErXPT];
    int64_t yo[kErXPT];
    uint32_t ya[kErXPT];
#pragma unroll
    for (int i = 0; i < kErXPT; ++i) {
      const int2 cf = chunk_split(min(tid + 256 * i, ytot - 1), inv4nb, 4 * Nb);
      const int prow = (int)(((float)(4 * cf.y) + 0.5f) * inv_nb);
      ya[i] = lds_addr(s_y + cf.x * kErYC + prow * kErRS + (4 * cf.y - prow * Nb));
      yo[i] = ybase + cf.x * chs + 4 * cf.y + coff;
    }
    lds_read7_f4(ya, zv);
#pragma unroll
    for (int i = 0; i < kErXPT; ++i) {
      if constexpr (MODE == 2) *reinterpret_cast<float4*>(a.zsave + yo[i]) = zv[i];
      float4 v = zv[i];
      if constexpr (BLK && G) {
        {
          v.x = gelu_as(zv[i].x);
          v.y = gelu_as(zv[i].y);
          v.z = gelu_as(zv[i].z);
          v.w = gelu_as(zv[i].w);
        }
      }
      if constexpr (H == 2) bad |= !finite4(v);
      *reinterpret_cast<float4*>(a.y + yo[i]) = v;
    }
  }
  if constexpr (H == 2) raise_half_flag(a.flag, bad);
}

// The fused row-axis epilogue applies when the contiguous axis is short, the retained rows and
// channels fit its register fragments, and every field pointer allows float4 access.
bool epilogue_rows_ok(const fno_plan* p, int mode, const float* x, const float* y,
                      const float* zsave) {
  const Geom& g = p->g;
  if (g.Nb > 32 || g.Nb % 4 != 0 || g.Na % kErRows != 0) return false;
  if (g.ma > kErMA || g.ma % 4 != 0 || g.mb > 8) return false;
  if (g.Cout > 4 * kErCPW || g.Cout * g.Nb > 64 * kErXPT) return false;
  if (mode != EPI_SPECTRAL && (g.Cin > 4 * kErKB || g.Cin * g.Nb > 64 * kErXPT)) return false;
  // the bypass here reads x as the block's input; a pre-activation input takes the line kernels
  if (mode != EPI_SPECTRAL && (p->desc.flags & FNO_FLAG_INPUT_GELU)) return false;
  if (g.B > 65535) return false;
  // 32-bit offsets within one batch entry's field
  const int64_t chs = g.O * (int64_t)g.Na * g.Nb;
  if (chs * (g.Cin > g.Cout ? g.Cin : g.Cout) >= ((int64_t)1 << 31)) return false;
  const int so = (2 * g.ma + 15) / 16 * 16;
  if (2 * so > 64) return false;
  auto al16 = [](const void* v) { return ((uintptr_t)v & 15u) == 0; };
  return al16(x) && al16(y) && al16(zsave);
}

template <int H, int MODE, bool G>
static hipError_t launch_rows_t(const RowsEpiArgs& a, int B, hipStream_t s) {
  const int RP = kErRows * a.Nb;
  const int xfl = 4 * kErKB * RP > 4 * 256 * kErXPT ? 4 * kErKB * RP : 4 * 256 * kErXPT;
  const size_t lds = sizeof(float) * ((size_t)(a.Cout + 1) * kErYC + (MODE >= 1 ? xfl : 0));
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_epi_rows<H, MODE, G>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_epi_rows<H, MODE, G>), dim3((unsigned)a.O, (unsigned)B), dim3(256), lds, s,
                     a);
  return hipGetLastError();
}

template <int H>
static hipError_t launch_rows_h(const RowsEpiArgs& a, int md, int B, hipStream_t s) {
  if (md == 0) return launch_rows_t<H, 0, false>(a, B, s);
  if (md == 1)
    return a.gelu ? launch_rows_t<H, 1, true>(a, B, s) : launch_rows_t<H, 1, false>(a, B, s);
  return a.gelu ? launch_rows_t<H, 2, true>(a, B, s) : launch_rows_t<H, 2, false>(a, B, s);
}

hipError_t launch_epilogue_rows(const fno_plan* p, int mode, const void* T, const float* x,
                                const float* wb, const float* bias, float* y, float* zsave,
                                hipStream_t s, bool t_half) {
  const Geom& g = p->g;
  RowsEpiArgs a{};
  a.Na = g.Na;
  a.Nb = g.Nb;
  a.ma = g.ma;
  a.mb = g.mb;
  a.Cin = g.Cin;
  a.Cout = g.Cout;
  a.SO = (2 * g.ma + 15) / 16 * 16;
  a.KA = 2 * a.SO;
  a.kpad = p->kpad;
  a.O = (int)g.O;
  a.gelu = (mode == EPI_BLOCK && (p->desc.flags & FNO_FLAG_GELU)) ? 1 : 0;
  if (t_half && !g.bf16) return hipErrorInvalidValue;
  a.T = t_half ? nullptr : static_cast<const float2*>(T);
  a.Th = t_half ? static_cast<const uint16_t*>(T) : nullptr;
  a.x = x;
  a.wb = wb;
  a.bias = (p->desc.flags & FNO_FLAG_BIAS) ? bias : nullptr;
  a.y = y;
  a.zsave = zsave;
  a.ainv = p->t.oinv[g.d - 2];
  a.ainv_bf = p->t.oinv_bf[g.d - 2];
  a.ainv_lo = p->t.oinv_bf_lo[g.d - 2];
  a.gt = p->t.gt_fwd;
  a.gt_bf = p->t.gt_fwd_bf;
  a.flag = p->g.half_flag;
  const int md = mode == EPI_SPECTRAL ? 0 : (zsave ? 2 : 1);
  if (g.half == 2) return launch_rows_h<2>(a, md, g.B, s);
  if (g.half == 1) return launch_rows_h<1>(a, md, g.B, s);
  return launch_rows_h<0>(a, md, g.B, s);
}

}  // namespace fno
