// Tucker-factorised spectral weights (TFNO; named on the mixed-precision neural-operator page,
// "Tiivistelmä", among the architectures trained in mixed precision, together with a greedy
// algorithm that orders the FNO block's half-precision tensor contractions).
//
// The retained-grid weight W[i, o, s_0..s_{d-1}] is held as a core G[R_in, R_out, R_0..] and
// factor matrices U_in [Cin, R_in], U_out [Cout, R_out], U_j [K_j, R_j] (K_j = 2 m_j on outer
// axes, m_{d-1} on the last):  W = G x_1 U_in x_2 U_out x_3 U_0 ..  (mode-n products).  The
// block's mix  yhat[b,o,k] = sum_i xhat[b,i,k] W[i,o,k]  is evaluated as a network of pairwise
// contractions without forming W where that is smaller:
//   - a factor applied to the core ("G*U"): a mode product on the core's lineage;
//   - U_in applied to the spectrum ("X*Uin"): xhat[b,i,k] -> [b,R_in,k];
//   - the per-mode channel mix ("mix") of the data tensor with the core once every mode
//     factor is applied: the dense mix kernels, reading the core tensor in its natural
//     [c_in][c_out][K] layout (the retained spectrum's mode order is that layout's);
//   - U_out applied to the mixed spectrum ("Y*Uout").
// The order is greedy: of the contractions available, the one with the smallest result is
// taken first.  Ties go to fewer flops, then to the mode factors (a channel factor can still
// act on the data side instead, so it waits), then to a fixed order.  Everything but the mix
// runs in float32 (small products); the mix uses the plan's operand precision.
#include "fno_internal.h"

#include <stdio.h>

namespace fno {

// ---- greedy contraction order (host) ---------------------------------------------------------
std::vector<TuckerStep> tucker_greedy_order(const TuckerDims& t) {
  const int D = t.d + 2;  // core axes: in, out, mode 0 .. mode d-1
  int64_t K = 1;
  for (int j = 0; j < t.d; ++j) K *= t.K[j];
  int64_t full[2 + kMaxDims];
  full[0] = t.Cin;
  full[1] = t.Cout;
  for (int j = 0; j < t.d; ++j) full[2 + j] = t.K[j];
  int64_t cur[2 + kMaxDims];  // current core extents
  bool todo[2 + kMaxDims];    // factor not yet applied anywhere
  for (int n = 0; n < D; ++n) {
    cur[n] = t.R[n];
    todo[n] = true;
  }
  bool in_on_data = false, mixed = false;
  std::vector<TuckerStep> steps;
  for (;;) {
    bool found = false;
    TuckerStep best{};
    int64_t best_size = 0, best_flops = 0;
    int best_prio = 0;
    // tie order: mode factors on the core, U_in on the spectrum, the mix, U_out on the mixed
    // spectrum, channel factors on the core
    auto prio = [](const TuckerStep& st) {
      return st.kind == TuckerStep::CORE ? (st.factor >= 2 ? 0 : 4) : (int)st.kind;
    };
    auto offer = [&](const TuckerStep& st, int64_t size, int64_t flops) {
      const int pr = prio(st);
      const bool better =
          !found || size < best_size ||
          (size == best_size &&
           (flops < best_flops || (flops == best_flops && pr < best_prio)));
      if (better) {
        found = true;
        best = st;
        best_size = size;
        best_flops = flops;
        best_prio = pr;
      }
    };
    int64_t core_size = 1;
    for (int n = 0; n < D; ++n) core_size *= cur[n];
    // factors on the core (U_in / U_out only while not yet applied on the data side)
    for (int n = 0; n < D; ++n) {
      if (!todo[n] || mixed) continue;
      TuckerStep st{};
      st.kind = TuckerStep::CORE;
      st.factor = n;
      st.an = full[n];
      st.cn = cur[n];
      st.pre = 1;
      for (int m = 0; m < n; ++m) st.pre *= cur[m];
      st.post = 1;
      for (int m = n + 1; m < D; ++m) st.post *= cur[m];
      const int64_t size = core_size / cur[n] * full[n];
      offer(st, size, size * cur[n]);
    }
    if (todo[0] && !mixed) {  // U_in on the spectrum
      TuckerStep st{};
      st.kind = TuckerStep::DATA_IN;
      st.factor = 0;
      st.pre = t.B;
      st.an = t.R[0];
      st.cn = t.Cin;
      st.post = K;
      const int64_t size = t.B * t.R[0] * K;
      offer(st, size, size * t.Cin);
    }
    bool modes_done = true;
    for (int n = 2; n < D; ++n) modes_done = modes_done && !todo[n];
    if (!mixed && modes_done && !todo[0]) {
      TuckerStep st{};
      st.kind = TuckerStep::MIX;
      st.factor = -1;
      st.pre = t.B;
      st.cn = in_on_data ? t.R[0] : t.Cin;  // contracted channels
      st.an = cur[1];                        // output channels (R_out or Cout)
      st.post = K;
      const int64_t size = t.B * cur[1] * K;
      offer(st, size, size * st.cn);
    }
    if (mixed && todo[1]) {  // U_out on the mixed spectrum
      TuckerStep st{};
      st.kind = TuckerStep::DATA_OUT;
      st.factor = 1;
      st.pre = t.B;
      st.an = t.Cout;
      st.cn = t.R[1];
      st.post = K;
      const int64_t size = t.B * t.Cout * K;
      offer(st, size, size * t.R[1]);
    }
    if (!found) break;
    steps.push_back(best);
    switch (best.kind) {
      case TuckerStep::CORE:
        cur[best.factor] = full[best.factor];
        todo[best.factor] = false;
        break;
      case TuckerStep::DATA_IN:
        todo[0] = false;
        in_on_data = true;
        break;
      case TuckerStep::MIX:
        mixed = true;
        break;
      case TuckerStep::DATA_OUT:
        todo[1] = false;
        break;
    }
    if (mixed && !todo[1]) break;
  }
  return steps;
}

std::string tucker_order_string(const std::vector<TuckerStep>& steps, int d) {
  std::string s;
  char buf[32];
  for (const TuckerStep& st : steps) {
    if (!s.empty()) s += ' ';
    switch (st.kind) {
      case TuckerStep::CORE:
        if (st.factor == 0) snprintf(buf, sizeof(buf), "G*Uin");
        else if (st.factor == 1) snprintf(buf, sizeof(buf), "G*Uout");
        else snprintf(buf, sizeof(buf), "G*U%d", st.factor - 2);
        s += buf;
        break;
      case TuckerStep::DATA_IN: s += "X*Uin"; break;
      case TuckerStep::MIX: s += "mix"; break;
      case TuckerStep::DATA_OUT: s += "Y*Uout"; break;
    }
  }
  (void)d;
  return s;
}

// ---- mode product ----------------------------------------------------------------------------
// out[p][a][q] = sum_c op(A)[a][c] T[p][c][q], complex.  op(A)[a][c] = A[a][c] (A stored
// [an][cn]) or A[c][a] (trans: A stored [cn][an]), conjugated when conj is set.  Grid: x over
// (p, q) columns, 256 per work-group; y over tiles of kMpRows output rows, whose op(A) rows are
// staged in LDS.  A thread owns one column: consecutive threads read consecutive q (coalesced
// for q-contiguous tensors), and the loads of kMpC consecutive c go out together (clamped
// indices, masked values: no branch around a load).  These tensors are a few MB, so the kernel
// is bound by load latency; the tiling keeps enough loads in flight.
constexpr int kMpRows = 8;
constexpr int kMpC = 8;

__global__ void __launch_bounds__(256)
k_mode_product(int64_t pre, int an, int cn, int64_t post, const float2* __restrict__ A,
               int trans, int conj, const float2* __restrict__ T, float2* __restrict__ out) {
  __shared__ float2 s_a[kMpRows * 64];
  const int tid = threadIdx.x;
  const int a0 = blockIdx.y * kMpRows;
  for (int e = tid; e < kMpRows * cn; e += 256) {
    const int a = min(a0 + e / cn, an - 1), c = e % cn;
    float2 v = trans ? A[(int64_t)c * an + a] : A[(int64_t)a * cn + c];
    if (conj) v.y = -v.y;
    s_a[e] = v;
  }
  __syncthreads();
  const int64_t col = (int64_t)blockIdx.x * 256 + tid;
  if (col >= pre * post) return;
  const int64_t p = col / post, q = col % post;
  const float2* tp = T + p * cn * post + q;
  float ar[kMpRows], ai[kMpRows];
#pragma unroll
  for (int j = 0; j < kMpRows; ++j) ar[j] = ai[j] = 0.f;
  for (int c0 = 0; c0 < cn; c0 += kMpC) {
    float2 tv[kMpC];
#pragma unroll
    for (int u = 0; u < kMpC; ++u) tv[u] = tp[(int64_t)min(c0 + u, cn - 1) * post];
#pragma unroll
    for (int u = 0; u < kMpC; ++u) {
      const bool ok = c0 + u < cn;
      const float tr = ok ? tv[u].x : 0.f, ti = ok ? tv[u].y : 0.f;
      const int c = min(c0 + u, cn - 1);
#pragma unroll
      for (int j = 0; j < kMpRows; ++j) {
        const float2 m = s_a[j * cn + c];
        ar[j] += m.x * tr - m.y * ti;
        ai[j] += m.x * ti + m.y * tr;
      }
    }
  }
  float2* op = out + p * an * post + q;
#pragma unroll
  for (int j = 0; j < kMpRows; ++j)
    if (a0 + j < an) op[(int64_t)(a0 + j) * post] = make_float2(ar[j], ai[j]);
}

// Short rows (post < kMpShortPost, e.g. the last mode of the core): one thread per output
// element in output order, so stores are contiguous; threads of one (p, q) read the same
// T values.  op(A) (at most 64 x 64) sits in LDS.
constexpr int kMpShortPost = 16;

__global__ void __launch_bounds__(256)
k_mode_product_short(int64_t pre, int an, int cn, int post, const float2* __restrict__ A,
                     int trans, int conj, const float2* __restrict__ T,
                     float2* __restrict__ out) {
  __shared__ float2 s_a[64 * 64];
  const int tid = threadIdx.x;
  for (int e = tid; e < an * cn; e += 256) {
    const int a = e / cn, c = e % cn;
    float2 v = trans ? A[(int64_t)c * an + a] : A[e];
    if (conj) v.y = -v.y;
    s_a[e] = v;
  }
  __syncthreads();
  const int64_t e = (int64_t)blockIdx.x * 256 + tid;
  if (e >= pre * an * post) return;
  const int q = (int)(e % post);
  const int64_t pa = e / post;
  const int a = (int)(pa % an);
  const int64_t p = pa / an;
  const float2* tp = T + p * cn * post + q;
  float ar = 0.f, ai = 0.f;
  for (int c0 = 0; c0 < cn; c0 += kMpC) {
    float2 tv[kMpC];
#pragma unroll
    for (int u = 0; u < kMpC; ++u) tv[u] = tp[(int64_t)min(c0 + u, cn - 1) * post];
#pragma unroll
    for (int u = 0; u < kMpC; ++u) {
      const bool ok = c0 + u < cn;
      const float tr = ok ? tv[u].x : 0.f, ti = ok ? tv[u].y : 0.f;
      const float2 m = s_a[a * cn + min(c0 + u, cn - 1)];
      ar += m.x * tr - m.y * ti;
      ai += m.x * ti + m.y * tr;
    }
  }
  out[e] = make_float2(ar, ai);
}

hipError_t launch_mode_product(int64_t pre, int an, int cn, int64_t post, const float2* A,
                               bool trans, bool conj, const float2* T, float2* out,
                               hipStream_t s) {
  if (an < 1 || cn < 1 || an > 64 || cn > 64 || pre < 1 || post < 1)
    return hipErrorInvalidValue;
  if (post < kMpShortPost) {
    const int64_t nblk = (pre * an * post + 255) / 256;
    if (nblk > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_mode_product_short, dim3((unsigned)nblk), dim3(256), 0, s, pre, an, cn,
                       (int)post, A, trans ? 1 : 0, conj ? 1 : 0, T, out);
    return hipGetLastError();
  }
  const int64_t blocks = (pre * post + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks, (unsigned)((an + kMpRows - 1) / kMpRows));
  hipLaunchKernelGGL(k_mode_product, grid, dim3(256), 0, s, pre, an, cn, post, A,
                     trans ? 1 : 0, conj ? 1 : 0, T, out);
  return hipGetLastError();
}

// ---- mode Gram product (factor gradients) ----------------------------------------------------
// out[a][c] = scale * sum_{p, q} X[p][a][q] w(q) conj(Y[p][c][q])   (conjugated when conj_out),
// X [pre][an][post], Y [pre][cn][post]; w(q) = gamma(q mod mb) * adj (the inverse transform's
// half-spectrum weight, when gamma_w) or 1.  Stage 1: work-group g sums the (p, q) range
// [g chunk, (g + 1) chunk) in tiles of kGramT staged in LDS (all of a tile's loads go out
// before any is stored); thread t owns a TA x TC block of outputs, sized so that the threads
// cover an x cn with as few idle as possible, and each LDS read serves TC (or TA) products.
// Stage 2 adds the partials of each output in a fixed order (deterministic) and applies
// scale / conj.
constexpr int kGramT = 32;
constexpr int kGramLd = (2 * 64 * kGramT) / 256;  // tile values loaded per thread (at most)

template <int TA, int TC>
__global__ void __launch_bounds__(256)
k_gram_part(int pre, int an, int cn, int post, const float2* __restrict__ X,
            const float2* __restrict__ Y, int gamma_w, int mb, int Nb, float adj, int chunk,
            float2* __restrict__ part) {
  __shared__ float2 s_x[64][kGramT + 1];
  __shared__ float2 s_y[64][kGramT + 1];
  const int tid = threadIdx.x;
  const int D = pre * post;
  const int lo = blockIdx.x * chunk;
  const int hi = min(D, lo + chunk);
  const int ncb = (cn + TC - 1) / TC;
  const int ab = tid / ncb, cb = tid % ncb;
  const bool active = ab * TA < an;
  const int rows = an + cn;
  // tile element t of this thread is fixed (256 u is a multiple of kGramT); its rows are
  // r0 + 8 u
  const int t = tid & (kGramT - 1);
  const int r0 = tid / kGramT;
  float ar[TA][TC], ai[TA][TC];
#pragma unroll
  for (int i = 0; i < TA; ++i)
#pragma unroll
    for (int j = 0; j < TC; ++j) ar[i][j] = ai[i][j] = 0.f;
  for (int base = lo; base < hi; base += kGramT) {
    const int idx = min(base + t, hi - 1);
    const int pp = idx / post, qq = idx - pp * post;
    float wq = base + t < hi ? 1.f : 0.f;
    if (gamma_w) {
      const int kb = qq % mb;
      wq *= ((kb == 0 || 2 * kb == Nb) ? 1.f : 2.f) * adj;
    }
    const float2* xs = X + (int64_t)pp * an * post + qq;
    const float2* ys = Y + (int64_t)pp * cn * post + qq;
    float2 v[kGramLd];
#pragma unroll
    for (int u = 0; u < kGramLd; ++u) {
      const int row = min(r0 + (256 / kGramT) * u, rows - 1);
      v[u] = row < an ? xs[(int64_t)row * post] : ys[(int64_t)(row - an) * post];
    }
    __syncthreads();  // the previous tile's products are done
#pragma unroll
    for (int u = 0; u < kGramLd; ++u) {
      const int row = r0 + (256 / kGramT) * u;
      if (row < an) s_x[row][t] = make_float2(v[u].x * wq, v[u].y * wq);
      else if (row < rows) s_y[row - an][t] = v[u];
    }
    __syncthreads();
    if (active) {
      for (int k = 0; k < kGramT; ++k) {
        float2 xv[TA], yv[TC];
#pragma unroll
        for (int i = 0; i < TA; ++i) xv[i] = s_x[min(TA * ab + i, 63)][k];
#pragma unroll
        for (int j = 0; j < TC; ++j) yv[j] = s_y[min(TC * cb + j, 63)][k];
#pragma unroll
        for (int i = 0; i < TA; ++i)
#pragma unroll
          for (int j = 0; j < TC; ++j) {
            ar[i][j] += xv[i].x * yv[j].x + xv[i].y * yv[j].y;  // x conj(y)
            ai[i][j] += xv[i].y * yv[j].x - xv[i].x * yv[j].y;
          }
      }
    }
  }
  const int nout = an * cn;
#pragma unroll
  for (int i = 0; i < TA; ++i)
#pragma unroll
    for (int j = 0; j < TC; ++j) {
      const int a = TA * ab + i, c = TC * cb + j;
      if (active && a < an && c < cn)
        part[(int64_t)blockIdx.x * nout + a * cn + c] = make_float2(ar[i][j], ai[i][j]);
    }
}

// 16 outputs per work-group; 16 thread groups each add every 16th partial (8 loads in flight
// per thread), then the 16 sums are combined in group order.
constexpr int kFinOut = 16;
constexpr int kFinGroups = 256 / kFinOut;

__global__ void __launch_bounds__(256)
k_gram_finish(int nparts, int nout, const float2* __restrict__ part, float scale, int conj_out,
              float2* __restrict__ out) {
  __shared__ float2 s_sum[kFinGroups][kFinOut];
  const int o = threadIdx.x % kFinOut, w = threadIdx.x / kFinOut;
  const int e = blockIdx.x * kFinOut + o;
  const int ec = min(e, nout - 1);
  float r = 0.f, i = 0.f;
  for (int g0 = w; g0 < nparts; g0 += kFinGroups * 8) {
    float2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = part[(int64_t)min(g0 + kFinGroups * u, nparts - 1) * nout + ec];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool ok = g0 + kFinGroups * u < nparts;
      r += ok ? v[u].x : 0.f;
      i += ok ? v[u].y : 0.f;
    }
  }
  s_sum[w][o] = make_float2(r, i);
  __syncthreads();
  if (w == 0 && e < nout) {
    float sr = 0.f, si = 0.f;
#pragma unroll
    for (int k = 0; k < kFinGroups; ++k) {
      sr += s_sum[k][o].x;
      si += s_sum[k][o].y;
    }
    out[e] = make_float2(scale * sr, (conj_out ? -scale : scale) * si);
  }
}

int gram_parts(int64_t pre, int64_t post, int an, int cn) {
  const int64_t D = pre * post;
  int64_t parts = (D + 2 * kGramT - 1) / (2 * kGramT);  // about two tiles per work-group
  const int64_t cap = kTuckerPartElems / ((int64_t)an * cn);
  if (parts > cap) parts = cap;
  if (parts > 2048) parts = 2048;
  if (parts < 1) parts = 1;
  return (int)parts;
}

hipError_t launch_gram(int64_t pre, int an, int cn, int64_t post, const float2* X,
                       const float2* Y, bool gamma_w, int mb, int Nb, float adj, float scale,
                       bool conj_out, float2* part, float2* out, hipStream_t s) {
  if (an < 1 || cn < 1 || an > 64 || cn > 64 || pre < 1 || post < 1 ||
      pre * post > 0x7fffffff || pre * (an > cn ? an : cn) * post > 0x7fffffff)
    return hipErrorInvalidValue;
  const int parts = gram_parts(pre, post, an, cn);
  const int64_t D = pre * post;
  int64_t chunk = (D + parts - 1) / parts;
  chunk = (chunk + kGramT - 1) / kGramT * kGramT;
  const int nparts = (int)((D + chunk - 1) / chunk);
  // the smallest per-thread output block whose thread grid fits 256 threads
  auto fits = [&](int ta, int tc) { return ((an + ta - 1) / ta) * ((cn + tc - 1) / tc) <= 256; };
  const dim3 grid((unsigned)nparts), blk(256);
  const int ip = (int)pre, iq = (int)post, ic = (int)chunk, gw = gamma_w ? 1 : 0;
  if (fits(1, 1))
    hipLaunchKernelGGL((k_gram_part<1, 1>), grid, blk, 0, s, ip, an, cn, iq, X, Y, gw, mb, Nb,
                       adj, ic, part);
  else if (fits(2, 1))
    hipLaunchKernelGGL((k_gram_part<2, 1>), grid, blk, 0, s, ip, an, cn, iq, X, Y, gw, mb, Nb,
                       adj, ic, part);
  else if (fits(2, 2))
    hipLaunchKernelGGL((k_gram_part<2, 2>), grid, blk, 0, s, ip, an, cn, iq, X, Y, gw, mb, Nb,
                       adj, ic, part);
  else if (fits(4, 2))
    hipLaunchKernelGGL((k_gram_part<4, 2>), grid, blk, 0, s, ip, an, cn, iq, X, Y, gw, mb, Nb,
                       adj, ic, part);
  else
    hipLaunchKernelGGL((k_gram_part<4, 4>), grid, blk, 0, s, ip, an, cn, iq, X, Y, gw, mb, Nb,
                       adj, ic, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nout = an * cn;
  hipLaunchKernelGGL(k_gram_finish, dim3((unsigned)((nout + kFinOut - 1) / kFinOut)), dim3(256),
                     0, s, nparts, nout, part, scale, conj_out ? 1 : 0, out);
  return hipGetLastError();
}

}  // namespace fno
