// libfno host runtime: descriptor validation, float64 table build, workspace layout and the
// launch sequence of each entry point.  All device work is enqueued on the caller's stream;
// nothing here allocates device memory except fno_plan_create (its tables, once) and the
// static scratch array of fno_block_fwd_static (the runtime places it when it loads the
// library's code on a device).
#include "fno_internal.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <new>
#include <cmath>
#include <string>
#include <vector>

namespace {

thread_local std::string g_last_error;

fno_status fail(fno_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
fno_status fail(fno_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

fno_status hip_fail(hipError_t e, const char* what) {
  return fail(FNO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define FNO_HIP(call, what)                       \
  do {                                            \
    hipError_t e_ = (call);                       \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

float round_bf16(float v) {
  uint32_t u;
  memcpy(&u, &v, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  u &= 0xffff0000u;
  float r;
  memcpy(&r, &u, 4);
  return r;
}

// float64 -> bfloat16 bits, round to nearest even (via the float32 rounding of the value)
uint16_t bf16_bits_host(double v) {
  const float f = round_bf16((float)v);
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

double bf16_value_host(uint16_t bits) {
  const uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

// float64 -> IEEE half bits, round to nearest even (one rounding)
uint16_t f16_bits_host(double v) {
  const _Float16 h = (_Float16)v;
  uint16_t b;
  memcpy(&b, &h, 2);
  return b;
}

double f16_value_host(uint16_t bits) {
  _Float16 h;
  memcpy(&h, &bits, 2);
  return (double)h;
}

// the plan's half format: bfloat16 or IEEE half
uint16_t half_bits_host(double v, bool f16) { return f16 ? f16_bits_host(v) : bf16_bits_host(v); }
double half_value_host(uint16_t b, bool f16) { return f16 ? f16_value_host(b) : bf16_value_host(b); }
float round_half_host(float v, bool f16) { return (float)half_value_host(half_bits_host(v, f16), f16); }

}  // namespace

extern "C" {

const char* fno_status_string(fno_status s) {
  switch (s) {
    case FNO_OK: return "FNO_OK";
    case FNO_ERR_INVALID_ARGUMENT: return "FNO_ERR_INVALID_ARGUMENT";
    case FNO_ERR_UNSUPPORTED: return "FNO_ERR_UNSUPPORTED";
    case FNO_ERR_HIP: return "FNO_ERR_HIP";
    case FNO_ERR_OUT_OF_MEMORY: return "FNO_ERR_OUT_OF_MEMORY";
    case FNO_ERR_INTERNAL: return "FNO_ERR_INTERNAL";
  }
  return "FNO_ERR_UNKNOWN";
}

const char* fno_last_error_message(void) { return g_last_error.c_str(); }

fno_status fno_plan_validate(const fno_plan_desc* d) {
  if (!d) return fail(FNO_ERR_INVALID_ARGUMENT, "descriptor is NULL");
  if (d->ndim < 2 || d->ndim > 4)
    return fail(FNO_ERR_INVALID_ARGUMENT, "ndim %d not in {2,3,4}", d->ndim);
  if (d->reserved != 0) return fail(FNO_ERR_INVALID_ARGUMENT, "reserved field must be 0");
  if (d->flags & ~(uint32_t)(FNO_FLAG_TANH_PREACT | FNO_FLAG_GELU | FNO_FLAG_BIAS |
                             FNO_FLAG_INPUT_GELU | FNO_FLAG_LAST_AXIS_FFT |
                             FNO_FLAG_LAST_AXIS_DENSE))
    return fail(FNO_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", d->flags);
  if ((d->flags & FNO_FLAG_LAST_AXIS_FFT) && (d->flags & FNO_FLAG_LAST_AXIS_DENSE))
    return fail(FNO_ERR_INVALID_ARGUMENT, "LAST_AXIS_FFT and LAST_AXIS_DENSE exclude each other");
  if (d->spectral_dtype != FNO_DTYPE_F32 && d->spectral_dtype != FNO_DTYPE_BF16 &&
      d->spectral_dtype != FNO_DTYPE_F16)
    return fail(FNO_ERR_INVALID_ARGUMENT, "unknown spectral dtype %d", d->spectral_dtype);
  if (d->batch < 1 || d->c_in < 1 || d->c_out < 1)
    return fail(FNO_ERR_INVALID_ARGUMENT, "batch/c_in/c_out must be >= 1");
  const int nd = d->ndim;
  for (int j = 0; j < 4; ++j) {
    if (j >= nd) {
      if (d->n[j] != 0 || d->modes[j] != 0)
        return fail(FNO_ERR_INVALID_ARGUMENT, "n[%d]/modes[%d] must be 0 beyond ndim", j, j);
      continue;
    }
    if (d->n[j] < 2) return fail(FNO_ERR_INVALID_ARGUMENT, "n[%d] = %lld < 2", j, (long long)d->n[j]);
    const int64_t mmax = (j == nd - 1) ? d->n[j] / 2 + 1 : d->n[j] / 2;
    if (d->modes[j] < 1 || d->modes[j] > mmax)
      return fail(FNO_ERR_INVALID_ARGUMENT, "modes[%d] = %lld outside [1, %lld]", j,
                  (long long)d->modes[j], (long long)mmax);
  }
  // limits of the kernels (valid FNO shapes beyond them are UNSUPPORTED)
  if (d->c_in > 64 || d->c_out > 64)
    return fail(FNO_ERR_UNSUPPORTED, "channels > 64 not implemented");
  const int64_t na = d->n[nd - 2], nb = d->n[nd - 1];
  const int64_t ma = d->modes[nd - 2], mb = d->modes[nd - 1];
  if (nb > 4096 || na > 65536)
    return fail(FNO_ERR_UNSUPPORTED, "last two axes (%lld, %lld) too long", (long long)na,
                (long long)nb);
  if (2 * ma * mb > 4096)
    return fail(FNO_ERR_UNSUPPORTED, "2*m_a*m_b = %lld > 4096", (long long)(2 * ma * mb));
  // LDS of the plane transform (root tables, 8 staged rows and their spectra)
  const int64_t lds_plane = 8 * (na + nb + 8 * mb) + 4 * 8 * nb;
  if (lds_plane > 65536)
    return fail(FNO_ERR_UNSUPPORTED, "plane transform needs %lld bytes of LDS", (long long)lds_plane);
  const int64_t lds_epi = 8 * nb + 4 * (d->c_in * d->c_out + d->c_out + 128 * d->c_in);
  if (lds_epi > 65536)
    return fail(FNO_ERR_UNSUPPORTED, "epilogue needs %lld bytes of LDS", (long long)lds_epi);
  double elems = (double)d->batch * (double)(d->c_in > d->c_out ? d->c_in : d->c_out);
  double wel = (double)(1 << (nd - 1)) * d->c_in * d->c_out;
  for (int j = 0; j < nd; ++j) {
    elems *= (double)d->n[j];
    wel *= (double)d->modes[j];
  }
  if (elems >= 2147483648.0) return fail(FNO_ERR_UNSUPPORTED, "field has >= 2^31 elements");
  if (wel >= 2147483648.0) return fail(FNO_ERR_UNSUPPORTED, "weights have >= 2^31 elements");
  return FNO_OK;
}

fno_status fno_plan_create(const fno_plan_desc* desc, fno_plan** out) {
  if (!out) return fail(FNO_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  fno_status st = fno_plan_validate(desc);
  if (st != FNO_OK) return st;
  fno_plan* p = new (std::nothrow) fno_plan();
  if (!p) return fail(FNO_ERR_OUT_OF_MEMORY, "host allocation failed");
  p->desc = *desc;
  fno::Geom& g = p->g;
  g.d = desc->ndim;
  g.B = (int)desc->batch;
  g.Cin = (int)desc->c_in;
  g.Cout = (int)desc->c_out;
  g.P = 1;
  g.Mprod = 1;
  g.K = 1;
  for (int j = 0; j < fno::kMaxDims; ++j) {
    g.N[j] = j < g.d ? (int)desc->n[j] : 0;
    g.M[j] = j < g.d ? (int)desc->modes[j] : 0;
  }
  for (int j = 0; j < g.d; ++j) {
    g.P *= g.N[j];
    g.Mprod *= g.M[j];
    g.K *= (j == g.d - 1) ? g.M[j] : 2 * g.M[j];
  }
  g.w_si = (int)(g.Cout * g.Mprod);
  g.w_so = (int)g.Mprod;
  g.Na = g.N[g.d - 2];
  g.Nb = g.N[g.d - 1];
  g.ma = g.M[g.d - 2];
  g.mb = g.M[g.d - 1];
  g.O = 1;
  for (int j = 0; j < g.d - 2; ++j) g.O *= g.N[j];
  g.ncorner = 1 << (g.d - 1);
  g.inv_ntot = (float)(1.0 / (double)g.P);
  g.half = desc->spectral_dtype == FNO_DTYPE_BF16 ? 1 : (desc->spectral_dtype == FNO_DTYPE_F16 ? 2 : 0);
  g.bf16 = g.half != 0;
  const bool f16 = g.half == 2;
  for (int j = 0; j < fno::kMaxDims; ++j)
    g.sc[j] = (f16 && j < g.d) ? (float)(1.0 / sqrt((double)g.N[j])) : 1.0f;
  g.adj_scale = f16 ? 1.0f : g.inv_ntot;
  {
    // the power of two nearest to v (v >= 1)
    auto pow2_near = [](double v) { return (float)std::ldexp(1.0, (int)std::lround(std::log2(v))); };
    g.mix_gain[0] = f16 ? pow2_near(std::sqrt((double)g.Cin) * g.Cout) : 1.0f;
    g.mix_gain[1] = f16 ? pow2_near(std::sqrt((double)g.Cout) * g.Cin) : 1.0f;
    g.inv_gain[0] = 1.0f / g.mix_gain[0];
    g.inv_gain[1] = 1.0f / g.mix_gain[1];
  }
  const int cmax = g.Cin > g.Cout ? g.Cin : g.Cout;

  p->kpad = (2 * g.mb + 31) / 32 * 32;
  p->jpad = (2 * g.mb + 15) / 16 * 16;
  // plane-transform chunking along axis a: at least 512 work-groups (two per CU), chunks of
  // 64-row multiples; fewer, longer chunks amortise each work-group's table load and final
  // combine, and a single chunk needs no partial-sum pass
  {
    const int64_t planes = (int64_t)g.B * cmax * g.O;
    int64_t want = (512 + planes - 1) / planes;
    if (want < 1) want = 1;
    int rows = (int)((g.Na + want - 1) / want);
    rows = (rows + 63) / 64 * 64;
    if (rows > g.Na) rows = g.Na;
    if (fno::plane_small_ok(p)) rows = g.Na;  // the short-row kernel never chunks
    p->plane_rows = rows;
    p->nch = (g.Na + rows - 1) / rows;
  }
  // forward transform of the contiguous axis on float32 plans: FFT or dense product
  {
    const bool fft_ok = fno::plane_fft_ok(p);
    if ((desc->flags & FNO_FLAG_LAST_AXIS_FFT) && !g.bf16 && !fft_ok) {
      delete p;
      return fail(FNO_ERR_UNSUPPORTED,
                  "LAST_AXIS_FFT needs a float32 plan with N_last in {128,256,512}, "
                  "m_last <= 32, m_{d-2} a multiple of 4 (<= 32) and N_{d-2} a multiple of 8");
    }
    p->plane_fft = fft_ok && !(desc->flags & FNO_FLAG_LAST_AXIS_DENSE) &&
                   ((desc->flags & FNO_FLAG_LAST_AXIS_FFT) || fno::plane_fft_default(p));
  }
  {
    const int64_t tiles = (g.P + 63) / 64;
    int64_t gpb = 1024 / g.B;
    if (gpb < 1) gpb = 1;
    if (gpb > tiles) gpb = tiles;
    p->nred = (int)(gpb * g.B);
  }
  // intermediate spectra: the largest is the fully expanded one before the epilogue
  {
    int64_t mx = 0;
    for (int j = -1; j <= g.d - 2; ++j) {
      int64_t v = (int64_t)g.B * cmax * g.mb;
      for (int i = 0; i <= g.d - 2; ++i) v *= (i <= j) ? g.N[i] : 2 * g.M[i];
      if (v > mx) mx = v;
    }
    p->complex_max = mx;
  }
  fno::Workspace& w = p->ws;
  size_t off = 0;
  const int64_t plane_out = (int64_t)g.B * cmax * g.O * 2 * g.ma * g.mb;
  w.plane_part = off;
  off += align_up(sizeof(float2) * (size_t)plane_out * p->nch);
  w.spec_a = off;
  off += align_up(sizeof(float2) * (size_t)p->complex_max);
  w.spec_b = off;
  off += align_up(sizeof(float2) * (size_t)p->complex_max);
  w.xhat = off;
  off += align_up(sizeof(float2) * (size_t)g.B * g.Cin * g.K);
  w.yhat = off;
  off += align_up(sizeof(float2) * (size_t)g.B * cmax * g.K);
  w.red_part = off;
  {
    const int nfast = fno::epilogue_bwd_fast_groups(p);
    const int nparts = nfast > p->nred ? nfast : p->nred;
    off += align_up(sizeof(float) * (size_t)nparts * (g.Cout * g.Cin + g.Cout));
  }
  w.loss_part = off;
  {
    const int nfast = fno::epilogue_fwd_fast_groups(p);
    off += align_up(sizeof(double) * (size_t)(nfast > fno::kMseParts ? nfast : fno::kMseParts));
  }
  w.total = off;
  p->save_off_z = align_up(sizeof(float2) * (size_t)g.B * g.Cin * g.K);
  p->save_bytes = p->save_off_z +
                  ((desc->flags & FNO_FLAG_GELU) ? align_up(sizeof(float) * (size_t)g.B *
                                                            g.Cout * g.P)
                                                 : 0);

  // ---- tables, built in float64 on the host
  std::vector<size_t> root_off(g.d), rootbf_off(g.d);
  size_t toff = 0;
  for (int j = 0; j < g.d; ++j) {
    root_off[j] = toff;
    toff += align_up(sizeof(float2) * g.N[j]);
    rootbf_off[j] = toff;
    toff += align_up(sizeof(float2) * g.N[j]);
  }
  // the epilogues read table fragments K = 64 wide whatever kpad is: the zero tail keeps the
  // last row's over-read in bounds (its products meet zero spectrum columns)
  const size_t gt_elems = (size_t)g.Nb * p->kpad + 64;
  const size_t gt_fwd_off = toff;
  toff += align_up(sizeof(float) * gt_elems);
  const size_t gt_unit_off = toff;
  toff += align_up(sizeof(float) * gt_elems);
  const size_t gt_fwd_bf_off = toff;
  toff += align_up(sizeof(uint16_t) * gt_elems);
  const size_t gt_unit_bf_off = toff;
  toff += align_up(sizeof(uint16_t) * gt_elems);
  const size_t t1_elems = (size_t)g.Nb * p->jpad;
  const size_t f2_elems = (size_t)4 * g.ma * g.Na;
  const size_t t1_off = toff;
  toff += align_up(sizeof(float) * t1_elems);
  const size_t t1_bf_off = toff;
  toff += align_up(sizeof(uint16_t) * t1_elems);
  const size_t t1t_bf_off = toff;  // the same table transposed, [jpad][Nb]
  toff += align_up(sizeof(uint16_t) * t1_elems);
  const size_t f2_off = toff;
  toff += align_up(sizeof(float) * f2_elems);
  const size_t f2_bf_off = toff;
  toff += align_up(sizeof(uint16_t) * f2_elems);
  const size_t f2_bf_lo_off = toff;
  toff += align_up(sizeof(uint16_t) * f2_elems);
  // outer-axis twiddle matrices (axes 0..d-2), rows padded to 16, K halves padded to 16
  size_t oinv_off[fno::kMaxDims][3] = {}, ofwd_off[fno::kMaxDims][3] = {};
  auto p16 = [](int v) { return (v + 15) / 16 * 16; };
  for (int j = 0; j <= g.d - 2; ++j) {
    const size_t ni = (size_t)p16(g.N[j]) * 2 * p16(2 * g.M[j]);
    const size_t nf = (size_t)p16(2 * g.M[j]) * 2 * p16(g.N[j]);
    oinv_off[j][0] = toff;
    toff += align_up(sizeof(float) * ni);
    oinv_off[j][1] = toff;
    toff += align_up(sizeof(uint16_t) * ni);
    oinv_off[j][2] = toff;
    toff += align_up(sizeof(uint16_t) * ni);
    ofwd_off[j][0] = toff;
    toff += align_up(sizeof(float) * nf);
    ofwd_off[j][1] = toff;
    toff += align_up(sizeof(uint16_t) * nf);
    ofwd_off[j][2] = toff;
    toff += align_up(sizeof(uint16_t) * nf);
  }
  const size_t woff_mode_elems = (size_t)g.ncorner * g.Mprod;
  const size_t mode_woff_off = toff;
  toff += align_up(sizeof(int32_t) * (size_t)g.K);
  const size_t woff_mode_off = toff;
  toff += align_up(sizeof(int32_t) * woff_mode_elems);
  const size_t half_flag_off = toff;  // the half-range flag word, uploaded as 0
  toff += align_up(sizeof(int32_t));
  std::vector<unsigned char> host(toff, 0);
  for (int j = 0; j < g.d; ++j) {
    float2* r = reinterpret_cast<float2*>(host.data() + root_off[j]);
    float2* rb = reinterpret_cast<float2*>(host.data() + rootbf_off[j]);
    for (int t = 0; t < g.N[j]; ++t) {
      const double ang = 2.0 * M_PI * (double)t / (double)g.N[j];
      const float c = (float)cos(ang), s = (float)sin(ang);
      r[t] = make_float2(c, s);
      rb[t] = make_float2(round_half_host(c, f16), round_half_host(s, f16));
    }
  }
  {
    // last-axis inverse tables: column 2k = g cos, 2k+1 = -g sin (angle 2 pi ((k p) mod Nb)/Nb)
    float* gf = reinterpret_cast<float*>(host.data() + gt_fwd_off);
    float* gu = reinterpret_cast<float*>(host.data() + gt_unit_off);
    uint16_t* gfb = reinterpret_cast<uint16_t*>(host.data() + gt_fwd_bf_off);
    uint16_t* gub = reinterpret_cast<uint16_t*>(host.data() + gt_unit_bf_off);
    // g / Ntot on unscaled plans; with 1/sqrt(N_j) tables both ways (IEEE half) the last-axis
    // inverse keeps only its own 1/sqrt(Nb), and its half tables also divide out the mix gain
    // (the last inverse stage of the forward and of the input gradient)
    const double inv_ntot = f16 ? 1.0 / sqrt((double)g.Nb) : 1.0 / (double)g.P;
    const double usc = f16 ? 1.0 / sqrt((double)g.Nb) : 1.0;
    const double hf = g.inv_gain[0], hu = g.inv_gain[1];
    for (int pt = 0; pt < g.Nb; ++pt)
      for (int k = 0; k < p->kpad / 2; ++k) {
        double c = 0.0, sn = 0.0, gam = 0.0;
        if (k < g.mb) {
          const double ang = 2.0 * M_PI * (double)(((int64_t)k * pt) % g.Nb) / (double)g.Nb;
          c = cos(ang);
          sn = sin(ang);
          gam = (k == 0 || 2 * k == g.Nb) ? 1.0 : 2.0;
        }
        const size_t e = (size_t)pt * p->kpad + 2 * k;
        gf[e] = (float)(gam * inv_ntot * c);
        gf[e + 1] = (float)(-gam * inv_ntot * sn);
        gu[e] = (float)(usc * c);
        gu[e + 1] = (float)(-usc * sn);
        gfb[e] = half_bits_host(hf * gam * inv_ntot * c, f16);
        gfb[e + 1] = half_bits_host(-hf * gam * inv_ntot * sn, f16);
        gub[e] = half_bits_host(hu * usc * c, f16);
        gub[e + 1] = half_bits_host(-hu * usc * sn, f16);
      }
  }
  {
    // forward plane tables
    float* t1 = reinterpret_cast<float*>(host.data() + t1_off);
    uint16_t* t1b = reinterpret_cast<uint16_t*>(host.data() + t1_bf_off);
    uint16_t* t1bt = reinterpret_cast<uint16_t*>(host.data() + t1t_bf_off);
    for (int c = 0; c < g.Nb; ++c)
      for (int k = 0; k < p->jpad / 2; ++k) {
        double cv = 0.0, sv = 0.0;
        if (k < g.mb) {
          const double ang = 2.0 * M_PI * (double)(((int64_t)k * c) % g.Nb) / (double)g.Nb;
          cv = g.sc[g.d - 1] * cos(ang);
          sv = -g.sc[g.d - 1] * sin(ang);
        }
        const size_t e = (size_t)c * p->jpad + 2 * k;
        t1[e] = (float)cv;
        t1[e + 1] = (float)sv;
        t1b[e] = half_bits_host(cv, f16);
        t1b[e + 1] = half_bits_host(sv, f16);
        t1bt[(size_t)(2 * k) * g.Nb + c] = half_bits_host(cv, f16);
        t1bt[(size_t)(2 * k + 1) * g.Nb + c] = half_bits_host(sv, f16);
      }
    float* f2 = reinterpret_cast<float*>(host.data() + f2_off);
    uint16_t* f2b = reinterpret_cast<uint16_t*>(host.data() + f2_bf_off);
    uint16_t* f2l = reinterpret_cast<uint16_t*>(host.data() + f2_bf_lo_off);
    for (int i = 0; i < 4 * g.ma; ++i) {
      const int sidx = i % (2 * g.ma);
      const int ka = sidx < g.ma ? sidx : g.Na - 2 * g.ma + sidx;
      for (int row = 0; row < g.Na; ++row) {
        const double ang = 2.0 * M_PI * (double)(((int64_t)ka * row) % g.Na) / (double)g.Na;
        const double v = g.sc[g.d - 2] * (i < 2 * g.ma ? cos(ang) : sin(ang));
        const size_t e = (size_t)i * g.Na + row;
        f2[e] = (float)v;
        f2b[e] = half_bits_host(v, f16);
        f2l[e] = half_bits_host(v - half_value_host(f2b[e], f16), f16);
      }
    }
  }
  for (int j = 0; j <= g.d - 2; ++j) {
    const int N = g.N[j], m = g.M[j];
    const int Np = p16(N), Mp = p16(2 * m);
    const double scj = g.sc[j];  // 1/sqrt(N_j) on IEEE-half plans, both directions
    auto put = [&](size_t* off, size_t e, double v0) {
      const double v = scj * v0;
      reinterpret_cast<float*>(host.data() + off[0])[e] = (float)v;
      const uint16_t hi = half_bits_host(v, f16);
      reinterpret_cast<uint16_t*>(host.data() + off[1])[e] = hi;
      reinterpret_cast<uint16_t*>(host.data() + off[2])[e] =
          half_bits_host(v - half_value_host(hi, f16), f16);
    };
    for (int pt = 0; pt < N; ++pt)
      for (int sidx = 0; sidx < 2 * m; ++sidx) {
        const int k = sidx < m ? sidx : N - 2 * m + sidx;
        const double ang = 2.0 * M_PI * (double)(((int64_t)k * pt) % N) / (double)N;
        // inverse: row pt, K = [cos | sin] over retained positions
        put(oinv_off[j], (size_t)pt * 2 * Mp + sidx, cos(ang));
        put(oinv_off[j], (size_t)pt * 2 * Mp + Mp + sidx, sin(ang));
        // forward: row sidx, K = [cos | -sin] over grid points
        put(ofwd_off[j], (size_t)sidx * 2 * Np + pt, cos(ang));
        put(ofwd_off[j], (size_t)sidx * 2 * Np + Np + pt, -sin(ang));
      }
  }
  {
    int32_t* mw = reinterpret_cast<int32_t*>(host.data() + mode_woff_off);
    int32_t* wm = reinterpret_cast<int32_t*>(host.data() + woff_mode_off);
    int dims[fno::kMaxDims];
    for (int j = 0; j < g.d; ++j) dims[j] = (j == g.d - 1) ? g.M[j] : 2 * g.M[j];
    for (int64_t t = 0; t < g.K; ++t) {
      int64_t r = t;
      int s[fno::kMaxDims];
      for (int j = g.d - 1; j >= 0; --j) {
        s[j] = (int)(r % dims[j]);
        r /= dims[j];
      }
      int corner = 0;
      int64_t kap = 0;
      for (int j = 0; j < g.d; ++j) {
        int kj = s[j];
        if (j < g.d - 1 && kj >= g.M[j]) {
          corner |= 1 << j;
          kj -= g.M[j];
        }
        kap = kap * g.M[j] + kj;
      }
      mw[t] = (int32_t)((int64_t)corner * g.Cin * g.Cout * g.Mprod + kap);
      wm[(int64_t)corner * g.Mprod + kap] = (int32_t)t;
    }
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    delete p;
    return hip_fail(e, "hipGetDevice");
  }
  p->device = dev;
  void* mem = nullptr;
  e = hipMalloc(&mem, toff);
  if (e != hipSuccess) {
    delete p;
    return hip_fail(e, "hipMalloc(plan tables)");
  }
  e = hipMemcpy(mem, host.data(), toff, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(mem);
    delete p;
    return hip_fail(e, "hipMemcpy(plan tables)");
  }
  p->table_mem = mem;
  unsigned char* base = static_cast<unsigned char*>(mem);
  for (int j = 0; j < fno::kMaxDims; ++j) {
    p->t.root[j] = j < g.d ? reinterpret_cast<const float2*>(base + root_off[j]) : nullptr;
    p->t.root_bf[j] = j < g.d ? reinterpret_cast<const float2*>(base + rootbf_off[j]) : nullptr;
  }
  p->t.gt_fwd = reinterpret_cast<const float*>(base + gt_fwd_off);
  p->t.gt_unit = reinterpret_cast<const float*>(base + gt_unit_off);
  p->t.gt_fwd_bf = reinterpret_cast<const uint16_t*>(base + gt_fwd_bf_off);
  p->t.gt_unit_bf = reinterpret_cast<const uint16_t*>(base + gt_unit_bf_off);
  p->t.t1 = reinterpret_cast<const float*>(base + t1_off);
  p->t.t1_bf = reinterpret_cast<const uint16_t*>(base + t1_bf_off);
  p->t.t1t_bf = reinterpret_cast<const uint16_t*>(base + t1t_bf_off);
  p->t.f2 = reinterpret_cast<const float*>(base + f2_off);
  p->t.f2_bf = reinterpret_cast<const uint16_t*>(base + f2_bf_off);
  p->t.f2_bf_lo = reinterpret_cast<const uint16_t*>(base + f2_bf_lo_off);
  for (int j = 0; j <= g.d - 2; ++j) {
    p->t.oinv[j] = reinterpret_cast<const float*>(base + oinv_off[j][0]);
    p->t.oinv_bf[j] = reinterpret_cast<const uint16_t*>(base + oinv_off[j][1]);
    p->t.oinv_bf_lo[j] = reinterpret_cast<const uint16_t*>(base + oinv_off[j][2]);
    p->t.ofwd[j] = reinterpret_cast<const float*>(base + ofwd_off[j][0]);
    p->t.ofwd_bf[j] = reinterpret_cast<const uint16_t*>(base + ofwd_off[j][1]);
    p->t.ofwd_bf_lo[j] = reinterpret_cast<const uint16_t*>(base + ofwd_off[j][2]);
  }
  p->t.mode_woff = reinterpret_cast<const int32_t*>(base + mode_woff_off);
  p->t.woff_mode = reinterpret_cast<const int32_t*>(base + woff_mode_off);
  p->g.half_flag = g.half == 2 ? reinterpret_cast<int*>(base + half_flag_off) : nullptr;
  *out = p;
  return FNO_OK;
}

fno_status fno_plan_destroy(fno_plan* p) {
  if (!p) return FNO_OK;
  hipError_t e = hipSuccess;
  if (p->table_mem) e = hipFree(p->table_mem);
  delete p;
  if (e != hipSuccess) return hip_fail(e, "hipFree(plan tables)");
  return FNO_OK;
}

fno_status fno_plan_half_range(const fno_plan* p, int* exceeded, int clear) {
  if (!p) return fail(FNO_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!exceeded) return fail(FNO_ERR_INVALID_ARGUMENT, "exceeded is NULL");
  *exceeded = 0;
  int* flag = p->g.half_flag;
  if (!flag) return FNO_OK;  // only IEEE-half plans keep the flag
  int dev = -1;
  FNO_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev != p->device)
    return fail(FNO_ERR_INVALID_ARGUMENT, "current device %d is not the plan's device %d", dev,
                p->device);
  int v = 0;
  FNO_HIP(hipMemcpy(&v, flag, sizeof(int), hipMemcpyDeviceToHost), "hipMemcpy(half flag)");
  *exceeded = v != 0;
  if (clear) FNO_HIP(hipMemset(flag, 0, sizeof(int)), "hipMemset(half flag)");
  return FNO_OK;
}

fno_status fno_plan_last_axis_fft(const fno_plan* p, int* fft) {
  if (!p) return fail(FNO_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!fft) return fail(FNO_ERR_INVALID_ARGUMENT, "fft is NULL");
  *fft = p->plane_fft ? 1 : 0;
  return FNO_OK;
}

fno_status fno_plan_query(const fno_plan* p, size_t* ws, size_t* save, size_t* wel) {
  if (!p) return fail(FNO_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (ws) *ws = p->ws.total;
  if (save) *save = p->save_bytes;
  if (wel) *wel = (size_t)p->g.ncorner * p->g.Cin * p->g.Cout * p->g.Mprod;
  return FNO_OK;
}

}  // extern "C"

namespace {

#define REQ(ptr, name)                                                       \
  do {                                                                       \
    if (!(ptr)) return fail(FNO_ERR_INVALID_ARGUMENT, "%s is NULL", name);   \
    if (!aligned16(ptr))                                                     \
      return fail(FNO_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name); \
  } while (0)

#define OPT(ptr, name)                                                       \
  do {                                                                       \
    if ((ptr) && !aligned16(ptr))                                            \
      return fail(FNO_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name); \
  } while (0)

// Every kernel launch goes through LAUNCH(name, stream, call): `name` keys the optional
// per-kernel event timer (fno_timing_*).
#define LAUNCH(name, strm, call)                                          \
  do {                                                                    \
    hipError_t e_ = timed_launch(name, strm, [&]() { return (call); });   \
    if (e_ != hipSuccess) return hip_fail(e_, name);                      \
  } while (0)

struct TimingState {
  std::mutex mu;
  bool on = false;
  std::string only;  // when not empty: time only the launches of this name
  struct Pending {
    const char* name;
    hipEvent_t a, b;
  };
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;
  std::vector<std::string> names;
  std::vector<int64_t> launches;
  std::vector<double> total_ms;
};

TimingState& timing_state() {
  static TimingState* t = new TimingState();  // never destroyed: usable at exit
  return *t;
}

hipEvent_t timing_event(TimingState& T) {
  if (!T.pool.empty()) {
    hipEvent_t e = T.pool.back();
    T.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Launch through `launch`; when the timer is on, bracket it with two events on `s`.
template <typename F>
hipError_t timed_launch(const char* name, hipStream_t s, F&& launch) {
  TimingState& T = timing_state();
  hipEvent_t a = nullptr, b = nullptr;
  {
    std::lock_guard<std::mutex> lk(T.mu);
    if (!T.on || (!T.only.empty() && T.only != name)) return launch();
    a = timing_event(T);
    b = timing_event(T);
  }
  if (!a || !b) return launch();
  hipError_t e = hipEventRecord(a, s);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, s);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(T.mu);
  T.pending.push_back({name, a, b});
  return hipSuccess;
}

// Wait for every recorded pair and fold it into the per-name totals (caller holds T.mu).
hipError_t timing_collect(TimingState& T) {
  for (auto& r : T.pending) {
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return e;
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return e;
    size_t i = 0;
    while (i < T.names.size() && T.names[i] != r.name) ++i;
    if (i == T.names.size()) {
      T.names.push_back(r.name);
      T.launches.push_back(0);
      T.total_ms.push_back(0.0);
    }
    T.launches[i] += 1;
    T.total_ms[i] += ms;
    T.pool.push_back(r.a);
    T.pool.push_back(r.b);
  }
  T.pending.clear();
  return hipSuccess;
}

const char* plane_name(int plane_in) {
  switch (plane_in) {
    case fno::PLANE_TANH: return "plane_fwd_tanh";
    case fno::PLANE_GELU: return "plane_fwd_gelu";
    case fno::PLANE_TANH_GELU: return "plane_fwd_tanh_gelu";
    case fno::PLANE_GELU_GRAD: return "plane_fwd_gelugrad";
    default: return "plane_fwd";
  }
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<unsigned char*>(base) + off);
}

// Forward transform of a field (channels `chans`) into the retained spectrum `dst`
// [B][chans][K]:  plane transform of the last two axes, then the remaining outer axes.
fno_status forward_transform(const fno_plan* p, int plane_in, int chans, const float* in0,
                             const float* in1, float2* dst, void* ws, hipStream_t s) {
  const fno::Geom& g = p->g;
  float2* part = at<float2>(ws, p->ws.plane_part);
  float2* ping = at<float2>(ws, p->ws.spec_a);
  float2* pong = at<float2>(ws, p->ws.spec_b);
  const int64_t plane_out = (int64_t)g.B * chans * g.O * 2 * g.ma * g.mb;
  const bool more = g.d > 2;
  float2* plane_dst = (p->nch == 1) ? (more ? ping : dst) : part;
  LAUNCH(plane_name(plane_in), s, fno::launch_plane_fwd(p, plane_in, chans, in0, in1, plane_dst, s));
  float2* cur = plane_dst;
  if (p->nch > 1) {
    float2* rd = more ? ping : dst;
    LAUNCH("reduce_parts", s, fno::launch_reduce_parts(part, p->nch, plane_out, plane_out, rd, s));
    cur = rd;
  }
  for (int j = g.d - 3; j >= 0; --j) {
    float2* nxt = (j == 0) ? dst : (cur == ping ? pong : ping);
    LAUNCH("outer_fwd", s, fno::launch_outer_fwd(p, j, chans, cur, 1, 0, nxt, s));
    cur = nxt;
  }
  return FNO_OK;
}

// Inverse transform of the outer axes 0..naxes-1 of a spectrum [B][chans][K]: all of
// 0..d-2 (naxes = d-1) gives T [B][chans][lines][mb]; returns the buffer holding the result
// (src itself when naxes = 0).
// half_last: the last axis's result in the plan's half format (see half_T).
fno_status inverse_outer(const fno_plan* p, int chans, const float2* src, void* ws,
                         hipStream_t s, const float2** T, int naxes, bool half_last = false) {
  float2* ping = at<float2>(ws, p->ws.spec_a);
  float2* pong = at<float2>(ws, p->ws.spec_b);
  const float2* cur = src;
  for (int j = 0; j < naxes; ++j) {
    float2* nxt = (cur == ping) ? pong : ping;
    if (half_last && j == naxes - 1)
      LAUNCH("outer_inv", s, fno::launch_outer_mfma_half(p, j, chans, cur,
                                                         reinterpret_cast<uint16_t*>(nxt), s));
    else
      LAUNCH("outer_inv", s, fno::launch_outer_inv(p, j, chans, cur, nxt, s));
    cur = nxt;
  }
  *T = cur;
  return FNO_OK;
}

// T (the spectrum after the outer inverses) goes to the width-64 matrix-core line epilogue of a
// half plan in that plan's half format: the epilogue rounds T to it when it stages a line, so
// the outer inverse rounds it instead (the same bits) and T's bytes halve.
bool half_T(const fno_plan* p, int chans) {
  const fno::Geom& g = p->g;
  return g.bf16 && chans == 64 && g.d >= 2 && fno::outer_fast_ok(p, g.d - 2, true) &&
         2 * g.mb >= 64;
}

fno_status check_ws(const fno_plan* p, void* ws, size_t ws_bytes) {
  REQ(ws, "workspace");
  if (ws_bytes < p->ws.total)
    return fail(FNO_ERR_INVALID_ARGUMENT, "workspace %zu bytes < required %zu", ws_bytes,
                p->ws.total);
  return FNO_OK;
}

int pre_mode(const fno_plan* p) {
  const bool t = (p->desc.flags & FNO_FLAG_TANH_PREACT) != 0;
  if (p->desc.flags & FNO_FLAG_INPUT_GELU) return t ? fno::PLANE_TANH_GELU : fno::PLANE_GELU;
  return t ? fno::PLANE_TANH : fno::PLANE_X;
}

// The spectral-weight step of a block: the dense per-mode mix, or a Tucker-factorised one.
struct WeightMix {
  virtual ~WeightMix() = default;
  // xhat [B][Cin][K] -> yhat [B][Cout][K]
  virtual fno_status fwd(const float2* xhat, float2* yhat, void* ws, hipStream_t s) const = 0;
  // ghat [B][Cout][K] -> ghx [B][Cin][K] (when ghx is non-null) and the weight gradients
  // (when wanted; they read xhat)
  virtual fno_status bwd(const float2* xhat, const float2* ghat, float2* ghx, void* ws,
                         hipStream_t s) const = 0;
  virtual bool wants_weight_grad() const = 0;
};

struct DenseMix final : WeightMix {
  const fno_plan* p;
  const float2* w;
  float2* grad_w;
  DenseMix(const fno_plan* p_, const float* w_, float* gw_)
      : p(p_), w(reinterpret_cast<const float2*>(w_)), grad_w(reinterpret_cast<float2*>(gw_)) {}
  fno_status fwd(const float2* xhat, float2* yhat, void*, hipStream_t s) const override {
    LAUNCH("mix_fwd", s, fno::launch_mix_fwd(p, xhat, 1, 0, w, yhat, s));
    return FNO_OK;
  }
  fno_status bwd(const float2* xhat, const float2* ghat, float2* ghx, void*,
                 hipStream_t s) const override {
    // one launch for both unless ghx overwrites the xhat that the weight gradient reads (a
    // recomputed spectrum shares its workspace region): then the weight gradient goes first
    if (grad_w && ghx && static_cast<const void*>(ghx) != static_cast<const void*>(xhat)) {
      LAUNCH("mix_bwd", s, fno::launch_mix_bwd_both(p, xhat, ghat, w, ghx, grad_w, s));
      return FNO_OK;
    }
    if (grad_w) LAUNCH("mix_bwd_dw", s, fno::launch_mix_bwd_dw(p, xhat, ghat, grad_w, s));
    if (ghx) LAUNCH("mix_bwd_dx", s, fno::launch_mix_bwd_dx(p, ghat, w, ghx, s));
    return FNO_OK;
  }
  bool wants_weight_grad() const override { return grad_w != nullptr; }
};

// The inverse of the outer axes and the forward epilogue of a block (mode EPI_BLOCK, or
// EPI_BLOCK_PREACT for z without the output GELU) from the mixed spectrum yhat.
fno_status block_epilogue_fwd(const fno_plan* p, int mode, const float2* yhat, const float* x,
                              const float* wb, const float* bias, float* y, float* zsave,
                              void* ws, hipStream_t s) {
  const float2* T = nullptr;
  fno_status st;
  if (fno::epilogue_rows_ok(p, mode, x, y, zsave)) {
    // half plans: the last outer inverse writes T in the half format the epilogue rounds it to
    const int d = p->g.d;
    const bool th = d >= 3 && fno::outer_inv_half_ok(p, d - 3);
    st = inverse_outer(p, p->g.Cout, yhat, ws, s, &T, d - 2, th);
    if (st != FNO_OK) return st;
    // timer names tell launches that also save z apart (their bytes differ)
    LAUNCH(zsave ? "epilogue_rows_fwd_zsave" : "epilogue_rows_fwd", s,
           fno::launch_epilogue_rows(p, mode, T, x, wb, bias, y, zsave, s, th));
    return FNO_OK;
  }
  const bool fast = fno::epilogue_fast_ok(p, mode, true);
  const bool th = fast && half_T(p, p->g.Cout);
  st = inverse_outer(p, p->g.Cout, yhat, ws, s, &T, p->g.d - 1, th);
  if (st != FNO_OK) return st;
  if (fast)
    LAUNCH(zsave ? "epilogue_fwd_zsave" : "epilogue_fwd", s,
           fno::launch_epilogue_fwd_fast(p, mode, T, x, wb, bias, y, zsave, s, th));
  else
    LAUNCH(zsave ? "epilogue_fwd_zsave" : "epilogue_fwd", s,
           fno::launch_epilogue_fwd(p, mode, T, x, wb, bias, y, zsave, s));
  return FNO_OK;
}

// Block forward after argument checks: transform, weight step, inverse + epilogue.
fno_status block_fwd_impl(const fno_plan* p, const float* x, const float* wb, const float* bias,
                          float* y, void* save, void* ws, hipStream_t s, const WeightMix& mix) {
  float2* xhat = save ? static_cast<float2*>(save) : at<float2>(ws, p->ws.xhat);
  fno_status st = forward_transform(p, pre_mode(p), p->g.Cin, x, nullptr, xhat, ws, s);
  if (st != FNO_OK) return st;
  float2* yhat = at<float2>(ws, p->ws.yhat);
  st = mix.fwd(xhat, yhat, ws, s);
  if (st != FNO_OK) return st;
  float* zsave = (save && (p->desc.flags & FNO_FLAG_GELU)) ? at<float>(save, p->save_off_z)
                                                            : nullptr;
  return block_epilogue_fwd(p, fno::EPI_BLOCK, yhat, x, wb, bias, y, zsave, ws, s);
}

// Block forward fused with the MSE loss against `tgt`: grad_z = grad_scale 2 (y - t) / n
// GELU'(z) and, when `loss` is given, loss = mean((y - t)^2).  The matrix-core epilogue does
// it in one pass over the field; the other epilogues write z into grad_z and a pointwise pass
// turns it into the gradient in place.
fno_status block_fwd_mse_impl(const fno_plan* p, const float* x, const float* wb,
                              const float* bias, const float* tgt, float grad_scale,
                              float* grad_z, float* loss, void* save, void* ws, hipStream_t s,
                              const WeightMix& mix) {
  const fno::Geom& g = p->g;
  float2* xhat = save ? static_cast<float2*>(save) : at<float2>(ws, p->ws.xhat);
  fno_status st = forward_transform(p, pre_mode(p), g.Cin, x, nullptr, xhat, ws, s);
  if (st != FNO_OK) return st;
  float2* yhat = at<float2>(ws, p->ws.yhat);
  st = mix.fwd(xhat, yhat, ws, s);
  if (st != FNO_OK) return st;
  const int64_t n = (int64_t)g.B * g.Cout * g.P;
  double* lpart = at<double>(ws, p->ws.loss_part);
  int nparts = fno::kMseParts;
  if (fno::epilogue_fast_ok(p, fno::EPI_BLOCK, true)) {
    const float2* T = nullptr;
    const bool th = half_T(p, g.Cout);
    st = inverse_outer(p, g.Cout, yhat, ws, s, &T, g.d - 1, th);
    if (st != FNO_OK) return st;
    const float msc = (float)(2.0 * (double)grad_scale / (double)n);
    LAUNCH("epilogue_fwd_mse", s,
           fno::launch_epilogue_fwd_mse(p, T, x, wb, bias, tgt, msc, grad_z, lpart, s, th));
    nparts = fno::epilogue_fwd_fast_groups(p);
  } else {
    st = block_epilogue_fwd(p, fno::EPI_BLOCK_PREACT, yhat, x, wb, bias, grad_z, nullptr, ws, s);
    if (st != FNO_OK) return st;
    const bool gelu = (p->desc.flags & FNO_FLAG_GELU) != 0;
    LAUNCH("mse_preact", s,
           fno::launch_mse_preact(n, tgt, grad_z, gelu, grad_scale, lpart, nparts, s));
  }
  if (loss) LAUNCH("mse_finish", s, fno::launch_mse_finish(n, nparts, lpart, loss, s));
  return FNO_OK;
}

// Block backward after argument checks.  With `preact`, gy is the gradient at the
// pre-activation z (the output GELU's derivative already applied) and z is not read.
fno_status block_bwd_impl(const fno_plan* p, const float* x, const float* wb, const void* save,
                          const float* gy, float* grad_x, float* grad_wb, float* grad_bias,
                          void* ws, hipStream_t s, const WeightMix& mix, bool preact = false) {
  const fno::Geom& g = p->g;
  const bool gelu = (p->desc.flags & FNO_FLAG_GELU) != 0 && !preact;
  const float* z = gelu ? at<const float>(const_cast<void*>(save), p->save_off_z) : nullptr;
  float2* ghat = at<float2>(ws, p->ws.yhat);
  fno_status st = forward_transform(p, gelu ? fno::PLANE_GELU_GRAD : fno::PLANE_X, g.Cout, gy,
                                    z, ghat, ws, s);
  if (st != FNO_OK) return st;
  float2* ghx = grad_x ? at<float2>(ws, p->ws.xhat) : nullptr;
  if (mix.wants_weight_grad() || ghx) {
    st = mix.bwd(static_cast<const float2*>(save), ghat, ghx, ws, s);
    if (st != FNO_OK) return st;
  }
  float* red = (grad_wb || grad_bias) ? at<float>(ws, p->ws.red_part) : nullptr;
  if (grad_x || red) {
    const float2* Tg = nullptr;
    const bool fast = fno::epilogue_bwd_fast(p, fno::EPI_BLOCK, grad_x);
    const bool th = fast && half_T(p, g.Cin);
    if (grad_x) {
      st = inverse_outer(p, g.Cin, ghx, ws, s, &Tg, g.d - 1, th);
      if (st != FNO_OK) return st;
    }
    // with the output GELU the epilogue also reads z (another field)
    if (fast)
      LAUNCH(z ? "epilogue_bwd_gelu" : "epilogue_bwd", s,
             fno::launch_epilogue_bwd_fast(p, fno::EPI_BLOCK, Tg, x, wb, gy, z, grad_x, red, s,
                                           th));
    else
      LAUNCH(z ? "epilogue_bwd_gelu" : "epilogue_bwd", s,
             fno::launch_epilogue_bwd(p, fno::EPI_BLOCK, Tg, x, wb, gy, z, grad_x, red, s));
    if (red)
      LAUNCH("bypass_grad_finish", s, fno::launch_bypass_grad_finish(p, red, grad_wb, grad_bias, grad_x, s));
  }
  return FNO_OK;
}

// Spectral convolution alone (no bypass, bias or GELU) after argument checks.
fno_status spectral_fwd_impl(const fno_plan* p, const float* x, float* y_spec, void* save,
                             void* ws, hipStream_t s, const WeightMix& mix) {
  float2* xhat = save ? static_cast<float2*>(save) : at<float2>(ws, p->ws.xhat);
  fno_status st = forward_transform(p, pre_mode(p), p->g.Cin, x, nullptr, xhat, ws, s);
  if (st != FNO_OK) return st;
  float2* yhat = at<float2>(ws, p->ws.yhat);
  st = mix.fwd(xhat, yhat, ws, s);
  if (st != FNO_OK) return st;
  const float2* T = nullptr;
  if (fno::epilogue_rows_ok(p, fno::EPI_SPECTRAL, x, y_spec, nullptr)) {
    st = inverse_outer(p, p->g.Cout, yhat, ws, s, &T, p->g.d - 2);
    if (st != FNO_OK) return st;
    LAUNCH("epilogue_rows_spec_fwd", s, fno::launch_epilogue_rows(p, fno::EPI_SPECTRAL, T, x, nullptr, nullptr, y_spec, nullptr, s));
    return FNO_OK;
  }
  st = inverse_outer(p, p->g.Cout, yhat, ws, s, &T, p->g.d - 1);
  if (st != FNO_OK) return st;
  LAUNCH("epilogue_spec_fwd", s, fno::launch_epilogue_fwd(p, fno::EPI_SPECTRAL, T, x, nullptr, nullptr, y_spec, nullptr,
                                  s));
  return FNO_OK;
}

// Its backward: the weight gradients read the retained spectrum (from save, else recomputed).
fno_status spectral_bwd_impl(const fno_plan* p, const float* x, const void* save,
                             const float* gys, float* grad_x, void* ws, hipStream_t s,
                             const WeightMix& mix) {
  const fno::Geom& g = p->g;
  float2* ghat = at<float2>(ws, p->ws.yhat);
  const float2* xhat = static_cast<const float2*>(save);
  fno_status st;
  if (mix.wants_weight_grad() && !xhat) {
    float2* xh = at<float2>(ws, p->ws.xhat);
    st = forward_transform(p, pre_mode(p), g.Cin, x, nullptr, xh, ws, s);
    if (st != FNO_OK) return st;
    xhat = xh;
  }
  st = forward_transform(p, fno::PLANE_X, g.Cout, gys, nullptr, ghat, ws, s);
  if (st != FNO_OK) return st;
  float2* ghx = grad_x ? at<float2>(ws, p->ws.xhat) : nullptr;
  if (mix.wants_weight_grad() || ghx) {
    st = mix.bwd(xhat, ghat, ghx, ws, s);
    if (st != FNO_OK) return st;
  }
  if (grad_x) {
    const float2* Tg = nullptr;
    st = inverse_outer(p, g.Cin, ghx, ws, s, &Tg, g.d - 1);
    if (st != FNO_OK) return st;
    LAUNCH("epilogue_spec_bwd", s, fno::launch_epilogue_bwd(p, fno::EPI_SPECTRAL, Tg, x, nullptr, nullptr, nullptr,
                                    grad_x, nullptr, s));
  }
  return FNO_OK;
}

}  // namespace

// A Tucker-factorised weight bound to a plan: the greedy contraction order, the mix geometry
// and the layout of its buffers behind the plan's own part of the workspace.
struct fno_tucker {
  const fno_plan* plan;
  fno::TuckerDims dims;
  int nf;                                   // factors: d + 2
  std::vector<fno::TuckerStep> steps;
  std::string order;
  int core_steps;
  bool in_on_data, out_on_data;
  fno::Geom gmix;                           // the plan's geometry with the mix's channels
  // U_in / U_out on the spectrum as fp32 mix launches with one weight for every mode:
  // g_in (C_in -> R_in; adjoint R_in -> C_in), g_out (R_out -> C_out; adjoint C_out -> R_out)
  fno::Geom g_in, g_out;
  int32_t* ident_woff;                      // device [2 K]: [0, K) t -> t, then K zeros
  const int32_t* zero_woff;
  int64_t K;
  int64_t core_elems;
  int64_t factor_elems[2 + fno::kMaxDims];
  std::vector<size_t> chain_off;            // result of each core step
  size_t g0_off, g1_off, x1_off, t2_off, u_off, v_off, part_off, total;
  // with `keep`, the save buffer continues after the plan's part with the forward's weight-step
  // intermediates (each core step's result, U_in xhat, the mix output before U_out), which the
  // backward then reads instead of recomputing
  bool keep = false;
  std::vector<size_t> keep_chain_off;
  size_t keep_x1_off = 0, keep_t2_off = 0, keep_total = 0;
};

namespace {

fno_status tucker_dims(const fno_plan_desc* d, const int32_t* ranks, fno::TuckerDims* t) {
  if (!ranks) return fail(FNO_ERR_INVALID_ARGUMENT, "ranks is NULL");
  fno_status st = fno_plan_validate(d);
  if (st != FNO_OK) return st;
  t->d = d->ndim;
  t->B = d->batch;
  t->Cin = (int)d->c_in;
  t->Cout = (int)d->c_out;
  for (int j = 0; j < t->d; ++j) t->K[j] = (int)(j < t->d - 1 ? 2 * d->modes[j] : d->modes[j]);
  const int ext[2] = {t->Cin, t->Cout};
  for (int n = 0; n < t->d + 2; ++n) {
    const int full = n < 2 ? ext[n] : t->K[n - 2];
    if (ranks[n] < 1 || ranks[n] > full)
      return fail(FNO_ERR_INVALID_ARGUMENT, "rank %d of mode %d outside 1..%d", ranks[n], n,
                  full);
    t->R[n] = ranks[n];
  }
  return FNO_OK;
}

const float2* f2c(const float* p) { return reinterpret_cast<const float2*>(p); }

// The Tucker-factorised weight step (the greedy order of tucker.hip).
struct TuckerMix final : WeightMix {
  const fno_tucker* t;
  const float2* core;
  const float* const* fac;
  float2* grad_core;
  float* const* grad_fac;  // may be null (forward)
  bool want_w;
  unsigned char* kept;     // the save buffer when it carries the kept intermediates, else null
  TuckerMix(const fno_tucker* t_, const float* core_, const float* const* fac_,
            float* gcore, float* const* gfac, const void* save = nullptr)
      : t(t_), core(f2c(core_)), fac(fac_), grad_core(reinterpret_cast<float2*>(gcore)),
        grad_fac(gfac) {
    want_w = grad_core != nullptr;
    for (int n = 0; gfac && n < t->nf; ++n) want_w = want_w || gfac[n] != nullptr;
    kept = (t->keep && save) ? static_cast<unsigned char*>(const_cast<void*>(save)) : nullptr;
  }
  // the buffer of core step si's result: the save buffer's slot when kept
  float2* chain_buf(void* ws, int si) const {
    return kept ? reinterpret_cast<float2*>(kept + t->keep_chain_off[si])
                : at<float2>(ws, t->chain_off[si]);
  }
  float2* gf(int n) const { return grad_fac ? reinterpret_cast<float2*>(grad_fac[n]) : nullptr; }
  bool wants_weight_grad() const override { return want_w; }

  // the core's lineage: every core step in order; in[si] = the input of step si
  // compute: run the products (else the kept results of the forward are only pointed at)
  fno_status core_chain(void* ws, hipStream_t s, std::vector<const float2*>* in,
                        const float2** H, bool compute = true) const {
    const float2* cur = core;
    int si = 0;
    for (const fno::TuckerStep& st : t->steps) {
      if (st.kind != fno::TuckerStep::CORE) continue;
      float2* out = chain_buf(ws, si);
      if (in) (*in)[si] = cur;
      if (compute)
        LAUNCH("tucker_core", s, fno::launch_mode_product(st.pre, st.an, st.cn, st.post,
                                                          f2c(fac[st.factor]), false, false,
                                                          cur, out, s));
      cur = out;
      ++si;
    }
    *H = cur;
    return FNO_OK;
  }

  fno_status fwd(const float2* xhat, float2* yhat, void* ws, hipStream_t s) const override {
    const float2* H = nullptr;
    fno_status st = core_chain(ws, s, nullptr, &H);
    if (st != FNO_OK) return st;
    const float2* data = xhat;
    if (t->in_on_data) {
      float2* x1 = kept ? reinterpret_cast<float2*>(kept + t->keep_x1_off)
                        : at<float2>(ws, t->x1_off);
      LAUNCH("tucker_data", s, fno::launch_mix_fwd_g(t->g_in, t->zero_woff, xhat, f2c(fac[0]),
                                                     x1, s));
      data = x1;
    }
    float2* mixed = !t->out_on_data ? yhat
                    : kept          ? reinterpret_cast<float2*>(kept + t->keep_t2_off)
                                    : at<float2>(ws, t->t2_off);
    LAUNCH("tucker_mix_fwd", s, fno::launch_mix_fwd_g(t->gmix, t->ident_woff, data, H, mixed, s));
    if (t->out_on_data)
      LAUNCH("tucker_data", s, fno::launch_mix_fwd_g(t->g_out, t->zero_woff, mixed, f2c(fac[1]),
                                                     yhat, s));
    return FNO_OK;
  }

  fno_status bwd(const float2* xhat, const float2* ghat, float2* ghx, void* ws,
                 hipStream_t s) const override {
    const fno::TuckerDims& d = t->dims;
    const fno::Geom& g = t->plan->g;
    float2* part = at<float2>(ws, t->part_off);
    std::vector<const float2*> chain_in(t->core_steps, nullptr);
    const float2* H = nullptr;
    fno_status st = core_chain(ws, s, &chain_in, &H, kept == nullptr);
    if (st != FNO_OK) return st;
    // u = ghat with U_out's conjugate applied (when U_out acts on the data side)
    const float2* u = ghat;
    if (t->out_on_data) {
      float2* ub = at<float2>(ws, t->u_off);
      LAUNCH("tucker_data", s, fno::launch_mix_bwd_dx_g(t->g_out, t->zero_woff, ghat,
                                                        f2c(fac[1]), ub, s));
      u = ub;
    }
    float2* gH = at<float2>(ws, t->g0_off);
    if (want_w) {
      const float2* data = xhat;
      if (t->in_on_data && kept) {
        data = reinterpret_cast<const float2*>(kept + t->keep_x1_off);
      } else if (t->in_on_data) {
        float2* x1 = at<float2>(ws, t->x1_off);
        LAUNCH("tucker_data", s, fno::launch_mix_fwd_g(t->g_in, t->zero_woff, xhat, f2c(fac[0]),
                                                       x1, s));
        data = x1;
      }
      // gradient of the core-side tensor the mix reads
      LAUNCH("tucker_mix_dw", s, fno::launch_mix_bwd_dw_g(t->gmix, t->ident_woff, data, u, gH, s));
      if (t->out_on_data && gf(1)) {
        float2* t2 = kept ? reinterpret_cast<float2*>(kept + t->keep_t2_off)
                          : at<float2>(ws, t->t2_off);
        if (!kept)
          LAUNCH("tucker_mix_fwd", s,
                 fno::launch_mix_fwd_g(t->gmix, t->ident_woff, data, H, t2, s));
        LAUNCH("tucker_gram_data", s, fno::launch_gram(d.B, d.Cout, d.R[1], t->K, ghat, t2, true,
                                                  g.mb, g.Nb, g.adj_scale, g.inv_gain[0], false,
                                                  part, gf(1), s));
      }
    }
    // v = the mix's adjoint of u; the input gradient spectrum, or it before U_in
    const bool need_v = ghx || (t->in_on_data && gf(0));
    if (need_v) {
      float2* v = t->in_on_data ? at<float2>(ws, t->v_off) : ghx;
      LAUNCH("tucker_mix_dx", s, fno::launch_mix_bwd_dx_g(t->gmix, t->ident_woff, u, H, v, s));
      if (t->in_on_data) {
        // the U_in gradient reads xhat, so it goes before ghx (which may reuse xhat's slot)
        if (gf(0))
          LAUNCH("tucker_gram_data", s, fno::launch_gram(d.B, d.Cin, d.R[0], t->K, xhat, v, false,
                                                    g.mb, g.Nb, 1.0f, g.inv_gain[1], true,
                                                    part, gf(0), s));
        if (ghx)
          LAUNCH("tucker_data", s, fno::launch_mix_bwd_dx_g(t->g_in, t->zero_woff, v,
                                                            f2c(fac[0]), ghx, s));
      }
    }
    if (!want_w) return FNO_OK;
    // the core's lineage in reverse: factor gradients, then the gradient of each step's input
    float2* cur = gH;
    float2* other = at<float2>(ws, t->g1_off);
    int si = t->core_steps - 1;
    for (int k = (int)t->steps.size() - 1; k >= 0; --k) {
      const fno::TuckerStep& stp = t->steps[k];
      if (stp.kind != fno::TuckerStep::CORE) continue;
      if (gf(stp.factor))
        LAUNCH("tucker_gram_core", s, fno::launch_gram(stp.pre, stp.an, stp.cn, stp.post, cur,
                                                  chain_in[si], false, g.mb, g.Nb, 1.0f, 1.0f,
                                                  false, part, gf(stp.factor), s));
      float2* dst = si == 0 ? grad_core : other;
      if (dst)
        LAUNCH("tucker_core_adj", s, fno::launch_mode_product(stp.pre, stp.cn, stp.an, stp.post,
                                                          f2c(fac[stp.factor]), true, true, cur,
                                                          dst, s));
      other = cur;
      cur = dst;
      --si;
    }
    return FNO_OK;
  }
};

fno_status check_tucker_args(const fno_tucker* t, const float* core, const float* const* fac,
                             void* ws, size_t ws_bytes) {
  if (!t) return fail(FNO_ERR_INVALID_ARGUMENT, "tucker is NULL");
  REQ(core, "core");
  if (!fac) return fail(FNO_ERR_INVALID_ARGUMENT, "factors is NULL");
  for (int n = 0; n < t->nf; ++n) REQ(fac[n], "factor");
  REQ(ws, "workspace");
  if (ws_bytes < t->total)
    return fail(FNO_ERR_INVALID_ARGUMENT, "workspace %zu bytes < required %zu", ws_bytes,
                t->total);
  return FNO_OK;
}

}  // namespace

// Device memory of fno_block_fwd_static, for callers that cannot allocate: one copy of this
// array per GPU, present from the library's load on that GPU until the process ends.  Host code
// never passes `scratch` itself to a kernel (on the host it names a stand-in, not the device
// copy); it takes the device address from hipGetSymbolAddress, once per device.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxScratchDevices];  // device address of `scratch` on each device

// The device address of `scratch` on device `dev` (the current device), looked up on the first
// call for that device.
fno_status static_scratch(int dev, void** out) {
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(FNO_ERR_UNSUPPORTED, "device %d: at most %d devices have a static scratch", dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(FNO_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return FNO_OK;
}

}  // namespace

extern "C" {

fno_status fno_spectral_conv_fwd(const fno_plan* p, const float* x, const float* w,
                                 float* y_spec, void* save, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (!p) return fail(FNO_ERR_INVALID_ARGUMENT, "plan is NULL");
  REQ(x, "x");
  REQ(w, "w");
  REQ(y_spec, "y_spec");
  OPT(save, "save");
  fno_status st = check_ws(p, ws, ws_bytes);
  if (st != FNO_OK) return st;
  return spectral_fwd_impl(p, x, y_spec, save, ws, static_cast<hipStream_t>(stream),
                           DenseMix(p, w, nullptr));
}

fno_status fno_block_fwd(const fno_plan* p, const float* x, const float* w, const float* wb,
                         const float* bias, float* y, void* save, void* ws, size_t ws_bytes,
                         void* stream) {
  if (!p) return fail(FNO_ERR_INVALID_ARGUMENT, "plan is NULL");
  REQ(x, "x");
  REQ(w, "w");
  REQ(wb, "w_bypass");
  REQ(y, "y");
  if (p->desc.flags & FNO_FLAG_BIAS) REQ(bias, "bias");
  OPT(save, "save");
  fno_status st = check_ws(p, ws, ws_bytes);
  if (st != FNO_OK) return st;
  return block_fwd_impl(p, x, wb, bias, y, save, ws, static_cast<hipStream_t>(stream),
                        DenseMix(p, w, nullptr));
}

fno_status fno_block_fwd_static(const fno_plan* p, const float* x, const float* w,
                                const float* wb, const float* bias, float* y, void* save,
                                void* stream) {
  if (!p) return fail(FNO_ERR_INVALID_ARGUMENT, "plan is NULL");
  REQ(x, "x");
  REQ(w, "w");
  REQ(wb, "w_bypass");
  REQ(y, "y");
  if (p->desc.flags & FNO_FLAG_BIAS) REQ(bias, "bias");
  OPT(save, "save");
  if (p->ws.total > kStaticScratchBytes)
    return fail(FNO_ERR_INVALID_ARGUMENT,
                "the plan's workspace (%zu bytes) exceeds the static scratch (%zu bytes); use "
                "fno_block_fwd with a caller workspace",
                p->ws.total, kStaticScratchBytes);
  int dev = -1;
  FNO_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev != p->device)
    return fail(FNO_ERR_INVALID_ARGUMENT, "current device %d is not the plan's device %d", dev,
                p->device);
  void* ws = nullptr;
  fno_status st = static_scratch(dev, &ws);
  if (st != FNO_OK) return st;
  return block_fwd_impl(p, x, wb, bias, y, save, ws, static_cast<hipStream_t>(stream),
                        DenseMix(p, w, nullptr));
}

fno_status fno_spectral_conv_bwd(const fno_plan* p, const float* x, const float* w,
                                 const void* save, const float* gys, float* grad_x,
                                 float* grad_w, void* ws, size_t ws_bytes, void* stream) {
  if (!p) return fail(FNO_ERR_INVALID_ARGUMENT, "plan is NULL");
  REQ(x, "x");
  REQ(w, "w");
  REQ(gys, "grad_y_spec");
  OPT(save, "save");
  OPT(grad_x, "grad_x");
  OPT(grad_w, "grad_w");
  fno_status st = check_ws(p, ws, ws_bytes);
  if (st != FNO_OK) return st;
  return spectral_bwd_impl(p, x, save, gys, grad_x, ws, static_cast<hipStream_t>(stream),
                           DenseMix(p, w, grad_w));
}

fno_status fno_block_bwd(const fno_plan* p, const float* x, const float* w, const float* wb,
                         const float* bias, const void* save, const float* gy, float* grad_x,
                         float* grad_w, float* grad_wb, float* grad_bias, void* ws,
                         size_t ws_bytes, void* stream) {
  (void)bias;
  if (!p) return fail(FNO_ERR_INVALID_ARGUMENT, "plan is NULL");
  REQ(x, "x");
  REQ(w, "w");
  REQ(wb, "w_bypass");
  REQ(gy, "grad_y");
  const bool gelu = (p->desc.flags & FNO_FLAG_GELU) != 0;
  if (gelu || grad_w) REQ(save, "save");
  OPT(save, "save");
  OPT(grad_x, "grad_x");
  OPT(grad_w, "grad_w");
  OPT(grad_wb, "grad_w_bypass");
  OPT(grad_bias, "grad_bias");
  fno_status st = check_ws(p, ws, ws_bytes);
  if (st != FNO_OK) return st;
  return block_bwd_impl(p, x, wb, save, gy, grad_x, grad_wb, grad_bias, ws,
                        static_cast<hipStream_t>(stream), DenseMix(p, w, grad_w));
}

fno_status fno_block_fwd_mse(const fno_plan* p, const float* x, const float* w, const float* wb,
                             const float* bias, const float* target, float grad_scale,
                             float* grad_z, float* loss, void* save, void* ws, size_t ws_bytes,
                             void* stream) {
  if (!p) return fail(FNO_ERR_INVALID_ARGUMENT, "plan is NULL");
  REQ(x, "x");
  REQ(w, "w");
  REQ(wb, "w_bypass");
  if (p->desc.flags & FNO_FLAG_BIAS) REQ(bias, "bias");
  REQ(target, "target");
  REQ(grad_z, "grad_z");
  OPT(loss, "loss");
  OPT(save, "save");
  if (!(grad_scale > 0.0f) || !std::isfinite(grad_scale))
    return fail(FNO_ERR_INVALID_ARGUMENT, "grad_scale must be finite and > 0");
  fno_status st = check_ws(p, ws, ws_bytes);
  if (st != FNO_OK) return st;
  return block_fwd_mse_impl(p, x, wb, bias, target, grad_scale, grad_z, loss, save, ws,
                            static_cast<hipStream_t>(stream), DenseMix(p, w, nullptr));
}

fno_status fno_block_bwd_preact(const fno_plan* p, const float* x, const float* w,
                                const float* wb, const float* bias, const void* save,
                                const float* grad_z, float* grad_x, float* grad_w,
                                float* grad_wb, float* grad_bias, void* ws, size_t ws_bytes,
                                void* stream) {
  (void)bias;
  if (!p) return fail(FNO_ERR_INVALID_ARGUMENT, "plan is NULL");
  REQ(x, "x");
  REQ(w, "w");
  REQ(wb, "w_bypass");
  REQ(grad_z, "grad_z");
  if (grad_w) REQ(save, "save");
  OPT(save, "save");
  OPT(grad_x, "grad_x");
  OPT(grad_w, "grad_w");
  OPT(grad_wb, "grad_w_bypass");
  OPT(grad_bias, "grad_bias");
  fno_status st = check_ws(p, ws, ws_bytes);
  if (st != FNO_OK) return st;
  return block_bwd_impl(p, x, wb, save, grad_z, grad_x, grad_wb, grad_bias, ws,
                        static_cast<hipStream_t>(stream), DenseMix(p, w, grad_w), true);
}

fno_status fno_tucker_order(const fno_plan_desc* desc, const int32_t* ranks, char* buf,
                            size_t len) {
  fno::TuckerDims d;
  fno_status st = tucker_dims(desc, ranks, &d);
  if (st != FNO_OK) return st;
  const std::string o = fno::tucker_order_string(fno::tucker_greedy_order(d), d.d);
  if (!buf || len < o.size() + 1)
    return fail(FNO_ERR_INVALID_ARGUMENT, "buffer of %zu bytes < %zu", len, o.size() + 1);
  memcpy(buf, o.c_str(), o.size() + 1);
  return FNO_OK;
}

fno_status fno_tucker_create(const fno_plan* p, const int32_t* ranks, fno_tucker** out) {
  if (!p || !out) return fail(FNO_ERR_INVALID_ARGUMENT, "plan or out is NULL");
  *out = nullptr;
  fno::TuckerDims d;
  fno_status st = tucker_dims(&p->desc, ranks, &d);
  if (st != FNO_OK) return st;
  fno_tucker* t = new (std::nothrow) fno_tucker();
  if (!t) return fail(FNO_ERR_OUT_OF_MEMORY, "host allocation");
  t->plan = p;
  t->dims = d;
  t->nf = d.d + 2;
  t->steps = fno::tucker_greedy_order(d);
  t->order = fno::tucker_order_string(t->steps, d.d);
  t->K = p->g.K;
  t->core_elems = 1;
  for (int n = 0; n < t->nf; ++n) t->core_elems *= d.R[n];
  const int ext[2] = {d.Cin, d.Cout};
  for (int n = 0; n < t->nf; ++n)
    t->factor_elems[n] = (int64_t)(n < 2 ? ext[n] : d.K[n - 2]) * d.R[n];
  // workspace: the plan's part, then the Tucker buffers
  size_t off = align_up(p->ws.total);
  auto take = [&](int64_t complex_elems) {
    const size_t o = off;
    off += align_up(sizeof(float2) * (size_t)complex_elems);
    return o;
  };
  int64_t gmax = t->core_elems;
  t->core_steps = 0;
  t->in_on_data = t->out_on_data = false;
  for (const fno::TuckerStep& stp : t->steps) {
    if (stp.kind == fno::TuckerStep::CORE) {
      const int64_t e = stp.pre * stp.an * stp.post;
      t->chain_off.push_back(take(e));
      gmax = e > gmax ? e : gmax;
      ++t->core_steps;
    } else if (stp.kind == fno::TuckerStep::DATA_IN) {
      t->in_on_data = true;
    } else if (stp.kind == fno::TuckerStep::DATA_OUT) {
      t->out_on_data = true;
    } else {
      t->gmix = p->g;
      t->gmix.Cin = stp.cn;
      t->gmix.Cout = stp.an;
      t->gmix.Mprod = p->g.K;
      t->gmix.w_si = (int)(stp.an * p->g.K);
      t->gmix.w_so = (int)p->g.K;
    }
  }
  t->g0_off = take(gmax);
  t->g1_off = take(gmax);
  const int64_t dR = (int64_t)d.B * t->K;
  t->x1_off = take(t->in_on_data ? dR * d.R[0] : 0);
  t->v_off = take(t->in_on_data ? dR * d.R[0] : 0);
  t->t2_off = take(t->out_on_data ? dR * d.R[1] : 0);
  t->u_off = take(t->out_on_data ? dR * d.R[1] : 0);
  t->part_off = take(fno::kTuckerPartElems);
  t->total = off;
  {
    size_t koff = align_up(p->save_bytes);
    auto keep_take = [&](int64_t complex_elems) {
      const size_t o = koff;
      koff += align_up(sizeof(float2) * (size_t)complex_elems);
      return o;
    };
    for (const fno::TuckerStep& stp : t->steps)
      if (stp.kind == fno::TuckerStep::CORE)
        t->keep_chain_off.push_back(keep_take(stp.pre * stp.an * stp.post));
    t->keep_x1_off = keep_take(t->in_on_data ? dR * d.R[0] : 0);
    t->keep_t2_off = keep_take(t->out_on_data ? dR * d.R[1] : 0);
    t->keep_total = koff;
  }
  // identity mode offsets (the core-side tensor [c_in][c_out][K] holds mode t at t), then
  // zero offsets (a factor matrix, the same for every mode)
  std::vector<int32_t> ident((size_t)(2 * t->K), 0);
  for (int64_t k = 0; k < t->K; ++k) ident[(size_t)k] = (int32_t)k;
  auto factor_geom = [&](int cin, int cout, int w_si, int w_so) {
    fno::Geom g = p->g;
    g.Cin = cin;
    g.Cout = cout;
    g.w_si = w_si;
    g.w_so = w_so;
    g.half = 0;  // factor products in float32
    g.bf16 = false;
    g.mb = 1;    // no half-spectrum weight and no adjoint scale on these launches
    g.adj_scale = 1.0f;
    g.mix_gain[0] = g.mix_gain[1] = g.inv_gain[0] = g.inv_gain[1] = 1.0f;
    return g;
  };
  t->g_in = factor_geom(d.Cin, d.R[0], d.R[0], 1);     // W[i][ri] = U_in[i][ri]
  t->g_out = factor_geom(d.R[1], d.Cout, 1, d.R[1]);   // W[ro][o] = U_out[o][ro]
  t->ident_woff = nullptr;
  hipError_t e = hipSetDevice(p->device);
  if (e == hipSuccess) e = hipMalloc(&t->ident_woff, sizeof(int32_t) * ident.size());
  if (e == hipSuccess)
    e = hipMemcpy(t->ident_woff, ident.data(), sizeof(int32_t) * ident.size(),
                  hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    if (t->ident_woff) (void)hipFree(t->ident_woff);
    delete t;
    return hip_fail(e, "fno_tucker_create");
  }
  t->zero_woff = t->ident_woff + t->K;
  *out = t;
  return FNO_OK;
}

fno_status fno_tucker_destroy(fno_tucker* t) {
  if (!t) return FNO_OK;
  hipError_t e = hipSuccess;
  if (t->ident_woff) e = hipFree(t->ident_woff);
  delete t;
  return e == hipSuccess ? FNO_OK : hip_fail(e, "fno_tucker_destroy");
}

fno_status fno_tucker_keep_intermediates(fno_tucker* t, int keep) {
  if (!t) return fail(FNO_ERR_INVALID_ARGUMENT, "tucker is NULL");
  t->keep = keep != 0;
  return FNO_OK;
}

fno_status fno_tucker_save_bytes(const fno_tucker* t, size_t* bytes) {
  if (!t || !bytes) return fail(FNO_ERR_INVALID_ARGUMENT, "tucker or bytes is NULL");
  *bytes = t->keep ? t->keep_total : t->plan->save_bytes;
  return FNO_OK;
}

fno_status fno_tucker_query(const fno_tucker* t, size_t* ws_bytes, int64_t* core_elems,
                            int64_t* factor_elems, char* order, size_t order_len) {
  if (!t) return fail(FNO_ERR_INVALID_ARGUMENT, "tucker is NULL");
  if (ws_bytes) *ws_bytes = t->total;
  if (core_elems) *core_elems = t->core_elems;
  if (factor_elems)
    for (int n = 0; n < t->nf; ++n) factor_elems[n] = t->factor_elems[n];
  if (order) {
    if (order_len < t->order.size() + 1)
      return fail(FNO_ERR_INVALID_ARGUMENT, "order buffer of %zu bytes < %zu", order_len,
                  t->order.size() + 1);
    memcpy(order, t->order.c_str(), t->order.size() + 1);
  }
  return FNO_OK;
}

fno_status fno_tucker_block_fwd(const fno_tucker* t, const float* x, const float* core,
                                const float* const* factors, const float* wb, const float* bias,
                                float* y, void* save, void* ws, size_t ws_bytes, void* stream) {
  fno_status st = check_tucker_args(t, core, factors, ws, ws_bytes);
  if (st != FNO_OK) return st;
  const fno_plan* p = t->plan;
  REQ(x, "x");
  REQ(wb, "w_bypass");
  REQ(y, "y");
  if (p->desc.flags & FNO_FLAG_BIAS) REQ(bias, "bias");
  OPT(save, "save");
  return block_fwd_impl(p, x, wb, bias, y, save, ws, static_cast<hipStream_t>(stream),
                        TuckerMix(t, core, factors, nullptr, nullptr, save));
}

fno_status fno_tucker_block_bwd(const fno_tucker* t, const float* x, const float* core,
                                const float* const* factors, const float* wb, const float* bias,
                                const void* save, const float* gy, float* grad_x,
                                float* grad_core, float* const* grad_factors, float* grad_wb,
                                float* grad_bias, void* ws, size_t ws_bytes, void* stream) {
  (void)bias;
  fno_status st = check_tucker_args(t, core, factors, ws, ws_bytes);
  if (st != FNO_OK) return st;
  const fno_plan* p = t->plan;
  REQ(x, "x");
  REQ(wb, "w_bypass");
  REQ(gy, "grad_y");
  OPT(grad_x, "grad_x");
  OPT(grad_core, "grad_core");
  OPT(grad_wb, "grad_w_bypass");
  OPT(grad_bias, "grad_bias");
  bool want_w = grad_core != nullptr;
  for (int n = 0; grad_factors && n < t->nf; ++n) {
    OPT(grad_factors[n], "grad_factor");
    want_w = want_w || grad_factors[n] != nullptr;
  }
  const bool gelu = (p->desc.flags & FNO_FLAG_GELU) != 0;
  if (gelu || want_w) REQ(save, "save");
  OPT(save, "save");
  return block_bwd_impl(p, x, wb, save, gy, grad_x, grad_wb, grad_bias, ws,
                        static_cast<hipStream_t>(stream),
                        TuckerMix(t, core, factors, grad_core, grad_factors, save));
}

fno_status fno_tucker_block_fwd_mse(const fno_tucker* t, const float* x, const float* core,
                                    const float* const* factors, const float* wb,
                                    const float* bias, const float* target, float grad_scale,
                                    float* grad_z, float* loss, void* save, void* ws,
                                    size_t ws_bytes, void* stream) {
  fno_status st = check_tucker_args(t, core, factors, ws, ws_bytes);
  if (st != FNO_OK) return st;
  const fno_plan* p = t->plan;
  REQ(x, "x");
  REQ(wb, "w_bypass");
  if (p->desc.flags & FNO_FLAG_BIAS) REQ(bias, "bias");
  REQ(target, "target");
  REQ(grad_z, "grad_z");
  OPT(loss, "loss");
  OPT(save, "save");
  if (!(grad_scale > 0.0f) || !std::isfinite(grad_scale))
    return fail(FNO_ERR_INVALID_ARGUMENT, "grad_scale must be finite and > 0");
  return block_fwd_mse_impl(p, x, wb, bias, target, grad_scale, grad_z, loss, save, ws,
                            static_cast<hipStream_t>(stream),
                            TuckerMix(t, core, factors, nullptr, nullptr, save));
}

fno_status fno_tucker_block_bwd_preact(const fno_tucker* t, const float* x, const float* core,
                                       const float* const* factors, const float* wb,
                                       const float* bias, const void* save,
                                       const float* grad_z, float* grad_x, float* grad_core,
                                       float* const* grad_factors, float* grad_wb,
                                       float* grad_bias, void* ws, size_t ws_bytes,
                                       void* stream) {
  (void)bias;
  fno_status st = check_tucker_args(t, core, factors, ws, ws_bytes);
  if (st != FNO_OK) return st;
  const fno_plan* p = t->plan;
  REQ(x, "x");
  REQ(wb, "w_bypass");
  REQ(grad_z, "grad_z");
  OPT(grad_x, "grad_x");
  OPT(grad_core, "grad_core");
  OPT(grad_wb, "grad_w_bypass");
  OPT(grad_bias, "grad_bias");
  bool want_w = grad_core != nullptr;
  for (int n = 0; grad_factors && n < t->nf; ++n) {
    OPT(grad_factors[n], "grad_factor");
    want_w = want_w || grad_factors[n] != nullptr;
  }
  if (want_w) REQ(save, "save");
  OPT(save, "save");
  return block_bwd_impl(p, x, wb, save, grad_z, grad_x, grad_wb, grad_bias, ws,
                        static_cast<hipStream_t>(stream),
                        TuckerMix(t, core, factors, grad_core, grad_factors, save), true);
}

fno_status fno_tucker_spectral_conv_fwd(const fno_tucker* t, const float* x, const float* core,
                                        const float* const* factors, float* y_spec, void* save,
                                        void* ws, size_t ws_bytes, void* stream) {
  fno_status st = check_tucker_args(t, core, factors, ws, ws_bytes);
  if (st != FNO_OK) return st;
  REQ(x, "x");
  REQ(y_spec, "y_spec");
  OPT(save, "save");
  return spectral_fwd_impl(t->plan, x, y_spec, save, ws, static_cast<hipStream_t>(stream),
                           TuckerMix(t, core, factors, nullptr, nullptr, save));
}

fno_status fno_tucker_spectral_conv_bwd(const fno_tucker* t, const float* x, const float* core,
                                        const float* const* factors, const void* save,
                                        const float* gys, float* grad_x, float* grad_core,
                                        float* const* grad_factors, void* ws, size_t ws_bytes,
                                        void* stream) {
  fno_status st = check_tucker_args(t, core, factors, ws, ws_bytes);
  if (st != FNO_OK) return st;
  REQ(x, "x");
  REQ(gys, "grad_y_spec");
  OPT(save, "save");
  OPT(grad_x, "grad_x");
  OPT(grad_core, "grad_core");
  for (int n = 0; grad_factors && n < t->nf; ++n) OPT(grad_factors[n], "grad_factor");
  return spectral_bwd_impl(t->plan, x, save, gys, grad_x, ws, static_cast<hipStream_t>(stream),
                           TuckerMix(t, core, factors, grad_core, grad_factors, save));
}

fno_status fno_pointwise_fwd(int64_t batch, int64_t npts, int64_t cin, int64_t hidden,
                             int64_t cout, const float* x, const float* w1, const float* b1,
                             const float* w2, const float* b2, float* y, void* stream) {
  if (batch < 1 || npts < 1 || cin < 1 || cout < 1 || hidden < 0)
    return fail(FNO_ERR_INVALID_ARGUMENT, "bad pointwise sizes");
  if (cin > 64 || cout > 128 || hidden > 256)
    return fail(FNO_ERR_UNSUPPORTED, "pointwise: c_in <= 64, c_out <= 128, hidden <= 256");
  if (batch > 65535) return fail(FNO_ERR_UNSUPPORTED, "pointwise: batch > 65535");
  REQ(x, "x");
  REQ(w1, "w1");
  REQ(y, "y");
  OPT(b1, "b1");
  if (hidden > 0) REQ(w2, "w2");
  OPT(b2, "b2");
  LAUNCH("pointwise", static_cast<hipStream_t>(stream), fno::launch_pointwise(batch, npts, (int)cin, (int)hidden, (int)cout, x, w1, b1, w2, b2,
                               y, static_cast<hipStream_t>(stream)));
  return FNO_OK;
}

static int mse_parts(int64_t n) {
  int64_t g = (n + 255) / 256;
  return (int)(g < fno::kMseParts ? (g < 1 ? 1 : g) : fno::kMseParts);
}

fno_status fno_mse_workspace_bytes(int64_t n, size_t* bytes) {
  if (n < 1 || !bytes) return fail(FNO_ERR_INVALID_ARGUMENT, "bad mse workspace query");
  *bytes = sizeof(double) * (size_t)mse_parts(n);
  return FNO_OK;
}

fno_status fno_mse_grad(int64_t n, const float* y, const float* t, float* grad, float* loss,
                        void* ws, size_t ws_bytes, void* stream) {
  return fno_mse_grad_scaled(n, y, t, grad, loss, 1.0f, ws, ws_bytes, stream);
}

fno_status fno_mse_grad_scaled(int64_t n, const float* y, const float* t, float* grad,
                               float* loss, float grad_scale, void* ws, size_t ws_bytes,
                               void* stream) {
  if (n < 1) return fail(FNO_ERR_INVALID_ARGUMENT, "n < 1");
  if (!(grad_scale > 0.0f) || !std::isfinite(grad_scale))
    return fail(FNO_ERR_INVALID_ARGUMENT, "grad_scale must be finite and > 0");
  REQ(y, "y");
  REQ(t, "t");
  REQ(grad, "grad");
  REQ(ws, "workspace");
  const int parts = mse_parts(n);
  if (ws_bytes < sizeof(double) * (size_t)parts)
    return fail(FNO_ERR_INVALID_ARGUMENT, "workspace too small");
  LAUNCH("mse", static_cast<hipStream_t>(stream), fno::launch_mse(n, y, t, grad, loss, grad_scale, static_cast<double*>(ws), parts,
                         static_cast<hipStream_t>(stream)));
  return FNO_OK;
}

fno_status fno_timing_enable(int enable) {
  TimingState& T = timing_state();
  std::lock_guard<std::mutex> lk(T.mu);
  T.on = enable != 0;
  return FNO_OK;
}

fno_status fno_timing_select(const char* name) {
  TimingState& T = timing_state();
  std::lock_guard<std::mutex> lk(T.mu);
  T.only = name ? name : "";
  return FNO_OK;
}

fno_status fno_timing_reset(void) {
  TimingState& T = timing_state();
  std::lock_guard<std::mutex> lk(T.mu);
  hipError_t e = T.pending.empty() ? hipSuccess : timing_collect(T);
  T.names.clear();
  T.launches.clear();
  T.total_ms.clear();
  if (e != hipSuccess) return hip_fail(e, "fno_timing_reset");
  return FNO_OK;
}

fno_status fno_timing_count(int* count) {
  if (!count) return fail(FNO_ERR_INVALID_ARGUMENT, "count is NULL");
  TimingState& T = timing_state();
  std::lock_guard<std::mutex> lk(T.mu);
  hipError_t e = T.pending.empty() ? hipSuccess : timing_collect(T);
  if (e != hipSuccess) return hip_fail(e, "fno_timing_count");
  *count = (int)T.names.size();
  return FNO_OK;
}

fno_status fno_timing_get(int index, const char** name, int64_t* launches, double* total_ms) {
  TimingState& T = timing_state();
  std::lock_guard<std::mutex> lk(T.mu);
  if (index < 0 || index >= (int)T.names.size())
    return fail(FNO_ERR_INVALID_ARGUMENT, "timing index %d out of range", index);
  if (name) *name = T.names[index].c_str();
  if (launches) *launches = T.launches[index];
  if (total_ms) *total_ms = T.total_ms[index];
  return FNO_OK;
}

}  // extern "C"

