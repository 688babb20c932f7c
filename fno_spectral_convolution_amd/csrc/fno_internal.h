// Internal declarations shared by the libfno host runtime and its kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <string>
#include <vector>

#include "fno.h"

namespace fno {

constexpr int kMaxDims = 4;
constexpr int kMaxChannels = 128;   // c_in, c_out limit of the epilogue/mix kernels
constexpr int kMaxBatchTile = 16;   // batch entries held in registers by the mix kernels

// Geometry of one plan, flattened for kernel arguments (passed by value).
struct Geom {
  int d;
  int B, Cin, Cout;
  int N[kMaxDims];
  int M[kMaxDims];
  int Na, Nb;          // the last two axes: rows (a = d-2) and contiguous (b = d-1)
  int ma, mb;          // modes per corner on those axes
  int64_t O;           // prod_{j < d-2} N_j (outer points; 1 in 2D)
  int64_t P;           // points per field = prod N_j
  int64_t K;           // retained modes per (batch, channel) = prod_{j<d-1} 2 m_j * m_b
  int64_t Mprod;       // prod m_j (weights per corner per (i, o))
  int w_si, w_so;      // mix weight strides of the input / output channel (Cout Mprod, Mprod
                       // in W's corner layout)
  int ncorner;
  float inv_ntot;      // 1 / P
  bool bf16;           // spectral operands in a 16-bit format (half)
  int half;            // 0: fp32 operands; 1: bfloat16; 2: IEEE half
  // IEEE-half plans scale every transform table by 1/sqrt(N_j) in both directions (sc[j]), so
  // spectra stay near unit size; 1 otherwise.  The mix's adjoint factor gamma * adj_scale is
  // gamma / Ntot (tables unscaled) or gamma (scaled tables).
  float sc[kMaxDims];
  float adj_scale;
  // IEEE-half plans also multiply the mixed spectra by a power of two near sqrt(Cin) Cout
  // (mix_gain[0], forward) or sqrt(Cout) Cin (mix_gain[1], input gradient).  It offsets the
  // 1/(Cin Cout) size of FNO spectral weights, so the spectra entering the inverse stay in
  // half's normal range; the last inverse stage takes it out again (inv_gain, folded into its
  // half table or applied in float).  Powers of two: both steps are exact.  1 otherwise.
  float mix_gain[2];
  float inv_gain[2];
  // IEEE-half plans: a device word the output-writing kernels set to 1 when they write a
  // non-finite value (half's range exceeded upstream); null on other plans
  int* half_flag;
};

// Device tables owned by a plan (all in one allocation).
struct Tables {
  const float2* root[kMaxDims];     // (cos, sin)(2 pi t / N_j), t < N_j  (fp32-rounded)
  const float2* root_bf[kMaxDims];  // same values rounded to bfloat16 (stored as float)
  const int32_t* mode_woff;         // [K]: offset of mode t in W for (i, o) = (0, 0)
  const int32_t* woff_mode;         // [ncorner * Mprod]: retained mode of each W element
  // last-axis inverse tables [Nb][kpad], interleaved (re, im) columns:
  // gt_fwd = g(k)/Ntot (cos, -sin)(2 pi k p / Nb); gt_unit = (cos, -sin) (adjoint scale)
  const float* gt_fwd;
  const float* gt_unit;
  const uint16_t* gt_fwd_bf;        // the same as 16-bit half operands (IEEE-half plans:
                                    // 1/sqrt(Nb) and 1/mix_gain instead of 1/Ntot)
  const uint16_t* gt_unit_bf;
  // forward plane tables: t1 [Nb][jpad] (col 2k = cos, 2k+1 = -sin of 2 pi k c / Nb) and
  // f2 [4 ma][Na] (rows < 2 ma: cos, rows >= 2 ma: sin of 2 pi ka(s) row / Na)
  const float* t1;
  const uint16_t* t1_bf;
  const uint16_t* t1t_bf;     // bf16 t1 transposed: [jpad][Nb]
  const float* f2;
  const uint16_t* f2_bf;      // bfloat16 of f2
  const uint16_t* f2_bf_lo;   // bfloat16 of (f2 - f2_bf): f2_bf + f2_bf_lo ~ f2 to 2^-16
  // outer-axis transforms of axes 0..d-2: A = [Mr | Mi] with rows = outputs, padded to 16:
  // oinv[j] [pad16(N_j)][2 pad16(2 m_j)]  (e^{+i theta}),  ofwd[j] [pad16(2 m_j)][2 pad16(N_j)]
  const float* oinv[kMaxDims];
  const uint16_t* oinv_bf[kMaxDims];
  const uint16_t* oinv_bf_lo[kMaxDims];
  const float* ofwd[kMaxDims];
  const uint16_t* ofwd_bf[kMaxDims];
  const uint16_t* ofwd_bf_lo[kMaxDims];
};

struct Workspace {
  // Offsets (bytes) of the buffers inside the caller's workspace.
  size_t plane_part;   // plane-transform partials [nch][B*C*O][2ma][mb] complex
  size_t spec_a;       // complex ping buffer (largest intermediate spectrum)
  size_t spec_b;       // complex pong buffer
  size_t xhat;         // [B][Cin][K] complex (when the caller gives no save buffer)
  size_t yhat;         // [B][Cout][K] complex
  size_t red_part;     // bypass-gradient partials [nred][Cout*Cin + Cout] float
  size_t loss_part;    // loss partial sums of the fused forward, [loss_parts] double
  size_t total;
};

}  // namespace fno

struct fno_plan {
  fno_plan_desc desc;
  fno::Geom g;
  fno::Tables t;
  void* table_mem;
  int device;
  int nch;              // chunks of the plane transform along axis a
  int nred;             // work-groups of the bypass-gradient reduction (generic kernels)
  int kpad;             // 2*mb rounded up to 32 (columns of the last-axis tables)
  int jpad;             // 2*mb rounded up to 16 (columns of the forward plane table t1)
  int plane_rows;       // rows of axis a per plane-transform chunk
  bool plane_fft;       // forward row transform by FFT (float32 plans), else dense products
  int64_t complex_max;  // largest intermediate spectrum (complex elements)
  fno::Workspace ws;
  size_t save_bytes;
  size_t save_off_z;    // offset of z inside the save buffer
};

namespace fno {

// ---- launchers (kernels_*.hip) -------------------------------------------------------------
// Prologue of the plane transform: how a field value becomes a transform operand.
enum PlaneIn {
  PLANE_X = 0,
  PLANE_TANH = 1,        // tanh(x)
  PLANE_GELU_GRAD = 2,   // g * GELU'(z)
  PLANE_GELU = 3,        // GELU(x): a block whose input is a pre-activation
  PLANE_TANH_GELU = 4    // tanh(GELU(x))
};

hipError_t launch_plane_fwd(const fno_plan* p, int plane_in, int chans, const float* in0,
                            const float* in1, float2* out, hipStream_t s);
// short contiguous axis (Nb <= 32): one wave per plane, unchunked output (nch == 1)
bool plane_small_ok(const fno_plan* p);
hipError_t launch_plane_small(const fno_plan* p, int plane_in, int chans, const float* in0,
                              const float* in1, float2* out, hipStream_t s);
hipError_t launch_outer_fwd(const fno_plan* p, int axis, int chans, const float2* in,
                            int nparts, int64_t part_stride, float2* out, hipStream_t s);
hipError_t launch_outer_inv(const fno_plan* p, int axis, int chans, const float2* in,
                            float2* out, hipStream_t s);
hipError_t launch_mix_fwd(const fno_plan* p, const float2* xhat, int nparts,
                          int64_t part_stride, const float2* w, float2* yhat, hipStream_t s);
hipError_t launch_mix_bwd_dx(const fno_plan* p, const float2* ghat, const float2* w,
                             float2* ghx, hipStream_t s);
hipError_t launch_mix_bwd_dw(const fno_plan* p, const float2* xhat, const float2* ghat,
                             float2* dw, hipStream_t s);
// both mix gradients (ghx and dw) in one launch
hipError_t launch_mix_bwd_both(const fno_plan* p, const float2* xhat, const float2* ghat,
                               const float2* w, float2* ghx, float2* dw, hipStream_t s);
// The same on an explicit geometry and per-mode weight offsets (woff[t] = offset of mode t
// inside one [Cin][Cout] weight slab; input-channel stride Cout * Mprod, output stride Mprod).
hipError_t launch_mix_fwd_g(const Geom& g, const int32_t* woff, const float2* xhat,
                            const float2* w, float2* yhat, hipStream_t s);
hipError_t launch_mix_bwd_dx_g(const Geom& g, const int32_t* woff, const float2* ghat,
                               const float2* w, float2* ghx, hipStream_t s);
hipError_t launch_mix_bwd_dw_g(const Geom& g, const int32_t* woff, const float2* xhat,
                               const float2* ghat, float2* dw, hipStream_t s);

// ---- Tucker-factorised weights (tucker.hip) ---------------------------------------------------
constexpr int kTuckerMaxMat = 4096;          // entries of a factor matrix (at most 64 x 64)
constexpr int64_t kTuckerPartElems = 1 << 20;  // complex partials of one factor gradient
struct TuckerDims {
  int d;
  int64_t B;
  int Cin, Cout;
  int K[kMaxDims];       // retained extent of each mode: 2 m_j (outer axes), m_{d-1} (last)
  int R[2 + kMaxDims];   // ranks: R_in, R_out, R_0 .. R_{d-1}
};
// One pairwise contraction of the Tucker network.  CORE: factor `factor` (0 in, 1 out, 2 + j
// mode j) applied to the core's lineage; DATA_IN: U_in on the spectrum; MIX: the per-mode
// channel mix; DATA_OUT: U_out on the mixed spectrum.  Mode products read [pre][cn][post] and
// write [pre][an][post]; for MIX, cn / an are the contracted / output channels.
struct TuckerStep {
  enum Kind { CORE = 0, DATA_IN = 1, MIX = 2, DATA_OUT = 3 } kind;
  int factor;
  int64_t pre, post;
  int an, cn;
};
std::vector<TuckerStep> tucker_greedy_order(const TuckerDims& t);
std::string tucker_order_string(const std::vector<TuckerStep>& steps, int d);
// out[p][a][q] = sum_c op(A)[a][c] T[p][c][q]; op(A) = A [an][cn], or A^T (A stored [cn][an])
// when trans, conjugated when conj
hipError_t launch_mode_product(int64_t pre, int an, int cn, int64_t post, const float2* A,
                               bool trans, bool conj, const float2* T, float2* out,
                               hipStream_t s);
// out[a][c] = scale sum_{p,q} X[p][a][q] w(q) conj(Y[p][c][q]) (conjugated when conj_out),
// w = gamma(q mod mb) * adj when gamma_w, else 1; part: kTuckerPartElems complex scratch
hipError_t launch_gram(int64_t pre, int an, int cn, int64_t post, const float2* X,
                       const float2* Y, bool gamma_w, int mb, int Nb, float adj, float scale,
                       bool conj_out, float2* part, float2* out, hipStream_t s);
hipError_t launch_reduce_parts(const float2* in, int nparts, int64_t part_stride, int64_t n,
                               float2* out, hipStream_t s);
// Epilogue: last-axis inverse of T [B][C][lines][mb] plus the pointwise part.
// EPI_BLOCK_PREACT: the block without its output GELU (y receives the pre-activation z).
enum EpiMode { EPI_SPECTRAL = 0, EPI_BLOCK = 1, EPI_BLOCK_PREACT = 2 };
hipError_t launch_epilogue_fwd(const fno_plan* p, int mode, const float2* T, const float* x,
                               const float* wb, const float* bias, float* y, float* zsave,
                               hipStream_t s);
hipError_t launch_epilogue_bwd(const fno_plan* p, int mode, const float2* Tg, const float* x,
                               const float* wb, const float* gy, const float* z,
                               float* grad_x, float* red_part, hipStream_t s);
bool epilogue_fast_ok(const fno_plan* p, int mode, bool fwd);
// Short contiguous axis: the forward epilogue fused with the inverse of axis a; T is the
// spectrum after the inverse of the outer axes 0..d-3 only, [B][Cout][O][2ma][mb].
bool epilogue_rows_ok(const fno_plan* p, int mode, const float* x, const float* y,
                      const float* zsave);
// t_half: T in the plan's half format (half plans; the rounding the epilogue applies to T)
hipError_t launch_epilogue_rows(const fno_plan* p, int mode, const void* T, const float* x,
                                const float* wb, const float* bias, float* y, float* zsave,
                                hipStream_t s, bool t_half = false);
// the backward epilogue takes the matrix-core kernel (which writes epilogue_bwd_fast_groups
// partial rows) only when grad_x is produced; otherwise the generic kernel (nred rows)
inline bool epilogue_bwd_fast(const fno_plan* p, int mode, const float* grad_x) {
  return grad_x != nullptr && epilogue_fast_ok(p, mode, false);
}
int epilogue_bwd_fast_groups(const fno_plan* p);
// The block's forward epilogue fused with the MSE loss (matrix-core kernel only): writes
// gz = msc (y - t) GELU'(z) (msc = grad_scale 2 / n; GELU' = 1 without the output GELU) and
// one partial sum of (y - t)^2 per work-group into lpart (epilogue_fwd_fast_groups of them).
int epilogue_fwd_fast_groups(const fno_plan* p);
hipError_t launch_epilogue_fwd_mse(const fno_plan* p, const void* T, const float* x,
                                   const float* wb, const float* bias, const float* tgt,
                                   float msc, float* gz, double* lpart, hipStream_t s,
                                   bool t_half = false);
// t_half: T is in the plan's half format (width 64, half operands; launch_outer_mfma_half)
hipError_t launch_epilogue_fwd_fast(const fno_plan* p, int mode, const void* T, const float* x,
                                    const float* wb, const float* bias, float* y, float* zsave,
                                    hipStream_t s, bool t_half = false);
hipError_t launch_epilogue_bwd_fast(const fno_plan* p, int mode, const void* Tg,
                                    const float* x, const float* wb, const float* gy,
                                    const float* z, float* grad_x, float* red_part,
                                    hipStream_t s, bool t_half = false);
bool plane_fast_ok(const fno_plan* p);
// float32 plans: the plane transform with an FFT along the contiguous axis
bool plane_fft_ok(const fno_plan* p);
bool plane_fft_default(const fno_plan* p);  // the shapes where it is the faster choice
hipError_t launch_plane_fft(const fno_plan* p, int plane_in, int chans, const float* in0,
                            const float* in1, float2* out, hipStream_t s);
hipError_t launch_plane_fwd_fast(const fno_plan* p, int plane_in, int chans, const float* in0,
                                 const float* in1, float2* out, hipStream_t s);
bool outer_fast_ok(const fno_plan* p, int axis, bool inv);
hipError_t launch_outer_mfma(const fno_plan* p, int axis, int chans, bool inv, const float2* in,
                             float2* out, hipStream_t s);
// The inverse of outer axis `axis` written in the plan's half format (half plans, outer_fast_ok):
// the rounding the matrix-core line epilogues apply to T when they stage it.
hipError_t launch_outer_mfma_half(const fno_plan* p, int axis, int chans, const float2* in,
                                  uint16_t* out, hipStream_t s);
// whether the forward's inverse of outer axis `axis` (Cout channels) streams column blocks of
// many wide slabs, so that launch_outer_mfma_half writes it in the half format with
// k_outer_inv_stream (half plans)
bool outer_inv_half_ok(const fno_plan* p, int axis);
hipError_t launch_bypass_grad_finish(const fno_plan* p, const float* red_part, float* dwb,
                                     float* dbias, const float* grad_x, hipStream_t s);
hipError_t launch_pointwise(int64_t batch, int64_t npts, int cin, int hidden, int cout,
                            const float* x, const float* w1, const float* b1, const float* w2,
                            const float* b2, float* y, hipStream_t s);
hipError_t launch_mse(int64_t n, const float* y, const float* t, float* g, float* loss,
                      float grad_scale, double* part, int nparts, hipStream_t s);
// In place on gz, which holds z [B][C][P]: y = GELU(z) (or z), gz = sc (y - t) GELU'(z) (or
// sc (y - t)) with sc = grad_scale 2 / n; partial sums of (y - t)^2 into part[nparts].
hipError_t launch_mse_preact(int64_t n, const float* t, float* gz, bool gelu, float grad_scale,
                             double* part, int nparts, hipStream_t s);
// loss = sum of part[0..nparts) / n, in a fixed order
hipError_t launch_mse_finish(int64_t n, int nparts, const double* part, float* loss,
                             hipStream_t s);
constexpr int kMseParts = 1024;  // work-groups of the stand-alone loss kernels

}  // namespace fno
