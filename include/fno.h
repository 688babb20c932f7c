/*
 * libfno -- FNO spectral-convolution block on AMD Instinct MI355X (gfx950).
 *
 * The operation is the spectral block of a Fourier Neural Operator: a truncated real DFT of a
 * [batch, channel, grid...] field, a per-mode complex channel mix, the zero-padded inverse,
 * a pointwise 1x1 bypass, a bias and an exact-erf GELU, plus the backward pass.
 *
 * Pages cited:
 *  [MPFNO] "Model-Parallel Fourier Neural Operators as Learned Surrogates for Large-Scale
 *          Parametric PDEs" (nubint.ai review), section "Proposed method": spectral
 *          convolution from FNO's linear-algebra form, 4 spectral blocks of width 20,
 *          gradients by automatic differentiation; "Main findings": 3D and 4D space-time grids.
 *  [MIXED] "Guaranteed Approximation Bounds and Efficient Mixed-Precision Training for Neural
 *          Operators" (linnk.ai insight), section "Tiivistelmä": half-precision Fourier
 *          transform and contraction, tanh pre-activation before the transform.
 *
 * Notation (d = ndim spatial axes, axis d-1 contiguous):
 *   Ntot = prod N_j;  theta_k(p) = 2 pi sum_j k_j p_j / N_j
 *   retained modes: axis j < d-1 keeps array indices {0..m_j-1} U {N_j-m_j..N_j-1};
 *                   axis d-1 keeps bins {0..m_{d-1}-1} of its half spectrum.
 *   xhat[b,i,k] = sum_p x'[b,i,p] e^{-i theta_k(p)},  x' = x or tanh(x) (FNO_FLAG_TANH_PREACT)
 *   yhat[b,o,k] = sum_i xhat[b,i,k] W[c(k),i,o,kappa(k)]
 *   y_spec[b,o,p] = (1/Ntot) sum_k gamma(k_{d-1}) Re(yhat[b,o,k] e^{+i theta_k(p)}),
 *                   gamma = 1 at the DC (and an even axis' Nyquist) bin, else 2
 *   z = y_spec + sum_i Wb[o,i] x[b,i,p] + bias[o];   y = GELU(z) = z/2 (1 + erf(z/sqrt 2))
 *
 * Layouts (all row-major, last index fastest, every pointer 16-byte aligned):
 *   x, y, grads ... float32 [B, C, N_0, ..., N_{d-1}]
 *   w, grad_w ..... complex float32 interleaved (re, im) -- the bytes of a complex64 tensor --
 *                   [2^(d-1) corners][C_in][C_out][m_0]...[m_{d-1}]; bit j of the corner
 *                   index is set when axis j (j < d-1) is in its high (negative-frequency)
 *                   range; local index q of a high range is frequency q - m_j.
 *   w_bypass ...... float32 [C_out][C_in];   bias ... float32 [C_out]
 *
 * Ownership: the caller allocates every tensor, the workspace and the save buffer (sizes from
 * fno_plan_query) on the plan's device and keeps them alive until the stream has run the
 * call.  A plan owns only its constant tables (and, on IEEE-half plans, one flag word).  Calls enqueue work on `stream` (a
 * hipStream_t; NULL = the null stream) and return without synchronising; they never
 * allocate device memory.  A plan is immutable after creation: concurrent calls on
 * different streams are safe when each has its own workspace.
 *
 * Errors: every function returns an fno_status; nothing aborts or throws across the ABI.
 *   FNO_ERR_INVALID_ARGUMENT  NULL/misaligned pointer, bad descriptor, workspace too small
 *   FNO_ERR_UNSUPPORTED       valid FNO shape outside what the kernels implement
 *   FNO_ERR_HIP               a HIP call or kernel launch failed (detail in
 *                             fno_last_error_message, thread-local)
 * Device faults surface at the caller's next synchronisation.
 */
#ifndef LIBFNO_FNO_H
#define LIBFNO_FNO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fno_status {
  FNO_OK = 0,
  FNO_ERR_INVALID_ARGUMENT = 1,
  FNO_ERR_UNSUPPORTED = 2,
  FNO_ERR_HIP = 3,
  FNO_ERR_OUT_OF_MEMORY = 4,
  FNO_ERR_INTERNAL = 5
} fno_status;

/* Arithmetic of the spectral path (transforms and channel mix).
 * F32:  float32 operands, float32 accumulation.
 * BF16: bfloat16 operands (pre-activated input, transform tables, spectra, weights rounded
 *       to nearest-even on load) with float32 accumulation -- the half-precision transform
 *       and contraction of [MIXED].  The bias, GELU and every HBM activation stay float32; the
 *       1x1 bypass and its weight gradient are float32 products, computed on plans with a
 *       multiple of 32 channels as three bfloat16 products of hi/lo split operands (each
 *       product exact to about 3 * 2^-18 relative, float32 accumulation).
 * F16:  the same with IEEE half operands.  Half's 5-bit exponent is kept in range by scaling
 *       every transform of the plan by 1/sqrt(N_j) per axis in both directions (tables built
 *       so), and by multiplying the mixed spectra by the power of two nearest sqrt(Cin) Cout
 *       (forward; sqrt(Cout) Cin for the input gradient), which the last inverse stage divides
 *       out.  The gain suits spectral weights of size about 1/(Cin Cout), the usual FNO
 *       initialisation; weights orders of magnitude larger can overflow half, and the
 *       outputs then hold inf or NaN: the plan records that (fno_plan_half_range).  Results
 *       are unchanged up to rounding.  Gradients far below half's range (a mean over 10^8
 *       elements) need a loss scale, see fno_mse_grad_scaled.  */
typedef enum fno_dtype { FNO_DTYPE_F32 = 0, FNO_DTYPE_BF16 = 1, FNO_DTYPE_F16 = 2 } fno_dtype;

enum {
  FNO_FLAG_TANH_PREACT = 1u, /* x' = tanh(x) feeds the spectral path only [MIXED] */
  FNO_FLAG_GELU = 2u,        /* block output y = GELU(z); without it y = z            */
  FNO_FLAG_BIAS = 4u,        /* bias pointer is read; without it bias is taken as 0    */
  FNO_FLAG_INPUT_GELU = 8u,  /* x is a pre-activation: the block's input is GELU(x), and
                                grad_x carries GELU'(x).  Lets a stack keep only each block's z
                                (the previous block runs without FNO_FLAG_GELU)           */
  /* How float32 plans take the forward transform of the contiguous axis (the forward and the
     input-gradient spectra).  Without either flag the plan picks the faster one for its
     shape.  FFT: a two-pass Stockham FFT in registers and LDS (N_{d-1} in {128, 256, 512},
     m_{d-1} <= 32, m_{d-2} a multiple of 4 up to 32, N_{d-2} a multiple of 8; otherwise
     fno_plan_create returns FNO_ERR_UNSUPPORTED).  DENSE: the truncated DFT as a matrix-core
     product.  The results agree to float32 rounding.  Half plans always use the dense
     products (at the half rate) and ignore both flags.                                    */
  FNO_FLAG_LAST_AXIS_FFT = 16u,
  FNO_FLAG_LAST_AXIS_DENSE = 32u
};

typedef struct fno_plan_desc {
  int32_t ndim;           /* spatial dimensions d: 2, 3 or 4                         */
  int32_t spectral_dtype; /* fno_dtype                                               */
  uint32_t flags;         /* FNO_FLAG_*                                              */
  int32_t reserved;       /* must be 0                                               */
  int64_t batch;          /* B >= 1                                                  */
  int64_t c_in;           /* input channels  (1..64)                                 */
  int64_t c_out;          /* output channels (1..64)                                 */
  int64_t n[4];           /* grid N_0..N_{d-1}; unused entries 0                    */
  int64_t modes[4];       /* modes per corner m_0..m_{d-1}; 1 <= m_j <= N_j/2 (j<d-1),
                             1 <= m_{d-1} <= N_{d-1}/2 + 1                           */
} fno_plan_desc;

typedef struct fno_plan fno_plan;

/* Host-only check of a descriptor (makes no HIP call). */
fno_status fno_plan_validate(const fno_plan_desc* desc);

/* Validate, build the transform tables in float64 on the host, round them and upload them
 * once to the current HIP device.  *out receives the plan. */
fno_status fno_plan_create(const fno_plan_desc* desc, fno_plan** out);

/* Free a plan's tables (NULL is accepted).  The caller must make sure no enqueued call still
 * uses the plan. */
fno_status fno_plan_destroy(fno_plan* plan);

/* Byte sizes of the caller-allocated workspace and save buffer of this plan, and the number
 * of complex elements of w.  Any output pointer may be NULL. */
fno_status fno_plan_query(const fno_plan* plan, size_t* workspace_bytes, size_t* save_bytes,
                          size_t* weight_elems);

/* Whether the plan takes the forward transform of its contiguous axis by FFT (*fft = 1) or by
 * dense matrix-core products (*fft = 0), as chosen at creation (FNO_FLAG_LAST_AXIS_FFT,
 * FNO_FLAG_LAST_AXIS_DENSE or the plan's own choice).  Host only. */
fno_status fno_plan_last_axis_fft(const fno_plan* plan, int* fft);

/* IEEE-half (F16) plans: whether a call made with this plan since its creation (or the last
 * clear) wrote a non-finite value into y, y_spec, z, grad_z, grad_x or the dense grad_w, i.e.
 * an operand left half's range on the way (*exceeded = 1, else 0).  The kernels that write
 * those outputs set a device word of the plan; this call reads it with a synchronous copy, so
 * the caller first synchronises the streams of the calls it asks about.  clear != 0 resets
 * the word after reading it.  Other plans: *exceeded = 0, no device access.  Calls on several
 * streams that share the plan share the word. */
fno_status fno_plan_half_range(const fno_plan* plan, int* exceeded, int clear);

/* Spectral convolution only: y_spec = inverse(mix(forward(x')))  (no bypass, bias or GELU).
 * `save` (nullable, save_bytes) receives the retained spectrum xhat for a later backward. */
fno_status fno_spectral_conv_fwd(const fno_plan* plan, const float* x, const float* w,
                                 float* y_spec, void* save, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Backward of fno_spectral_conv_fwd for the incoming gradient grad_y_spec:
 *   grad_x = s(x) * adjoint(grad_y_spec) with s = 1 - tanh(x)^2 under FNO_FLAG_TANH_PREACT,
 *   grad_w = sum_b conj(xhat) ghat  (complex64, W's layout).
 * `save` (nullable) is the buffer filled by the forward with the same x and w; when NULL the
 * spectrum is recomputed from x.  grad_x / grad_w may be NULL to skip that output.  Outputs
 * are overwritten, not accumulated. */
fno_status fno_spectral_conv_bwd(const fno_plan* plan, const float* x, const float* w,
                                 const void* save, const float* grad_y_spec, float* grad_x,
                                 float* grad_w, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Full block forward: y = GELU(y_spec + Wb x + bias).  `save` (nullable) receives what
 * fno_block_bwd needs (the retained spectrum and the pre-activation z). */
fno_status fno_block_fwd(const fno_plan* plan, const float* x, const float* w,
                         const float* w_bypass, const float* bias, float* y, void* save,
                         void* workspace, size_t workspace_bytes, void* stream);

/* fno_block_fwd without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * workspace is a static device array of 64 MiB inside libfno, one per GPU, present from the
 * library's load on that GPU until the process ends; this call allocates nothing and frees
 * nothing.  Its limit: plans whose fno_plan_query workspace exceeds 64 MiB are rejected with
 * FNO_ERR_INVALID_ARGUMENT (use fno_block_fwd).  The current device must be the plan's
 * (else FNO_ERR_INVALID_ARGUMENT).  Every call on one GPU uses the same array, which keeps the
 * last call's contents (nothing in it needs to start at zero: the forward writes every byte
 * it reads): calls that overlap on one GPU (other streams, other threads) race, so the caller
 * orders them (one stream, or events).  Other arguments, results and errors as fno_block_fwd. */
fno_status fno_block_fwd_static(const fno_plan* plan, const float* x, const float* w,
                                const float* w_bypass, const float* bias, float* y, void* save,
                                void* stream);

/* Full block backward for the incoming gradient grad_y.  `save` must come from
 * fno_block_fwd with the same inputs (required when FNO_FLAG_GELU is set).
 * Outputs (each may be NULL to skip): grad_x [B,C_in,N..], grad_w (complex64, W's layout),
 * grad_w_bypass [C_out][C_in], grad_bias [C_out].  Overwritten, not accumulated; the
 * reductions over batch and grid are deterministic (bitwise run-to-run). */
fno_status fno_block_bwd(const fno_plan* plan, const float* x, const float* w,
                         const float* w_bypass, const float* bias, const void* save,
                         const float* grad_y, float* grad_x, float* grad_w,
                         float* grad_w_bypass, float* grad_bias, void* workspace,
                         size_t workspace_bytes, void* stream);

/* The last block of a training step fused with the mean-squared-error loss against `target`
 * (same shape as y): with z = y_spec + Wb x + bias and y = GELU(z) (y = z without
 * FNO_FLAG_GELU), writes
 *   grad_z = grad_scale * 2 (y - target) / n * GELU'(z)   (n = batch * C_out * prod N),
 * the gradient of grad_scale * mean((y - target)^2) with respect to z, and, when `loss` (a
 * device float) is non-NULL, loss = mean((y - target)^2) (unscaled; fixed-order reduction).
 * y itself is not written.  It equals fno_block_fwd, then fno_mse_grad_scaled on y, then the
 * output GELU's chain rule, in one pass over the field when the plan's matrix-core epilogue
 * applies (else the epilogue writes z into grad_z and a pointwise pass rewrites it).
 * `save` (nullable) receives the retained spectrum only: the pre-activation is not needed
 * afterwards, since fno_block_bwd_preact takes grad_z.  grad_scale must be finite and > 0. */
fno_status fno_block_fwd_mse(const fno_plan* plan, const float* x, const float* w,
                             const float* w_bypass, const float* bias, const float* target,
                             float grad_scale, float* grad_z, float* loss, void* save,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Block backward from the gradient at the pre-activation z (the output GELU's derivative
 * already applied, as fno_block_fwd_mse returns it): fno_block_bwd without the GELU' step, so
 * z is never read.  `save` is one filled by fno_block_fwd or fno_block_fwd_mse with the same
 * inputs (its spectrum is read); it is required only for grad_w (else NULL recomputes). */
fno_status fno_block_bwd_preact(const fno_plan* plan, const float* x, const float* w,
                                const float* w_bypass, const float* bias, const void* save,
                                const float* grad_z, float* grad_x, float* grad_w,
                                float* grad_w_bypass, float* grad_bias, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ---- Tucker-factorised spectral weights (TFNO) ----------------------------------------------
 * TFNO is one of the architectures trained in mixed precision on the mixed-precision
 * neural-operator page ("Tiivistelmä"), together with a greedy algorithm ordering the block's
 * half-precision tensor contractions.  The weight on the retained grid,
 *   W[i, o, s_0, .., s_{d-1}]   (s_j < 2 m_j on outer axes, low modes first; s_{d-1} < m_{d-1}),
 * is a Tucker form: W = G x_1 U_in x_2 U_out x_3 U_0 .. x_{d+2} U_{d-1}, where the mode-n
 * product replaces a core index r by a: (T x_n U)[.., a, ..] = sum_r T[.., r, ..] U[a, r].
 * Device layouts (interleaved complex64, row-major): core G [R_in][R_out][R_0]..[R_{d-1}],
 * U_in [C_in][R_in], U_out [C_out][R_out], U_j [2 m_j][R_j] (j < d-1), U_{d-1} [m_{d-1}][R_{d-1}].
 * A dense weight w of fno_block_fwd equals W with corner c taking s_j in the high half of
 * axis j exactly when bit j of c is set.
 * The block computes the mix without forming W where that is smaller: a greedy order takes,
 * of the contractions available (a factor applied to the core, U_in applied to the spectrum,
 * the per-mode channel mix once the core carries every mode, U_out applied to the mixed
 * spectrum), the one with the smallest result first (ties: fewer flops).  The mix runs in the
 * plan's spectral precision; the factor products in float32.  ranks: d + 2 values R_in, R_out,
 * R_0 .. R_{d-1}, each in 1 .. its mode's extent (else INVALID_ARGUMENT). */
typedef struct fno_tucker fno_tucker;

/* Host only (no HIP call): the greedy contraction order for a descriptor and ranks, as a
 * space-separated list of steps, e.g. "G*U1 G*U0 X*Uin mix Y*Uout" (G*Un: factor n of the
 * modes applied to the core; G*Uin / G*Uout: a channel factor applied to the core; X*Uin:
 * U_in on the spectrum; mix; Y*Uout: U_out on the mixed spectrum).  buf receives it with its
 * terminating NUL (INVALID_ARGUMENT when len is too small). */
fno_status fno_tucker_order(const fno_plan_desc* desc, const int32_t* ranks, char* buf,
                            size_t len);

/* Bind Tucker ranks to a plan (which must outlive the result): the order above, the workspace
 * layout, and one small device table (K int32).  *out receives the object. */
fno_status fno_tucker_create(const fno_plan* plan, const int32_t* ranks, fno_tucker** out);
fno_status fno_tucker_destroy(fno_tucker* tucker);  /* NULL accepted */

/* Workspace bytes of the Tucker calls (they replace the plan's own workspace size), complex
 * elements of the core and of each of the d + 2 factors, and the contraction order (as
 * fno_tucker_order).  Any output pointer may be NULL. */
fno_status fno_tucker_query(const fno_tucker* tucker, size_t* workspace_bytes,
                            int64_t* core_elems, int64_t* factor_elems, char* order,
                            size_t order_len);

/* Keep the weight step's intermediates for the backward (keep != 0; off after create): every
 * Tucker call then takes save buffers of fno_tucker_save_bytes bytes, the plan's save followed
 * by the forward's core-chain results, U_in applied to the spectrum and the mix output before
 * U_out, which the backward reads instead of recomputing (its results are the same bits).  Off,
 * save buffers are the plan's and the backward recomputes them.  A backward must see the same
 * setting as the forward that filled its save buffer. */
fno_status fno_tucker_keep_intermediates(fno_tucker* tucker, int keep);
fno_status fno_tucker_save_bytes(const fno_tucker* tucker, size_t* bytes);

/* fno_block_fwd with the Tucker weight (core + factors: a host array of d + 2 device
 * pointers, in the order U_in, U_out, U_0 .. U_{d-1}).  The save buffer is the plan's
 * (fno_tucker_save_bytes with kept intermediates). */
fno_status fno_tucker_block_fwd(const fno_tucker* tucker, const float* x, const float* core,
                                const float* const* factors, const float* w_bypass,
                                const float* bias, float* y, void* save, void* workspace,
                                size_t workspace_bytes, void* stream);

/* fno_spectral_conv_fwd / _bwd with the Tucker weight (the spectral convolution alone; save is
 * optional as there: without it the backward recomputes the spectrum). */
fno_status fno_tucker_spectral_conv_fwd(const fno_tucker* tucker, const float* x,
                                        const float* core, const float* const* factors,
                                        float* y_spec, void* save, void* workspace,
                                        size_t workspace_bytes, void* stream);
fno_status fno_tucker_spectral_conv_bwd(const fno_tucker* tucker, const float* x,
                                        const float* core, const float* const* factors,
                                        const void* save, const float* grad_y_spec,
                                        float* grad_x, float* grad_core,
                                        float* const* grad_factors, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* fno_block_bwd with the Tucker weight: grad_core (the core's layout) and grad_factors (a host
 * array of d + 2 device pointers, each nullable; the array itself may be NULL) replace grad_w.
 * The gradient convention is W's (dL/dRe + i dL/dIm); save is required when FNO_FLAG_GELU is
 * set or any weight gradient is asked for. */
fno_status fno_tucker_block_bwd(const fno_tucker* tucker, const float* x, const float* core,
                                const float* const* factors, const float* w_bypass,
                                const float* bias, const void* save, const float* grad_y,
                                float* grad_x, float* grad_core, float* const* grad_factors,
                                float* grad_w_bypass, float* grad_bias, void* workspace,
                                size_t workspace_bytes, void* stream);

/* fno_block_fwd_mse / fno_block_bwd_preact with the Tucker weight (arguments as in
 * fno_tucker_block_fwd / _bwd; save is required for any weight gradient). */
fno_status fno_tucker_block_fwd_mse(const fno_tucker* tucker, const float* x, const float* core,
                                    const float* const* factors, const float* w_bypass,
                                    const float* bias, const float* target, float grad_scale,
                                    float* grad_z, float* loss, void* save, void* workspace,
                                    size_t workspace_bytes, void* stream);
fno_status fno_tucker_block_bwd_preact(const fno_tucker* tucker, const float* x,
                                       const float* core, const float* const* factors,
                                       const float* w_bypass, const float* bias,
                                       const void* save, const float* grad_z, float* grad_x,
                                       float* grad_core, float* const* grad_factors,
                                       float* grad_w_bypass, float* grad_bias, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* Pointwise layers used to lift into and project out of the block stack.
 * hidden == 0: y = w1 x + b1            (w1 [c_out][c_in], b1 [c_out])
 * hidden  > 0: y = w2 GELU(w1 x + b1) + b2 (w1 [hidden][c_in], w2 [c_out][hidden])
 * x [batch][c_in][npts], y [batch][c_out][npts]; biases may be NULL. c_in <= 64, c_out <= 128,
 * hidden <= 256. */
fno_status fno_pointwise_fwd(int64_t batch, int64_t npts, int64_t c_in, int64_t hidden,
                             int64_t c_out, const float* x, const float* w1, const float* b1,
                             const float* w2, const float* b2, float* y, void* stream);

/* Mean squared error: grad = 2 (y - t) / n and loss = mean((y - t)^2) written to the device
 * float *loss (deterministic two-stage reduction; nullable).  Workspace size from
 * fno_mse_workspace_bytes. */
fno_status fno_mse_workspace_bytes(int64_t n, size_t* bytes);
fno_status fno_mse_grad(int64_t n, const float* y, const float* t, float* grad, float* loss,
                        void* workspace, size_t workspace_bytes, void* stream);
/* The same with grad = grad_scale * 2 (y - t) / n (the loss itself unscaled): a static loss
 * scale, which keeps the gradients of an IEEE-half (F16) plan's backward inside half's range;
 * every gradient the backward then returns is scaled by grad_scale as well.  grad_scale must
 * be finite and > 0 (else INVALID_ARGUMENT). */
fno_status fno_mse_grad_scaled(int64_t n, const float* y, const float* t, float* grad,
                               float* loss, float grad_scale, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Per-kernel timing with HIP events, for measurement (off by default).  While enabled, every
 * kernel launch of libfno is bracketed by two events recorded on the stream it is launched
 * on, keyed by the kernel's name (e.g. "plane_fwd_tanh", "epilogue_bwd").  fno_timing_count
 * waits for the recorded events, folds them into per-name totals and returns the number of
 * names; fno_timing_get returns name, launch count and summed duration (ms) of entry
 * `index`.  The name pointer stays valid until the next fno_timing_reset.  Process-wide. */
fno_status fno_timing_enable(int enable);
/* Restrict the timer to the launches of one kernel name (NULL or "" = every launch), so that a
 * measurement can time one kernel while the others run without events.  Process-wide. */
fno_status fno_timing_select(const char* name);
fno_status fno_timing_reset(void);
fno_status fno_timing_count(int* count);
fno_status fno_timing_get(int index, const char** name, int64_t* launches, double* total_ms);

const char* fno_status_string(fno_status status);
const char* fno_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBFNO_FNO_H */
