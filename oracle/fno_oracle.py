"""Plain fp64 CPU oracle of the FNO spectral-convolution block.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (libfno and its Python binding) may
import, call or link this module; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or helper with the HIP
path: every transform here is a naive O(N*m) sum written with ``np.exp`` DFT matrices; no FFT
routine is called.

Pages cited (short names used in the docstrings below):

[MPFNO]  "Model-Parallel Fourier Neural Operators as Learned Surrogates for Large-Scale
         Parametric PDEs" (nubint.ai review page).  Section "Proposed method": the spectral
         convolution is derived from FNO's linear-algebra form; the network has 4 spectral
         blocks of embedding width 20; gradients come from automatic differentiation.
         Section "Main findings": 3D/4D space-time problems (512^3 x 20).
[MIXED]  "Guaranteed Approximation Bounds and Efficient Mixed-Precision Training for Neural
         Operators" (linnk.ai insight page).  Section "Tiivistelmä" (summary), key insights:
         the Fourier transform and the tensor contraction of the FNO block may run in half
         precision; a tanh pre-activation is applied before the Fourier transform.

The pages never print the layer's formula.  What is computed here is the standard FNO
spectral block, in this notation (d spatial axes, the last one contiguous):

  theta_k(p) = 2*pi * sum_j k_j p_j / N_j,      Ntot = prod_j N_j
  S_j        = {0..m_j-1} U {N_j-m_j..N_j-1}  for the outer axes j < d-1
  S_{d-1}    = {0..m_{d-1}-1}                  (half spectrum of the real transform)

  F1  xhat[b,i,k] = sum_p x'[b,i,p] exp(-i theta_k(p)),  k in S_0 x .. x S_{d-1},
      x' = x, or tanh(x) on the mixed-precision path [MIXED].
  F2  yhat[b,o,k] = sum_i xhat[b,i,k] W[c(k), i, o, kappa(k)]; corner c has bit j set when
      k_j lies in the high range of axis j; kappa_j = k_j (low) or k_j - (N_j - m_j) (high).
  F3  y_spec[b,o,p] = (1/Ntot) sum_k gamma(k_{d-1}) Re(yhat[b,o,k] exp(+i theta_k(p))),
      gamma = 1 for k_{d-1} = 0 or N_{d-1}/2, else 2  (the real part of the inverse of the
      zero-padded half spectrum, i.e. what irfftn returns).
  F4  z = y_spec + sum_i Wb[o,i] x[b,i,p] + bias[o];  y = GELU(z) = z/2 (1 + erf(z/sqrt2)).

Backward (gradient of a complex quantity = dL/dRe + i dL/dIm):

  B1  g_z   = g_y * (Phi(z) + z phi(z))
  B2  ghat  = (gamma/Ntot) sum_p g_z exp(-i theta_k(p))
  B3  ghx   = sum_o ghat[o] conj(W[i,o]);   dW[i,o] = sum_b conj(xhat[b,i]) ghat[b,o]
  B4  gxs   = sum_k Re(ghx exp(+i theta_k(p)))           (unit scale)
  B5  grad_x = sum_o Wb[o,i] g_z[o] + s(x) gxs,   s = 1 - tanh(x)^2 (mixed) or 1
  B6  dWb[o,i] = sum_{b,p} g_z[o] x[i];   dbias[o] = sum_{b,p} g_z[o]

Tucker-factorised weights (TFNO, one of the architectures [MIXED] "Tiivistelmä" trains in mixed
precision; the page names it only).  The weight on the retained grid, W_full[i, o, s_0..s_{d-1}]
(``expand_weights``' layout: s_j in 0..2m_j-1 on outer axes, 0..m_{d-1}-1 on the last), is held
in Tucker form (core tensor times one factor matrix per mode):

  T1  W_full = G x_1 U_in x_2 U_out x_3 U_0 .. x_{d+2} U_{d-1},
      (T x_n U)[.., a, ..] = sum_r T[.., r, ..] U[a, r]   (mode-n product: index r_n -> a)
      G complex [R_in, R_out, R_0, .., R_{d-1}], U_n complex [I_n, R_n].
  T2  grad_G   = grad_W x_1 conj(U_in)^T x_2 conj(U_out)^T .. (every mode)
  T3  grad_U_n[a, r] = sum over all other indices of grad_W[.., a, ..] conj(B_n[.., r, ..]),
      B_n = G x_m U_m over every m != n
  (W is complex-linear in each of G and the U_n, so each gradient is grad_W pulled back through
  the conjugated Jacobian.)  The block is F1-F4 with W = fold(W_full).

Input activation (a layout of the same network, not another network): a block may take a
pre-activation x and apply GELU to it first, so that the previous block need not store both
its z and y = GELU(z).  Then every use of x above uses GELU(x) and

  B7  grad_x = GELU'(x) * (grad_x of the block on GELU(x))

Layouts: fields are [B, C, N_0, .., N_{d-1}] float; ``W`` is complex
[2^(d-1), Cin, Cout, m_0, .., m_{d-1}]; ``Wb`` is [Cout, Cin]; ``bias`` is [Cout].
Everything is evaluated in float64 / complex128.
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "retained_indices", "dft_matrix", "gamma_weights", "spectrum", "expand_weights",
    "fold_weights", "channel_mix", "inverse_spectrum", "inverse_at_points", "adjoint_inverse",
    "gelu",
    "gelu_prime", "spectral_conv_fwd", "spectral_conv_bwd", "block_fwd", "block_at_points",
    "block_bwd",
    "pointwise_linear", "projection_fwd", "mse_loss_grad", "stack_fwd", "train_step",
    "mode_product", "tucker_to_full", "tucker_block_fwd", "tucker_block_bwd", "tucker_grads",
    "tucker_spectral_conv_fwd", "tucker_spectral_conv_bwd",
]


# ----------------------------------------------------------------------------- index sets
def retained_indices(n: int, m: int, last: bool) -> np.ndarray:
    """Array indices of the retained modes of one axis (S_j above), in array order.

    Outer axes keep the m lowest non-negative and the m most negative frequencies (array
    indices N-m..N-1, i.e. frequencies -m..-1); the contiguous axis keeps bins 0..m-1 of its
    half spectrum.
    """
    if last:
        return np.arange(m, dtype=np.int64)
    return np.concatenate([np.arange(m), np.arange(n - m, n)]).astype(np.int64)


def dft_matrix(n: int, ks: np.ndarray, sign: int) -> np.ndarray:
    """E[k, p] = exp(sign * 2*pi*i * ((k*p) mod n) / n) for k in ``ks``, p = 0..n-1.

    The product k*p is reduced modulo n in integers before the angle is formed, so every
    entry is the exact root of unity up to one rounding of cos/sin.
    """
    p = np.arange(n, dtype=np.int64)
    kp = np.outer(np.asarray(ks, dtype=np.int64), p) % n
    return np.exp(sign * 2j * np.pi * kp.astype(np.float64) / n)


def gamma_weights(n_last: int, m_last: int) -> np.ndarray:
    """gamma(k) of F3: 1 for the DC bin and the Nyquist bin of an even axis, else 2."""
    g = np.full(m_last, 2.0)
    g[0] = 1.0
    if n_last % 2 == 0 and m_last > n_last // 2:
        g[n_last // 2] = 1.0
    return g


def _apply_axis(a: np.ndarray, mat: np.ndarray, axis: int) -> np.ndarray:
    """out[.., k, ..] = sum_p mat[k, p] a[.., p, ..] along ``axis`` (a plain matrix product)."""
    if np.isrealobj(a):
        re = np.tensordot(a, mat.real, axes=([axis], [1]))
        im = np.tensordot(a, mat.imag, axes=([axis], [1]))
        out = re + 1j * im
    else:
        out = np.tensordot(a, mat, axes=([axis], [1]))
    return np.moveaxis(out, -1, axis)


# ----------------------------------------------------------------------------- forward
def spectrum(xp: np.ndarray, modes) -> np.ndarray:
    """F1: truncated forward DFT of a real field over all spatial axes.

    ``xp`` is [B, C, N_0..N_{d-1}] (already pre-activated); returns complex
    [B, C, 2m_0, .., 2m_{d-2}, m_{d-1}] with each axis in ``retained_indices`` order.
    Written as one naive DFT matrix product per axis (exact re-association of the
    d-dimensional sum).  [MPFNO] "Proposed method".
    """
    xp = np.asarray(xp, dtype=np.float64)
    d = xp.ndim - 2
    out = xp
    for j in reversed(range(d)):
        n = xp.shape[2 + j]
        ks = retained_indices(n, modes[j], last=(j == d - 1))
        out = _apply_axis(out, dft_matrix(n, ks, -1), 2 + j)
    return out


def _corner_slices(modes, corner: int):
    d = len(modes)
    sl = []
    for j in range(d - 1):
        h = (corner >> j) & 1
        sl.append(slice(h * modes[j], h * modes[j] + modes[j]))
    sl.append(slice(0, modes[d - 1]))
    return tuple(sl)


def expand_weights(w: np.ndarray, modes) -> np.ndarray:
    """Place the per-corner weights W[c,i,o,m..] on the retained grid (F2's c(k), kappa(k)).

    Returns complex [Cin, Cout, 2m_0, .., 2m_{d-2}, m_{d-1}]: corner c covers the low half
    (index < m_j) of axis j when bit j of c is clear and the high half when it is set.
    """
    d = len(modes)
    ncorner = 1 << (d - 1)
    assert w.shape[0] == ncorner, (w.shape, modes)
    cin, cout = w.shape[1], w.shape[2]
    full_shape = [cin, cout] + [2 * m for m in modes[:-1]] + [modes[-1]]
    full = np.zeros(full_shape, dtype=np.complex128)
    for c in range(ncorner):
        full[(slice(None), slice(None)) + _corner_slices(modes, c)] = w[c]
    return full


def fold_weights(wfull: np.ndarray, modes) -> np.ndarray:
    """Inverse of ``expand_weights``: gather the per-corner blocks back into W's layout."""
    d = len(modes)
    ncorner = 1 << (d - 1)
    return np.stack([wfull[(slice(None), slice(None)) + _corner_slices(modes, c)]
                     for c in range(ncorner)], axis=0)


def channel_mix(xhat: np.ndarray, w: np.ndarray, modes) -> np.ndarray:
    """F2: yhat[b,o,k] = sum_i xhat[b,i,k] W[c(k),i,o,kappa(k)] (per-mode complex matmul)."""
    wfull = expand_weights(np.asarray(w, dtype=np.complex128), modes)
    return np.einsum("bi...,io...->bo...", xhat, wfull)


def inverse_spectrum(yhat: np.ndarray, shape, modes, unit_scale: bool = False) -> np.ndarray:
    """F3 (and B4): real field from a truncated half spectrum.

    Default: (1/Ntot) sum_k gamma(k_last) Re(yhat_k exp(+i theta_k(p))), the inverse of the
    zero-padded half spectrum.  With ``unit_scale`` (the adjoint of F1, used by B4) the
    1/Ntot factor and gamma are both dropped.
    """
    d = len(shape)
    out = np.asarray(yhat, dtype=np.complex128)
    for j in range(d - 1):
        n = shape[j]
        ks = retained_indices(n, modes[j], last=False)
        out = _apply_axis(out, dft_matrix(n, ks, +1).T, 2 + j)
    n = shape[d - 1]
    ks = retained_indices(n, modes[d - 1], last=True)
    e = dft_matrix(n, ks, +1)  # [m, N]
    if unit_scale:
        wk = np.ones(len(ks))
        scale = 1.0
    else:
        wk = gamma_weights(n, modes[d - 1])
        scale = 1.0 / float(np.prod(shape))
    out = out * wk  # broadcasts over the last (mode) axis
    # Re(Y e^{i theta}) = Re Y cos - Im Y sin
    real = np.tensordot(out.real, e.real, axes=([out.ndim - 1], [0])) \
        - np.tensordot(out.imag, e.imag, axes=([out.ndim - 1], [0]))
    return real * scale


def inverse_at_points(yhat: np.ndarray, shape, modes, points) -> np.ndarray:
    """F3 evaluated directly at given grid points (non-separable sum over every retained mode).

    ``points`` is an int array [P, d]; returns [B, C, P].  Used to check outputs of fields too
    large to invert whole.
    """
    d = len(shape)
    pts = np.asarray(points, dtype=np.int64)
    sets = [retained_indices(shape[j], modes[j], last=(j == d - 1)) for j in range(d)]
    grids = np.meshgrid(*sets, indexing="ij")
    ntot = float(np.prod(shape))
    # phase[k, p] = 2 pi sum_j ((k_j p_j) mod N_j) / N_j
    phase = np.zeros((grids[0].size, pts.shape[0]))
    for j in range(d):
        kp = np.outer(grids[j].ravel(), pts[:, j]) % shape[j]
        phase += 2.0 * np.pi * kp / shape[j]
    gam = np.broadcast_to(gamma_weights(shape[d - 1], modes[d - 1]), grids[0].shape).ravel()
    yk = np.asarray(yhat, dtype=np.complex128).reshape(yhat.shape[0], yhat.shape[1], -1)
    e = np.exp(1j * phase) * gam[:, None]
    return np.real(np.tensordot(yk, e, axes=([2], [0]))) / ntot


def adjoint_inverse(g: np.ndarray, modes) -> np.ndarray:
    """B2: ghat = (gamma(k_last)/Ntot) sum_p g exp(-i theta_k(p)), the adjoint of F3."""
    d = g.ndim - 2
    shape = g.shape[2:]
    gh = spectrum(g, modes)
    wk = gamma_weights(shape[d - 1], modes[d - 1]) / float(np.prod(shape))
    return gh * wk


# ----------------------------------------------------------------------------- GELU
def gelu(z: np.ndarray) -> np.ndarray:
    """Exact-erf GELU: z/2 (1 + erf(z/sqrt 2))."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def gelu_prime(z: np.ndarray) -> np.ndarray:
    """d GELU/dz = Phi(z) + z phi(z)."""
    z = np.asarray(z, dtype=np.float64)
    cdf = 0.5 * (1.0 + _erf(z / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)
    return cdf + z * pdf


def _bcast(v: np.ndarray, nd: int) -> np.ndarray:
    return np.asarray(v, dtype=np.float64).reshape((1, -1) + (1,) * (nd - 2))


def _pointwise(wmat: np.ndarray, f: np.ndarray) -> np.ndarray:
    """out[b,o,p] = sum_i wmat[o,i] f[b,i,p] (a 1x1 convolution), as one matrix product."""
    out = np.tensordot(np.asarray(wmat, dtype=np.float64), f, axes=([1], [1]))
    return np.moveaxis(out, 0, 1)


# ----------------------------------------------------------------------------- spectral conv
def spectral_conv_fwd(x, w, modes, tanh: bool = False, input_gelu: bool = False):
    """F1-F3 only (no bypass, bias or activation).  Returns dict(y_spec, xhat, yhat)."""
    x = np.asarray(x, dtype=np.float64)
    if input_gelu:
        x = gelu(x)
    xp = np.tanh(x) if tanh else x
    xhat = spectrum(xp, modes)
    yhat = channel_mix(xhat, w, modes)
    y_spec = inverse_spectrum(yhat, x.shape[2:], modes)
    return {"y_spec": y_spec, "xhat": xhat, "yhat": yhat}


def spectral_conv_bwd(x, w, modes, g_yspec, tanh: bool = False, input_gelu: bool = False):
    """Adjoint of ``spectral_conv_fwd`` (B2-B4, times tanh' on the mixed path; B7 with an
    input activation).

    Returns dict(grad_x, grad_w) with grad_w in W's corner layout.
    """
    x = np.asarray(x, dtype=np.float64)
    if input_gelu:
        r = spectral_conv_bwd(gelu(x), w, modes, g_yspec, tanh=tanh)
        r["grad_x"] = gelu_prime(x) * r["grad_x"]
        return r
    g = np.asarray(g_yspec, dtype=np.float64)
    xp = np.tanh(x) if tanh else x
    xhat = spectrum(xp, modes)
    ghat = adjoint_inverse(g, modes)
    wfull = expand_weights(np.asarray(w, dtype=np.complex128), modes)
    ghx = np.einsum("bo...,io...->bi...", ghat, np.conj(wfull))
    dwfull = np.einsum("bi...,bo...->io...", np.conj(xhat), ghat)
    gxs = inverse_spectrum(ghx, x.shape[2:], modes, unit_scale=True)
    if tanh:
        gxs = gxs * (1.0 - np.tanh(x) ** 2)
    return {"grad_x": gxs, "grad_w": fold_weights(dwfull, modes), "ghat": ghat, "ghx": ghx}


# ----------------------------------------------------------------------------- block
def block_fwd(x, w, wb, bias, modes, tanh: bool = False, act: bool = True,
              input_gelu: bool = False):
    """F1-F4: one FNO block (input GELU(x) when input_gelu).  Returns dict(y, z, y_spec,
    xhat, yhat)."""
    x = np.asarray(x, dtype=np.float64)
    if input_gelu:
        x = gelu(x)
    out = spectral_conv_fwd(x, w, modes, tanh=tanh)
    z = out["y_spec"] + _pointwise(wb, x)
    if bias is not None:
        z = z + _bcast(bias, x.ndim)
    out["z"] = z
    out["y"] = gelu(z) if act else z
    return out


def block_at_points(x, w, wb, bias, modes, points, tanh: bool = False, act: bool = True,
                    input_gelu: bool = False):
    """F1-F4 evaluated only at given grid points: the spectrum of the whole field (F1, F2),
    then F3 by ``inverse_at_points`` and the bypass, bias and GELU of F4 at those points alone.

    For fields too large to invert whole (the 4D space-time share).  ``points`` is an int
    array [P, d]; returns dict(y_spec, z, y), each [B, Cout, P].
    """
    x = gelu(x) if input_gelu else np.asarray(x)
    grid = x.shape[2:]
    xp = np.tanh(np.asarray(x, dtype=np.float64)) if tanh else x
    yhat = channel_mix(spectrum(xp, modes), w, modes)
    del xp
    pts = np.asarray(points, dtype=np.int64)
    y_spec = inverse_at_points(yhat, grid, modes, pts)
    flat = np.ravel_multi_index(tuple(pts.T), grid)
    xs = x.reshape(x.shape[0], x.shape[1], -1)[:, :, flat].astype(np.float64)
    z = y_spec + _pointwise(wb, xs)
    if bias is not None:
        z = z + _bcast(bias, 3)
    return {"y_spec": y_spec, "z": z, "y": gelu(z) if act else z}


def block_bwd(x, w, wb, bias, modes, g_y, tanh: bool = False, act: bool = True,
              input_gelu: bool = False):
    """B1-B6 for one block (B7 with an input activation).  Returns dict(grad_x, grad_w,
    grad_wb, grad_bias, g_z, gx_spec)."""
    x = np.asarray(x, dtype=np.float64)
    if input_gelu:
        r = block_bwd(gelu(x), w, wb, bias, modes, g_y, tanh=tanh, act=act)
        r["grad_x"] = gelu_prime(x) * r["grad_x"]
        r["gx_spec"] = gelu_prime(x) * r["gx_spec"]
        return r
    g_y = np.asarray(g_y, dtype=np.float64)
    fwd = block_fwd(x, w, wb, bias, modes, tanh=tanh, act=act)
    g_z = g_y * gelu_prime(fwd["z"]) if act else g_y
    sp = spectral_conv_bwd(x, w, modes, g_z, tanh=tanh)
    grad_x = _pointwise(np.asarray(wb, dtype=np.float64).T, g_z) + sp["grad_x"]
    red = (0,) + tuple(range(2, x.ndim))
    grad_wb = np.tensordot(g_z, x, axes=(red, red))
    grad_bias = g_z.sum(axis=red)
    return {"grad_x": grad_x, "grad_w": sp["grad_w"], "grad_wb": grad_wb,
            "grad_bias": grad_bias, "g_z": g_z, "gx_spec": sp["grad_x"],
            "ghat": sp["ghat"], "ghx": sp["ghx"], "fwd": fwd}


# ----------------------------------------------------------------------------- lift / projection / loss
def pointwise_linear(x, wmat, bias):
    """Lift (1x1 linear layer, no activation): out = wmat x + bias."""
    x = np.asarray(x, dtype=np.float64)
    out = _pointwise(wmat, x)
    if bias is not None:
        out = out + _bcast(bias, x.ndim)
    return out


def projection_fwd(x, w1, b1, w2, b2):
    """Projection head: Linear(C -> H), GELU, Linear(H -> Cout), pointwise."""
    h = gelu(pointwise_linear(x, w1, b1))
    return pointwise_linear(h, w2, b2)


def mse_loss_grad(y, t):
    """L = mean((y - t)^2) and dL/dy = 2 (y - t) / numel."""
    y = np.asarray(y, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    diff = y - t
    return float(np.mean(diff * diff)), 2.0 * diff / diff.size


def block_fwd_mse(x, w, wb, bias, modes, target, grad_scale: float = 1.0, tanh: bool = False,
                  act: bool = True, input_gelu: bool = False):
    """The last block of a training step followed by the loss (F1-F4, then A12), reported at
    the block's pre-activation: loss = mean((y - t)^2) and grad_z = grad_scale * dloss/dz,
    i.e. the loss gradient 2 (y - t) / numel through the output GELU's derivative (B1).
    Returns dict(loss, grad_z, fwd)."""
    fwd = block_fwd(x, w, wb, bias, modes, tanh=tanh, act=act, input_gelu=input_gelu)
    loss, g_y = mse_loss_grad(fwd["y"], target)
    g_z = g_y * gelu_prime(fwd["z"]) if act else g_y
    return {"loss": loss, "grad_z": grad_scale * g_z, "fwd": fwd}


def block_bwd_preact(x, w, wb, bias, modes, g_z, tanh: bool = False, input_gelu: bool = False):
    """B2-B6 (and B7) of one block from the gradient at its pre-activation z: block_bwd with
    the output GELU's derivative already applied."""
    return block_bwd(x, w, wb, bias, modes, g_z, tanh=tanh, act=False, input_gelu=input_gelu)


# ----------------------------------------------------------------------------- stacks
def stack_fwd(x, blocks, modes, tanh: bool = False, lift=None, proj=None):
    """Lift (optional) -> FNO blocks (GELU after each) -> projection (optional).

    ``blocks`` is a list of dicts with keys w, wb, bias.  [MPFNO] "Proposed method":
    4 spectral blocks.
    """
    h = np.asarray(x, dtype=np.float64)
    if lift is not None:
        h = pointwise_linear(h, lift["w"], lift["b"])
    for blk in blocks:
        h = block_fwd(h, blk["w"], blk["wb"], blk["bias"], modes, tanh=tanh)["y"]
    if proj is not None:
        h = projection_fwd(h, proj["w1"], proj["b1"], proj["w2"], proj["b2"])
    return h


def train_step(x, target, blocks, modes, tanh: bool = False):
    """Forward through the blocks, MSE against ``target``, backward through the blocks.

    Returns dict(loss, y, grad_x, grads=[per block dict(grad_w, grad_wb, grad_bias)]).
    """
    acts = [np.asarray(x, dtype=np.float64)]
    for blk in blocks:
        acts.append(block_fwd(acts[-1], blk["w"], blk["wb"], blk["bias"], modes,
                              tanh=tanh)["y"])
    loss, g = mse_loss_grad(acts[-1], target)
    grads = [None] * len(blocks)
    for li in reversed(range(len(blocks))):
        blk = blocks[li]
        r = block_bwd(acts[li], blk["w"], blk["wb"], blk["bias"], modes, g, tanh=tanh)
        grads[li] = {"grad_w": r["grad_w"], "grad_wb": r["grad_wb"],
                     "grad_bias": r["grad_bias"]}
        g = r["grad_x"]
    return {"loss": loss, "y": acts[-1], "grad_x": g, "grads": grads}


# ----------------------------------------------------------------------------- Tucker weights
def mode_product(t: np.ndarray, u: np.ndarray, n: int) -> np.ndarray:
    """T1's mode-n product: (T x_n U)[.., a, ..] = sum_r T[.., r, ..] U[a, r]."""
    t = np.asarray(t, dtype=np.complex128)
    u = np.asarray(u, dtype=np.complex128)
    assert t.shape[n] == u.shape[1], (t.shape, u.shape, n)
    r = np.tensordot(t, u, axes=([n], [1]))  # the new index a comes last
    return np.moveaxis(r, -1, n)


def tucker_to_full(core, factors) -> np.ndarray:
    """T1: the retained-grid weight W_full [Cin, Cout, 2m_0, .., m_{d-1}] of a Tucker core and
    its factors [U_in, U_out, U_0, .., U_{d-1}]."""
    t = np.asarray(core, dtype=np.complex128)
    assert t.ndim == len(factors), (t.shape, len(factors))
    for n, u in enumerate(factors):
        t = mode_product(t, u, n)
    return t


def _check_tucker_shapes(core, factors, cin, cout, modes):
    want = [cin, cout] + [2 * m for m in modes[:-1]] + [modes[-1]]
    assert len(factors) == len(want) == np.ndim(core)
    for n, u in enumerate(factors):
        assert np.shape(u) == (want[n], np.shape(core)[n]), (n, np.shape(u), want[n])


def tucker_block_fwd(x, core, factors, wb, bias, modes, tanh: bool = False, act: bool = True):
    """One FNO block whose spectral weight is T1's Tucker form (F1-F4 on W = fold(W_full))."""
    x = np.asarray(x, dtype=np.float64)
    _check_tucker_shapes(core, factors, x.shape[1], np.shape(wb)[0], modes)
    w = fold_weights(tucker_to_full(core, factors), modes)
    return block_fwd(x, w, wb, bias, modes, tanh=tanh, act=act)


def tucker_block_bwd(x, core, factors, wb, bias, modes, g_y, tanh: bool = False,
                     act: bool = True):
    """B1-B6 with T2 / T3 for the Tucker factors.  Returns block_bwd's dict plus grad_core
    and grad_factors (same order as ``factors``)."""
    x = np.asarray(x, dtype=np.float64)
    _check_tucker_shapes(core, factors, x.shape[1], np.shape(wb)[0], modes)
    core = np.asarray(core, dtype=np.complex128)
    factors = [np.asarray(u, dtype=np.complex128) for u in factors]
    w = fold_weights(tucker_to_full(core, factors), modes)
    r = block_bwd(x, w, wb, bias, modes, g_y, tanh=tanh, act=act)
    r["grad_core"], r["grad_factors"] = tucker_grads(core, factors,
                                                     expand_weights(r["grad_w"], modes))
    return r


def tucker_grads(core, factors, gw):
    """T2 and T3: the core and factor gradients from the retained-grid weight gradient gw."""
    core = np.asarray(core, dtype=np.complex128)
    factors = [np.asarray(u, dtype=np.complex128) for u in factors]
    # T2: every mode contracted with the conjugated factor
    gcore = gw
    for n, u in enumerate(factors):
        gcore = mode_product(gcore, np.conj(u).T, n)
    # T3: B_n = G with every factor but the n-th applied; contract all indices except n
    gfac = []
    for n in range(len(factors)):
        bn = core
        for m, u in enumerate(factors):
            if m != n:
                bn = mode_product(bn, u, m)
        axes = [a for a in range(gw.ndim) if a != n]
        gfac.append(np.tensordot(gw, np.conj(bn), axes=(axes, axes)))
    return gcore, gfac


def tucker_spectral_conv_fwd(x, core, factors, modes, tanh: bool = False):
    """F1-F3 with T1's Tucker weight."""
    x = np.asarray(x, dtype=np.float64)
    _check_tucker_shapes(core, factors, x.shape[1], np.shape(factors[1])[0], modes)
    return spectral_conv_fwd(x, fold_weights(tucker_to_full(core, factors), modes), modes,
                             tanh=tanh)


def tucker_spectral_conv_bwd(x, core, factors, modes, g_yspec, tanh: bool = False):
    """The adjoint of tucker_spectral_conv_fwd: grad_x, grad_core, grad_factors (T2 / T3)."""
    x = np.asarray(x, dtype=np.float64)
    _check_tucker_shapes(core, factors, x.shape[1], np.shape(factors[1])[0], modes)
    r = spectral_conv_bwd(x, fold_weights(tucker_to_full(core, factors), modes), modes, g_yspec,
                          tanh=tanh)
    r["grad_core"], r["grad_factors"] = tucker_grads(core, factors,
                                                     expand_weights(r["grad_w"], modes))
    return r
