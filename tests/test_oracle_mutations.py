"""Plant plausible mistakes in the oracle (on the CPU) and show that a pin catches each.

Every mutation below replaces one oracle function with a subtly wrong copy (a flipped
sign, an index off by one, a dropped term, a transposed or unconjugated operand).  The
named pin must then fail.  This is what makes the pins meaningful: a pin that passes on a
broken oracle pins nothing.
"""
import math

import numpy as np
import pytest

import oracle.fno_oracle as O
from tests import oracle_pins as P

_orig = {name: getattr(O, name) for name in dir(O) if not name.startswith("__")}


def _dft_sign_flipped(n, ks, sign):
    return _orig["dft_matrix"](n, ks, -sign)


def _retained_off_by_one(n, m, last):
    if last:
        return np.arange(m, dtype=np.int64)
    return np.concatenate([np.arange(m), np.arange(n - m - 1, n - 1)]).astype(np.int64)


def _gamma_all_two(n_last, m_last):
    return np.full(m_last, 2.0)


def _gamma_no_nyquist(n_last, m_last):
    g = np.full(m_last, 2.0)
    g[0] = 1.0
    return g


def _expand_bits_reversed(w, modes):
    d = len(modes)
    if d < 3:
        return _orig["expand_weights"](w, modes)
    ncorner = 1 << (d - 1)
    perm = []
    for c in range(ncorner):
        r = 0
        for j in range(d - 1):
            if (c >> j) & 1:
                r |= 1 << (d - 2 - j)
        perm.append(r)
    return _orig["expand_weights"](w[perm], modes)


def _mix_conj(xhat, w, modes):
    return _orig["channel_mix"](xhat, np.conj(w), modes)


def _inverse_imag_sign(yhat, shape, modes, unit_scale=False):
    return _orig["inverse_spectrum"](np.conj(yhat), shape, modes, unit_scale)


def _adjoint_no_gamma(g, modes):
    d = g.ndim - 2
    return _orig["spectrum"](g, modes) / float(np.prod(g.shape[2:]))


def _gelu_prime_no_pdf(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * (1.0 + np.vectorize(math.erf)(z / math.sqrt(2.0)))


def _bwd_no_conj(x, w, modes, g_yspec, tanh=False):
    return _orig["spectral_conv_bwd"](x, np.conj(w), modes, g_yspec, tanh)


def _block_bwd_no_tanh_prime(x, w, wb, bias, modes, g_y, tanh=False, act=True):
    r = _orig["block_bwd"](x, w, wb, bias, modes, g_y, tanh=tanh, act=act)
    if tanh:
        r = dict(r)
        r["grad_x"] = r["grad_x"] - r["gx_spec"] + r["gx_spec"] / np.maximum(
            1.0 - np.tanh(x) ** 2, 1e-300)
    return r


def _block_no_bias(x, w, wb, bias, modes, tanh=False, act=True):
    return _orig["block_fwd"](x, w, wb, None, modes, tanh=tanh, act=act)


def _mode_product_transposed(t, u, n):
    return _orig["mode_product"](t, np.asarray(u).T, n)


def _mode_product_conj(t, u, n):
    return _orig["mode_product"](t, np.conj(u), n)


def _tucker_bwd_factor_unconj(x, core, factors, wb, bias, modes, g_y, tanh=False, act=True):
    r = _orig["tucker_block_bwd"](x, core, factors, wb, bias, modes, g_y, tanh, act)
    r = dict(r)
    r["grad_factors"] = [np.conj(gf) for gf in r["grad_factors"]]
    return r


def _tucker_bwd_core_one_mode_short(x, core, factors, wb, bias, modes, g_y, tanh=False,
                                    act=True):
    r = _orig["tucker_block_bwd"](x, core, factors, wb, bias, modes, g_y, tanh, act)
    r = dict(r)
    # the last mode's conjugated factor left out of T2 (replaced by its plain transpose)
    u = np.asarray(factors[-1])
    n = len(factors) - 1
    gw = O.expand_weights(r["grad_w"], modes)
    gc = gw
    for m, um in enumerate(factors):
        gc = _orig["mode_product"](gc, (np.conj(um) if m != n else um).T, m)
    r["grad_core"] = gc
    return r


def _block_bwd_input_gelu_no_prime(x, w, wb, bias, modes, g_y, tanh=False, act=True,
                                   input_gelu=False):
    if not input_gelu:
        return _orig["block_bwd"](x, w, wb, bias, modes, g_y, tanh=tanh, act=act)
    return _orig["block_bwd"](O.gelu(x), w, wb, bias, modes, g_y, tanh=tanh, act=act)


def _fused_loss_no_gelu_prime(x, w, wb, bias, modes, target, grad_scale=1.0, tanh=False,
                              act=True, input_gelu=False):
    # the loss gradient handed on as if y were z (the output GELU's derivative dropped)
    r = _orig["block_fwd_mse"](x, w, wb, bias, modes, target, grad_scale, tanh, False,
                               input_gelu)
    fwd = _orig["block_fwd"](x, w, wb, bias, modes, tanh=tanh, act=act, input_gelu=input_gelu)
    r = dict(r)
    r["loss"] = float(np.mean((fwd["y"] - np.asarray(target, dtype=np.float64)) ** 2))
    r["grad_z"] = grad_scale * 2.0 * (fwd["y"] - target) / fwd["y"].size
    r["fwd"] = fwd
    return r


def _preact_bwd_gelu_twice(x, w, wb, bias, modes, g_z, tanh=False, input_gelu=False):
    # the output GELU's derivative applied again on top of the pre-activation gradient
    return _orig["block_bwd"](x, w, wb, bias, modes, g_z, tanh=tanh, act=True,
                              input_gelu=input_gelu)


def _lift_no_bias(x, wmat, bias):
    return _orig["pointwise_linear"](x, wmat, None)


def _projection_gelu_after_second(x, w1, b1, w2, b2):
    h = _orig["pointwise_linear"](x, w1, b1)
    return O.gelu(_orig["pointwise_linear"](h, w2, b2))


def _block_points_common(x, w, wb, bias, modes, points, tanh, act, input_gelu, bypass_src,
                         flip_points):
    x = np.asarray(x, dtype=np.float64)
    if input_gelu:
        x = O.gelu(x)
    grid = x.shape[2:]
    xp = np.tanh(x) if tanh else x
    yhat = O.channel_mix(O.spectrum(xp, modes), w, modes)
    pts = np.asarray(points, dtype=np.int64)
    y_spec = O.inverse_at_points(yhat, grid, modes, pts)
    if flip_points:
        flat = np.ravel_multi_index(tuple(pts[:, ::-1].T), grid[::-1])
    else:
        flat = np.ravel_multi_index(tuple(pts.T), grid)
    src = xp if bypass_src == "preact" else x
    xs = src.reshape(x.shape[0], x.shape[1], -1)[:, :, flat]
    z = y_spec + np.einsum("oi,bip->bop", wb, xs) + np.asarray(bias)[None, :, None]
    return {"y_spec": y_spec, "z": z, "y": O.gelu(z) if act else z}


def _block_points_bypass_on_tanh(x, w, wb, bias, modes, points, tanh=False, act=True,
                                 input_gelu=False):
    # the bypass fed the tanh pre-activated field instead of the block's input
    return _block_points_common(x, w, wb, bias, modes, points, tanh, act, input_gelu,
                                "preact", False)


def _block_points_index_order(x, w, wb, bias, modes, points, tanh=False, act=True,
                              input_gelu=False):
    # the bypass gathers x with the point coordinates in reversed axis order
    return _block_points_common(x, w, wb, bias, modes, points, tanh, act, input_gelu, "x",
                                True)


MUTATIONS = [
    ("pointwise_linear", _lift_no_bias, P.check_pointwise_lift_projection),
    ("projection_fwd", _projection_gelu_after_second, P.check_pointwise_lift_projection),
    ("block_at_points", _block_points_bypass_on_tanh, P.check_block_at_points),
    ("block_at_points", _block_points_index_order, P.check_block_at_points),
    ("block_fwd_mse", _fused_loss_no_gelu_prime, P.check_fused_loss),
    ("block_bwd_preact", _preact_bwd_gelu_twice, P.check_fused_loss),
    ("dft_matrix", _dft_sign_flipped, P.check_spectrum_bruteforce),
    ("retained_indices", _retained_off_by_one, P.check_spectrum_numpy_fft),
    ("gamma_weights", _gamma_all_two, P.check_roundtrip_identity),
    ("gamma_weights", _gamma_no_nyquist, P.check_parseval_and_dc),
    ("expand_weights", _expand_bits_reversed, P.check_single_mode_closed_form),
    ("channel_mix", _mix_conj, P.check_single_mode_closed_form),
    ("inverse_spectrum", _inverse_imag_sign, P.check_inverse_numpy_irfftn),
    ("adjoint_inverse", _adjoint_no_gamma, P.check_adjoint_identities),
    ("gelu_prime", _gelu_prime_no_pdf, P.check_gelu),
    ("spectral_conv_bwd", _bwd_no_conj, P.check_adjoint_identities),
    ("block_bwd", _block_bwd_no_tanh_prime, P.check_block_finite_differences),
    ("block_fwd", _block_no_bias, P.check_zero_weight_block),
    ("block_bwd", _block_bwd_input_gelu_no_prime, P.check_input_activation),
    ("mode_product", _mode_product_transposed, P.check_tucker_hosvd),
    ("mode_product", _mode_product_conj, P.check_tucker_hosvd),
    ("tucker_block_bwd", _tucker_bwd_factor_unconj, P.check_tucker_block_finite_differences),
    ("tucker_block_bwd", _tucker_bwd_core_one_mode_short,
     P.check_tucker_block_finite_differences),
]


@pytest.mark.parametrize("name,bad,check", MUTATIONS,
                         ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_pin_catches_mutation(monkeypatch, name, bad, check):
    monkeypatch.setattr(O, name, bad)
    with pytest.raises((AssertionError, ValueError)):
        check(O)


def _inverse_points_no_gamma(yhat, shape, modes, points):
    import numpy as _np
    d = len(shape)
    pts = _np.asarray(points)
    sets = [O.retained_indices(shape[j], modes[j], last=(j == d - 1)) for j in range(d)]
    grids = _np.meshgrid(*sets, indexing="ij")
    phase = sum(2 * _np.pi * _np.outer(grids[j].ravel(), pts[:, j]) / shape[j] for j in range(d))
    yk = yhat.reshape(yhat.shape[0], yhat.shape[1], -1)
    return _np.real(_np.tensordot(yk, _np.exp(1j * phase), axes=([2], [0]))) / _np.prod(shape)


def test_point_inverse_pin_catches_missing_gamma(monkeypatch):
    monkeypatch.setattr(O, "inverse_at_points", _inverse_points_no_gamma)
    with pytest.raises(AssertionError):
        P.check_inverse_at_points(O)
