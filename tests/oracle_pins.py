"""Pin checks for the fp64 oracle.

Each ``check_*`` function raises AssertionError when the oracle disagrees with something the
definition or the mathematics fixes independently of the oracle's own code: brute-force
non-separable sums, a library FFT, Parseval, closed forms for single Fourier modes, the
cutoff, symmetries, adjoint identities and finite differences.  ``test_oracle_pins.py`` runs
them on the oracle as it is; ``test_oracle_mutations.py`` runs them on deliberately broken
copies of it to show that the pins catch plausible mistakes.
"""
from __future__ import annotations

import itertools
import math

import numpy as np


def _rng(seed):
    return np.random.default_rng(np.random.SeedSequence([77, seed]))


def _rand_w(g, d, cin, cout, modes):
    shape = (1 << (d - 1), cin, cout) + tuple(modes)
    return g.standard_normal(shape) + 1j * g.standard_normal(shape)


def _close(a, b, tol, what):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)
    assert err <= tol, f"{what}: rel max err {err:.3e} > {tol:.1e}"


# ------------------------------------------------------------------ F1: forward transform
GRIDS = [((8, 8), (3, 3)), ((4, 4, 4), (1, 2, 2)), ((4, 4, 4, 6), (2, 1, 2, 3))]


def check_spectrum_bruteforce(O):
    """Non-separable sum over all points for every retained mode (8x8, 4^3, 4^3x6)."""
    for gi, (grid, modes) in enumerate(GRIDS):
        g = _rng(gi)
        d = len(grid)
        x = g.standard_normal((2, 3) + grid)
        got = O.spectrum(x, modes)
        sets = []
        for j in range(d):
            n, m = grid[j], modes[j]
            sets.append(list(range(m)) if j == d - 1 else list(range(m)) + list(range(n - m, n)))
        pts = np.stack(np.meshgrid(*[np.arange(n) for n in grid], indexing="ij"), axis=0)
        want = np.zeros(got.shape, dtype=np.complex128)
        for pos in itertools.product(*[range(len(s)) for s in sets]):
            k = [sets[j][pos[j]] for j in range(d)]
            phase = sum(2.0 * math.pi * k[j] * pts[j] / grid[j] for j in range(d))
            kern = np.exp(-1j * phase)
            want[(slice(None), slice(None)) + pos] = np.tensordot(x, kern, axes=(
                tuple(range(2, 2 + d)), tuple(range(d))))
        _close(got, want, 1e-12, f"brute force F1 {grid}")


def check_spectrum_numpy_fft(O):
    """Library pin: the retained entries of numpy.fft.rfftn (test-side only)."""
    for gi, (grid, modes) in enumerate(GRIDS + [((12, 10), (4, 5)), ((6, 8, 10), (3, 2, 6))]):
        g = _rng(10 + gi)
        d = len(grid)
        x = g.standard_normal((2, 2) + grid)
        full = np.fft.rfftn(x, axes=tuple(range(2, 2 + d)))
        idx = []
        for j in range(d):
            n, m = grid[j], modes[j]
            idx.append(np.arange(m) if j == d - 1 else np.r_[0:m, n - m:n])
        want = full[np.ix_(range(2), range(2), *idx)]
        _close(O.spectrum(x, modes), want, 1e-12, f"rfftn pin {grid}")


def check_parseval_and_dc(O):
    """Full modes: sum x^2 = (1/Ntot) sum_half gamma |X|^2; X_0 = sum x."""
    for gi, grid in enumerate([(8, 8), (6, 10), (4, 4, 6), (4, 2, 4, 6)]):
        g = _rng(20 + gi)
        d = len(grid)
        modes = tuple(n // 2 for n in grid[:-1]) + (grid[-1] // 2 + 1,)
        x = g.standard_normal((1, 1) + grid)
        X = O.spectrum(x, modes)
        ntot = float(np.prod(grid))
        gam = O.gamma_weights(grid[-1], modes[-1])
        lhs = float(np.sum(x * x))
        rhs = float(np.sum(gam * np.abs(X) ** 2) / ntot)
        assert abs(lhs - rhs) <= 1e-11 * lhs, ("Parseval", grid, lhs, rhs)
        assert abs(X[(0, 0) + (0,) * d] - np.sum(x)) <= 1e-11 * np.sum(np.abs(x)), "DC"


# ------------------------------------------------------------------ F3: inverse
def check_roundtrip_identity(O):
    """Full modes and W = identity on every mode: y_spec = x exactly (up to rounding)."""
    for gi, grid in enumerate([(8, 8), (6, 10), (4, 6, 8), (4, 2, 4, 6), (8, 5)]):
        g = _rng(30 + gi)
        d = len(grid)
        modes = tuple(n // 2 for n in grid[:-1]) + (grid[-1] // 2 + 1,)
        c = 3
        x = g.standard_normal((2, c) + grid)
        w = np.zeros((1 << (d - 1), c, c) + modes, dtype=np.complex128)
        for i in range(c):
            w[:, i, i] = 1.0
        y = O.spectral_conv_fwd(x, w, modes)["y_spec"]
        _close(y, x, 1e-12, f"round trip {grid}")


def check_inverse_numpy_irfftn(O):
    """R3 pin: the inverse equals numpy.fft.irfftn of the zero-padded (non-Hermitian) half
    spectrum, which keeps only the real part of the DC/Nyquist bins of the last axis."""
    for gi, (grid, modes) in enumerate([((8, 8), (3, 3)), ((6, 10), (2, 4)),
                                        ((4, 6, 8), (2, 3, 4)), ((4, 4, 4, 6), (2, 1, 2, 3))]):
        g = _rng(40 + gi)
        d = len(grid)
        shp = (2, 3) + tuple(2 * m for m in modes[:-1]) + (modes[-1],)
        Y = g.standard_normal(shp) + 1j * g.standard_normal(shp)
        pad = np.zeros((2, 3) + tuple(grid[:-1]) + (grid[-1] // 2 + 1,), dtype=np.complex128)
        idx = []
        for j in range(d):
            n, m = grid[j], modes[j]
            idx.append(np.arange(m) if j == d - 1 else np.r_[0:m, n - m:n])
        pad[np.ix_(range(2), range(3), *idx)] = Y
        want = np.fft.irfftn(pad, s=grid, axes=tuple(range(2, 2 + d)))
        _close(O.inverse_spectrum(Y, grid, modes), want, 1e-12, f"irfftn pin {grid}")


# ------------------------------------------------------------------ F2: mix + corners
def _theta(grid, k):
    pts = np.meshgrid(*[np.arange(n) for n in grid], indexing="ij")
    return sum(2.0 * math.pi * k[j] * pts[j] / grid[j] for j in range(len(grid)))


def check_single_mode_closed_form(O):
    """x_i = A cos(theta_k + phi) on channel i only, 0 < k_last < N_last/2, k retained in
    corner c  =>  y_spec_o = A Re(W[c,i,o,kappa] exp(i (theta_k + phi))).  One case per
    corner, in 2D, 3D and 4D, with Cin != Cout so a transposed W cannot pass."""
    cases = [((12, 10), (3, 4)), ((8, 10, 12), (2, 3, 5)), ((6, 8, 4, 10), (2, 3, 1, 4))]
    for gi, (grid, modes) in enumerate(cases):
        g = _rng(50 + gi)
        d = len(grid)
        cin, cout = 3, 2
        w = _rand_w(g, d, cin, cout, modes)
        for corner in range(1 << (d - 1)):
            kappa = [int(g.integers(0, modes[j])) for j in range(d - 1)]
            kappa.append(int(g.integers(1, modes[-1])))
            k = []
            for j in range(d - 1):
                high = (corner >> j) & 1
                k.append(kappa[j] - modes[j] if high else kappa[j])  # signed frequency
            k.append(kappa[-1])
            i = int(g.integers(0, cin))
            amp, phi = 1.7, 0.3 + corner
            x = np.zeros((1, cin) + grid)
            th = _theta(grid, k)
            x[0, i] = amp * np.cos(th + phi)
            y = O.spectral_conv_fwd(x, w, modes)["y_spec"]
            wk = w[(corner, i, slice(None)) + tuple(kappa)]
            want = amp * np.real(wk[:, None] * np.exp(1j * (th.reshape(1, -1) + phi)))
            _close(y[0].reshape(cout, -1), want, 1e-11,
                   f"single mode grid={grid} corner={corner} k={k}")


def check_single_mode_dc_plane(O):
    """k_last = 0: the output takes both +k and -k, i.e.
    (A/2) Re(W_k e^{i(theta+phi)} + W_{-k} e^{-i(theta+phi)}), with the -k term dropped
    when -k is not retained (k_j = -m_j)."""
    grid, modes = (12, 10), (3, 4)
    g = _rng(60)
    cin, cout = 2, 3
    w = _rand_w(g, 2, cin, cout, modes)
    wfull = O.expand_weights(w, modes)  # index by retained position
    pos_of = {kk: p for p, kk in enumerate(list(range(3)) + list(range(-3, 0)))}
    for k0 in [1, 2, -1, -3, 0]:
        k = (k0, 0)
        th = _theta(grid, k)
        amp, phi = 0.9, -0.4
        x = np.zeros((1, cin) + grid)
        x[0, 1] = amp * np.cos(th + phi)
        y = O.spectral_conv_fwd(x, w, modes)["y_spec"][0]
        if k0 == 0:
            want = amp * np.cos(phi) * np.real(wfull[1, :, pos_of[0], 0])[:, None, None] \
                * np.ones((1,) + grid)
        else:
            wp = wfull[1, :, pos_of[k0], 0]
            term = wp[:, None, None] * np.exp(1j * (th + phi))[None]
            if -k0 in pos_of:
                wm = wfull[1, :, pos_of[-k0], 0]
                term = term + wm[:, None, None] * np.exp(-1j * (th + phi))[None]
            want = 0.5 * amp * np.real(term)
        _close(y, want, 1e-11, f"dc-plane mode k0={k0}")


def check_cutoff(O):
    """Any mode outside the retained set (with 0 < k_last < N_last/2) gives y_spec = 0."""
    grid, modes = (16, 12), (3, 4)
    g = _rng(70)
    w = _rand_w(g, 2, 2, 2, modes)
    for k in [(5, 1), (0, 4), (3, 2), (-4, 3), (8, 5), (4, 4)]:
        x = np.zeros((1, 2) + grid)
        x[0, 0] = np.cos(_theta(grid, k) + 0.2)
        y = O.spectral_conv_fwd(x, w, modes)["y_spec"]
        assert np.max(np.abs(y)) < 1e-13, ("cutoff", k, np.max(np.abs(y)))
    grid3, modes3 = (8, 10, 12), (2, 3, 4)
    w3 = _rand_w(g, 3, 2, 2, modes3)
    for k in [(2, 0, 1), (0, 3, 1), (1, 1, 4), (-3, 1, 2)]:
        x = np.zeros((1, 2) + grid3)
        x[0, 1] = np.cos(_theta(grid3, k))
        y = O.spectral_conv_fwd(x, w3, modes3)["y_spec"]
        assert np.max(np.abs(y)) < 1e-13, ("cutoff 3D", k, np.max(np.abs(y)))


def check_linearity_equivariance_selfadjoint(O):
    grid, modes = (10, 12), (3, 4)
    g = _rng(80)
    c = 3
    w = _rand_w(g, 2, c, c, modes)
    w2 = _rand_w(g, 2, c, c, modes)
    x1 = g.standard_normal((2, c) + grid)
    x2 = g.standard_normal((2, c) + grid)
    f = lambda x, ww: O.spectral_conv_fwd(x, ww, modes)["y_spec"]  # noqa: E731
    _close(f(2.0 * x1 - 3.0 * x2, w), 2.0 * f(x1, w) - 3.0 * f(x2, w), 1e-12, "linear in x")
    _close(f(x1, w + 2.0 * w2), f(x1, w) + 2.0 * f(x1, w2), 1e-12, "linear in W")
    sh = (3, 5)
    _close(f(np.roll(x1, sh, axis=(2, 3)), w), np.roll(f(x1, w), sh, axis=(2, 3)), 1e-12,
           "translation equivariance")
    wb = g.standard_normal((c, c))
    bias = g.standard_normal(c)
    blk = lambda x: O.block_fwd(x, w, wb, bias, modes)["y"]  # noqa: E731
    _close(blk(np.roll(x1, sh, axis=(2, 3))), np.roll(blk(x1), sh, axis=(2, 3)), 1e-12,
           "block translation equivariance")
    # W = identity on every retained mode: the map is an orthogonal projection (symmetric)
    eye = np.zeros_like(w)
    for i in range(c):
        eye[:, i, i] = 1.0
    lhs = np.sum(f(x1, eye) * x2)
    rhs = np.sum(x1 * f(x2, eye))
    assert abs(lhs - rhs) <= 1e-12 * (abs(lhs) + 1.0), ("self-adjoint", lhs, rhs)


# ------------------------------------------------------------------ F4: epilogue
def check_gelu(O):
    import random
    z = np.linspace(-6, 6, 241)
    _close(O.gelu(z) - O.gelu(-z), z, 1e-14, "GELU(z)-GELU(-z)=z")
    assert O.gelu(np.array([0.0]))[0] == 0.0
    r = random.Random(5)
    for _ in range(50):
        v = r.uniform(-8, 8)
        want = 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0)))
        assert abs(O.gelu(np.array([v]))[0] - want) <= 1e-15 * max(1.0, abs(want)), v
    h = 1e-6
    fd = (O.gelu(z + h) - O.gelu(z - h)) / (2 * h)
    _close(O.gelu_prime(z), fd, 1e-8, "GELU' vs central difference")


def check_zero_weight_block(O):
    """W = 0: the block is GELU(Wb x + b) computed pointwise with explicit loops."""
    g = _rng(90)
    grid, modes = (4, 6), (2, 2)
    cin, cout = 3, 2
    x = g.standard_normal((2, cin) + grid)
    w = np.zeros((2, cin, cout) + modes, dtype=np.complex128)
    wb = g.standard_normal((cout, cin))
    bias = g.standard_normal(cout)
    y = O.block_fwd(x, w, wb, bias, modes)["y"]
    for b in range(2):
        for o in range(cout):
            for p0 in range(grid[0]):
                for p1 in range(grid[1]):
                    z = bias[o] + sum(wb[o, i] * x[b, i, p0, p1] for i in range(cin))
                    want = 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0)))
                    assert abs(y[b, o, p0, p1] - want) < 1e-13 * max(1, abs(want))


# ------------------------------------------------------------------ backward
def check_adjoint_identities(O):
    """<A x, g> = <x, A^T g> for the x-map and <dy[dW], g> = sum Re(conj(dW) dW') for the
    W-map, in 2D, 3D and 4D."""
    for gi, (grid, modes) in enumerate([((10, 12), (3, 4)), ((6, 8, 10), (2, 3, 4)),
                                        ((4, 6, 4, 8), (2, 2, 1, 3))]):
        g = _rng(100 + gi)
        d = len(grid)
        cin, cout = 3, 2
        w = _rand_w(g, d, cin, cout, modes)
        x = g.standard_normal((2, cin) + grid)
        gy = g.standard_normal((2, cout) + grid)
        y = O.spectral_conv_fwd(x, w, modes)["y_spec"]
        bw = O.spectral_conv_bwd(x, w, modes, gy)
        lhs = np.sum(y * gy)
        rhs = np.sum(x * bw["grad_x"])
        assert abs(lhs - rhs) <= 1e-11 * (abs(lhs) + np.sqrt(np.sum(y * y))), ("x-adjoint", lhs, rhs)
        dw = _rand_w(g, d, cin, cout, modes)
        ydw = O.spectral_conv_fwd(x, dw, modes)["y_spec"]  # y is linear in W
        lhs = np.sum(ydw * gy)
        rhs = np.sum(np.real(np.conj(bw["grad_w"]) * dw))
        assert abs(lhs - rhs) <= 1e-11 * (abs(lhs) + 1.0), ("W-adjoint", lhs, rhs)


def check_block_finite_differences(O):
    """fp64 central differences of L = <y, g> through the whole block (tanh, GELU, bypass,
    bias), in 2D and 3D, for sampled entries of x, W (re and im), Wb and bias."""
    for gi, (grid, modes, tanh) in enumerate([((6, 8), (2, 3), False), ((6, 8), (2, 3), True),
                                              ((4, 4, 6), (1, 2, 2), True)]):
        g = _rng(120 + gi)
        d = len(grid)
        cin, cout = 2, 3
        x = g.standard_normal((2, cin) + grid)
        w = _rand_w(g, d, cin, cout, modes) * 0.5
        wb = g.standard_normal((cout, cin))
        bias = g.standard_normal(cout)
        gy = g.standard_normal((2, cout) + grid)
        L = lambda x_, w_, wb_, b_: float(np.sum(  # noqa: E731
            O.block_fwd(x_, w_, wb_, b_, modes, tanh=tanh)["y"] * gy))
        r = O.block_bwd(x, w, wb, bias, modes, gy, tanh=tanh)
        h = 1e-6

        def fd(arr, idx, setter):
            a_p = arr.copy()
            a_m = arr.copy()
            setter(a_p, idx, h)
            setter(a_m, idx, -h)
            return a_p, a_m

        def add_real(a, idx, dlt):
            a[idx] += dlt

        def add_imag(a, idx, dlt):
            a[idx] += 1j * dlt

        for _ in range(6):
            idx = tuple(int(g.integers(0, s)) for s in x.shape)
            xp, xm = fd(x, idx, add_real)
            num = (L(xp, w, wb, bias) - L(xm, w, wb, bias)) / (2 * h)
            assert abs(num - r["grad_x"][idx]) < 1e-6 * max(1, abs(num)), ("dx", idx, num, r["grad_x"][idx])
        for _ in range(6):
            idx = tuple(int(g.integers(0, s)) for s in w.shape)
            for setter, part in ((add_real, np.real), (add_imag, np.imag)):
                wp, wm = fd(w, idx, setter)
                num = (L(x, wp, wb, bias) - L(x, wm, wb, bias)) / (2 * h)
                ana = part(r["grad_w"][idx])
                assert abs(num - ana) < 1e-6 * max(1, abs(num)), ("dW", idx, num, ana)
        for _ in range(4):
            idx = (int(g.integers(0, cout)), int(g.integers(0, cin)))
            p, m = fd(wb, idx, add_real)
            num = (L(x, w, p, bias) - L(x, w, m, bias)) / (2 * h)
            assert abs(num - r["grad_wb"][idx]) < 1e-6 * max(1, abs(num)), ("dWb", idx)
        for o in range(cout):
            p, m = fd(bias, (o,), add_real)
            num = (L(x, w, wb, p) - L(x, w, wb, m)) / (2 * h)
            assert abs(num - r["grad_bias"][o]) < 1e-6 * max(1, abs(num)), ("dbias", o)


def check_mse_and_stack(O):
    """MSE gradient by central differences; a 2-block train step's input gradient by FD."""
    g = _rng(140)
    y = g.standard_normal((2, 3, 4, 5))
    t = g.standard_normal((2, 3, 4, 5))
    loss, gr = O.mse_loss_grad(y, t)
    assert abs(loss - np.mean((y - t) ** 2)) < 1e-15 * 10
    h = 1e-6
    for _ in range(5):
        idx = tuple(int(g.integers(0, s)) for s in y.shape)
        yp = y.copy()
        ym = y.copy()
        yp[idx] += h
        ym[idx] -= h
        num = (O.mse_loss_grad(yp, t)[0] - O.mse_loss_grad(ym, t)[0]) / (2 * h)
        assert abs(num - gr[idx]) < 1e-8
    grid, modes = (6, 8), (2, 3)
    c = 2
    blocks = [{"w": _rand_w(g, 2, c, c, modes) * 0.3, "wb": g.standard_normal((c, c)),
               "bias": g.standard_normal(c)} for _ in range(2)]
    x = g.standard_normal((1, c) + grid)
    tgt = g.standard_normal((1, c) + grid)
    res = O.train_step(x, tgt, blocks, modes, tanh=True)
    for _ in range(4):
        idx = tuple(int(g.integers(0, s)) for s in x.shape)
        xp = x.copy()
        xm = x.copy()
        xp[idx] += h
        xm[idx] -= h
        lp = O.mse_loss_grad(O.stack_fwd(xp, blocks, modes, tanh=True), tgt)[0]
        lm = O.mse_loss_grad(O.stack_fwd(xm, blocks, modes, tanh=True), tgt)[0]
        num = (lp - lm) / (2 * h)
        assert abs(num - res["grad_x"][idx]) < 1e-6 * max(1e-3, abs(num)), ("stack dx", num)


def check_fused_loss(O):
    """The last block fused with the loss: grad_z by central differences of the loss in z
    (the output GELU between them), and the pre-activation backward's grad_x, grad_Wb and
    grad_bias by central differences of loss(block(x)) (input GELU on and off); grad_scale
    only scales the gradient."""
    h = 1e-6
    for gi, (grid, modes, tanh, ig) in enumerate([((6, 8), (2, 3), True, False),
                                                  ((4, 4, 6), (1, 2, 2), False, True)]):
        g = _rng(160 + gi)
        d = len(grid)
        c = 2
        x = g.standard_normal((2, c) + grid)
        w = _rand_w(g, d, c, c, modes) * 0.4
        wb = g.standard_normal((c, c))
        bias = g.standard_normal(c)
        tgt = g.standard_normal((2, c) + grid)
        r = O.block_fwd_mse(x, w, wb, bias, modes, tgt, tanh=tanh, input_gelu=ig)
        z = r["fwd"]["z"]
        loss_z = lambda z_: float(np.mean((O.gelu(z_) - tgt) ** 2))  # noqa: E731
        assert abs(r["loss"] - loss_z(z)) < 1e-12 * max(1.0, r["loss"])
        for _ in range(5):
            idx = tuple(int(g.integers(0, s)) for s in z.shape)
            zp = z.copy()
            zm = z.copy()
            zp[idx] += h
            zm[idx] -= h
            num = (loss_z(zp) - loss_z(zm)) / (2 * h)
            assert abs(num - r["grad_z"][idx]) < 1e-6 * max(1e-3, abs(num)), \
                ("grad_z", idx, num, r["grad_z"][idx])
        r8 = O.block_fwd_mse(x, w, wb, bias, modes, tgt, grad_scale=8.0, tanh=tanh,
                             input_gelu=ig)
        _close(r8["grad_z"], 8.0 * r["grad_z"], 1e-15, "grad_scale")
        b = O.block_bwd_preact(x, w, wb, bias, modes, r["grad_z"], tanh=tanh, input_gelu=ig)
        L = lambda x_, wb_, b_: O.block_fwd_mse(  # noqa: E731
            x_, w, wb_, b_, modes, tgt, tanh=tanh, input_gelu=ig)["loss"]
        for _ in range(5):
            idx = tuple(int(g.integers(0, s)) for s in x.shape)
            xp = x.copy()
            xm = x.copy()
            xp[idx] += h
            xm[idx] -= h
            num = (L(xp, wb, bias) - L(xm, wb, bias)) / (2 * h)
            assert abs(num - b["grad_x"][idx]) < 1e-6 * max(1e-3, abs(num)), ("dx", idx, num)
        for _ in range(3):
            idx = (int(g.integers(0, c)), int(g.integers(0, c)))
            p = wb.copy()
            m = wb.copy()
            p[idx] += h
            m[idx] -= h
            num = (L(x, p, bias) - L(x, m, bias)) / (2 * h)
            assert abs(num - b["grad_wb"][idx]) < 1e-6 * max(1e-3, abs(num)), ("dWb", idx)
        for o in range(c):
            p = bias.copy()
            m = bias.copy()
            p[o] += h
            m[o] -= h
            num = (L(x, wb, p) - L(x, wb, m)) / (2 * h)
            assert abs(num - b["grad_bias"][o]) < 1e-6 * max(1e-3, abs(num)), ("dbias", o)


def check_inverse_at_points(O):
    """The point-wise inverse agrees with numpy's irfftn of the zero-padded spectrum at
    every sampled point (2D, 3D, 4D)."""
    for gi, (grid, modes) in enumerate([((8, 10), (3, 4)), ((6, 8, 10), (2, 3, 4)),
                                        ((4, 6, 4, 8), (2, 2, 1, 3))]):
        g = _rng(150 + gi)
        d = len(grid)
        shp = (1, 2) + tuple(2 * m for m in modes[:-1]) + (modes[-1],)
        Y = g.standard_normal(shp) + 1j * g.standard_normal(shp)
        pad = np.zeros((1, 2) + tuple(grid[:-1]) + (grid[-1] // 2 + 1,), dtype=np.complex128)
        idx = [np.arange(modes[j]) if j == d - 1 else
               np.r_[0:modes[j], grid[j] - modes[j]:grid[j]] for j in range(d)]
        pad[np.ix_(range(1), range(2), *idx)] = Y
        full = np.fft.irfftn(pad, s=grid, axes=tuple(range(2, 2 + d)))
        pts = np.stack([g.integers(0, n, 9) for n in grid], axis=1)
        got = O.inverse_at_points(Y, grid, modes, pts)
        want = np.stack([full[(slice(None), slice(None)) + tuple(p)] for p in pts], axis=-1)
        _close(got, want, 1e-12, f"inverse at points {grid}")


def check_input_activation(O):
    """A block on a pre-activation x with input_gelu is the same block on GELU(x) (forward),
    and its grad_x obeys the chain rule (fp64 central differences through the whole block,
    tanh path, with and without the output GELU)."""
    g = _rng(300)
    grid, modes = (6, 8), (2, 3)
    cin, cout = 2, 3
    x = g.standard_normal((2, cin) + grid)
    w = _rand_w(g, 2, cin, cout, modes) * 0.5
    wb = g.standard_normal((cout, cin))
    bias = g.standard_normal(cout)
    gy = g.standard_normal((2, cout) + grid)
    xg = O.gelu(x)
    for act in (True, False):
        a = O.block_fwd(x, w, wb, bias, modes, tanh=True, act=act, input_gelu=True)["y"]
        b = O.block_fwd(xg, w, wb, bias, modes, tanh=True, act=act)["y"]
        assert np.array_equal(a, b)
        r = O.block_bwd(x, w, wb, bias, modes, gy, tanh=True, act=act, input_gelu=True)
        h = 1e-6
        for _ in range(6):
            idx = tuple(int(g.integers(0, s_)) for s_ in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            L = lambda xx: float(np.sum(O.block_fwd(xx, w, wb, bias, modes, tanh=True,  # noqa: E731
                                                    act=act, input_gelu=True)["y"] * gy))
            num = (L(xp) - L(xm)) / (2 * h)
            assert abs(num - r["grad_x"][idx]) < 1e-6 * max(1, abs(num)), (act, idx, num)
        sp = O.spectral_conv_bwd(x, w, modes, gy, tanh=True, input_gelu=True)
        for _ in range(3):
            idx = tuple(int(g.integers(0, s_)) for s_ in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            Ls = lambda xx: float(np.sum(O.spectral_conv_fwd(xx, w, modes, tanh=True,  # noqa: E731
                                                             input_gelu=True)["y_spec"] * gy))
            num = (Ls(xp) - Ls(xm)) / (2 * h)
            assert abs(num - sp["grad_x"][idx]) < 1e-6 * max(1, abs(num)), ("spec", idx, num)


# ------------------------------------------------------------------ T1-T3: Tucker weights
def _crand(g, shape):
    return g.standard_normal(shape) + 1j * g.standard_normal(shape)


def _apply_mode(t, m, n):
    """t with matrix m[a, r] applied on axis n, written with an explicit einsum subscript."""
    letters = "abcdefgh"[:t.ndim]
    out = letters[:n] + "z" + letters[n + 1:]
    return np.einsum(f"{letters},z{letters[n]}->{out}", t, m)


def check_tucker_identity_factors(O):
    """Square identity factors leave the core unchanged."""
    g = _rng(200)
    shape = (3, 2, 4, 5)
    core = _crand(g, shape)
    got = O.tucker_to_full(core, [np.eye(n) for n in shape])
    assert np.array_equal(got, core)


def check_tucker_hosvd(O):
    """Higher-order SVD (Kolda and Bader, "Tensor decompositions and applications"): with U_n
    the left singular vectors of the mode-n unfolding and core = W x_n conj(U_n)^T for every n,
    the full-rank Tucker form reconstructs W, and truncating mode n to R_n columns costs at most
    the sum over modes of the discarded squared singular values.  The factors are unitary and
    not symmetric, so a transposed or conjugated factor in the oracle's product fails."""
    g = _rng(201)
    for shape in [(3, 4, 6, 5), (2, 3, 4, 4, 3)]:
        W = _crand(g, shape)
        Us, svals = [], []
        for n in range(len(shape)):
            unf = np.moveaxis(W, n, 0).reshape(shape[n], -1)
            U, sv, _ = np.linalg.svd(unf, full_matrices=True)
            Us.append(U)
            svals.append(sv)
        core = W
        for n, U in enumerate(Us):
            core = _apply_mode(core, np.conj(U).T, n)
        _close(O.tucker_to_full(core, Us), W, 1e-12, f"HOSVD round trip {shape}")
        ranks = [max(1, n - 1) for n in shape]
        tcore = core[tuple(slice(0, r) for r in ranks)]
        approx = O.tucker_to_full(tcore, [U[:, :r] for U, r in zip(Us, ranks)])
        bound = sum(float(np.sum(sv[r:] ** 2)) for sv, r in zip(svals, ranks))
        err = float(np.sum(np.abs(W - approx) ** 2))
        assert 0.0 < err <= bound * (1 + 1e-12), (shape, err, bound)


def check_tucker_rank_one(O):
    """A rank-1 Tucker form is the scaled outer product of its factor vectors."""
    g = _rng(202)
    dims = (3, 4, 6, 5)
    c = complex(g.standard_normal(), g.standard_normal())
    vecs = [_crand(g, (n,)) for n in dims]
    want = c * vecs[0]
    for v in vecs[1:]:
        want = np.multiply.outer(want, v)
    got = O.tucker_to_full(np.full((1,) * len(dims), c), [v[:, None] for v in vecs])
    _close(got, want, 1e-13, "rank-1 Tucker")


def check_tucker_block_finite_differences(O):
    """fp64 central differences of L = <y, g> through a whole block (tanh, GELU, bypass) with
    Tucker weights, for the real and imaginary parts of sampled core and factor entries, in 2D
    and 3D."""
    for gi, (grid, modes, ranks) in enumerate([((6, 8), (2, 3), (2, 3, 3, 2)),
                                               ((4, 4, 6), (1, 2, 2), (2, 2, 2, 3, 1))]):
        g = _rng(210 + gi)
        cin, cout = 2, 3
        dims = [cin, cout] + [2 * m for m in modes[:-1]] + [modes[-1]]
        x = g.standard_normal((2, cin) + grid)
        core = _crand(g, ranks) * 0.5
        facs = [_crand(g, (n, r)) * 0.5 for n, r in zip(dims, ranks)]
        wb = g.standard_normal((cout, cin))
        bias = g.standard_normal(cout)
        gy = g.standard_normal((2, cout) + grid)

        def L(core_, facs_):
            return float(np.sum(O.tucker_block_fwd(x, core_, facs_, wb, bias, modes,
                                                   tanh=True)["y"] * gy))

        r = O.tucker_block_bwd(x, core, facs, wb, bias, modes, gy, tanh=True)
        h = 1e-6
        targets = [("core", None)] + [("factor", n) for n in range(len(facs))]
        for what, n in targets:
            arr = core if n is None else facs[n]
            ana_all = r["grad_core"] if n is None else r["grad_factors"][n]
            for _ in range(3):
                idx = tuple(int(g.integers(0, s_)) for s_ in arr.shape)
                for dlt, part in ((h, np.real), (1j * h, np.imag)):
                    ap, am = arr.copy(), arr.copy()
                    ap[idx] += dlt
                    am[idx] -= dlt
                    if n is None:
                        num = (L(ap, facs) - L(am, facs)) / (2 * h)
                    else:
                        fp = list(facs)
                        fm = list(facs)
                        fp[n], fm[n] = ap, am
                        num = (L(core, fp) - L(core, fm)) / (2 * h)
                    ana = part(ana_all[idx])
                    assert abs(num - ana) < 1e-6 * max(1, abs(num)), (what, n, idx, num, ana)



def check_pointwise_lift_projection(O):
    """The lift (1x1 linear layer with bias) and the projection head (Linear, GELU, Linear)
    evaluated point by point with explicit loops and math.erf."""
    g = _rng(170)
    b, cin, hid, cout = 2, 3, 5, 2
    grid = (3, 4)
    x = g.standard_normal((b, cin) + grid)
    w1 = g.standard_normal((hid, cin))
    b1 = g.standard_normal(hid)
    w2 = g.standard_normal((cout, hid))
    b2 = g.standard_normal(cout)
    lift = O.pointwise_linear(x, w1, b1)
    proj = O.projection_fwd(x, w1, b1, w2, b2)
    for bi in range(b):
        for p0 in range(grid[0]):
            for p1 in range(grid[1]):
                h = []
                for k in range(hid):
                    a = b1[k] + sum(w1[k, i] * x[bi, i, p0, p1] for i in range(cin))
                    assert abs(lift[bi, k, p0, p1] - a) < 1e-13 * max(1.0, abs(a)), ("lift", k)
                    h.append(0.5 * a * (1.0 + math.erf(a / math.sqrt(2.0))))
                for o in range(cout):
                    want = b2[o] + sum(w2[o, k] * h[k] for k in range(hid))
                    got = proj[bi, o, p0, p1]
                    assert abs(got - want) < 1e-13 * max(1.0, abs(want)), ("projection", o)
    assert np.array_equal(O.pointwise_linear(x, w1, None),
                          O.pointwise_linear(x, w1, np.zeros(hid)))


def check_block_at_points(O):
    """The point-wise block (spectrum, mix, point-wise inverse, bypass, bias, GELU at sampled
    points only) equals the whole-field block at those points: 2D, 3D and 4D, with and without
    tanh and input GELU."""
    cases = [((8, 10), (3, 4), False, False), ((6, 8, 10), (2, 3, 4), True, False),
             ((4, 6, 4, 8), (2, 2, 1, 3), False, True)]
    for gi, (grid, modes, tanh, ig) in enumerate(cases):
        g = _rng(180 + gi)
        d = len(grid)
        cin, cout = 3, 2
        x = g.standard_normal((2, cin) + grid)
        w = _rand_w(g, d, cin, cout, modes)
        wb = g.standard_normal((cout, cin))
        bias = g.standard_normal(cout)
        full = O.block_fwd(x, w, wb, bias, modes, tanh=tanh, input_gelu=ig)
        pts = np.stack([g.integers(0, n, 11) for n in grid], axis=1)
        got = O.block_at_points(x, w, wb, bias, modes, pts, tanh=tanh, input_gelu=ig)
        for key in ("y_spec", "z", "y"):
            want = np.stack([full[key][(slice(None), slice(None)) + tuple(p)] for p in pts],
                            axis=-1)
            _close(got[key], want, 1e-12, f"block at points {grid} {key}")


ALL_CHECKS = [
    check_inverse_at_points,
    check_spectrum_bruteforce, check_spectrum_numpy_fft, check_parseval_and_dc,
    check_roundtrip_identity, check_inverse_numpy_irfftn, check_single_mode_closed_form,
    check_single_mode_dc_plane, check_cutoff, check_linearity_equivariance_selfadjoint,
    check_gelu, check_zero_weight_block, check_adjoint_identities,
    check_block_finite_differences, check_mse_and_stack,
    check_input_activation, check_fused_loss,
    check_tucker_identity_factors, check_tucker_hosvd, check_tucker_rank_one,
    check_tucker_block_finite_differences,
    check_pointwise_lift_projection, check_block_at_points,
]
