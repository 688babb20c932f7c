"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and the oracle.

This module only draws numbers: it holds none of the spectral block's arithmetic (no
transform, mix, bypass or activation), and neither the oracle nor the HIP binding imports
the other through it.  Every array is generated on the host in float64 from
``np.random.default_rng(SeedSequence([cfg_id, stream, index]))`` and returned as float32,
so the GPU and the oracle receive byte-identical values.

Streams: 0 input field, 1 spectral weights, 2 bypass weights, 3 bias, 4 target field,
5 lift/projection weights, 6 permeability layers, 7 Tucker core and factors.

The pages' datasets (CO2 plume simulations, the mixed-precision study's PDE datasets) are
not available; these fields stand in for them with the same shapes:
* Gaussian random fields with power spectral density proportional to (|k|^2 + 9)^-2 over
  integer wavenumbers (amplitude (|k|^2+9)^-1), zero mean and unit variance per channel.
* Coordinate channels p_j / N_j on the periodic grid.
* A layered log-normal permeability channel: 8 layers along axis 0 separated by 7 sorted
  uniform random interfaces, values exp(N(0, 1)).
"""
from __future__ import annotations

import numpy as np
import scipy.fft as _sfft

(STREAM_INPUT, STREAM_W, STREAM_WB, STREAM_BIAS, STREAM_TARGET, STREAM_PROJ, STREAM_LAYERS,
 STREAM_TUCKER) = range(8)


def rng(cfg_id: int, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg_id, stream, index]))


def _grf_filter(grid):
    """Amplitude (|k|^2 + 9)^-1 on the rfftn grid of ``grid`` (integer wavenumbers)."""
    ks = []
    for j, n in enumerate(grid):
        if j == len(grid) - 1:
            k = np.arange(n // 2 + 1, dtype=np.float64)
        else:
            k = np.fft.fftfreq(n, d=1.0 / n)
        shape = [1] * len(grid)
        shape[j] = k.size
        ks.append((k * k).reshape(shape))
    k2 = sum(ks)
    return 1.0 / (k2 + 9.0)


def grf(g: np.random.Generator, lead: int, grid) -> np.ndarray:
    """``lead`` independent Gaussian random fields on ``grid`` -> float32 [lead, *grid].

    Fields are built one at a time (white noise, spectral filter, back to space) and
    normalised to zero mean and unit variance.
    """
    grid = tuple(int(n) for n in grid)
    axes = tuple(range(len(grid)))
    filt = _grf_filter(grid).astype(np.float32)
    out = np.empty((lead,) + grid, dtype=np.float32)
    for i in range(lead):
        w = g.standard_normal(grid, dtype=np.float32)
        f = _sfft.rfftn(w, axes=axes, workers=-1)
        f *= filt
        f.flat[0] = 0.0
        v = _sfft.irfftn(f, s=grid, axes=axes, workers=-1).astype(np.float64)
        v -= v.mean()
        v /= max(v.std(), 1e-30)
        out[i] = v.astype(np.float32)
    return out


def normal(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    return (g.standard_normal(shape) * std).astype(np.float32)


def field(w, stream: int = STREAM_INPUT, channels=None) -> np.ndarray:
    """Input (stream 0) or target (stream 4) field of workload ``w`` -> float32 [B, C, *grid]."""
    c = channels if channels is not None else (w.lift_in if (w.lift_in and stream == STREAM_INPUT)
                                               else w.width)
    shape = (w.batch, c) + tuple(w.grid)
    g = rng(w.cfg_id, stream)
    if w.input_kind == "normal":
        return normal(g, shape)
    x = grf(g, w.batch * c, w.grid).reshape(shape)
    if stream != STREAM_INPUT:
        return x
    if w.input_kind == "grf_coords":
        # channel 0 a GRF, channels 1.. the coordinates p_j / N_j of the first axes
        for j in range(1, c):
            n = w.grid[j - 1]
            coord = (np.arange(n, dtype=np.float64) / n).astype(np.float32)
            shp = [1] * len(w.grid)
            shp[j - 1] = n
            x[:, j] = np.broadcast_to(coord.reshape(shp), w.grid)
    elif w.input_kind == "grf_layered":
        gl = rng(w.cfg_id, STREAM_LAYERS)
        n0 = w.grid[0]
        for b in range(w.batch):
            cuts = np.sort(gl.uniform(0.0, 1.0, 7)) * n0
            vals = np.exp(gl.standard_normal(8))
            layer = np.searchsorted(cuts, np.arange(n0) + 0.5)
            prof = vals[layer].astype(np.float32)
            shp = [n0] + [1] * (len(w.grid) - 1)
            x[b, 0] = np.broadcast_to(prof.reshape(shp), w.grid)
    return x


def spectral_weights(w, block: int = 0, cin=None, cout=None, modes=None) -> np.ndarray:
    """Complex weights [2^(d-1), Cin, Cout, m_0..m_{d-1}] as complex64; real and imaginary
    parts U(0, 1) / (Cin * Cout)."""
    cin = cin or w.width
    cout = cout or w.width
    modes = tuple(modes or w.modes)
    shape = (1 << (len(modes) - 1), cin, cout) + modes
    g = rng(w.cfg_id, STREAM_W, block)
    scale = 1.0 / (cin * cout)
    re = g.uniform(0.0, 1.0, shape) * scale
    im = g.uniform(0.0, 1.0, shape) * scale
    return (re + 1j * im).astype(np.complex64)


def bypass_weights(w, block: int = 0, cin=None, cout=None) -> np.ndarray:
    """1x1 bypass weight [Cout, Cin] ~ N(0, 1/Cin)."""
    cin = cin or w.width
    cout = cout or w.width
    return normal(rng(w.cfg_id, STREAM_WB, block), (cout, cin), std=1.0 / np.sqrt(cin))


def bias(w, block: int = 0, cin=None, cout=None) -> np.ndarray:
    """Bias [Cout]: zero when the workload says so, else U(-1/sqrt(Cin), 1/sqrt(Cin))."""
    cin = cin or w.width
    cout = cout or w.width
    if w.zero_bias:
        return np.zeros(cout, dtype=np.float32)
    lim = 1.0 / np.sqrt(cin)
    return rng(w.cfg_id, STREAM_BIAS, block).uniform(-lim, lim, cout).astype(np.float32)


def tucker_params(w, block: int = 0, cin=None, cout=None, modes=None, ranks=None):
    """Tucker core [R_in, R_out, R_0..] and factors [C_in, R_in], [C_out, R_out], [2 m_j, R_j],
    [m_{d-1}, R_{d-1}] as complex64: factor entries complex normal with variance 1/extent (unit
    expected column norm), core entries complex normal times 1/(C_in C_out)."""
    cin = cin or w.width
    cout = cout or w.width
    modes = tuple(modes or w.modes)
    ranks = tuple(ranks or w.tucker_ranks)
    ext = [cin, cout] + [2 * m for m in modes[:-1]] + [modes[-1]]
    g = rng(w.cfg_id, STREAM_TUCKER, block)
    factors = []
    for n, r in zip(ext, ranks):
        u = (g.standard_normal((n, r)) + 1j * g.standard_normal((n, r))) / np.sqrt(2.0 * n)
        factors.append(u.astype(np.complex64))
    core = (g.standard_normal(ranks) + 1j * g.standard_normal(ranks)) / (cin * cout)
    return core.astype(np.complex64), factors


def block_params(w, n_blocks=None):
    """Per-block parameter dicts for ``n_blocks`` blocks: (w, wb, bias), or (core, factors,
    wb, bias) for workloads with Tucker-factorised spectral weights."""
    n = w.blocks if n_blocks is None else n_blocks
    out = []
    for i in range(n):
        blk = {"wb": bypass_weights(w, i), "bias": bias(w, i)}
        if getattr(w, "tucker_ranks", None):
            blk["core"], blk["factors"] = tucker_params(w, i)
        else:
            blk["w"] = spectral_weights(w, i)
        out.append(blk)
    return out


def lift_proj_params(w):
    """Lift [C, Cin0] ~ N(0, 1/Cin0) and projection [H, C], [Cout, H] ~ N(0, 1/fan_in)."""
    g = rng(w.cfg_id, STREAM_PROJ)
    c, cin0, hid, cout = w.width, w.lift_in, w.proj_hidden, w.proj_out

    def lin(fan_in, fan_out):
        wm = (g.standard_normal((fan_out, fan_in)) / np.sqrt(fan_in)).astype(np.float32)
        lim = 1.0 / np.sqrt(fan_in)
        bv = g.uniform(-lim, lim, fan_out).astype(np.float32)
        return wm, bv

    lw, lb = lin(cin0, c)
    w1, b1 = lin(c, hid)
    w2, b2 = lin(hid, cout)
    return {"lift": {"w": lw, "b": lb}, "proj": {"w1": w1, "b1": b1, "w2": w2, "b2": b2}}


def small_case(seed: int, batch: int, cin: int, cout: int, grid, modes, zero_bias=False):
    """Random small problem for parity tests: x ~ N(0,1), W, Wb, bias as above."""
    g = np.random.default_rng(np.random.SeedSequence([1000, seed]))
    grid = tuple(grid)
    modes = tuple(modes)
    x = g.standard_normal((batch, cin) + grid).astype(np.float32)
    shape = (1 << (len(modes) - 1), cin, cout) + modes
    scale = 1.0 / (cin * cout)
    wc = ((g.uniform(0, 1, shape) + 1j * g.uniform(0, 1, shape)) * scale).astype(np.complex64)
    wb = (g.standard_normal((cout, cin)) / np.sqrt(cin)).astype(np.float32)
    lim = 1.0 / np.sqrt(cin)
    bv = np.zeros(cout, np.float32) if zero_bias else g.uniform(-lim, lim, cout).astype(np.float32)
    return x, wc, wb, bv


def normal_like(seed: int, shape) -> np.ndarray:
    g = np.random.default_rng(np.random.SeedSequence([2000, seed]))
    return g.standard_normal(shape).astype(np.float32)
