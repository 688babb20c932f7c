"""The contiguous-axis FFT of float32 plans (FNO_FLAG_LAST_AXIS_FFT) against the fp64 oracle.

Rows of 128, 256 and 512 points (L = 4, 8 and 16 lanes per row in the kernel), every column
tile count of the row spectra (16, 32 and 64 columns, with zero columns past m_b), the most
bins a row holds (32), a single bin, chunked planes whose last chunk is a ragged part of a
64-row block, 2D, 3D and 4D fields, and every operand prologue the transform takes: plain x,
tanh(x), GELU(x) of a pre-activation input, tanh(GELU(x)), and g * GELU'(z) in the backward.
Each output on its own, relative L2 <= 1e-5.  The dense and the FFT plans of one shape are
also compared with each other.
"""
import zlib

import numpy as np
import pytest

import oracle.fno_oracle as O
from fno_spectral_convolution_amd import inputs
from tests.gpu_helpers import TOL_F32, announce, check, rel_l2

pytestmark = pytest.mark.gpu

FFT_CASES = [
    # name, batch, cin, cout, grid, modes
    ("nb128_ragged_rows", 2, 16, 16, (40, 128), (8, 10)),
    ("nb128_mb32", 1, 4, 4, (16, 128), (4, 32)),
    ("nb128_chunked_ragged", 1, 3, 2, (200, 128), (12, 16)),
    ("nb256_c32", 3, 32, 32, (24, 256), (4, 16)),
    ("nb256_one_bin", 2, 2, 2, (16, 256), (4, 1)),
    ("nb512_c64", 2, 64, 64, (64, 512), (8, 32)),
    ("nb512_chunked", 1, 2, 2, (256, 512), (16, 32)),
    ("nb512_mb8", 2, 5, 3, (32, 512), (8, 8)),
    ("3d_nb256", 2, 4, 3, (6, 16, 256), (2, 4, 12)),
    ("4d_nb128", 1, 3, 4, (4, 6, 8, 128), (2, 2, 4, 8)),
]


def _torch():
    import torch
    return torch


def _dev(a):
    return _torch().from_numpy(np.ascontiguousarray(a)).to("cuda")


def _host(t):
    return t.detach().cpu().numpy()


@pytest.fixture(scope="module")
def L():
    from fno_spectral_convolution_amd import binding
    return binding


@pytest.mark.parametrize("tanh", [False, True], ids=["x", "tanh"])
@pytest.mark.parametrize("case", FFT_CASES, ids=[c[0] for c in FFT_CASES])
def test_fft_block_fwd_bwd(L, case, tanh):
    name, batch, cin, cout, grid, modes = case
    announce("fft block", name, tanh)
    seed = 3100 + zlib.crc32(name.encode()) % 1000
    x, w, wb, b = inputs.small_case(seed, batch, cin, cout, grid, modes)
    gy = inputs.normal_like(seed, (batch, cout) + grid)
    plan = L.Plan(batch, cin, cout, grid, modes, tanh=tanh, last_axis="fft")
    assert plan.last_axis_fft
    tx, tw, twb, tb, tg = (_dev(a) for a in (x, w, wb, b, gy))
    save = plan.new_save()
    y = plan.block_fwd(tx, tw, twb, tb, save=save)
    g = plan.block_bwd(tx, tw, twb, tb, save, tg)
    _torch().cuda.synchronize()
    ref = O.block_bwd(x, w, wb, b, modes, gy, tanh=tanh)
    check("y", _host(y), ref["fwd"]["y"], TOL_F32)
    check("grad_x", _host(g["x"]), ref["grad_x"], TOL_F32)
    check("grad_w", _host(g["w"]), ref["grad_w"], TOL_F32)
    check("grad_wb", _host(g["wb"]), ref["grad_wb"], TOL_F32)
    check("grad_bias", _host(g["bias"]), ref["grad_bias"], TOL_F32)
    plan.close()


@pytest.mark.parametrize("case", FFT_CASES, ids=[c[0] for c in FFT_CASES])
def test_fft_spectral_conv(L, case):
    """The spectral path alone, where no bypass term hides a transform error."""
    name, batch, cin, cout, grid, modes = case
    announce("fft spectral", name)
    seed = 4100 + zlib.crc32(name.encode()) % 1000
    x, w, _, _ = inputs.small_case(seed, batch, cin, cout, grid, modes)
    gy = inputs.normal_like(seed, (batch, cout) + grid)
    plan = L.Plan(batch, cin, cout, grid, modes, gelu=False, bias=False, last_axis="fft")
    tx, tw, tg = (_dev(a) for a in (x, w, gy))
    save = plan.new_save()
    ys = plan.spectral_conv_fwd(tx, tw, save=save)
    gx, gw = plan.spectral_conv_bwd(tx, tw, tg, save=save)
    _torch().cuda.synchronize()
    fwd = O.spectral_conv_fwd(x, w, modes)
    bwd = O.spectral_conv_bwd(x, w, modes, gy)
    check("y_spec", _host(ys), fwd["y_spec"], TOL_F32)
    check("grad_x", _host(gx), bwd["grad_x"], TOL_F32)
    check("grad_w", _host(gw), bwd["grad_w"], TOL_F32)
    plan.close()


@pytest.mark.parametrize("tanh", [False, True], ids=["gelu", "tanh_gelu"])
@pytest.mark.parametrize("case", FFT_CASES[::3], ids=[c[0] for c in FFT_CASES[::3]])
def test_fft_input_gelu(L, case, tanh):
    """A block whose input is a pre-activation: the transform's prologue is GELU(x) or
    tanh(GELU(x)), and the backward's is g * GELU'(z) of the block's output."""
    name, batch, cin, cout, grid, modes = case
    announce("fft input_gelu", name, tanh)
    seed = 5100 + zlib.crc32(name.encode()) % 1000
    x, w, wb, b = inputs.small_case(seed, batch, cin, cout, grid, modes)
    gy = inputs.normal_like(seed, (batch, cout) + grid)
    plan = L.Plan(batch, cin, cout, grid, modes, tanh=tanh, input_gelu=True, last_axis="fft")
    tx, tw, twb, tb, tg = (_dev(a) for a in (x, w, wb, b, gy))
    save = plan.new_save()
    y = plan.block_fwd(tx, tw, twb, tb, save=save)
    g = plan.block_bwd(tx, tw, twb, tb, save, tg)
    _torch().cuda.synchronize()
    ref = O.block_bwd(x, w, wb, b, modes, gy, tanh=tanh, input_gelu=True)
    check("y", _host(y), ref["fwd"]["y"], TOL_F32)
    check("grad_x", _host(g["x"]), ref["grad_x"], TOL_F32)
    check("grad_w", _host(g["w"]), ref["grad_w"], TOL_F32)
    check("grad_wb", _host(g["wb"]), ref["grad_wb"], TOL_F32)
    check("grad_bias", _host(g["bias"]), ref["grad_bias"], TOL_F32)
    plan.close()


@pytest.mark.parametrize("case", FFT_CASES[::2], ids=[c[0] for c in FFT_CASES[::2]])
def test_fft_and_dense_agree(L, case):
    """The two transforms of one shape agree to float32 rounding (and each with the oracle,
    above); the dense plan is asked for explicitly."""
    name, batch, cin, cout, grid, modes = case
    announce("fft vs dense", name)
    seed = 6100 + zlib.crc32(name.encode()) % 1000
    x, w, _, _ = inputs.small_case(seed, batch, cin, cout, grid, modes)
    tx, tw = _dev(x), _dev(w)
    outs = {}
    for mode in ("fft", "dense"):
        plan = L.Plan(batch, cin, cout, grid, modes, gelu=False, bias=False, last_axis=mode)
        assert plan.last_axis_fft == (mode == "fft")
        outs[mode] = _host(plan.spectral_conv_fwd(tx, tw))
        plan.close()
    e = rel_l2(outs["fft"], outs["dense"])
    print(f"    fft vs dense: rel_l2={e:.3e}", flush=True)
    assert e <= 2 * TOL_F32
    check("y_spec dense", outs["dense"], O.spectral_conv_fwd(x, w, modes)["y_spec"], TOL_F32)


def test_default_choice(L):
    """Without a flag a float32 plan takes the FFT for rows of 256 or 512 points and the
    dense products for rows of 128; half plans always take the dense products."""
    for grid, modes, mixed, want in [((64, 512), (8, 32), False, True),
                                     ((24, 256), (4, 16), False, True),
                                     ((40, 128), (8, 10), False, False),
                                     ((64, 512), (8, 32), True, False),
                                     ((64, 512), (8, 32), "f16", False)]:
        plan = L.Plan(1, 4, 4, grid, modes, mixed=mixed)
        assert plan.last_axis_fft == want, (grid, mixed)
        plan.close()
    plan = L.Plan(1, 4, 4, (64, 512), (8, 32), mixed=True, last_axis="fft")
    assert not plan.last_axis_fft  # half plans ignore the flag
    plan.close()
