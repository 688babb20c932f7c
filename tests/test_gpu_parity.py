"""HIP path (through the C-ABI) against the fp64 oracle, element by element, on seeded inputs.

Shapes span several work-group tiles with ragged tails, every dimensionality (2D, 3D, 4D
with a 20-point contiguous axis), odd grids, the largest allowed mode counts, one mode,
Cin != Cout and batches beyond one register tile.  Each output is compared on its own
(y_spec, y, grad_x, grad_w, grad_w_bypass, grad_bias): relative L2 <= 1e-5 on the fp32 path,
<= 1e-2 on the tanh + bf16 path, <= 1.25e-3 on the tanh + IEEE-half path.
"""
import zlib

import numpy as np
import pytest

import oracle.fno_oracle as O
from fno_spectral_convolution_amd import inputs
from tests.gpu_helpers import TOL_F32, announce, check, tol_for

pytestmark = pytest.mark.gpu

CASES = [
    # name, batch, cin, cout, grid, modes
    ("2d_ragged", 2, 3, 5, (24, 20), (5, 4)),
    ("2d_c1shape", 4, 20, 20, (64, 64), (12, 12)),
    ("2d_odd_maxmodes", 1, 2, 3, (15, 9), (7, 5)),
    ("2d_full_spectrum", 1, 3, 3, (8, 8), (4, 5)),
    ("2d_one_mode", 3, 1, 1, (16, 32), (1, 1)),
    ("2d_batch20", 20, 2, 2, (8, 16), (2, 3)),
    ("2d_wide", 2, 64, 64, (32, 64), (8, 16)),
    ("3d_ragged", 2, 4, 3, (12, 10, 16), (3, 2, 5)),
    ("4d_t20", 1, 3, 4, (6, 8, 10, 20), (2, 3, 4, 8)),
    # shapes taken by the matrix-core kernels (contiguous axis a multiple of 64)
    ("2d_mc_c16", 2, 16, 16, (40, 128), (6, 10)),
    ("2d_mc_c32", 3, 32, 32, (24, 256), (5, 16)),
    ("2d_mc_c48", 2, 48, 48, (16, 64), (4, 8)),
    ("2d_mc_c64", 2, 64, 64, (64, 512), (8, 32)),
    ("3d_mc_c20", 1, 20, 20, (10, 12, 64), (3, 4, 8)),
    ("4d_mc_c16", 1, 16, 16, (4, 6, 8, 64), (2, 2, 3, 6)),
    # few planes and long outer axes: the plane transform splits each plane into row chunks
    # and adds their partial spectra
    ("2d_chunked_nb64", 1, 4, 4, (256, 64), (8, 8)),
    ("2d_chunked_nb512", 1, 2, 2, (256, 512), (16, 32)),
    # half plans: 64 kept bins on rows of 128 take the eight-wave plane kernel
    ("2d_mc_nb128_jp64", 2, 6, 6, (48, 128), (4, 32)),
    # shapes taken by the short-row plane kernel (contiguous axis <= 32, a multiple of 4)
    ("4d_short_t20", 1, 3, 4, (4, 6, 16, 20), (2, 2, 4, 8)),
    ("3d_short_t20_jp32", 2, 5, 3, (6, 32, 20), (3, 8, 10)),
    ("3d_short_na128", 1, 2, 3, (4, 128, 12), (2, 12, 6)),
    ("2d_short_max", 2, 3, 2, (128, 32), (32, 16)),
    # shapes taken by the fused row-axis epilogue (rows a multiple of 16, ma <= 12, mb <= 8)
    ("2d_rows_c20", 2, 20, 20, (32, 20), (8, 8)),
    ("3d_rows_c9_17", 2, 9, 17, (4, 48, 24), (2, 8, 7)),
    ("2d_rows_nb32", 1, 12, 5, (64, 32), (12, 8)),
    # 1024 wide slabs for the second outer inverse: the streaming inverse, whose half plans
    # write the row epilogue's spectrum in the half format
    ("4d_rows_stream_inv", 1, 16, 16, (64, 8, 16, 20), (2, 2, 8, 8)),
]


def _torch():
    import torch
    return torch


def _dev(a):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _host(t):
    return t.detach().cpu().numpy()


# spectral precision of a plan (Plan's `mixed`) and its tanh pre-activation; "f32_tanh" is the
# plan a precision schedule switches to (fp32 arithmetic, the model's tanh kept)
PRECISIONS = [("f32", False, False), ("mixed", True, True), ("f16", "f16", True),
              ("f32_tanh", False, True)]


@pytest.fixture(scope="module")
def L():
    from fno_spectral_convolution_amd import binding
    return binding


@pytest.mark.parametrize("prec", PRECISIONS, ids=[p[0] for p in PRECISIONS])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_block_fwd_bwd(L, case, prec):
    name, batch, cin, cout, grid, modes = case
    pname, mixed, tanh = prec
    announce("block", name, pname)
    seed = zlib.crc32(name.encode()) % 1000
    x, w, wb, b = inputs.small_case(seed, batch, cin, cout, grid, modes)
    gy = inputs.normal_like(seed, (batch, cout) + grid)
    tol = tol_for(mixed)
    plan = L.Plan(batch, cin, cout, grid, modes, mixed=mixed, tanh=tanh)
    tx, tw, twb, tb, tg = (_dev(a) for a in (x, w, wb, b, gy))
    save = plan.new_save()
    y = plan.block_fwd(tx, tw, twb, tb, save=save)
    g = plan.block_bwd(tx, tw, twb, tb, save, tg)
    _torch().cuda.synchronize()
    ref = O.block_bwd(x, w, wb, b, modes, gy, tanh=tanh)
    check("y", _host(y), ref["fwd"]["y"], tol)
    check("grad_x", _host(g["x"]), ref["grad_x"], tol)
    check("grad_w", _host(g["w"]), ref["grad_w"], tol)
    check("grad_wb", _host(g["wb"]), ref["grad_wb"], tol)
    check("grad_bias", _host(g["bias"]), ref["grad_bias"], tol)
    plan.close()


@pytest.mark.parametrize("prec", PRECISIONS, ids=[p[0] for p in PRECISIONS])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_spectral_conv_fwd_bwd(L, case, prec):
    """The spectral path alone (no bypass to mask its errors), with and without a save."""
    name, batch, cin, cout, grid, modes = case
    pname, mixed, tanh = prec
    announce("spectral", name, pname)
    seed = 500 + zlib.crc32(name.encode()) % 1000
    x, w, _, _ = inputs.small_case(seed, batch, cin, cout, grid, modes)
    gy = inputs.normal_like(seed, (batch, cout) + grid)
    tol = tol_for(mixed)
    plan = L.Plan(batch, cin, cout, grid, modes, mixed=mixed, tanh=tanh, gelu=False,
                  bias=False)
    tx, tw, tg = (_dev(a) for a in (x, w, gy))
    save = plan.new_save()
    ys = plan.spectral_conv_fwd(tx, tw, save=save)
    gx, gw = plan.spectral_conv_bwd(tx, tw, tg, save=save)
    gx2, gw2 = plan.spectral_conv_bwd(tx, tw, tg, save=None)
    _torch().cuda.synchronize()
    fwd = O.spectral_conv_fwd(x, w, modes, tanh=tanh)
    bwd = O.spectral_conv_bwd(x, w, modes, gy, tanh=tanh)
    check("y_spec", _host(ys), fwd["y_spec"], tol)
    check("grad_x", _host(gx), bwd["grad_x"], tol)
    check("grad_w", _host(gw), bwd["grad_w"], tol)
    assert np.array_equal(_host(gx), _host(gx2)), "recomputed spectrum changed grad_x"
    assert np.array_equal(_host(gw), _host(gw2)), "recomputed spectrum changed grad_w"
    plan.close()


# Many narrow float32 slabs on the row axis of a 3D field (batch x channels x first-axis
# length >= 4096, at most 32 kept rows in, at most 128 rows out, at most 64 floats per row):
# the inverse of that axis runs on work-groups that walk several slabs each with the table in
# registers.  One case per column-tile width, one with idle row-tile waves (32 output rows).
SLAB_CASES = [
    # name, batch, cin, cout, grid, modes
    ("3d_slabs_nt1", 1, 16, 16, (256, 32, 64), (2, 8, 8)),
    ("3d_slabs_nt2", 2, 16, 16, (128, 128, 32), (4, 16, 16)),
]


@pytest.mark.parametrize("case", SLAB_CASES, ids=[c[0] for c in SLAB_CASES])
def test_many_slab_outer_inverse(L, case):
    name, batch, cin, cout, grid, modes = case
    announce("slabs", name)
    seed = zlib.crc32(name.encode()) % 1000
    x, w, _, _ = inputs.small_case(seed, batch, cin, cout, grid, modes)
    gy = inputs.normal_like(seed, (batch, cout) + grid)
    plan = L.Plan(batch, cin, cout, grid, modes, mixed=False, tanh=False, gelu=False,
                  bias=False)
    tx, tw, tg = (_dev(a) for a in (x, w, gy))
    ys = plan.spectral_conv_fwd(tx, tw)
    gx, gw = plan.spectral_conv_bwd(tx, tw, tg)
    _torch().cuda.synchronize()
    fwd = O.spectral_conv_fwd(x, w, modes)
    bwd = O.spectral_conv_bwd(x, w, modes, gy)
    check("y_spec", _host(ys), fwd["y_spec"], TOL_F32)
    check("grad_x", _host(gx), bwd["grad_x"], TOL_F32)
    check("grad_w", _host(gw), bwd["grad_w"], TOL_F32)
    plan.close()


@pytest.mark.parametrize("mixed", [False, True, "f16"], ids=["f32", "mixed", "f16"])
def test_bitwise_deterministic(L, mixed):
    announce("determinism", mixed)
    grid, modes = (48, 40), (9, 7)
    x, w, wb, b = inputs.small_case(11, 3, 6, 6, grid, modes)
    gy = inputs.normal_like(11, (3, 6) + grid)
    plan = L.Plan(3, 6, 6, grid, modes, mixed=mixed)
    tx, tw, twb, tb, tg = (_dev(a) for a in (x, w, wb, b, gy))
    outs = []
    for _ in range(2):
        save = plan.new_save()
        y = plan.block_fwd(tx, tw, twb, tb, save=save)
        g = plan.block_bwd(tx, tw, twb, tb, save, tg)
        _torch().cuda.synchronize()
        outs.append([_host(y)] + [_host(g[k]) for k in ("x", "w", "wb", "bias")])
    for a, c in zip(outs[0], outs[1]):
        assert np.array_equal(a, c)
    plan.close()



# On half plans with a multiple of 32 channels the bypass products (Wb x forward, Wb^T g_z and
# dWb backward) run as three bfloat16 products of hi / lo split operands, each product exact to
# about 3 * 2^-18 relative.  With W = 0 the spectral path contributes exactly zero, so these
# outputs are the bypass alone and must agree with the oracle nearly as closely as float32.
TOL_SPLIT = 2e-5


@pytest.mark.parametrize("mixed", [True, "f16"], ids=["bf16", "f16"])
@pytest.mark.parametrize("ig", [False, True], ids=["x", "input_gelu"])
@pytest.mark.parametrize("case", [c for c in CASES if c[0] in ("2d_wide", "2d_mc_c32",
                                                               "2d_mc_c64")],
                         ids=lambda c: c[0])
def test_half_plan_bypass_split(L, case, mixed, ig):
    name, batch, cin, cout, grid, modes = case
    announce("bypass split", name, mixed, "input_gelu" if ig else "x")
    seed = 900 + zlib.crc32(name.encode()) % 1000
    x, w, wb, b = inputs.small_case(seed, batch, cin, cout, grid, modes)
    w = np.zeros_like(w)
    gy = inputs.normal_like(seed, (batch, cout) + grid)
    plan = L.Plan(batch, cin, cout, grid, modes, mixed=mixed, input_gelu=ig)
    tx, tw, twb, tb, tg = (_dev(a) for a in (x, w, wb, b, gy))
    save = plan.new_save()
    y = plan.block_fwd(tx, tw, twb, tb, save=save)
    g = plan.block_bwd(tx, tw, twb, tb, save, tg)
    _torch().cuda.synchronize()
    ref = O.block_bwd(x, w, wb, b, modes, gy, tanh=True, input_gelu=ig)
    check("y", _host(y), ref["fwd"]["y"], TOL_SPLIT)
    check("grad_x", _host(g["x"]), ref["grad_x"], TOL_SPLIT)
    check("grad_wb", _host(g["wb"]), ref["grad_wb"], TOL_SPLIT)
    check("grad_bias", _host(g["bias"]), ref["grad_bias"], TOL_SPLIT)
    plan.close()


# The spectral-dominant variant: spectral weights scaled by C^2 (about U(0,1) per entry instead
# of U(0,1)/(Cin Cout)), so the spectral path dominates the block output.  fp32 and bf16 plans
# keep their tolerances.  An IEEE-half plan may leave half's range: then its outputs hold inf /
# NaN and the plan must say so (fno_plan_half_range); otherwise it meets its tolerance.
@pytest.mark.parametrize("prec", [("f32", False), ("bf16", True), ("f16", "f16")],
                         ids=lambda p: p[0])
@pytest.mark.parametrize("case", [c for c in CASES if c[0] in (
    "2d_mc_c64", "2d_wide", "2d_mc_c32", "3d_mc_c20", "4d_short_t20", "2d_c1shape")],
    ids=lambda c: c[0])
def test_spectral_dominant_weights(L, case, prec):
    name, batch, cin, cout, grid, modes = case
    pname, mixed = prec
    announce("spectral-dominant", name, pname)
    seed = 1300 + zlib.crc32(name.encode()) % 1000
    x, w, wb, b = inputs.small_case(seed, batch, cin, cout, grid, modes)
    w = (w * np.float32(cin * cout)).astype(w.dtype)
    gy = inputs.normal_like(seed, (batch, cout) + grid)
    plan = L.Plan(batch, cin, cout, grid, modes, mixed=mixed)
    assert not plan.half_range_exceeded()
    tx, tw, twb, tb, tg = (_dev(a) for a in (x, w, wb, b, gy))
    save = plan.new_save()
    y = plan.block_fwd(tx, tw, twb, tb, save=save)
    g = plan.block_bwd(tx, tw, twb, tb, save, tg)
    _torch().cuda.synchronize()
    outs = {"y": _host(y), "grad_x": _host(g["x"]), "grad_w": _host(g["w"]),
            "grad_wb": _host(g["wb"]), "grad_bias": _host(g["bias"])}
    nonfinite = [k for k in ("y", "grad_x", "grad_w") if not np.all(np.isfinite(outs[k]))]
    flagged = plan.half_range_exceeded(clear=True)
    print(f"    half range exceeded: {flagged}; non-finite outputs: {nonfinite}", flush=True)
    assert flagged == bool(nonfinite), (flagged, nonfinite)
    if mixed != "f16":
        assert not flagged
    if not flagged:
        ref = O.block_bwd(x, w, wb, b, modes, gy, tanh=bool(mixed))
        tol = tol_for(mixed)
        check("y", outs["y"], ref["fwd"]["y"], tol)
        check("grad_x", outs["grad_x"], ref["grad_x"], tol)
        check("grad_w", outs["grad_w"], ref["grad_w"], tol)
        check("grad_wb", outs["grad_wb"], ref["grad_wb"], tol)
        check("grad_bias", outs["grad_bias"], ref["grad_bias"], tol)
    # the flag was cleared: a call at the usual weight scale leaves it clear
    x2, w2, wb2, b2 = inputs.small_case(seed + 1, batch, cin, cout, grid, modes)
    plan.block_fwd(_dev(x2), _dev(w2), _dev(wb2), _dev(b2))
    _torch().cuda.synchronize()
    assert not plan.half_range_exceeded()
    plan.close()


@pytest.mark.parametrize("case", [c for c in CASES if c[0] in (
    "2d_mc_c64", "2d_ragged", "4d_short_t20", "3d_mc_c20")], ids=lambda c: c[0])
def test_f16_overflow_is_reported(L, case):
    """Spectral weights far beyond half's range on an IEEE-half plan: the outputs are
    non-finite and the plan reports it; a bfloat16 plan (float32's exponent range) keeps the
    same inputs finite."""
    name, batch, cin, cout, grid, modes = case
    announce("f16 overflow", name)
    seed = 1700 + zlib.crc32(name.encode()) % 1000
    x, w, wb, b = inputs.small_case(seed, batch, cin, cout, grid, modes)
    w = (w * np.float32(cin * cout * 65536.0)).astype(w.dtype)
    gy = inputs.normal_like(seed, (batch, cout) + grid)
    for mixed in ("f16", True):
        plan = L.Plan(batch, cin, cout, grid, modes, mixed=mixed)
        tx, tw, twb, tb, tg = (_dev(a) for a in (x, w, wb, b, gy))
        save = plan.new_save()
        y = plan.block_fwd(tx, tw, twb, tb, save=save)
        g = plan.block_bwd(tx, tw, twb, tb, save, tg)
        _torch().cuda.synchronize()
        finite = all(bool(np.all(np.isfinite(_host(t)))) for t in (y, g["x"], g["w"]))
        flagged = plan.half_range_exceeded()
        print(f"    {mixed}: finite outputs {finite}, half range exceeded {flagged}", flush=True)
        if mixed == "f16":
            assert flagged and not finite
        else:
            assert finite and not flagged
        plan.close()

@pytest.mark.parametrize("prec", PRECISIONS[:3], ids=[p[0] for p in PRECISIONS[:3]])
def test_gelu_off_and_bias_off(L, prec):
    """Flags: without GELU the block returns z; without BIAS the bias pointer is ignored.  The
    grid's 24-point contiguous axis takes the fused row-axis epilogue."""
    pname, mixed, tanh = prec
    announce("flags", pname)
    tol = tol_for(mixed)
    grid, modes = (16, 24), (4, 6)
    x, w, wb, b = inputs.small_case(21, 2, 3, 4, grid, modes)
    gy = inputs.normal_like(21, (2, 4) + grid)
    plan = L.Plan(2, 3, 4, grid, modes, mixed=mixed, tanh=tanh, gelu=False, bias=False)
    tx, tw, twb, tg = (_dev(a) for a in (x, w, wb, gy))
    save = plan.new_save()
    y = plan.block_fwd(tx, tw, twb, None, save=save)
    g = plan.block_bwd(tx, tw, twb, None, save, tg)
    _torch().cuda.synchronize()
    ref = O.block_bwd(x, w, wb, None, modes, gy, tanh=tanh, act=False)
    check("z", _host(y), ref["fwd"]["y"], tol)
    check("grad_x", _host(g["x"]), ref["grad_x"], tol)
    check("grad_w", _host(g["w"]), ref["grad_w"], tol)
    check("grad_wb", _host(g["wb"]), ref["grad_wb"], tol)
    check("grad_bias", _host(g["bias"]), ref["grad_bias"], tol)
    plan.close()


def test_pointwise_and_mse(L):
    announce("pointwise+mse")
    torch = _torch()
    g = np.random.default_rng(5)
    x = g.standard_normal((3, 5, 7, 33)).astype(np.float32)
    w1 = g.standard_normal((12, 5)).astype(np.float32)
    b1 = g.standard_normal(12).astype(np.float32)
    w2 = g.standard_normal((2, 12)).astype(np.float32)
    b2 = g.standard_normal(2).astype(np.float32)
    lift = L.pointwise(_dev(x), _dev(w1), _dev(b1))
    proj = L.pointwise(_dev(x), _dev(w1), _dev(b1), _dev(w2), _dev(b2))
    t = g.standard_normal((3, 2, 7, 33)).astype(np.float32)
    loss, grad = L.mse_grad(proj, _dev(t))
    torch.cuda.synchronize()
    check("lift", _host(lift), O.pointwise_linear(x, w1, b1), TOL_F32)
    pref = O.projection_fwd(x, w1, b1, w2, b2)
    check("projection", _host(proj), pref, TOL_F32)
    lref, gref = O.mse_loss_grad(_host(proj), t)
    check("mse_grad", _host(grad), gref, TOL_F32)
    assert abs(float(_host(loss)[0]) - lref) <= 1e-6 * lref
    # a power-of-two loss scale multiplies the gradient exactly and leaves the loss alone
    loss2, grad2 = L.mse_grad(proj, _dev(t), grad_scale=65536.0)
    torch.cuda.synchronize()
    assert np.array_equal(_host(grad2), _host(grad) * np.float32(65536.0))
    assert float(_host(loss2)[0]) == float(_host(loss)[0])



@pytest.mark.parametrize("cin,npts,bias", [(1, 2304, True), (2, 2304, False), (3, 4100, True),
                                          (4, 2304, True), (3, 2302, True)])
def test_lift_few_input_channels(L, cin, npts, bias):
    """Lifts from at most four channels (point counts that are multiples of 4 take the VALU
    lift, the last case the matrix-core path), with and without a bias."""
    announce("lift", cin, npts, bias)
    g = np.random.default_rng(60 + cin)
    cout = 20
    x = g.standard_normal((3, cin, npts)).astype(np.float32)
    w1 = g.standard_normal((cout, cin)).astype(np.float32)
    b1 = g.standard_normal(cout).astype(np.float32) if bias else None
    lift = L.pointwise(_dev(x), _dev(w1), _dev(b1) if bias else None)
    _torch().cuda.synchronize()
    ref = O.pointwise_linear(x, w1, b1)
    check("lift", _host(lift), ref, TOL_F32)


@pytest.mark.parametrize("cout,hidden", [(1, 128), (3, 20), (4, 64), (5, 40)])
def test_projection_narrow_outputs(L, cout, hidden):
    """Projection heads around the narrow-output path (<= 4 outputs take the VALU second
    product), with a point count that leaves a ragged last tile."""
    announce("projection", cout, hidden)
    g = np.random.default_rng(40 + cout)
    cin, npts = 32, 3 * 64 + 9
    x = g.standard_normal((2, cin, npts)).astype(np.float32)
    w1 = (g.standard_normal((hidden, cin)) / np.sqrt(cin)).astype(np.float32)
    b1 = g.standard_normal(hidden).astype(np.float32)
    w2 = (g.standard_normal((cout, hidden)) / np.sqrt(hidden)).astype(np.float32)
    b2 = g.standard_normal(cout).astype(np.float32)
    proj = L.pointwise(_dev(x), _dev(w1), _dev(b1), _dev(w2), _dev(b2))
    _torch().cuda.synchronize()
    check("projection", _host(proj), O.projection_fwd(x, w1, b1, w2, b2), TOL_F32)

@pytest.mark.parametrize("cout,hidden,cin,batch,npts", [
    (1, 128, 32, 3, 64 * 1000),   # 3000 tiles: work-groups walk more than one
    (2, 64, 32, 2, 64 * 5),       # four M-tiles: one per wave
    (3, 100, 20, 2, 64 * 1100),   # hidden rows and input channels padded inside the tiles
    (4, 128, 7, 1, 64 * 2500),
    (4, 40, 32, 5, 64),           # one tile per batch entry
])
def test_projection_narrow_whole_tiles(L, cout, hidden, cin, batch, npts):
    """Narrow projection heads on whole 64-point tiles (cin <= 32, hidden <= 128): the
    grid-stride path that keeps the weights in registers and loads the next tile ahead."""
    announce("projection whole tiles", cout, hidden, cin, batch, npts)
    g = np.random.default_rng(400 + 10 * cout + cin)
    x = g.standard_normal((batch, cin, npts)).astype(np.float32)
    w1 = (g.standard_normal((hidden, cin)) / np.sqrt(cin)).astype(np.float32)
    b1 = g.standard_normal(hidden).astype(np.float32)
    w2 = (g.standard_normal((cout, hidden)) / np.sqrt(hidden)).astype(np.float32)
    b2 = g.standard_normal(cout).astype(np.float32)
    proj = L.pointwise(_dev(x), _dev(w1), _dev(b1), _dev(w2), _dev(b2))
    nob = L.pointwise(_dev(x), _dev(w1), None, _dev(w2), None)
    _torch().cuda.synchronize()
    # the first product runs on the bfloat16 matrix cores as six products of exactly split
    # operands: float32 grade (about 1e-7 here, as the float32 tile kernel).  Dropping one
    # term product of order 2 (about 2^-16 |ab| each) would exceed this bound.
    tol = 1e-6
    check("projection", _host(proj), O.projection_fwd(x, w1, b1, w2, b2), tol)
    check("projection, no biases", _host(nob), O.projection_fwd(x, w1, None, w2, None), tol)


def test_pointwise_widest(L):
    """The widest pointwise layers the boundary accepts (64 -> 256 -> 128), ragged point count."""
    announce("pointwise widest")
    g = np.random.default_rng(6)
    x = g.standard_normal((2, 64, 70)).astype(np.float32)
    w1 = (g.standard_normal((256, 64)) / 8).astype(np.float32)
    b1 = g.standard_normal(256).astype(np.float32)
    w2 = (g.standard_normal((128, 256)) / 16).astype(np.float32)
    b2 = g.standard_normal(128).astype(np.float32)
    proj = L.pointwise(_dev(x), _dev(w1), _dev(b1), _dev(w2), _dev(b2))
    lift = L.pointwise(_dev(x), _dev(w2[:, :64].copy()), _dev(b2))
    _torch().cuda.synchronize()
    check("projection", _host(proj), O.projection_fwd(x, w1, b1, w2, b2), TOL_F32)
    check("lift", _host(lift), O.pointwise_linear(x, w2[:, :64], b2), TOL_F32)


def test_bad_workspace_is_an_error(L):
    announce("workspace-too-small")
    torch = _torch()
    plan = L.Plan(1, 2, 2, (16, 16), (3, 3))
    x = torch.zeros((1, 2, 16, 16), device="cuda")
    w = torch.zeros((2, 2, 2, 3, 3), dtype=torch.complex64, device="cuda")
    y = torch.empty_like(x)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.FnoError) as ei:
        L.fno_spectral_conv_fwd(plan.handle, x.data_ptr(), w.data_ptr(), y.data_ptr(), None,
                                ws.data_ptr(), 16, 0)
    assert ei.value.status == L.FNO_ERR_INVALID_ARGUMENT
    with pytest.raises(L.FnoError) as ei:
        L.fno_spectral_conv_fwd(plan.handle, x.data_ptr() + 4, w.data_ptr(), y.data_ptr(), None,
                                plan.workspace().data_ptr(), plan.ws_bytes, 0)
    assert ei.value.status == L.FNO_ERR_INVALID_ARGUMENT
    plan.close()


# shapes for the pre-activation input: each line-epilogue width, the generic kernels, a short
# contiguous axis (line kernels decline, generic epilogue), 3D and 4D
IG_CASES = [c for c in CASES if c[0] in (
    "2d_ragged", "2d_c1shape", "2d_mc_c16", "2d_mc_c32", "2d_mc_c64", "3d_mc_c20",
    "4d_short_t20", "2d_rows_c20", "2d_odd_maxmodes", "4d_t20", "2d_mc_nb128_jp64")]


@pytest.mark.parametrize("act", [True, False], ids=["gelu_out", "z_out"])
@pytest.mark.parametrize("prec", PRECISIONS[:3], ids=[p[0] for p in PRECISIONS[:3]])
@pytest.mark.parametrize("case", IG_CASES, ids=[c[0] for c in IG_CASES])
def test_block_input_gelu(L, case, prec, act):
    """A block whose input is a pre-activation (FNO_FLAG_INPUT_GELU): forward, backward."""
    name, batch, cin, cout, grid, modes = case
    pname, mixed, tanh = prec
    announce("block input_gelu", name, pname, act)
    seed = 900 + zlib.crc32(name.encode()) % 1000
    x, w, wb, b = inputs.small_case(seed, batch, cin, cout, grid, modes)
    gy = inputs.normal_like(seed, (batch, cout) + grid)
    tol = tol_for(mixed)
    plan = L.Plan(batch, cin, cout, grid, modes, mixed=mixed, tanh=tanh, gelu=act,
                  input_gelu=True)
    tx, tw, twb, tb, tg = (_dev(a) for a in (x, w, wb, b, gy))
    save = plan.new_save()
    y = plan.block_fwd(tx, tw, twb, tb, save=save)
    g = plan.block_bwd(tx, tw, twb, tb, save, tg)
    _torch().cuda.synchronize()
    ref = O.block_bwd(x, w, wb, b, modes, gy, tanh=tanh, act=act, input_gelu=True)
    check("y", _host(y), ref["fwd"]["y"], tol)
    check("grad_x", _host(g["x"]), ref["grad_x"], tol)
    check("grad_w", _host(g["w"]), ref["grad_w"], tol)
    check("grad_wb", _host(g["wb"]), ref["grad_wb"], tol)
    check("grad_bias", _host(g["bias"]), ref["grad_bias"], tol)
    plan.close()


@pytest.mark.parametrize("prec", PRECISIONS[:2], ids=[p[0] for p in PRECISIONS[:2]])
@pytest.mark.parametrize("case", IG_CASES[:6], ids=[c[0] for c in IG_CASES[:6]])
def test_spectral_conv_input_gelu(L, case, prec):
    name, batch, cin, cout, grid, modes = case
    pname, mixed, tanh = prec
    announce("spectral input_gelu", name, pname)
    seed = 1900 + zlib.crc32(name.encode()) % 1000
    x, w, _, _ = inputs.small_case(seed, batch, cin, cout, grid, modes)
    gy = inputs.normal_like(seed, (batch, cout) + grid)
    tol = tol_for(mixed)
    plan = L.Plan(batch, cin, cout, grid, modes, mixed=mixed, tanh=tanh, gelu=False, bias=False,
                  input_gelu=True)
    tx, tw, tg = (_dev(a) for a in (x, w, gy))
    ys = plan.spectral_conv_fwd(tx, tw)
    gx, gw = plan.spectral_conv_bwd(tx, tw, tg)
    _torch().cuda.synchronize()
    fwd = O.spectral_conv_fwd(x, w, modes, tanh=tanh, input_gelu=True)
    bwd = O.spectral_conv_bwd(x, w, modes, gy, tanh=tanh, input_gelu=True)
    check("y_spec", _host(ys), fwd["y_spec"], tol)
    check("grad_x", _host(gx), bwd["grad_x"], tol)
    check("grad_w", _host(gw), bwd["grad_w"], tol)
    plan.close()


def _fused_loss_case(L, case, prec, ig, act, seed0):
    """fno_block_fwd_mse then fno_block_bwd_preact against the oracle's loss, grad_z and the
    block backward from it; f16 plans take the static loss scale 2^16."""
    name, batch, cin, cout, grid, modes = case
    pname, mixed, tanh = prec
    announce("block fused loss", name, pname, "input_gelu" if ig else "", "gelu" if act else "z")
    seed = seed0 + zlib.crc32(name.encode()) % 1000
    x, w, wb, b = inputs.small_case(seed, batch, cin, cout, grid, modes)
    tgt = inputs.normal_like(seed + 1, (batch, cout) + grid)
    scale = 65536.0 if mixed == "f16" else 1.0
    tol = tol_for(mixed)
    plan = L.Plan(batch, cin, cout, grid, modes, mixed=mixed, tanh=tanh, gelu=act,
                  input_gelu=ig)
    tx, tw, twb, tb, tt = (_dev(a) for a in (x, w, wb, b, tgt))
    save = plan.new_save()
    gz, loss = plan.block_fwd_mse(tx, tw, twb, tb, tt, grad_scale=scale, save=save)
    g = plan.block_bwd_preact(tx, tw, twb, tb, save, gz)
    # from the oracle's grad_z, without a save (the spectrum recomputed; grad_x only)
    ref = O.block_fwd_mse(x, w, wb, b, modes, tgt, tanh=tanh, act=act, input_gelu=ig)
    g2 = plan.block_bwd_preact(tx, tw, twb, tb, None,
                               _dev((ref["grad_z"] * scale).astype(np.float32)),
                               want=("x",))
    _torch().cuda.synchronize()
    refb = O.block_bwd_preact(x, w, wb, b, modes, ref["grad_z"], tanh=tanh, input_gelu=ig)
    check("grad_z", _host(gz) / scale, ref["grad_z"], tol)
    got_loss = float(_host(loss)[0])
    print(f"    loss: {got_loss:.7e} (oracle {ref['loss']:.7e})", flush=True)
    assert abs(got_loss - ref["loss"]) <= tol * ref["loss"], (got_loss, ref["loss"])
    check("grad_x", _host(g["x"]) / scale, refb["grad_x"], tol)
    check("grad_w", _host(g["w"]) / scale, refb["grad_w"], tol)
    check("grad_wb", _host(g["wb"]) / scale, refb["grad_wb"], tol)
    check("grad_bias", _host(g["bias"]) / scale, refb["grad_bias"], tol)
    check("grad_x (recomputed spectrum)", _host(g2["x"]) / scale, refb["grad_x"], tol)
    plan.close()


@pytest.mark.parametrize("prec", PRECISIONS[:3], ids=[p[0] for p in PRECISIONS[:3]])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_block_fused_loss(L, case, prec):
    """The last block fused with the MSE loss (the matrix-core epilogue where it applies, the
    generic and row-axis epilogues plus a pointwise pass elsewhere)."""
    _fused_loss_case(L, case, prec, False, True, 2900)


@pytest.mark.parametrize("ig,act", [(True, True), (True, False), (False, False)],
                         ids=["input_gelu", "input_gelu_z_out", "z_out"])
@pytest.mark.parametrize("prec", PRECISIONS[:2], ids=[p[0] for p in PRECISIONS[:2]])
@pytest.mark.parametrize("case", IG_CASES, ids=[c[0] for c in IG_CASES])
def test_block_fused_loss_activations(L, case, prec, ig, act):
    _fused_loss_case(L, case, prec, ig, act, 3900)


@pytest.mark.parametrize("scale_exp", [-40, 40], ids=["2^-40", "2^40"])
@pytest.mark.parametrize("case", [c for c in CASES if c[0] in (
    "4d_short_t20", "3d_short_na128", "2d_mc_c64", "2d_chunked_nb512")],
    ids=lambda c: c[0])
def test_f32_far_from_unit_scale(L, case, scale_exp):
    """Float32 plans on fields far from unit size: the short-row transform's products run as
    split bfloat16 products and the long rows take the FFT; both must keep float32's relative
    accuracy at any exponent (the spectral path is linear in x, so the oracle is scaled)."""
    name, batch, cin, cout, grid, modes = case
    announce("f32 scale", name, scale_exp)
    seed = 7100 + zlib.crc32(name.encode()) % 1000
    x, w, _, _ = inputs.small_case(seed, batch, cin, cout, grid, modes)
    xs = (x * np.float32(2.0 ** scale_exp)).astype(np.float32)
    plan = L.Plan(batch, cin, cout, grid, modes, gelu=False, bias=False)
    ys = plan.spectral_conv_fwd(_dev(xs), _dev(w))
    _torch().cuda.synchronize()
    ref = O.spectral_conv_fwd(xs.astype(np.float64), w, modes)["y_spec"]
    check("y_spec", _host(ys), ref, TOL_F32)
    plan.close()
