"""Tucker-factorised (TFNO) block through the C-ABI against the fp64 oracle.

Each case runs fno_tucker_block_fwd / _bwd and compares y, grad_x, grad_core, every factor
gradient, grad_w_bypass and grad_bias with the oracle's tucker_block_fwd / _bwd (relative L2,
the tolerances of the plain block: 1e-5 fp32, 1e-2 tanh + bf16, 1.25e-3 tanh + IEEE half).
The shapes take both forms of the greedy order: factors applied to the spectrum around a
rank-sized mix, and every factor applied to the core (the dense weight formed) when the batch
is large; also rank 1, C_in != C_out, 3D and a 4D grid with a 20-point last axis.
"""
import zlib

import numpy as np
import pytest

import oracle.fno_oracle as O
from fno_spectral_convolution_amd import inputs
from tests.gpu_helpers import announce, check, tol_for

pytestmark = pytest.mark.gpu

CASES = [
    # name, batch, cin, cout, grid, modes, ranks, expected fragment of the order
    ("2d_half_ranks", 2, 16, 16, (24, 64), (5, 12), (8, 8, 6, 6), "X*Uin"),
    ("2d_core_side", 64, 4, 4, (16, 32), (4, 8), (4, 4, 8, 8), "G*Uin"),
    ("2d_rank_one", 3, 5, 7, (16, 20), (3, 6), (1, 1, 1, 1), None),
    ("2d_ragged", 2, 6, 3, (15, 9), (7, 5), (4, 2, 9, 3), None),
    ("3d", 2, 6, 5, (8, 12, 16), (2, 3, 5), (3, 4, 2, 3, 4), None),
    ("4d_t20", 1, 3, 4, (4, 6, 8, 20), (2, 2, 3, 8), (2, 3, 2, 3, 4, 5), None),
    ("2d_wide", 2, 64, 64, (32, 64), (8, 16), (32, 32, 8, 8), "X*Uin"),
]
PRECISIONS = [("f32", False), ("mixed", True), ("f16", "f16")]


def _torch():
    import torch
    return torch


def _dev(a):
    return _torch().from_numpy(np.ascontiguousarray(a)).to("cuda")


def _host(t):
    return t.detach().cpu().numpy()


def _tucker_params(seed, cin, cout, modes, ranks):
    """Seeded core and factors: unit-column factors and a core of size 1/(C_in C_out)."""
    g = np.random.default_rng(np.random.SeedSequence([3000, seed]))
    ext = [cin, cout] + [2 * m for m in modes[:-1]] + [modes[-1]]
    facs = []
    for n, r in zip(ext, ranks):
        u = (g.standard_normal((n, r)) + 1j * g.standard_normal((n, r))) / np.sqrt(2.0 * n)
        facs.append(u.astype(np.complex64))
    core = ((g.standard_normal(ranks) + 1j * g.standard_normal(ranks))
            / (cin * cout)).astype(np.complex64)
    return core, facs


@pytest.fixture(scope="module")
def L():
    from fno_spectral_convolution_amd import binding
    return binding


@pytest.mark.parametrize("prec", PRECISIONS, ids=[p[0] for p in PRECISIONS])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_tucker_block_fwd_bwd(L, case, prec):
    name, batch, cin, cout, grid, modes, ranks, frag = case
    pname, mixed = prec
    seed = zlib.crc32(name.encode()) % 1000
    x, _, wb, b = inputs.small_case(seed, batch, cin, cout, grid, modes)
    gy = inputs.normal_like(seed, (batch, cout) + grid)
    core, facs = _tucker_params(seed, cin, cout, modes, ranks)
    plan = L.Plan(batch, cin, cout, grid, modes, mixed=mixed)
    tk = L.Tucker(plan, ranks)
    announce("tucker", name, pname, tk.order)
    if frag is not None:
        assert frag in tk.order.split(), tk.order
    tol = tol_for(mixed)
    tx, twb, tb, tg, tcore = (_dev(a) for a in (x, wb, b, gy, core))
    tfac = [_dev(u) for u in facs]
    save = plan.new_save()
    y = tk.block_fwd(tx, tcore, tfac, twb, tb, save=save)
    gr = tk.block_bwd(tx, tcore, tfac, twb, tb, save, tg)
    _torch().cuda.synchronize()
    ref = O.tucker_block_bwd(x, core, facs, wb, b, modes, gy, tanh=bool(mixed))
    check("y", _host(y), ref["fwd"]["y"], tol)
    check("grad_x", _host(gr["x"]), ref["grad_x"], tol)
    check("grad_core", _host(gr["core"]), ref["grad_core"], tol)
    for n, (got, want) in enumerate(zip(gr["factors"], ref["grad_factors"])):
        check(f"grad_factor {n}", _host(got), want, tol)
    check("grad_wb", _host(gr["wb"]), ref["grad_wb"], tol)
    check("grad_bias", _host(gr["bias"]), ref["grad_bias"], tol)
    tk.close()
    plan.close()


def test_tucker_partial_outputs_and_determinism(L):
    """grad_x alone (no weight gradients, no save read for them), weight gradients alone, and
    a second call giving bit-identical results."""
    name, batch, cin, cout, grid, modes, ranks, _ = CASES[0]
    announce("tucker partial", name)
    x, _, wb, b = inputs.small_case(7, batch, cin, cout, grid, modes)
    gy = inputs.normal_like(7, (batch, cout) + grid)
    core, facs = _tucker_params(7, cin, cout, modes, ranks)
    plan = L.Plan(batch, cin, cout, grid, modes)
    tk = L.Tucker(plan, ranks)
    tx, twb, tb, tg, tcore = (_dev(a) for a in (x, wb, b, gy, core))
    tfac = [_dev(u) for u in facs]
    save = plan.new_save()
    tk.block_fwd(tx, tcore, tfac, twb, tb, save=save)
    full = tk.block_bwd(tx, tcore, tfac, twb, tb, save, tg)
    only_x = tk.block_bwd(tx, tcore, tfac, twb, tb, save, tg, want_w=False)
    only_w = tk.block_bwd(tx, tcore, tfac, twb, tb, save, tg, want_x=False)
    again = tk.block_bwd(tx, tcore, tfac, twb, tb, save, tg)
    _torch().cuda.synchronize()
    assert np.array_equal(_host(full["x"]), _host(only_x["x"]))
    assert np.array_equal(_host(full["core"]), _host(only_w["core"]))
    for a, c in zip(full["factors"], only_w["factors"]):
        assert np.array_equal(_host(a), _host(c))
    for k in ("x", "core", "wb", "bias"):
        assert np.array_equal(_host(full[k]), _host(again[k]))
    tk.close()
    plan.close()


@pytest.mark.parametrize("use_save", [True, False], ids=["save", "recompute"])
@pytest.mark.parametrize("prec", PRECISIONS[:2], ids=[p[0] for p in PRECISIONS[:2]])
@pytest.mark.parametrize("case", CASES[:5], ids=[c[0] for c in CASES[:5]])
def test_tucker_spectral_conv(L, case, prec, use_save):
    """The spectral convolution alone with Tucker weights (no bypass to mask its errors), with
    the spectrum saved by the forward or recomputed by the backward."""
    name, batch, cin, cout, grid, modes, ranks, _ = case
    pname, mixed = prec
    seed = 400 + zlib.crc32(name.encode()) % 1000
    x, _, _, _ = inputs.small_case(seed, batch, cin, cout, grid, modes)
    gy = inputs.normal_like(seed, (batch, cout) + grid)
    core, facs = _tucker_params(seed, cin, cout, modes, ranks)
    plan = L.Plan(batch, cin, cout, grid, modes, mixed=mixed, gelu=False, bias=False)
    tk = L.Tucker(plan, ranks)
    announce("tucker spectral", name, pname, use_save, tk.order)
    tol = tol_for(mixed)
    tx, tg, tcore = (_dev(a) for a in (x, gy, core))
    tfac = [_dev(u) for u in facs]
    save = plan.new_save() if use_save else None
    ys = tk.spectral_conv_fwd(tx, tcore, tfac, save=save)
    gx, gcore, gfac = tk.spectral_conv_bwd(tx, tcore, tfac, tg, save=save)
    _torch().cuda.synchronize()
    fwd = O.tucker_spectral_conv_fwd(x, core, facs, modes, tanh=bool(mixed))
    bwd = O.tucker_spectral_conv_bwd(x, core, facs, modes, gy, tanh=bool(mixed))
    check("y_spec", _host(ys), fwd["y_spec"], tol)
    check("grad_x", _host(gx), bwd["grad_x"], tol)
    check("grad_core", _host(gcore), bwd["grad_core"], tol)
    for n, want in enumerate(bwd["grad_factors"]):
        check(f"grad_factor {n}", _host(gfac[n]), want, tol)
    tk.close()
    plan.close()


@pytest.mark.parametrize("prec", PRECISIONS, ids=[p[0] for p in PRECISIONS])
@pytest.mark.parametrize("case", CASES[:5] + CASES[6:], ids=[c[0] for c in CASES[:5] + CASES[6:]])
def test_tucker_fused_loss(L, case, prec):
    """fno_tucker_block_fwd_mse then fno_tucker_block_bwd_preact against the oracle's loss,
    grad_z and the Tucker block backward from it (f16: static loss scale 2^16)."""
    name, batch, cin, cout, grid, modes, ranks, _ = case
    pname, mixed = prec
    seed = 40 + zlib.crc32(name.encode()) % 1000
    x, _, wb, b = inputs.small_case(seed, batch, cin, cout, grid, modes)
    tgt = inputs.normal_like(seed + 1, (batch, cout) + grid)
    core, facs = _tucker_params(seed, cin, cout, modes, ranks)
    scale = 65536.0 if mixed == "f16" else 1.0
    plan = L.Plan(batch, cin, cout, grid, modes, mixed=mixed, input_gelu=True)
    tk = L.Tucker(plan, ranks)
    announce("tucker fused loss", name, pname, tk.order)
    tol = tol_for(mixed)
    tx, twb, tb, tt, tcore = (_dev(a) for a in (x, wb, b, tgt, core))
    tfac = [_dev(u) for u in facs]
    save = plan.new_save()
    gz, loss = tk.block_fwd_mse(tx, tcore, tfac, twb, tb, tt, grad_scale=scale, save=save)
    gr = tk.block_bwd_preact(tx, tcore, tfac, twb, tb, save, gz)
    _torch().cuda.synchronize()
    w = O.fold_weights(O.tucker_to_full(core, facs), modes)
    ref = O.block_fwd_mse(x, w, wb, b, modes, tgt, tanh=bool(mixed), input_gelu=True)
    refb = O.block_bwd_preact(x, w, wb, b, modes, ref["grad_z"], tanh=bool(mixed),
                              input_gelu=True)
    gcore, gfac = O.tucker_grads(core, facs, O.expand_weights(refb["grad_w"], modes))
    check("grad_z", _host(gz) / scale, ref["grad_z"], tol)
    got_loss = float(_host(loss)[0])
    assert abs(got_loss - ref["loss"]) <= tol * ref["loss"], (got_loss, ref["loss"])
    check("grad_x", _host(gr["x"]) / scale, refb["grad_x"], tol)
    check("grad_core", _host(gr["core"]) / scale, gcore, tol)
    for n, (got, want) in enumerate(zip(gr["factors"], gfac)):
        check(f"grad_factor {n}", _host(got) / scale, want, tol)
    check("grad_wb", _host(gr["wb"]) / scale, refb["grad_wb"], tol)
    check("grad_bias", _host(gr["bias"]) / scale, refb["grad_bias"], tol)
    tk.close()
    plan.close()


@pytest.mark.parametrize("prec", PRECISIONS[:2], ids=[p[0] for p in PRECISIONS[:2]])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_tucker_kept_intermediates(L, case, prec):
    """fno_tucker_keep_intermediates: the backward reads the forward's core-chain results,
    U_in xhat and the mix output from the save buffer instead of recomputing them; every output
    is the same bits as without, for the plain and the loss-fused block."""
    name, batch, cin, cout, grid, modes, ranks, _ = case
    pname, mixed = prec
    seed = 70 + zlib.crc32(name.encode()) % 1000
    x, _, wb, b = inputs.small_case(seed, batch, cin, cout, grid, modes)
    gy = inputs.normal_like(seed, (batch, cout) + grid)
    core, facs = _tucker_params(seed, cin, cout, modes, ranks)
    plan = L.Plan(batch, cin, cout, grid, modes, mixed=mixed)
    tk = L.Tucker(plan, ranks)
    announce("tucker kept", name, pname, tk.order)
    tx, twb, tb, tg, tcore = (_dev(a) for a in (x, wb, b, gy, core))
    tfac = [_dev(u) for u in facs]

    def run():
        save = tk.new_save()
        y = tk.block_fwd(tx, tcore, tfac, twb, tb, save=save)
        g = tk.block_bwd(tx, tcore, tfac, twb, tb, save, tg)
        gz, loss = tk.block_fwd_mse(tx, tcore, tfac, twb, tb, tg, save=save)
        gp = tk.block_bwd_preact(tx, tcore, tfac, twb, tb, save, gz)
        _torch().cuda.synchronize()
        out = {"y": _host(y), "gz": _host(gz), "loss": _host(loss)}
        for tag, d in (("bwd", g), ("pre", gp)):
            for k in ("x", "core", "wb", "bias"):
                out[f"{tag}_{k}"] = _host(d[k])
            for n, u in enumerate(d["factors"]):
                out[f"{tag}_factor{n}"] = _host(u)
        return out

    plain_bytes = tk.save_bytes
    plain = run()
    tk.keep_intermediates(True)
    assert tk.save_bytes > plain_bytes
    kept = run()
    for k in plain:
        assert np.array_equal(plain[k], kept[k]), k
    tk.close()
    plan.close()
