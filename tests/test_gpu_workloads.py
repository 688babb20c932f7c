"""Parity at the workloads' full sizes, in the launch configuration bench.py times.

Inputs are the workloads' own seeded fields (Gaussian random fields, coordinate and layered
permeability channels) and block parameters.  Where the oracle can evaluate the whole field in
seconds it does (the 2D single layer; the 2D and 3D training workloads one block forward +
backward over the full batch; the 2D stack on sampled batch entries, which the stack never
mixes).  For the 4D space-time share (3.4 GB per field) the oracle computes the full retained spectrum and then the block output
directly at sampled grid points.  The spectral path is also compared on its own (y_spec and the
spectral part of grad_x), since at these weight scales the bypass dominates the block output.
"""
import zlib

import numpy as np
import pytest

import oracle.fno_oracle as O
from fno_spectral_convolution_amd import configs, inputs
from tests.gpu_helpers import TOL_F32, announce, check, tol_for

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _dev(a):
    return _torch().from_numpy(np.ascontiguousarray(a)).to("cuda")


def _host(t):
    return t.detach().cpu().numpy()


_FIELDS = {}


def _field(wl):
    """The workload's seeded input field, generated once per module (the fp32 and bf16 4D workloads share it)."""
    key = (wl.cfg_id, wl.batch, wl.width, tuple(wl.grid), wl.input_kind)
    if key not in _FIELDS:
        _FIELDS.clear()
        _FIELDS[key] = inputs.field(wl, inputs.STREAM_INPUT, channels=wl.width)
    return _FIELDS[key]


@pytest.fixture(scope="module")
def L():
    from fno_spectral_convolution_amd import binding
    return binding


def _grad_in(wl, scale):
    g = np.random.default_rng(np.random.SeedSequence([wl.cfg_id, 77]))
    return (g.standard_normal((wl.batch, wl.width) + tuple(wl.grid)) * scale).astype(np.float32)


def _block_case(L, name, grad_scale):
    """One block of the workload at full size: forward, backward and the spectral path alone."""
    wl = configs.get(name)
    tol = tol_for(wl.mixed)
    announce("workload block", name, wl.batch, wl.width, wl.grid, wl.modes)
    x = _field(wl)
    blk = inputs.block_params(wl, 1)[0]
    gy = _grad_in(wl, grad_scale)
    plan = L.Plan(wl.batch, wl.width, wl.width, wl.grid, wl.modes, mixed=wl.mixed)
    tx, tw, twb, tb, tg = (_dev(a) for a in (x, blk["w"], blk["wb"], blk["bias"], gy))
    save = plan.new_save()
    y = plan.block_fwd(tx, tw, twb, tb, save=save)
    g = plan.block_bwd(tx, tw, twb, tb, save, tg)
    _torch().cuda.synchronize()
    y, gx, gw, gwb, gb = _host(y), _host(g["x"]), _host(g["w"]), _host(g["wb"]), _host(g["bias"])
    del save, g
    ref = O.block_bwd(x, blk["w"], blk["wb"], blk["bias"], wl.modes, gy, tanh=bool(wl.mixed))
    check("y", y, ref["fwd"]["y"], tol)
    check("grad_x", gx, ref["grad_x"], tol)
    check("grad_w", gw, ref["grad_w"], tol)
    check("grad_wb", gwb, ref["grad_wb"], tol)
    check("grad_bias", gb, ref["grad_bias"], tol)
    # the spectral path on its own: forward y_spec and the adjoint applied to the oracle's g_z
    sp = L.Plan(wl.batch, wl.width, wl.width, wl.grid, wl.modes, mixed=wl.mixed, gelu=False,
                bias=False)
    ys = sp.spectral_conv_fwd(tx, tw)
    gxs, _ = sp.spectral_conv_bwd(tx, tw, _dev(ref["g_z"].astype(np.float32)), want_w=False)
    _torch().cuda.synchronize()
    check("y_spec", _host(ys), ref["fwd"]["y_spec"], tol)
    check("grad_x spectral part", _host(gxs), ref["gx_spec"], tol)
    plan.close()
    sp.close()


def _tucker_block_case(L, name, grad_scale):
    """One Tucker-factorised block of the workload at full size, forward and backward."""
    wl = configs.get(name)
    tol = tol_for(wl.mixed)
    x = _field(wl)
    blk = inputs.block_params(wl, 1)[0]
    gy = _grad_in(wl, grad_scale)
    plan = L.Plan(wl.batch, wl.width, wl.width, wl.grid, wl.modes, mixed=wl.mixed)
    tk = L.Tucker(plan, wl.tucker_ranks)
    announce("workload tucker block", name, wl.batch, wl.width, wl.grid, wl.modes,
             wl.tucker_ranks, tk.order)
    tx, twb, tb, tg, tcore = (_dev(a) for a in (x, blk["wb"], blk["bias"], gy, blk["core"]))
    tfac = [_dev(u) for u in blk["factors"]]
    save = plan.new_save()
    y = tk.block_fwd(tx, tcore, tfac, twb, tb, save=save)
    g = tk.block_bwd(tx, tcore, tfac, twb, tb, save, tg)
    _torch().cuda.synchronize()
    got = {"y": _host(y), "grad_x": _host(g["x"]), "grad_core": _host(g["core"]),
           "grad_wb": _host(g["wb"]), "grad_bias": _host(g["bias"]),
           "grad_factors": [_host(u) for u in g["factors"]]}
    del save, g
    ref = O.tucker_block_bwd(x, blk["core"], blk["factors"], blk["wb"], blk["bias"], wl.modes,
                             gy, tanh=bool(wl.mixed))
    check("y", got["y"], ref["fwd"]["y"], tol)
    check("y error against |y_spec|", got["y"] - ref["fwd"]["y"] + ref["fwd"]["y_spec"],
          ref["fwd"]["y_spec"],
          tol)
    check("grad_x", got["grad_x"], ref["grad_x"], tol)
    check("grad_core", got["grad_core"], ref["grad_core"], tol)
    for n, (a, b) in enumerate(zip(got["grad_factors"], ref["grad_factors"])):
        check(f"grad_factor {n}", a, b, tol)
    check("grad_wb", got["grad_wb"], ref["grad_wb"], tol)
    check("grad_bias", got["grad_bias"], ref["grad_bias"], tol)
    tk.close()
    plan.close()


def test_layer2d_64_block_full(L):
    _block_case(L, "layer2d_64", 1.0)


def test_train2d_512_block_full(L):
    _block_case(L, "train2d_512", 1e-3)


def test_train2d_512_f16_block_full(L):
    _block_case(L, "train2d_512_f16", 1e-3)


def test_train2d_512_tfno_block_full(L):
    _tucker_block_case(L, "train2d_512_tfno", 1e-3)


def test_train3d_128_block_full(L):
    _block_case(L, "train3d_128", 1e-3)


@pytest.mark.parametrize("name", ["train2d_512", "train3d_128"])
def test_last_block_fused_loss_full(L, name):
    """The last block of the training stack at full size, as the step runs it: input GELU,
    output GELU, the loss against the workload's target fused into the forward epilogue
    (fno_block_fwd_mse) and the backward from the pre-activation gradient
    (fno_block_bwd_preact), against the oracle's loss, grad_z and block backward."""
    wl = configs.get(name)
    tol = tol_for(wl.mixed)
    announce("workload fused loss", name, wl.batch, wl.width, wl.grid, wl.modes)
    x = _field(wl)
    tgt = inputs.field(wl, inputs.STREAM_TARGET)
    blk = inputs.block_params(wl, 1)[0]
    plan = L.Plan(wl.batch, wl.width, wl.width, wl.grid, wl.modes, mixed=wl.mixed,
                  input_gelu=True)
    tx, tw, twb, tb, tt = (_dev(a) for a in (x, blk["w"], blk["wb"], blk["bias"], tgt))
    save = plan.new_save()
    gz, loss = plan.block_fwd_mse(tx, tw, twb, tb, tt, save=save)
    g = plan.block_bwd_preact(tx, tw, twb, tb, save, gz)
    _torch().cuda.synchronize()
    got = {"grad_z": _host(gz), "loss": float(_host(loss)[0]), "grad_x": _host(g["x"]),
           "grad_w": _host(g["w"]), "grad_wb": _host(g["wb"]), "grad_bias": _host(g["bias"])}
    del save, g, gz, tt
    ref = O.block_fwd_mse(x, blk["w"], blk["wb"], blk["bias"], wl.modes, tgt,
                          tanh=bool(wl.mixed), input_gelu=True)
    print(f"    loss: {got['loss']:.7e} (oracle {ref['loss']:.7e})", flush=True)
    assert abs(got["loss"] - ref["loss"]) <= tol * ref["loss"], (got["loss"], ref["loss"])
    check("grad_z", got["grad_z"], ref["grad_z"], tol)
    refb = O.block_bwd_preact(x, blk["w"], blk["wb"], blk["bias"], wl.modes, ref["grad_z"],
                              tanh=bool(wl.mixed), input_gelu=True)
    del ref
    for k in ("grad_x", "grad_w", "grad_wb", "grad_bias"):
        check(k, got[k], refb[k], tol)
    plan.close()


def test_stack2d_256_sampled_batches(L):
    """The full 2D stack (lift, 4 blocks, projection) on the GPU, as bench.py runs it; the
    oracle evaluates the same stack for batch entries 0 and 15."""
    from fno_spectral_convolution_amd.stack import StackRunner
    wl = configs.get("stack2d_256")
    announce("workload stack stack2d_256")
    runner = StackRunner(wl, device="cuda")
    out = _host(runner.step())
    _torch().cuda.synchronize()
    hi = runner.host
    for b in (0, wl.batch - 1):
        want = O.stack_fwd(hi["x"][b:b + 1], hi["blocks"], wl.modes,
                           lift=hi["lift_proj"]["lift"], proj=hi["lift_proj"]["proj"])
        check(f"stack output batch {b}", out[b:b + 1], want, TOL_F32)


@pytest.mark.parametrize("name", ["st4d_128x20", "st4d_128x20_bf16", "st4d_128x20_f16"])
def test_st4d_128x20_block_sampled_points(L, name):
    """4D space-time share [1, 20, 128^3 x 20]: y and y_spec at 512 sampled grid points."""
    wl = configs.get(name)
    tol = tol_for(wl.mixed)
    announce("workload block sampled", name)
    torch = _torch()
    x = _field(wl)
    blk = inputs.block_params(wl, 1)[0]
    plan = L.Plan(wl.batch, wl.width, wl.width, wl.grid, wl.modes, mixed=wl.mixed)
    tx = _dev(x)
    tw, twb, tb = _dev(blk["w"]), _dev(blk["wb"]), _dev(blk["bias"])
    y = plan.block_fwd(tx, tw, twb, tb)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    pts = np.stack([rng.integers(0, n, 512) for n in wl.grid], axis=1)
    flat = np.ravel_multi_index(tuple(pts.T), wl.grid)
    idx = torch.from_numpy(flat).to("cuda")
    y_s = _host(y.reshape(wl.batch, wl.width, -1)[:, :, idx])
    del y
    sp = L.Plan(wl.batch, wl.width, wl.width, wl.grid, wl.modes, mixed=wl.mixed, gelu=False,
                bias=False)
    ys = sp.spectral_conv_fwd(tx, tw)
    ys_s = _host(ys.reshape(wl.batch, wl.width, -1)[:, :, idx])
    del ys, tx
    torch.cuda.synchronize()
    want = O.block_at_points(x, blk["w"], blk["wb"], blk["bias"], wl.modes, pts,
                             tanh=bool(wl.mixed))
    want_spec = want["y_spec"]
    check("y_spec (sampled)", ys_s, want_spec, tol)
    check("y (sampled)", y_s, want["y"], tol)
    plan.close()
    sp.close()
