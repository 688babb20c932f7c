"""Precision scheduling on the GPU (mixed-precision neural-operator page, "Tiivistelmä":
training moves from mixed to full precision): a two-block 2D training stack (dense or
Tucker-factorised weights) runs four steps through StackRunner.run, two with half operands,
two in fp32 with the tanh pre-activation kept, once with the loss fused into the last block
and once with the stand-alone loss kernel.  Every step's loss, gradients and (with the loss
kernel) output are compared with the oracle's training step (tanh on) at the tolerance of the
precision the step ran in; steps of one precision must agree bit for bit (no weight update runs
between them)."""
import numpy as np
import pytest

import oracle.fno_oracle as O
from fno_spectral_convolution_amd import configs
from tests.gpu_helpers import announce, check, tol_for

pytestmark = pytest.mark.gpu

# width 16 and a 64-point contiguous axis take the matrix-core kernels
_WL = dict(name="sched2d_24x64", cfg_id=11, batch=2, width=16, grid=(24, 64), modes=(5, 12),
           blocks=2, train=True)


def _host(t):
    return t.detach().cpu().numpy().copy()


def _tucker_train_ref(hi, modes):
    """The oracle's training step of a stack of Tucker blocks (GELU after every block, MSE)."""
    acts = [np.asarray(hi["x"], dtype=np.float64)]
    for blk in hi["blocks"]:
        acts.append(O.tucker_block_fwd(acts[-1], blk["core"], blk["factors"], blk["wb"],
                                       blk["bias"], modes, tanh=True)["y"])
    loss, g = O.mse_loss_grad(acts[-1], hi["target"])
    grads = [None] * len(hi["blocks"])
    for i in reversed(range(len(hi["blocks"]))):
        blk = hi["blocks"][i]
        r = O.tucker_block_bwd(acts[i], blk["core"], blk["factors"], blk["wb"], blk["bias"],
                               modes, g, tanh=True)
        grads[i] = {"grad_core": r["grad_core"], "grad_factors": r["grad_factors"],
                    "grad_wb": r["grad_wb"], "grad_bias": r["grad_bias"]}
        g = r["grad_x"]
    return {"loss": loss, "y": acts[-1], "grad_x": g, "grads": grads}


@pytest.mark.parametrize("fuse", [True, False], ids=["fused_loss", "loss_kernel"])
@pytest.mark.parametrize("weights", ["dense", "tucker"])
@pytest.mark.parametrize("half", ["bf16", "f16"])
def test_precision_schedule_training_run(half, weights, fuse):
    import torch
    from fno_spectral_convolution_amd.stack import PrecisionSchedule, StackRunner
    announce("schedule", half, weights, "fused loss" if fuse else "loss kernel")
    extra = {"tucker_ranks": (8, 8, 6, 6)} if weights == "tucker" else {}
    wl = configs.Workload(mixed=True if half == "bf16" else "f16", **_WL, **extra)
    runner = StackRunner(wl, device="cuda", fuse_loss=fuse)
    assert runner.fuse_loss == fuse
    hi = runner.host
    if weights == "tucker":
        ref = _tucker_train_ref(hi, wl.modes)
    else:
        ref = O.train_step(hi["x"], hi["target"], hi["blocks"], wl.modes, tanh=True)
    wkeys = ("core", "wb", "bias") if weights == "tucker" else ("w", "wb", "bias")
    seen = []

    def on_step(i, out):
        torch.cuda.synchronize()
        s = runner.grad_scale
        grads = []
        for g in runner.grads:
            d = {k: _host(g[k]) / s for k in wkeys}
            if weights == "tucker":
                d["factors"] = [_host(u) / s for u in g["factors"]]
            grads.append(d)
        # the fused loss never writes the output field
        assert (out is None) == fuse
        seen.append({"precision": runner.precision, "scale": s,
                     "y": None if out is None else _host(out),
                     "loss": float(_host(runner.loss)[0]), "grad_x": _host(runner.grad_x) / s,
                     "grads": grads})

    runner.run(PrecisionSchedule(2, half), 4, on_step=on_step)
    assert [r["precision"] for r in seen] == [half, half, "f32", "f32"]
    assert [r["scale"] for r in seen] == ([65536.0] * 2 if half == "f16" else [1.0] * 2) + [1.0] * 2
    for i, r in enumerate(seen):
        tol = tol_for(False if r["precision"] == "f32" else ("f16" if half == "f16" else True))
        print(f"  step {i} ({r['precision']})", flush=True)
        if not fuse:
            check("y", r["y"], ref["y"], tol)
        assert abs(r["loss"] - ref["loss"]) <= tol * ref["loss"], (r["loss"], ref["loss"])
        check("grad_x", r["grad_x"], ref["grad_x"], tol)
        for b, (g, gr) in enumerate(zip(r["grads"], ref["grads"])):
            if weights == "tucker":
                check(f"block {b} grad_core", g["core"], gr["grad_core"], tol)
                for n, (u, ur) in enumerate(zip(g["factors"], gr["grad_factors"])):
                    check(f"block {b} grad_factor {n}", u, ur, tol)
            else:
                check(f"block {b} grad_w", g["w"], gr["grad_w"], tol)
            check(f"block {b} grad_wb", g["wb"], gr["grad_wb"], tol)
            check(f"block {b} grad_bias", g["bias"], gr["grad_bias"], tol)
    for a, b in ((seen[0], seen[1]), (seen[2], seen[3])):
        assert a["loss"] == b["loss"] and np.array_equal(a["grad_x"], b["grad_x"])
        if not fuse:
            assert np.array_equal(a["y"], b["y"])
        for ga, gb in zip(a["grads"], b["grads"]):
            assert all(np.array_equal(ga[k], gb[k]) for k in wkeys)
    # the fp32 steps after the switch differ from the half steps before it
    assert not np.array_equal(seen[1]["grad_x"], seen[2]["grad_x"])
