"""A stack of FNO blocks driven through libfno, with every buffer allocated up front.

``StackRunner(workload).step()`` runs one pass of a workload: an optional pointwise lift,
the spectral blocks (GELU after each), an optional projection head, and for training
workloads the MSE loss against a target and the backward through every block (input,
spectral-weight, bypass-weight and bias gradients).  Workloads with Tucker ranks hold each
block's spectral weight as a Tucker core and factors (TFNO) and run the Tucker entry points.  Torch provides device memory and the
stream; all arithmetic runs in libfno's kernels.

``PrecisionSchedule`` with ``StackRunner.run`` moves a training run from a half-precision
spectral path to fp32 at a chosen step (precision scheduling, mixed-precision neural-operator
page, "Tiivistelmä").
"""
from __future__ import annotations

import numpy as np

from . import binding as L
from . import inputs
from .configs import F16_LOSS_SCALE, precision


SPECTRAL_PRECISIONS = ("f32", "bf16", "f16")
_PLAN_MIXED = {"f32": False, "bf16": "bf16", "f16": "f16"}


class PrecisionSchedule:
    """Mixed-to-full precision switch of a training run (mixed-precision neural-operator page,
    "Tiivistelmä": precision scheduling).  Steps 0 .. switch_step - 1 run the spectral path
    with `half` operands ("bf16" or "f16"), every later step in fp32.  The page gives only the
    direction of the switch, so the step is the caller's.  The tanh pre-activation is part of
    the model and stays on after the switch: only the arithmetic changes."""

    def __init__(self, switch_step: int, half: str = "bf16"):
        if half not in ("bf16", "f16"):
            raise ValueError(f"half must be 'bf16' or 'f16', not {half!r}")
        if isinstance(switch_step, bool) or int(switch_step) != switch_step or switch_step < 0:
            raise ValueError(f"switch_step must be an integer >= 0, not {switch_step!r}")
        self.switch_step = int(switch_step)
        self.half = half

    @classmethod
    def from_fraction(cls, total_steps: int, half_fraction: float, half: str = "bf16"):
        """The first floor(half_fraction * total_steps) steps in half precision."""
        if total_steps < 0 or not 0.0 <= half_fraction <= 1.0:
            raise ValueError("need total_steps >= 0 and 0 <= half_fraction <= 1")
        return cls(int(half_fraction * total_steps), half)

    def precision_at(self, step: int) -> str:
        if step < 0:
            raise ValueError("step must be >= 0")
        return self.half if step < self.switch_step else "f32"


class StackRunner:
    """fuse_loss (training stacks without a projection head): the last block's forward
    computes the loss and the gradient at its pre-activation in one pass (fno_block_fwd_mse)
    and its backward starts from that gradient (fno_block_bwd_preact), so the output field y
    is never written; step() then returns None.  With fuse_loss=False the step writes y and
    runs the stand-alone loss kernel between the two passes."""

    def __init__(self, wl, device="cuda", host_inputs=None, fuse_loss=True, last_axis=None):
        import torch
        self.torch = torch
        self.wl = wl
        dev = torch.device(device)
        self.device = dev
        C = wl.width
        # one plan per spectral precision the run has used and block role (a plan holds only
        # its tables and workspace); the workload's tanh pre-activation is kept by all of them
        self._tanh = bool(wl.mixed)
        self._last_axis = last_axis  # float32 plans: None (plan picks), "fft" or "dense"
        self._plans = {}
        self._tuckers = {}
        self.tucker = bool(wl.tucker_ranks)
        self.precision = precision(wl)
        self._use_precision(self.precision)
        # IEEE-half training takes a static loss scale: every gradient the step returns
        # (weights, bypass, bias, input) comes out multiplied by grad_scale
        self.grad_scale = F16_LOSS_SCALE if self.precision == "f16" else 1.0
        hi = host_inputs or make_host_inputs(wl)
        self.host = hi
        def to(a):
            if isinstance(a, list):
                return [to(v) for v in a]
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        self.params = [{k: to(v) for k, v in blk.items()} for blk in hi["blocks"]]
        self.x_in = to(hi["x"])
        self.target = to(hi["target"]) if wl.train else None
        self.lp = None
        if wl.lift_in:
            lp = hi["lift_proj"]
            self.lp = {"lift": {k: to(v) for k, v in lp["lift"].items()},
                       "proj": {k: to(v) for k, v in lp["proj"].items()}}
        shape = (wl.batch, C) + tuple(wl.grid)
        nb = wl.blocks
        self.fuse_loss = bool(fuse_loss and wl.train and self.lp is None)
        if wl.train:
            self.acts = [torch.empty(shape, dtype=torch.float32, device=dev)
                         for _ in range(nb + 1)]
            self.saves = [self._saver(i).new_save() for i in range(nb)]
            self._save_bytes = [self._saver(i).save_bytes for i in range(nb)]
            self.g = [torch.empty(shape, dtype=torch.float32, device=dev) for _ in range(2)]
            self.grads = []
            for p in self.params:
                gr = {"wb": torch.empty_like(p["wb"]), "bias": torch.empty_like(p["bias"])}
                if self.tucker:
                    gr["core"] = torch.empty_like(p["core"])
                    gr["factors"] = [torch.empty_like(u) for u in p["factors"]]
                else:
                    gr["w"] = torch.empty_like(p["w"])
                self.grads.append(gr)
            self.loss = torch.empty(1, dtype=torch.float32, device=dev)
            self.mse_ws = torch.empty(max(L.fno_mse_workspace_bytes(self.acts[-1].numel()), 16),
                                      dtype=torch.uint8, device=dev)
        else:
            # forward only: two activation buffers used in turn
            self.acts = [torch.empty(shape, dtype=torch.float32, device=dev) for _ in range(2)]
            self.saves = [None] * nb
        if self.lp is not None:
            out_shape = (wl.batch, wl.proj_out) + tuple(wl.grid)
            self.out = torch.empty(out_shape, dtype=torch.float32, device=dev)
    def role(self, i):
        """(input GELU, output GELU) of block i.  A training stack moves the GELU between two
        blocks to the start of the later one: each inner block then keeps only its
        pre-activation z, and its backward reads z and the incoming gradient once instead of
        twice.  The network, its outputs and its gradients are those of the plain stack."""
        nb = self.wl.blocks
        if not self.wl.train or nb == 1:
            return (False, True)
        return (i > 0, i == nb - 1)

    def _plan_for(self, prec, role=(False, True)):
        key = (prec, role)
        if key not in self._plans:
            wl = self.wl
            plan = L.Plan(wl.batch, wl.width, wl.width, wl.grid, wl.modes,
                          mixed=_PLAN_MIXED[prec], tanh=self._tanh, gelu=role[1],
                          input_gelu=role[0], device=self.device,
                          last_axis=self._last_axis if prec == "f32" else None)
            if wl.tucker_ranks:
                tk = L.Tucker(plan, wl.tucker_ranks)
                tk.workspace()
                if wl.train:  # the backward reads the forward's weight-step intermediates
                    tk.keep_intermediates(True)
                self._tuckers[key] = tk
            else:
                plan.workspace()
            self._plans[key] = plan
        return self._plans[key]

    def _use_precision(self, prec):
        nb = self.wl.blocks
        self.block_plans = [self._plan_for(prec, self.role(i)) for i in range(nb)]
        self.block_tuckers = [self._tuckers.get((prec, self.role(i))) for i in range(nb)]
        self.plan = self.block_plans[-1]
        self.tk = self.block_tuckers[-1]

    def set_precision(self, prec):
        """Run the following steps with spectral precision `prec` ("f32", "bf16", "f16").
        The first switch to a precision builds its plan (host tables, one upload); the saved
        spectra buffers grow if the new plan needs more.  Enqueued work is not affected."""
        if prec not in SPECTRAL_PRECISIONS:
            raise ValueError(f"spectral precision must be one of {SPECTRAL_PRECISIONS}")
        if prec == self.precision:
            return
        self._use_precision(prec)
        if self.wl.train:
            for i in range(len(self.block_plans)):
                sv = self._saver(i)
                if sv.save_bytes > self._save_bytes[i]:
                    self.saves[i] = sv.new_save()
                    self._save_bytes[i] = sv.save_bytes
        self.precision = prec
        self.grad_scale = F16_LOSS_SCALE if prec == "f16" else 1.0

    def run(self, schedule, steps, start=0, on_step=None):
        """Steps start .. start + steps - 1 of a training run, each at the precision the
        schedule gives it; on_step(step_index, output) is called after each step is enqueued."""
        out = None
        for i in range(start, start + steps):
            self.set_precision(schedule.precision_at(i))
            out = self.step()
            if on_step is not None:
                on_step(i, out)
        return out

    def _saver(self, i):
        """What sizes block i's save buffer: its Tucker weight (with the kept intermediates)
        or its plan."""
        return self.block_tuckers[i] if self.tucker else self.block_plans[i]

    def _act(self, i):
        return self.acts[i] if self.wl.train else self.acts[i % 2]

    def step(self):
        """One pass of the workload; returns the output field (None when the loss is fused
        into the last block) and enqueues the backward of a training workload."""
        wl = self.wl
        if self.lp is not None:
            lift = self.lp["lift"]
            L.pointwise(self.x_in, lift["w"], lift["b"], out=self._act(0))
            src0 = self._act(0)
        else:
            src0 = self.x_in
        h = src0
        nb = len(self.params)
        for i, p in enumerate(self.params):
            dst = self._act(i + 1)
            if self.fuse_loss and i == nb - 1:
                # loss and the gradient at the last pre-activation, into g[0]; y is not stored
                if self.tucker:
                    self.block_tuckers[i].block_fwd_mse(
                        h, p["core"], p["factors"], p["wb"], p["bias"], self.target,
                        self.grad_scale, save=self.saves[i], grad_z=self.g[0], loss=self.loss)
                else:
                    self.block_plans[i].block_fwd_mse(
                        h, p["w"], p["wb"], p["bias"], self.target, self.grad_scale,
                        save=self.saves[i], grad_z=self.g[0], loss=self.loss)
                h = None
                break
            if self.tucker:
                self.block_tuckers[i].block_fwd(h, p["core"], p["factors"], p["wb"], p["bias"],
                                                save=self.saves[i], out=dst)
            else:
                self.block_plans[i].block_fwd(h, p["w"], p["wb"], p["bias"], save=self.saves[i],
                                              out=dst)
            h = dst
        if self.lp is not None:
            pr = self.lp["proj"]
            L.pointwise(h, pr["w1"], pr["b1"], pr["w2"], pr["b2"], out=self.out)
            h = self.out
        if wl.train:
            if not self.fuse_loss:
                L.mse_grad(h, self.target, grad=self.g[0], loss=self.loss, ws=self.mse_ws,
                           grad_scale=self.grad_scale)
            gin = 0
            for i in reversed(range(len(self.params))):
                p = self.params[i]
                x_i = src0 if i == 0 else self.acts[i]
                gout = 1 - gin
                if self.fuse_loss and i == nb - 1:
                    if self.tucker:
                        self.block_tuckers[i].block_bwd_preact(
                            x_i, p["core"], p["factors"], p["wb"], p["bias"], self.saves[i],
                            self.g[gin], out={"x": self.g[gout], **self.grads[i]})
                    else:
                        self.block_plans[i].block_bwd_preact(
                            x_i, p["w"], p["wb"], p["bias"], self.saves[i], self.g[gin],
                            out={"x": self.g[gout], **self.grads[i]})
                elif self.tucker:
                    self.block_tuckers[i].block_bwd(x_i, p["core"], p["factors"], p["wb"],
                                                    p["bias"], self.saves[i], self.g[gin],
                                                    out={"x": self.g[gout], **self.grads[i]})
                else:
                    self.block_plans[i].block_bwd(x_i, p["w"], p["wb"], p["bias"], self.saves[i],
                                                  self.g[gin],
                                                  out={"x": self.g[gout], **self.grads[i]})
                gin = gout
            self.grad_x = self.g[gin]
        return h


def make_host_inputs(wl):
    """Seeded host arrays (float32 / complex64) of a workload."""
    hi = {"x": inputs.field(wl, inputs.STREAM_INPUT),
          "blocks": inputs.block_params(wl)}
    if wl.train:
        hi["target"] = inputs.field(wl, inputs.STREAM_TARGET)
    if wl.lift_in:
        hi["lift_proj"] = inputs.lift_proj_params(wl)
    return hi
