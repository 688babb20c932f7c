"""A stack of FNO blocks driven through libfno, with every buffer allocated up front.

``StackRunner(workload).step()`` runs one pass of a workload: an optional pointwise lift,
the spectral blocks (GELU after each), an optional projection head, and for training
workloads the MSE loss against a target and the backward through every block (input,
spectral-weight, bypass-weight and bias gradients).  Torch provides device memory and the
stream; all arithmetic runs in libfno's kernels.
"""
from __future__ import annotations

import numpy as np

from . import binding as L
from . import inputs


class StackRunner:
    def __init__(self, wl, device="cuda", host_inputs=None):
        import torch
        self.torch = torch
        self.wl = wl
        dev = torch.device(device)
        self.device = dev
        C = wl.width
        self.plan = L.Plan(wl.batch, C, C, wl.grid, wl.modes, mixed=wl.mixed, device=dev)
        hi = host_inputs or make_host_inputs(wl)
        self.host = hi
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
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
        if wl.train:
            self.acts = [torch.empty(shape, dtype=torch.float32, device=dev)
                         for _ in range(nb + 1)]
            self.saves = [self.plan.new_save() for _ in range(nb)]
            self.g = [torch.empty(shape, dtype=torch.float32, device=dev) for _ in range(2)]
            self.grads = [{"w": torch.empty_like(p["w"]), "wb": torch.empty_like(p["wb"]),
                           "bias": torch.empty_like(p["bias"])} for p in self.params]
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
        self.plan.workspace()

    def _act(self, i):
        return self.acts[i] if self.wl.train else self.acts[i % 2]

    def step(self):
        """One pass of the workload; returns the output field (and enqueues the backward)."""
        wl = self.wl
        if self.lp is not None:
            lift = self.lp["lift"]
            L.pointwise(self.x_in, lift["w"], lift["b"], out=self._act(0))
            src0 = self._act(0)
        else:
            src0 = self.x_in
        h = src0
        for i, p in enumerate(self.params):
            dst = self._act(i + 1)
            self.plan.block_fwd(h, p["w"], p["wb"], p["bias"], save=self.saves[i], out=dst)
            h = dst
        if self.lp is not None:
            pr = self.lp["proj"]
            L.pointwise(h, pr["w1"], pr["b1"], pr["w2"], pr["b2"], out=self.out)
            h = self.out
        if wl.train:
            L.mse_grad(h, self.target, grad=self.g[0], loss=self.loss, ws=self.mse_ws)
            gin = 0
            for i in reversed(range(len(self.params))):
                p = self.params[i]
                x_i = src0 if i == 0 else self.acts[i]
                gout = 1 - gin
                self.plan.block_bwd(x_i, p["w"], p["wb"], p["bias"], self.saves[i], self.g[gin],
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
