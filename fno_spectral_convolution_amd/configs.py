"""Workload registry: the FNO workloads this library is checked and measured on.

Pure data.  Shapes follow the FNO of the model-parallel FNO page ("Proposed method": 4
spectral blocks, width 20; "Main findings": 3D and 4D space-time grids) and the
mixed-precision neural-operator page ("Tiivistelmä": tanh pre-activation, half-precision
transform and contraction).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int                   # seed namespace of the input generators
    batch: int
    width: int                    # channels inside the blocks (Cin = Cout)
    grid: Tuple[int, ...]         # spatial grid N_0..N_{d-1}; the last axis is contiguous
    modes: Tuple[int, ...]        # modes per corner m_0..m_{d-1}
    blocks: int                   # number of spectral blocks
    mixed: object                 # False: fp32; True / "bf16" or "f16": tanh pre-activation
                                  # + bfloat16 or IEEE-half spectral operands
    train: bool                   # forward + MSE + backward (else forward only)
    lift_in: Optional[int] = None     # pointwise lift input channels (2D stack)
    proj_hidden: Optional[int] = None  # projection hidden width (2D stack)
    proj_out: Optional[int] = None
    zero_bias: bool = False
    input_kind: str = "grf"       # grf | normal | grf_coords | grf_layered
    tucker_ranks: Optional[Tuple[int, ...]] = None  # Tucker-factorised spectral weights
                                  # (TFNO): ranks R_in, R_out, R_0..R_{d-1}
    notes: str = ""

    @property
    def ndim(self) -> int:
        return len(self.grid)

    @property
    def points(self) -> int:
        p = 1
        for n in self.grid:
            p *= n
        return p

    @property
    def units(self) -> int:
        """Grid points x channels x batch x blocks: the throughput unit."""
        return self.batch * self.width * self.points * self.blocks


WORKLOADS = {
    "layer2d_64": Workload("layer2d_64", 1, 4, 20, (64, 64), (12, 12), 1, False, False,
                   zero_bias=True, input_kind="normal",
                   notes="2D single spectral layer, forward only, fp32"),
    "stack2d_256": Workload("stack2d_256", 2, 16, 32, (256, 256), (16, 16), 4, False, False,
                   lift_in=3, proj_hidden=128, proj_out=1, input_kind="grf_coords",
                   notes="2D FNO stack forward, fp32, lift 3->32, projection 32->128->1"),
    "train2d_512": Workload("train2d_512", 3, 8, 64, (512, 512), (32, 32), 4, True, True,
                   notes="2D FNO training step, tanh + bf16 spectral path, fwd+bwd, MSE"),
    "train3d_128": Workload("train3d_128", 4, 2, 20, (128, 128, 128), (16, 16, 16), 4, False, True,
                   input_kind="grf_layered",
                   notes="3D FNO stack fwd+bwd, fp32, layered permeability channel"),
    "st4d_128x20": Workload("st4d_128x20", 5, 1, 20, (128, 128, 128, 20), (12, 12, 12, 8), 4, False, False,
                   notes="4D space-time block stack forward, fp32"),
    "st4d_128x20_bf16": Workload("st4d_128x20_bf16", 5, 1, 20, (128, 128, 128, 20), (12, 12, 12, 8), 4, True, False,
                    notes="4D space-time block stack forward, tanh + bf16"),
    # the IEEE-half variants of the two mixed-precision workloads
    "train2d_512_f16": Workload("train2d_512_f16", 3, 8, 64, (512, 512), (32, 32), 4, "f16", True,
                   notes="2D FNO training step, tanh + fp16 spectral path (static loss scale 2^16), fwd+bwd, MSE"),
    "st4d_128x20_f16": Workload("st4d_128x20_f16", 5, 1, 20, (128, 128, 128, 20), (12, 12, 12, 8), 4, "f16", False,
                    notes="4D space-time block stack forward, tanh + fp16"),
    # TFNO: the 2D mixed-precision training step with Tucker-factorised spectral weights, every
    # rank half its mode's extent (64 channels, 2 x 32 and 32 retained modes)
    "train2d_512_tfno": Workload("train2d_512_tfno", 6, 8, 64, (512, 512), (32, 32), 4, True, True,
                    tucker_ranks=(32, 32, 32, 16),
                    notes="2D TFNO training step (Tucker ranks 32/32/32/16), tanh + bf16, fwd+bwd, MSE"),
}

# static loss scale of the IEEE-half training step: MSE gradients of a mean over ~10^8 elements
# are ~1e-8, below half's smallest subnormal (6e-8); scaled by 2^16 they sit near 1e-3
F16_LOSS_SCALE = 65536.0


def precision(wl) -> str:
    """Spectral arithmetic of a workload: "f32", "bf16" or "f16"."""
    if wl.mixed == "f16":
        return "f16"
    return "bf16" if wl.mixed else "f32"


def get(name: str) -> Workload:
    return WORKLOADS[name.lower()]
