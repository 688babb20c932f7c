"""Shared helpers of the GPU parity tests (no oracle arithmetic here)."""
import sys

import numpy as np

TOL_F32 = 1e-5    # relative L2, fp32 spectral path
TOL_MIXED = 1e-2  # relative L2, tanh + bf16 spectral path
# tanh + IEEE-half spectral path: the operand rounding error scales with the unit roundoff,
# 2^-11 for half against 2^-8 for bfloat16, so the bfloat16 bound divided by 8.  A half path
# that rounded its operands to bfloat16 by mistake shows errors eight times larger.
TOL_F16 = TOL_MIXED / 8


def tol_for(mixed) -> float:
    """Tolerance of a spectral precision as the plans take it: False, True / "bf16", "f16"."""
    if not mixed:
        return TOL_F32
    return TOL_F16 if mixed == "f16" else TOL_MIXED


def rel_l2(got, want) -> float:
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (got.shape, want.shape)
    g = got.astype(np.complex128 if np.iscomplexobj(got) or np.iscomplexobj(want) else np.float64)
    w = want.astype(g.dtype)
    den = np.linalg.norm(w.ravel())
    return float(np.linalg.norm((g - w).ravel()) / max(den, 1e-300))


def check(name, got, want, tol):
    e = rel_l2(got, want)
    print(f"    {name}: rel_l2={e:.3e} (tol {tol:.0e})", flush=True)
    assert e <= tol, f"{name}: rel L2 {e:.3e} > {tol:.1e}"
    return e


def announce(*parts):
    print("CASE " + " ".join(str(p) for p in parts), flush=True)
    sys.stdout.flush()
