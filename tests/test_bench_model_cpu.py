"""bench.py's step floors: the method's compulsory bytes and flops of each workload, against
the figures worked out by hand from the same definitions (CPU only)."""
import pytest

import bench
from fno_spectral_convolution_amd import configs

# workload: (GB, spectral GF, pointwise GF, t_hbm us, t_flop us, bound)
EXPECTED = {
    "stack2d_256": (1.376, 9.9, 17.6, 172.0, 175.3, "mfma"),
    "train2d_512": (12.080, 123.5, 206.2, 1510.0, 1359.7, "hbm"),
    "train3d_128": (7.676, 78.4, 40.3, 959.4, 754.6, "hbm"),
    "st4d_128x20": (28.259, 704.1, 134.2, 3532.4, 5329.3, "mfma"),
    "st4d_128x20_bf16": (28.259, 704.1, 134.2, 3532.4, 1133.0, "hbm"),
}


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_step_floor(name):
    wl = configs.get(name)
    gb, spec, pw, th, tf, bound = EXPECTED[name]
    w = bench.method_work(wl)
    assert abs(w["bytes"] / 1e9 - gb) < 0.001
    assert abs(w["flops_spectral"] / 1e9 - spec) < 0.1
    assert abs(w["flops_pointwise"] / 1e9 - pw) < 0.1
    r = bench.step_roofline(wl, configs.precision(wl), 2.0)
    assert abs(r["t_hbm_us"] - th) < 0.2 and abs(r["t_flop_us"] - tf) < 0.2
    assert r["bound"] == bound
    assert r["t_roof_us"] == max(r["t_hbm_us"], r["t_flop_us"])
    assert abs(r["frac"] - r["t_roof_us"] / 2000.0) < 1e-4


def test_kernel_floor_split_bypass():
    """The width-64 half-plan backward epilogue: 12 B per element + the half-format line
    spectra, its two bypass products priced as three bf16 products each."""
    wl = configs.get("train2d_512")
    row = bench.kernel_model(wl, "bf16")["epilogue_bwd"]
    U = 8 * 64 * 512 * 512
    assert row[0] == 12 * U + 8 * 64 * 512 * 32 * 4
    assert row[3] is True
    t_hbm, t_flop = bench.kernel_floor(row, "bf16")
    assert t_hbm > t_flop
    row32 = bench.kernel_model(wl, "f32")["epilogue_bwd"]
    assert row32[3] is False
    assert bench.kernel_floor(row32, "f32")[1] > t_hbm  # float32: the bypass binds
