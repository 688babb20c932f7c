"""C-ABI boundary checks that need no GPU: the library loads, exports every symbol the
header declares, and validates descriptors on the host."""
import ctypes
import os
import re

import pytest

from fno_spectral_convolution_amd import binding as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "fno.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fno_[a-z0-9_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert _header_functions() == sorted(L.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in _header_functions():
        assert hasattr(lib, name), name


def test_desc_layout_matches_header():
    # int32 x4, int64 x3, int64[4] x2
    assert ctypes.sizeof(L.fno_plan_desc) == 16 + 24 + 64


def _desc(**kw):
    base = dict(batch=4, c_in=20, c_out=20, grid=(64, 64), modes=(12, 12), dtype=0, flags=6)
    base.update(kw)
    return L.make_desc(base["batch"], base["c_in"], base["c_out"], base["grid"], base["modes"],
                       base["dtype"], base["flags"])


@pytest.mark.parametrize("kw", [
    dict(), dict(grid=(128, 128, 128), modes=(16, 16, 16)),
    dict(grid=(128, 128, 128, 20), modes=(12, 12, 12, 8), batch=1),
    dict(grid=(512, 512), modes=(32, 32), c_in=64, c_out=64, dtype=1, flags=7),
    dict(grid=(512, 512), modes=(32, 32), c_in=64, c_out=64, dtype=2, flags=7),
    dict(grid=(512, 512), modes=(32, 32), c_in=64, c_out=64, dtype=1, flags=15),
    dict(grid=(256, 256), modes=(16, 16), flags=16 | 7), dict(flags=32),
    dict(grid=(8, 8), modes=(4, 5)), dict(grid=(15, 9), modes=(7, 5)),
])
def test_validate_accepts(kw):
    assert L.fno_plan_validate(_desc(**kw)) == L.FNO_OK, L.last_error_message()


@pytest.mark.parametrize("kw,status", [
    (dict(grid=(64,), modes=(12,)), L.FNO_ERR_INVALID_ARGUMENT),
    (dict(modes=(33, 12)), L.FNO_ERR_INVALID_ARGUMENT),
    (dict(modes=(12, 34)), L.FNO_ERR_INVALID_ARGUMENT),
    (dict(modes=(0, 12)), L.FNO_ERR_INVALID_ARGUMENT),
    (dict(batch=0), L.FNO_ERR_INVALID_ARGUMENT),
    (dict(c_in=0), L.FNO_ERR_INVALID_ARGUMENT),
    (dict(flags=64), L.FNO_ERR_INVALID_ARGUMENT),
    (dict(flags=16 | 32), L.FNO_ERR_INVALID_ARGUMENT),
    (dict(dtype=7), L.FNO_ERR_INVALID_ARGUMENT),
    (dict(c_in=65), L.FNO_ERR_UNSUPPORTED),
    (dict(grid=(64, 8192), modes=(12, 12)), L.FNO_ERR_UNSUPPORTED),
])
def test_validate_rejects(kw, status):
    assert L.fno_plan_validate(_desc(**kw)) == status
    assert L.last_error_message()


def test_reserved_and_unused_dims_rejected():
    d = _desc()
    d.reserved = 1
    assert L.fno_plan_validate(d) == L.FNO_ERR_INVALID_ARGUMENT
    d = _desc()
    d.n[3] = 5
    assert L.fno_plan_validate(d) == L.FNO_ERR_INVALID_ARGUMENT


def test_null_arguments_rejected_on_host():
    assert L._lib.fno_plan_validate(None) == L.FNO_ERR_INVALID_ARGUMENT
    assert L._lib.fno_plan_create(None, None) == L.FNO_ERR_INVALID_ARGUMENT
    assert L._lib.fno_plan_destroy(None) == L.FNO_OK
    assert L._lib.fno_plan_query(None, None, None, None) == L.FNO_ERR_INVALID_ARGUMENT
    assert L._lib.fno_block_fwd(None, None, None, None, None, None, None, None, 0, None) == \
        L.FNO_ERR_INVALID_ARGUMENT
    assert L._lib.fno_mse_grad(0, None, None, None, None, None, 0, None) == \
        L.FNO_ERR_INVALID_ARGUMENT
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert L._lib.fno_mse_grad_scaled(4, None, None, None, None, bad, None, 0, None) == \
            L.FNO_ERR_INVALID_ARGUMENT
    assert L._lib.fno_pointwise_fwd(1, 1, 1, 0, 300, None, None, None, None, None, None,
                                    None) == L.FNO_ERR_UNSUPPORTED
    assert L._lib.fno_tucker_keep_intermediates(None, 1) == L.FNO_ERR_INVALID_ARGUMENT
    assert L._lib.fno_tucker_save_bytes(None, None) == L.FNO_ERR_INVALID_ARGUMENT
    assert L._lib.fno_block_fwd_mse(None, None, None, None, None, None, 1.0, None, None, None,
                                    None, 0, None) == L.FNO_ERR_INVALID_ARGUMENT
    assert L._lib.fno_block_bwd_preact(None, None, None, None, None, None, None, None, None,
                                       None, None, None, 0, None) == L.FNO_ERR_INVALID_ARGUMENT
    assert L._lib.fno_tucker_block_fwd_mse(None, None, None, None, None, None, None, 1.0, None,
                                           None, None, None, 0, None) == \
        L.FNO_ERR_INVALID_ARGUMENT
    assert L._lib.fno_tucker_block_bwd_preact(None, None, None, None, None, None, None, None,
                                              None, None, None, None, None, None, 0, None) == \
        L.FNO_ERR_INVALID_ARGUMENT


def test_status_strings():
    for s in range(6):
        assert L.status_string(s).startswith("FNO_")


@pytest.mark.parametrize("kw", [
    dict(), dict(grid=(24, 20), modes=(5, 4), c_in=3, c_out=5),
    dict(grid=(15, 9), modes=(7, 5)), dict(grid=(8, 8), modes=(4, 5)),
    dict(grid=(64, 512), modes=(8, 32), c_in=64, c_out=64, dtype=1, flags=7),
    dict(grid=(12, 10, 16), modes=(3, 2, 5)), dict(grid=(10, 12, 64), modes=(3, 4, 8)),
    dict(grid=(6, 8, 10, 20), modes=(2, 3, 4, 8), batch=1),
    dict(grid=(128, 128, 128, 20), modes=(12, 12, 12, 8), batch=1),
    dict(grid=(512, 512), modes=(32, 32), c_in=64, c_out=64, batch=8, dtype=1, flags=7),
    dict(grid=(512, 512), modes=(32, 32), c_in=64, c_out=64, batch=8, dtype=2, flags=7),
    dict(grid=(128, 128, 128, 20), modes=(12, 12, 12, 8), batch=1, dtype=2, flags=7),
    dict(grid=(16, 32), modes=(1, 1), c_in=1, c_out=1),
    dict(grid=(256, 256), modes=(16, 16), c_in=32, c_out=32, batch=16, flags=16 | 7),
    dict(grid=(128, 128, 128), modes=(16, 16, 16), c_in=20, c_out=20, batch=2, flags=16),
    dict(grid=(512, 512), modes=(32, 32), c_in=64, c_out=64, batch=8, flags=16 | 7),
    dict(grid=(512, 512), modes=(32, 32), c_in=64, c_out=64, batch=8, flags=32 | 7),
    dict(grid=(512, 512), modes=(32, 32), c_in=64, c_out=64, batch=8, dtype=1, flags=16 | 7),
])
def test_plan_create_host_logic(kw):
    """fno_plan_create runs its whole host-side part (geometry, chunking, workspace sizing,
    float64 table build) before its first HIP call; without a GPU it must then fail cleanly
    with FNO_ERR_HIP, never crash."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: plan creation succeeds instead")
    with pytest.raises(L.FnoError) as ei:
        L.fno_plan_create(_desc(**kw))
    assert ei.value.status == L.FNO_ERR_HIP


@pytest.mark.parametrize("kw", [
    dict(grid=(64, 64), modes=(12, 12), flags=16),           # rows of 64 points
    dict(grid=(256, 1024), modes=(16, 16), flags=16),        # rows of 1024 points
    dict(grid=(256, 256), modes=(16, 33), flags=16),         # more than 32 kept bins
    dict(grid=(256, 256), modes=(14, 16), flags=16),         # m_a not a multiple of 4
])
def test_last_axis_fft_rejected_where_unsupported(kw):
    """A float32 plan that asks for the contiguous-axis FFT outside the shapes it covers is
    refused at creation, before any HIP call."""
    with pytest.raises(L.FnoError) as ei:
        L.fno_plan_create(_desc(**kw))
    assert ei.value.status == L.FNO_ERR_UNSUPPORTED
    assert "LAST_AXIS_FFT" in L.last_error_message()


def test_last_axis_query_null_arguments():
    assert L._lib.fno_plan_last_axis_fft(None, None) == L.FNO_ERR_INVALID_ARGUMENT
