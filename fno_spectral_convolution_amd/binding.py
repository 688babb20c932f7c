"""ctypes binding of libfno (argument marshalling only).

Every function of ``include/fno.h`` is exposed under its C name and takes plain integers
for pointers (``tensor.data_ptr()``) and streams (``torch.cuda.current_stream().cuda_stream``).
``Plan`` wraps a plan for torch tensors: it allocates outputs, workspace and save buffers
with torch on the plan's device and forwards pointers; every step of the computation runs
in libfno's HIP kernels.  There is no fallback: if libfno.so is missing or fails to load,
importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import (POINTER, byref, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t,
                    c_uint32, c_void_p)

_HERE = os.path.dirname(os.path.abspath(__file__))
# FNO_LIBRARY names another build of libfno (e.g. the host-sanitized one for CPU checks)
LIB_PATH = os.environ.get("FNO_LIBRARY") or os.path.join(_HERE, "libfno.so")

FNO_OK = 0
FNO_ERR_INVALID_ARGUMENT = 1
FNO_ERR_UNSUPPORTED = 2
FNO_ERR_HIP = 3
FNO_ERR_OUT_OF_MEMORY = 4
FNO_ERR_INTERNAL = 5

FNO_DTYPE_F32 = 0
FNO_DTYPE_BF16 = 1
FNO_DTYPE_F16 = 2

FNO_FLAG_TANH_PREACT = 1
FNO_FLAG_GELU = 2
FNO_FLAG_BIAS = 4
FNO_FLAG_INPUT_GELU = 8
FNO_FLAG_LAST_AXIS_FFT = 16
FNO_FLAG_LAST_AXIS_DENSE = 32

EXPORTS = [
    "fno_plan_validate", "fno_plan_create", "fno_plan_destroy", "fno_plan_query",
    "fno_plan_half_range", "fno_plan_last_axis_fft",
    "fno_spectral_conv_fwd", "fno_spectral_conv_bwd", "fno_block_fwd", "fno_block_fwd_static",
    "fno_block_bwd",
    "fno_block_fwd_mse", "fno_block_bwd_preact", "fno_pointwise_fwd", "fno_mse_workspace_bytes", "fno_mse_grad", "fno_mse_grad_scaled",
    "fno_tucker_order", "fno_tucker_create", "fno_tucker_destroy", "fno_tucker_query",
    "fno_tucker_keep_intermediates", "fno_tucker_save_bytes",
    "fno_tucker_block_fwd", "fno_tucker_block_bwd", "fno_tucker_spectral_conv_fwd",
    "fno_tucker_spectral_conv_bwd", "fno_tucker_block_fwd_mse", "fno_tucker_block_bwd_preact",
    "fno_timing_enable", "fno_timing_select",
    "fno_timing_reset", "fno_timing_count", "fno_timing_get", "fno_status_string",
    "fno_last_error_message",
]


class fno_plan_desc(ctypes.Structure):
    _fields_ = [("ndim", c_int32), ("spectral_dtype", c_int32), ("flags", c_uint32),
                ("reserved", c_int32), ("batch", c_int64), ("c_in", c_int64),
                ("c_out", c_int64), ("n", c_int64 * 4), ("modes", c_int64 * 4)]


class FnoError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {status_string(status)}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libfno.so not built ({LIB_PATH}); run "
                           "`python -m fno_spectral_convolution_amd.build`")
    # torch brings its own HIP runtime; load it first so that libfno's libamdhip64
    # dependency resolves to that same, already loaded runtime (one HIP runtime per process:
    # libfno's kernels then run on torch's streams and memory).
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    sig = {
        "fno_plan_validate": (c_int, [POINTER(fno_plan_desc)]),
        "fno_plan_create": (c_int, [POINTER(fno_plan_desc), POINTER(c_void_p)]),
        "fno_plan_destroy": (c_int, [P]),
        "fno_plan_query": (c_int, [P, POINTER(c_size_t), POINTER(c_size_t), POINTER(c_size_t)]),
        "fno_plan_half_range": (c_int, [P, POINTER(c_int), c_int]),
        "fno_plan_last_axis_fft": (c_int, [P, POINTER(c_int)]),
        "fno_spectral_conv_fwd": (c_int, [P, P, P, P, P, P, c_size_t, P]),
        "fno_spectral_conv_bwd": (c_int, [P, P, P, P, P, P, P, P, c_size_t, P]),
        "fno_block_fwd": (c_int, [P, P, P, P, P, P, P, P, c_size_t, P]),
        "fno_block_fwd_static": (c_int, [P, P, P, P, P, P, P, P]),
        "fno_block_bwd": (c_int, [P, P, P, P, P, P, P, P, P, P, P, P, c_size_t, P]),
        "fno_block_fwd_mse": (c_int, [P, P, P, P, P, P, c_float, P, P, P, P, c_size_t, P]),
        "fno_block_bwd_preact": (c_int, [P, P, P, P, P, P, P, P, P, P, P, P, c_size_t, P]),
        "fno_pointwise_fwd": (c_int, [c_int64, c_int64, c_int64, c_int64, c_int64,
                                      P, P, P, P, P, P, P]),
        "fno_mse_workspace_bytes": (c_int, [c_int64, POINTER(c_size_t)]),
        "fno_mse_grad": (c_int, [c_int64, P, P, P, P, P, c_size_t, P]),
        "fno_mse_grad_scaled": (c_int, [c_int64, P, P, P, P, c_float, P, c_size_t, P]),
        "fno_tucker_order": (c_int, [POINTER(fno_plan_desc), POINTER(c_int32), c_char_p,
                                     c_size_t]),
        "fno_tucker_create": (c_int, [P, POINTER(c_int32), POINTER(c_void_p)]),
        "fno_tucker_destroy": (c_int, [P]),
        "fno_tucker_keep_intermediates": (c_int, [P, c_int]),
        "fno_tucker_save_bytes": (c_int, [P, POINTER(c_size_t)]),
        "fno_tucker_query": (c_int, [P, POINTER(c_size_t), POINTER(c_int64), POINTER(c_int64),
                                     c_char_p, c_size_t]),
        "fno_tucker_block_fwd": (c_int, [P, P, P, POINTER(c_void_p), P, P, P, P, P, c_size_t,
                                         P]),
        "fno_tucker_block_bwd": (c_int, [P, P, P, POINTER(c_void_p), P, P, P, P, P, P,
                                         POINTER(c_void_p), P, P, P, c_size_t, P]),
        "fno_tucker_spectral_conv_fwd": (c_int, [P, P, P, POINTER(c_void_p), P, P, P, c_size_t,
                                                 P]),
        "fno_tucker_spectral_conv_bwd": (c_int, [P, P, P, POINTER(c_void_p), P, P, P, P,
                                                 POINTER(c_void_p), P, c_size_t, P]),
        "fno_tucker_block_fwd_mse": (c_int, [P, P, P, POINTER(c_void_p), P, P, P, c_float, P,
                                             P, P, P, c_size_t, P]),
        "fno_tucker_block_bwd_preact": (c_int, [P, P, P, POINTER(c_void_p), P, P, P, P, P, P,
                                                POINTER(c_void_p), P, P, P, c_size_t, P]),
        "fno_timing_enable": (c_int, [c_int]),
        "fno_timing_select": (c_int, [c_char_p]),
        "fno_timing_reset": (c_int, []),
        "fno_timing_count": (c_int, [POINTER(c_int)]),
        "fno_timing_get": (c_int, [c_int, POINTER(c_char_p), POINTER(c_int64),
                                   POINTER(ctypes.c_double)]),
        "fno_status_string": (c_char_p, [c_int]),
        "fno_last_error_message": (c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def status_string(status: int) -> str:
    return _lib.fno_status_string(status).decode()


def last_error_message() -> str:
    return _lib.fno_last_error_message().decode()


def _check(status: int, where: str):
    if status != FNO_OK:
        raise FnoError(status, where, last_error_message())


def make_desc(batch, c_in, c_out, grid, modes, dtype=FNO_DTYPE_F32, flags=0) -> fno_plan_desc:
    d = fno_plan_desc()
    d.ndim = len(grid)
    d.spectral_dtype = dtype
    d.flags = flags
    d.reserved = 0
    d.batch, d.c_in, d.c_out = batch, c_in, c_out
    for j in range(4):
        d.n[j] = grid[j] if j < len(grid) else 0
        d.modes[j] = modes[j] if j < len(modes) else 0
    return d


# ---- raw C entry points (same names as the header) ----------------------------------------
def fno_plan_validate(desc: fno_plan_desc) -> int:
    return _lib.fno_plan_validate(byref(desc))


def fno_plan_create(desc: fno_plan_desc) -> int:
    out = c_void_p()
    _check(_lib.fno_plan_create(byref(desc), byref(out)), "fno_plan_create")
    return out.value


def fno_plan_destroy(plan: int) -> None:
    _check(_lib.fno_plan_destroy(plan), "fno_plan_destroy")


def fno_plan_query(plan: int):
    ws, sv, we = c_size_t(), c_size_t(), c_size_t()
    _check(_lib.fno_plan_query(plan, byref(ws), byref(sv), byref(we)), "fno_plan_query")
    return ws.value, sv.value, we.value


def fno_plan_half_range(plan: int, clear: bool = False) -> bool:
    """Whether a call on this IEEE-half plan wrote a non-finite output (synchronous read)."""
    v = c_int()
    _check(_lib.fno_plan_half_range(plan, byref(v), int(bool(clear))), "fno_plan_half_range")
    return bool(v.value)


def fno_plan_last_axis_fft(plan: int) -> bool:
    """Whether the plan takes its contiguous-axis forward transform by FFT (host only)."""
    v = c_int()
    _check(_lib.fno_plan_last_axis_fft(plan, byref(v)), "fno_plan_last_axis_fft")
    return bool(v.value)


def fno_spectral_conv_fwd(plan, x, w, y_spec, save, ws, ws_bytes, stream):
    _check(_lib.fno_spectral_conv_fwd(plan, x, w, y_spec, save, ws, ws_bytes, stream),
           "fno_spectral_conv_fwd")


def fno_spectral_conv_bwd(plan, x, w, save, grad_y_spec, grad_x, grad_w, ws, ws_bytes, stream):
    _check(_lib.fno_spectral_conv_bwd(plan, x, w, save, grad_y_spec, grad_x, grad_w, ws,
                                      ws_bytes, stream), "fno_spectral_conv_bwd")


def fno_block_fwd(plan, x, w, w_bypass, bias, y, save, ws, ws_bytes, stream):
    _check(_lib.fno_block_fwd(plan, x, w, w_bypass, bias, y, save, ws, ws_bytes, stream),
           "fno_block_fwd")


def fno_block_fwd_static(plan, x, w, w_bypass, bias, y, save, stream):
    _check(_lib.fno_block_fwd_static(plan, x, w, w_bypass, bias, y, save, stream),
           "fno_block_fwd_static")


def fno_block_bwd(plan, x, w, w_bypass, bias, save, grad_y, grad_x, grad_w, grad_w_bypass,
                  grad_bias, ws, ws_bytes, stream):
    _check(_lib.fno_block_bwd(plan, x, w, w_bypass, bias, save, grad_y, grad_x, grad_w,
                              grad_w_bypass, grad_bias, ws, ws_bytes, stream), "fno_block_bwd")


def fno_block_fwd_mse(plan, x, w, w_bypass, bias, target, grad_scale, grad_z, loss, save, ws,
                      ws_bytes, stream):
    _check(_lib.fno_block_fwd_mse(plan, x, w, w_bypass, bias, target, grad_scale, grad_z, loss,
                                  save, ws, ws_bytes, stream), "fno_block_fwd_mse")


def fno_block_bwd_preact(plan, x, w, w_bypass, bias, save, grad_z, grad_x, grad_w,
                         grad_w_bypass, grad_bias, ws, ws_bytes, stream):
    _check(_lib.fno_block_bwd_preact(plan, x, w, w_bypass, bias, save, grad_z, grad_x, grad_w,
                                     grad_w_bypass, grad_bias, ws, ws_bytes, stream),
           "fno_block_bwd_preact")


def fno_pointwise_fwd(batch, npts, c_in, hidden, c_out, x, w1, b1, w2, b2, y, stream):
    _check(_lib.fno_pointwise_fwd(batch, npts, c_in, hidden, c_out, x, w1, b1, w2, b2, y,
                                  stream), "fno_pointwise_fwd")


def fno_mse_workspace_bytes(n: int) -> int:
    b = c_size_t()
    _check(_lib.fno_mse_workspace_bytes(n, byref(b)), "fno_mse_workspace_bytes")
    return b.value


def fno_mse_grad(n, y, t, grad, loss, ws, ws_bytes, stream):
    _check(_lib.fno_mse_grad(n, y, t, grad, loss, ws, ws_bytes, stream), "fno_mse_grad")


def fno_mse_grad_scaled(n, y, t, grad, loss, grad_scale, ws, ws_bytes, stream):
    _check(_lib.fno_mse_grad_scaled(n, y, t, grad, loss, grad_scale, ws, ws_bytes, stream),
           "fno_mse_grad_scaled")


def fno_timing_enable(enable: bool) -> None:
    _check(_lib.fno_timing_enable(1 if enable else 0), "fno_timing_enable")


def fno_timing_select(name=None) -> None:
    """Time only the launches of kernel `name` (None: every launch)."""
    _check(_lib.fno_timing_select(name.encode() if name else None), "fno_timing_select")


def fno_timing_reset() -> None:
    _check(_lib.fno_timing_reset(), "fno_timing_reset")


def fno_timing_count() -> int:
    n = c_int()
    _check(_lib.fno_timing_count(byref(n)), "fno_timing_count")
    return n.value


def fno_timing_get(index: int):
    name, launches, ms = c_char_p(), c_int64(), ctypes.c_double()
    _check(_lib.fno_timing_get(index, byref(name), byref(launches), byref(ms)), "fno_timing_get")
    return name.value.decode(), launches.value, ms.value


def timing_report() -> dict:
    """{kernel name: (launches, total ms)} of everything recorded since the last reset."""
    return {nm: (n, ms) for nm, n, ms in (fno_timing_get(i) for i in range(fno_timing_count()))}


# ---- torch-facing convenience (allocation + pointer marshalling only) ---------------------
def spectral_dtype(mixed):
    """fno_dtype of a plan: False -> F32, True / "bf16" -> BF16, "f16" -> F16."""
    if mixed is False or mixed is None:
        return FNO_DTYPE_F32
    if mixed is True or mixed == "bf16":
        return FNO_DTYPE_BF16
    if mixed == "f16":
        return FNO_DTYPE_F16
    raise ValueError(f"unknown spectral precision {mixed!r}")


def _ptr(t):
    return None if t is None else t.data_ptr()


class Plan:
    """One FNO block shape.  Tensors are torch tensors on the plan's device: fields float32
    [B, C, *grid], spectral weights complex64 [2^(d-1), Cin, Cout, *modes], bypass float32
    [Cout, Cin], bias float32 [Cout]."""

    def __init__(self, batch, c_in, c_out, grid, modes, mixed=False, tanh=None, gelu=True,
                 bias=True, device=None, input_gelu=False, last_axis=None):
        """mixed: False (fp32 spectral path), True or "bf16" (bfloat16 operands), "f16" (IEEE
        half operands); a mixed plan takes the tanh pre-activation unless tanh says otherwise.
        input_gelu: x is a pre-activation and the block's input is GELU(x).
        last_axis: None (the plan picks), "fft" or "dense": how a float32 plan takes the
        forward transform of the contiguous axis."""
        import torch
        self.torch = torch
        self.device = torch.device(device) if device is not None else torch.device("cuda")
        tanh = bool(mixed) if tanh is None else tanh
        flags = (FNO_FLAG_TANH_PREACT if tanh else 0) | (FNO_FLAG_GELU if gelu else 0) | \
            (FNO_FLAG_BIAS if bias else 0) | (FNO_FLAG_INPUT_GELU if input_gelu else 0)
        if last_axis not in (None, "fft", "dense"):
            raise ValueError(f"last_axis must be None, 'fft' or 'dense', not {last_axis!r}")
        flags |= {None: 0, "fft": FNO_FLAG_LAST_AXIS_FFT,
                  "dense": FNO_FLAG_LAST_AXIS_DENSE}[last_axis]
        self.desc = make_desc(batch, c_in, c_out, tuple(grid), tuple(modes),
                              spectral_dtype(mixed), flags)
        self.batch, self.c_in, self.c_out = batch, c_in, c_out
        self.grid, self.modes = tuple(grid), tuple(modes)
        self.flags = flags
        with torch.cuda.device(self.device):
            self.handle = fno_plan_create(self.desc)
        self.ws_bytes, self.save_bytes, self.weight_elems = fno_plan_query(self.handle)
        self._ws = None

    def close(self):
        if getattr(self, "handle", None):
            fno_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def half_range_exceeded(self, clear=False):
        """IEEE-half plans: whether a call since creation (or the last clear) wrote a
        non-finite output; synchronise the calls' streams first."""
        return fno_plan_half_range(self.handle, clear)

    @property
    def last_axis_fft(self):
        """True when the plan takes its contiguous-axis forward transform by FFT."""
        return fno_plan_last_axis_fft(self.handle)

    # buffers
    def workspace(self):
        if self._ws is None:
            self._ws = self.torch.empty(max(self.ws_bytes, 16), dtype=self.torch.uint8,
                                        device=self.device)
        return self._ws

    def new_save(self):
        return self.torch.empty(max(self.save_bytes, 16), dtype=self.torch.uint8,
                                device=self.device)

    def _field(self, c):
        return self.torch.empty((self.batch, c) + self.grid, dtype=self.torch.float32,
                                device=self.device)

    def _stream(self):
        return self.torch.cuda.current_stream(self.device).cuda_stream

    # entry points
    def spectral_conv_fwd(self, x, w, save=None, out=None):
        y = out if out is not None else self._field(self.c_out)
        ws = self.workspace()
        fno_spectral_conv_fwd(self.handle, x.data_ptr(), w.data_ptr(), y.data_ptr(), _ptr(save),
                              ws.data_ptr(), self.ws_bytes, self._stream())
        return y

    def spectral_conv_bwd(self, x, w, grad_y_spec, save=None, want_x=True, want_w=True):
        gx = self._field(self.c_in) if want_x else None
        gw = self.torch.empty_like(w) if want_w else None
        ws = self.workspace()
        fno_spectral_conv_bwd(self.handle, x.data_ptr(), w.data_ptr(), _ptr(save),
                              grad_y_spec.data_ptr(), _ptr(gx), _ptr(gw), ws.data_ptr(),
                              self.ws_bytes, self._stream())
        return gx, gw

    def block_fwd(self, x, w, wb, bias=None, save=None, out=None):
        y = out if out is not None else self._field(self.c_out)
        ws = self.workspace()
        fno_block_fwd(self.handle, x.data_ptr(), w.data_ptr(), wb.data_ptr(), _ptr(bias),
                      y.data_ptr(), _ptr(save), ws.data_ptr(), self.ws_bytes, self._stream())
        return y

    def block_fwd_static(self, x, w, wb, bias=None, save=None, out=None):
        """block_fwd on libfno's static scratch (no workspace is allocated for it)."""
        y = out if out is not None else self._field(self.c_out)
        fno_block_fwd_static(self.handle, x.data_ptr(), w.data_ptr(), wb.data_ptr(), _ptr(bias),
                             y.data_ptr(), _ptr(save), self._stream())
        return y

    def block_bwd(self, x, w, wb, bias, save, grad_y, want=("x", "w", "wb", "bias"), out=None):
        t = self.torch
        o = out or {}
        # an output is allocated only when the caller passes none for it
        gx = o["x"] if "x" in o else (self._field(self.c_in) if "x" in want else None)
        gw = o["w"] if "w" in o else (t.empty_like(w) if "w" in want else None)
        gwb = o["wb"] if "wb" in o else (t.empty_like(wb) if "wb" in want else None)
        gb = o["bias"] if "bias" in o else (
            t.empty(self.c_out, dtype=t.float32, device=self.device) if "bias" in want
            else None)
        ws = self.workspace()
        fno_block_bwd(self.handle, x.data_ptr(), w.data_ptr(), wb.data_ptr(), _ptr(bias),
                      _ptr(save), grad_y.data_ptr(), _ptr(gx), _ptr(gw), _ptr(gwb), _ptr(gb),
                      ws.data_ptr(), self.ws_bytes, self._stream())
        return {"x": gx, "w": gw, "wb": gwb, "bias": gb}

    def block_fwd_mse(self, x, w, wb, bias, target, grad_scale=1.0, save=None, grad_z=None,
                      loss=None):
        """Block forward fused with the MSE loss; returns (grad_z, loss) (device tensors)."""
        t = self.torch
        gz = grad_z if grad_z is not None else self._field(self.c_out)
        ls = loss if loss is not None else t.empty(1, dtype=t.float32, device=self.device)
        ws = self.workspace()
        fno_block_fwd_mse(self.handle, x.data_ptr(), w.data_ptr(), wb.data_ptr(), _ptr(bias),
                          target.data_ptr(), float(grad_scale), gz.data_ptr(), ls.data_ptr(),
                          _ptr(save), ws.data_ptr(), self.ws_bytes, self._stream())
        return gz, ls

    def block_bwd_preact(self, x, w, wb, bias, save, grad_z, want=("x", "w", "wb", "bias"),
                         out=None):
        """Block backward from the gradient at the pre-activation (block_bwd's outputs)."""
        t = self.torch
        o = out or {}
        # an output is allocated only when the caller passes none for it
        gx = o["x"] if "x" in o else (self._field(self.c_in) if "x" in want else None)
        gw = o["w"] if "w" in o else (t.empty_like(w) if "w" in want else None)
        gwb = o["wb"] if "wb" in o else (t.empty_like(wb) if "wb" in want else None)
        gb = o["bias"] if "bias" in o else (
            t.empty(self.c_out, dtype=t.float32, device=self.device) if "bias" in want
            else None)
        ws = self.workspace()
        fno_block_bwd_preact(self.handle, x.data_ptr(), w.data_ptr(), wb.data_ptr(), _ptr(bias),
                             _ptr(save), grad_z.data_ptr(), _ptr(gx), _ptr(gw), _ptr(gwb),
                             _ptr(gb), ws.data_ptr(), self.ws_bytes, self._stream())
        return {"x": gx, "w": gw, "wb": gwb, "bias": gb}


def _ranks_arr(ranks):
    return (c_int32 * len(ranks))(*[int(r) for r in ranks])


def _ptr_arr(ptrs):
    return (c_void_p * len(ptrs))(*[p if p else None for p in ptrs])


def fno_tucker_order(desc, ranks) -> str:
    """The greedy contraction order of a descriptor and Tucker ranks (host only)."""
    buf = ctypes.create_string_buffer(512)
    _check(_lib.fno_tucker_order(byref(desc), _ranks_arr(ranks), buf, len(buf)),
           "fno_tucker_order")
    return buf.value.decode()


def fno_tucker_create(plan_handle, ranks):
    h = c_void_p()
    _check(_lib.fno_tucker_create(plan_handle, _ranks_arr(ranks), byref(h)), "fno_tucker_create")
    return h.value


def fno_tucker_destroy(handle):
    _check(_lib.fno_tucker_destroy(handle), "fno_tucker_destroy")


def fno_tucker_query(handle, nfactors):
    ws = c_size_t()
    core = c_int64()
    fac = (c_int64 * nfactors)()
    buf = ctypes.create_string_buffer(512)
    _check(_lib.fno_tucker_query(handle, byref(ws), byref(core), fac, buf, len(buf)),
           "fno_tucker_query")
    return ws.value, core.value, list(fac), buf.value.decode()


def fno_tucker_block_fwd(h, x, core, factors, wb, bias, y, save, ws, ws_bytes, stream):
    _check(_lib.fno_tucker_block_fwd(h, x, core, _ptr_arr(factors), wb, bias, y, save, ws,
                                     ws_bytes, stream), "fno_tucker_block_fwd")


def fno_tucker_block_bwd(h, x, core, factors, wb, bias, save, gy, gx, gcore, gfactors, gwb, gb,
                         ws, ws_bytes, stream):
    gf = _ptr_arr(gfactors) if gfactors is not None else None
    _check(_lib.fno_tucker_block_bwd(h, x, core, _ptr_arr(factors), wb, bias, save, gy, gx,
                                     gcore, gf, gwb, gb, ws, ws_bytes, stream),
           "fno_tucker_block_bwd")


def fno_tucker_block_fwd_mse(h, x, core, factors, wb, bias, target, grad_scale, grad_z, loss,
                             save, ws, ws_bytes, stream):
    _check(_lib.fno_tucker_block_fwd_mse(h, x, core, _ptr_arr(factors), wb, bias, target,
                                         grad_scale, grad_z, loss, save, ws, ws_bytes, stream),
           "fno_tucker_block_fwd_mse")


def fno_tucker_block_bwd_preact(h, x, core, factors, wb, bias, save, gz, gx, gcore, gfactors,
                                gwb, gb, ws, ws_bytes, stream):
    gf = _ptr_arr(gfactors) if gfactors is not None else None
    _check(_lib.fno_tucker_block_bwd_preact(h, x, core, _ptr_arr(factors), wb, bias, save, gz,
                                            gx, gcore, gf, gwb, gb, ws, ws_bytes, stream),
           "fno_tucker_block_bwd_preact")


def fno_tucker_spectral_conv_fwd(h, x, core, factors, y, save, ws, ws_bytes, stream):
    _check(_lib.fno_tucker_spectral_conv_fwd(h, x, core, _ptr_arr(factors), y, save, ws,
                                             ws_bytes, stream), "fno_tucker_spectral_conv_fwd")


def fno_tucker_spectral_conv_bwd(h, x, core, factors, save, gys, gx, gcore, gfactors, ws,
                                 ws_bytes, stream):
    gf = _ptr_arr(gfactors) if gfactors is not None else None
    _check(_lib.fno_tucker_spectral_conv_bwd(h, x, core, _ptr_arr(factors), save, gys, gx, gcore,
                                             gf, ws, ws_bytes, stream),
           "fno_tucker_spectral_conv_bwd")


class Tucker:
    """Tucker-factorised spectral weights bound to a ``Plan``: core complex64
    [R_in, R_out, R_0, .., R_{d-1}], factors complex64 [C_in, R_in], [C_out, R_out],
    [2 m_j, R_j] (outer axes), [m_{d-1}, R_{d-1}]."""

    def __init__(self, plan, ranks):
        self.plan = plan
        self.ranks = tuple(int(r) for r in ranks)
        self.nf = len(plan.grid) + 2
        if len(self.ranks) != self.nf:
            raise ValueError(f"need {self.nf} ranks (in, out, one per axis)")
        self.handle = fno_tucker_create(plan.handle, self.ranks)
        self.ws_bytes, self.core_elems, self.factor_elems, self.order = \
            fno_tucker_query(self.handle, self.nf)
        self._ws = None

    def close(self):
        if getattr(self, "handle", None):
            fno_tucker_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def factor_shapes(self):
        p = self.plan
        full = [p.c_in, p.c_out] + [2 * m for m in p.modes[:-1]] + [p.modes[-1]]
        return [(n, r) for n, r in zip(full, self.ranks)]

    def workspace(self):
        if self._ws is None:
            t = self.plan.torch
            self._ws = t.empty(max(self.ws_bytes, 16), dtype=t.uint8, device=self.plan.device)
        return self._ws

    def keep_intermediates(self, keep=True):
        """Keep the forward's weight-step intermediates in the save buffer for the backward
        (save buffers then come from new_save())."""
        _check(_lib.fno_tucker_keep_intermediates(self.handle, 1 if keep else 0),
               "fno_tucker_keep_intermediates")

    @property
    def save_bytes(self):
        b = c_size_t()
        _check(_lib.fno_tucker_save_bytes(self.handle, byref(b)), "fno_tucker_save_bytes")
        return b.value

    def new_save(self):
        t = self.plan.torch
        return t.empty(max(self.save_bytes, 16), dtype=t.uint8, device=self.plan.device)

    def block_fwd(self, x, core, factors, wb, bias=None, save=None, out=None):
        p = self.plan
        y = out if out is not None else p._field(p.c_out)
        ws = self.workspace()
        fno_tucker_block_fwd(self.handle, x.data_ptr(), core.data_ptr(),
                             [f.data_ptr() for f in factors], wb.data_ptr(), _ptr(bias),
                             y.data_ptr(), _ptr(save), ws.data_ptr(), self.ws_bytes,
                             p._stream())
        return y

    def spectral_conv_fwd(self, x, core, factors, save=None, out=None):
        p = self.plan
        y = out if out is not None else p._field(p.c_out)
        ws = self.workspace()
        fno_tucker_spectral_conv_fwd(self.handle, x.data_ptr(), core.data_ptr(),
                                     [f.data_ptr() for f in factors], y.data_ptr(), _ptr(save),
                                     ws.data_ptr(), self.ws_bytes, p._stream())
        return y

    def spectral_conv_bwd(self, x, core, factors, grad_y_spec, save=None, want_x=True,
                          want_w=True):
        """Returns (grad_x, grad_core, grad_factors) (None where not asked)."""
        p = self.plan
        t = p.torch
        gx = p._field(p.c_in) if want_x else None
        gcore = t.empty_like(core) if want_w else None
        gfac = [t.empty_like(f) for f in factors] if want_w else None
        ws = self.workspace()
        fno_tucker_spectral_conv_bwd(self.handle, x.data_ptr(), core.data_ptr(),
                                     [f.data_ptr() for f in factors], _ptr(save),
                                     grad_y_spec.data_ptr(), _ptr(gx), _ptr(gcore),
                                     [_ptr(g) for g in gfac] if gfac is not None else None,
                                     ws.data_ptr(), self.ws_bytes, p._stream())
        return gx, gcore, gfac

    def block_bwd(self, x, core, factors, wb, bias, save, grad_y, want_x=True, want_w=True,
                  out=None):
        """Returns dict(x, core, factors, wb, bias) of gradients (None where not asked)."""
        p = self.plan
        t = p.torch
        o = out or {}
        # an output is allocated only when the caller passes none for it
        gx = o["x"] if "x" in o else (p._field(p.c_in) if want_x else None)
        gcore = o["core"] if "core" in o else (t.empty_like(core) if want_w else None)
        gfac = o["factors"] if "factors" in o else (
            [t.empty_like(f) for f in factors] if want_w else None)
        gwb = o["wb"] if "wb" in o else t.empty_like(wb)
        gb = o["bias"] if "bias" in o else t.empty(p.c_out, dtype=t.float32, device=p.device)
        ws = self.workspace()
        fno_tucker_block_bwd(self.handle, x.data_ptr(), core.data_ptr(),
                             [f.data_ptr() for f in factors], wb.data_ptr(), _ptr(bias),
                             _ptr(save), grad_y.data_ptr(), _ptr(gx), _ptr(gcore),
                             [_ptr(g) for g in gfac] if gfac is not None else None,
                             _ptr(gwb), _ptr(gb), ws.data_ptr(), self.ws_bytes, p._stream())
        return {"x": gx, "core": gcore, "factors": gfac, "wb": gwb, "bias": gb}

    def block_fwd_mse(self, x, core, factors, wb, bias, target, grad_scale=1.0, save=None,
                      grad_z=None, loss=None):
        """block_fwd fused with the MSE loss; returns (grad_z, loss) (device tensors)."""
        p = self.plan
        t = p.torch
        gz = grad_z if grad_z is not None else p._field(p.c_out)
        ls = loss if loss is not None else t.empty(1, dtype=t.float32, device=p.device)
        ws = self.workspace()
        fno_tucker_block_fwd_mse(self.handle, x.data_ptr(), core.data_ptr(),
                                 [f.data_ptr() for f in factors], wb.data_ptr(), _ptr(bias),
                                 target.data_ptr(), float(grad_scale), gz.data_ptr(),
                                 ls.data_ptr(), _ptr(save), ws.data_ptr(), self.ws_bytes,
                                 p._stream())
        return gz, ls

    def block_bwd_preact(self, x, core, factors, wb, bias, save, grad_z, want_x=True,
                         want_w=True, out=None):
        """block_bwd from the gradient at the pre-activation (block_bwd's outputs)."""
        p = self.plan
        t = p.torch
        o = out or {}
        # an output is allocated only when the caller passes none for it
        gx = o["x"] if "x" in o else (p._field(p.c_in) if want_x else None)
        gcore = o["core"] if "core" in o else (t.empty_like(core) if want_w else None)
        gfac = o["factors"] if "factors" in o else (
            [t.empty_like(f) for f in factors] if want_w else None)
        gwb = o["wb"] if "wb" in o else t.empty_like(wb)
        gb = o["bias"] if "bias" in o else t.empty(p.c_out, dtype=t.float32, device=p.device)
        ws = self.workspace()
        fno_tucker_block_bwd_preact(self.handle, x.data_ptr(), core.data_ptr(),
                                    [f.data_ptr() for f in factors], wb.data_ptr(), _ptr(bias),
                                    _ptr(save), grad_z.data_ptr(), _ptr(gx), _ptr(gcore),
                                    [_ptr(g) for g in gfac] if gfac is not None else None,
                                    _ptr(gwb), _ptr(gb), ws.data_ptr(), self.ws_bytes,
                                    p._stream())
        return {"x": gx, "core": gcore, "factors": gfac, "wb": gwb, "bias": gb}


def pointwise(x, w1, b1=None, w2=None, b2=None, out=None):
    """Lift (w2 None) or projection head on a torch field [B, Cin, *grid]."""
    import torch
    batch, cin = x.shape[0], x.shape[1]
    npts = x[0, 0].numel()
    hidden = 0 if w2 is None else w1.shape[0]
    cout = w1.shape[0] if w2 is None else w2.shape[0]
    y = out if out is not None else torch.empty((batch, cout) + tuple(x.shape[2:]),
                                                dtype=torch.float32, device=x.device)
    fno_pointwise_fwd(batch, npts, cin, hidden, cout, x.data_ptr(), w1.data_ptr(), _ptr(b1),
                      _ptr(w2), _ptr(b2), y.data_ptr(),
                      torch.cuda.current_stream(x.device).cuda_stream)
    return y


def mse_grad(y, t, grad=None, loss=None, ws=None, grad_scale=1.0):
    """loss = mean((y - t)^2), grad = grad_scale * 2 (y - t) / n (grad_scale: a static loss
    scale for IEEE-half plans)."""
    import torch
    n = y.numel()
    g = grad if grad is not None else torch.empty_like(y)
    lo = loss if loss is not None else torch.empty(1, dtype=torch.float32, device=y.device)
    nb = fno_mse_workspace_bytes(n)
    w = ws if ws is not None else torch.empty(max(nb, 16), dtype=torch.uint8, device=y.device)
    stream = torch.cuda.current_stream(y.device).cuda_stream
    if grad_scale == 1.0:
        fno_mse_grad(n, y.data_ptr(), t.data_ptr(), g.data_ptr(), lo.data_ptr(), w.data_ptr(),
                     w.numel(), stream)
    else:
        fno_mse_grad_scaled(n, y.data_ptr(), t.data_ptr(), g.data_ptr(), lo.data_ptr(),
                            float(grad_scale), w.data_ptr(), w.numel(), stream)
    return lo, g
