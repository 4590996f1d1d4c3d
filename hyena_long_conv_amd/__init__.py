"""Hyena order-N forward on MI355X: Python binding of the C ABI in include/hyena.h.

Argument marshalling only: every step of the operator runs in the HIP kernels
of libhyena_mi355x.so.  Tensors are torch CUDA (ROCm) tensors; work is
enqueued on torch's current stream of the tensors' device.  There is no CPU
fallback: without the built library every call raises.

    h    = filter_gen(params, L)          # [N, D, L] fp32
    spec = filter_spectrum(h)             # opaque spectrum, reused across calls
    y    = forward(v, [x1, ..., xN], spec)

    # the block around the operator (projections, short convolutions)
    v, xs = in_projection(u, bp)          # u [B, L, D] -> v, x_n [B, D, L]
    out   = out_projection(y, bp)         # [B, D, L] -> [B, L, D]
    out   = block_forward(u, bp, spec)    # all three in one call
"""
from __future__ import annotations

import ctypes
import os
import re

__all__ = ["HyenaError", "lib", "plan", "filter_gen", "filter_spectrum", "spectrum_export",
           "forward", "forward_static", "forward_workspace_bytes", "spectrum_bytes", "spectrum_workspace_bytes",
           "LIB_PATH", "HEADER_PATH", "header_functions", "PreparedForward", "BlockParams",
           "in_projection", "out_projection", "block_forward", "block_workspace_bytes", "PreparedCall",
           "prepare_in_projection", "prepare_out_projection", "prepare_block_forward", "backward",
           "backward_workspace_bytes", "filter_gen_li", "filter_gen_mr", "forward_fir", "nd_plan",
           "nd_spectrum_bytes", "nd_workspace_bytes", "nd_filter_spectrum", "prepare_nd_forward", "nd_forward"]

# HYENA_LIB names another build of the same library (tuning variants, the
# host-sanitized build of the argument checks); the in-tree build otherwise.
LIB_PATH = os.environ.get("HYENA_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                       "libhyena_mi355x.so")
HEADER_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "hyena.h")

HYENA_FP32, HYENA_BF16 = 0, 1
STATUS = {0: "HYENA_OK", 1: "HYENA_ERR_NULL", 2: "HYENA_ERR_SHAPE", 3: "HYENA_ERR_UNSUPPORTED",
          4: "HYENA_ERR_ALIGN", 5: "HYENA_ERR_WORKSPACE", 6: "HYENA_ERR_ALIAS", 7: "HYENA_ERR_HIP"}


class HyenaError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {STATUS.get(code, code)}")


class FilterParams(ctypes.Structure):
    _fields_ = [("D", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32), ("H", ctypes.c_int32),
                ("W1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("W2", ctypes.c_void_p),
                ("b2", ctypes.c_void_p), ("W3", ctypes.c_void_p), ("b3", ctypes.c_void_p),
                ("alpha", ctypes.c_void_p)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int64), ("M", ctypes.c_int64), ("path", ctypes.c_int32),
                ("n1", ctypes.c_int32), ("n2", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("spec_stride", ctypes.c_int64)]


class BlockParams(ctypes.Structure):
    _fields_ = [("D", ctypes.c_int32), ("N", ctypes.c_int32), ("T", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("W_in", ctypes.c_void_p), ("b_in", ctypes.c_void_p), ("w_short", ctypes.c_void_p),
                ("W_out", ctypes.c_void_p), ("b_out", ctypes.c_void_p)]



def _poison(t):
    """Buffers the binding allocates for the library to fill (outputs,
    spectra, workspaces) start as NaN -- every byte 0xFF -- when HYENA_POISON=1
    is set, so a kernel that reads memory it never wrote shows up as NaN
    instead of passing on stale values.  A test instrument, off by default."""
    if os.environ.get("HYENA_POISON") == "1":
        import torch
        t.fill_(255 if t.dtype == torch.uint8 else float("nan"))
    return t


def _empty(*args, **kw):
    import torch
    return _poison(torch.empty(*args, **kw))


def _empty_like(t):
    import torch
    return _poison(torch.empty_like(t))

_lib = None


def lib() -> ctypes.CDLL:
    """Load libhyena_mi355x.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m hyena_long_conv_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    L.hyena_plan.argtypes = [i64, ctypes.POINTER(PlanInfo)]
    L.hyena_plan.restype = i32
    L.hyena_filter_gen.argtypes = [ctypes.POINTER(FilterParams), i64, vp, vp]
    L.hyena_filter_gen.restype = i32
    L.hyena_spectrum_bytes.argtypes = [i32, i32, i64]
    L.hyena_spectrum_bytes.restype = i64
    L.hyena_spectrum_workspace_bytes.argtypes = [i32, i32, i64]
    L.hyena_spectrum_workspace_bytes.restype = i64
    L.hyena_filter_spectrum.argtypes = [vp, i32, i32, i64, vp, vp, i64, vp]
    L.hyena_filter_spectrum.restype = i32
    L.hyena_spectrum_export.argtypes = [vp, i32, i32, i64, vp, vp]
    L.hyena_spectrum_export.restype = i32
    L.hyena_forward_workspace_bytes.argtypes = [i64, i32, i32, i64, i32]
    L.hyena_forward_workspace_bytes.restype = i64
    L.hyena_forward.argtypes = [vp, ctypes.POINTER(vp), vp, vp, i64, i32, i32, i64, i32, vp, i64, vp]
    L.hyena_forward.restype = i32
    L.hyena_forward_static.argtypes = [vp, ctypes.POINTER(vp), vp, vp, i64, i32, i32, i64, i32, vp]
    L.hyena_forward_static.restype = i32
    bp = ctypes.POINTER(BlockParams)
    L.hyena_in_projection.argtypes = [vp, bp, ctypes.POINTER(vp), i64, i64, i32, vp]
    L.hyena_in_projection.restype = i32
    L.hyena_out_projection.argtypes = [vp, bp, vp, i64, i64, i32, vp]
    L.hyena_out_projection.restype = i32
    L.hyena_block_workspace_bytes.argtypes = [i64, i32, i32, i64, i32]
    L.hyena_block_workspace_bytes.restype = i64
    L.hyena_block_forward.argtypes = [vp, bp, vp, vp, i64, i64, i32, vp, i64, vp]
    L.hyena_block_forward.restype = i32
    L.hyena_backward_workspace_bytes.argtypes = [i64, i32, i32, i64, i32]
    L.hyena_backward_workspace_bytes.restype = i64
    L.hyena_backward.argtypes = [vp, ctypes.POINTER(vp), vp, vp, vp, ctypes.POINTER(vp), vp, i64, i32, i32, i64, i32,
                                 vp, i64, vp]
    L.hyena_backward.restype = i32
    L.hyena_filter_gen_li.argtypes = [vp, vp, i32, i32, i32, i64, vp, vp]
    L.hyena_filter_gen_li.restype = i32
    L.hyena_filter_gen_mr.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    L.hyena_filter_gen_mr.restype = i32
    L.hyena_forward_fir.argtypes = [vp, ctypes.POINTER(vp), vp, i32, vp, i64, i32, i32, i64, i32, vp]
    L.hyena_forward_fir.restype = i32
    L.hyena_plan_ex.argtypes = [i64, i32, ctypes.POINTER(PlanInfo)]
    L.hyena_plan_ex.restype = i32
    L.hyena_spectrum_bytes_ex.argtypes = [i32, i32, i64, i32]
    L.hyena_spectrum_bytes_ex.restype = i64
    L.hyena_spectrum_workspace_bytes_ex.argtypes = [i32, i32, i64, i32]
    L.hyena_spectrum_workspace_bytes_ex.restype = i64
    L.hyena_filter_spectrum_ex.argtypes = [vp, i32, i32, i64, i32, vp, vp, i64, vp]
    L.hyena_filter_spectrum_ex.restype = i32
    L.hyena_spectrum_export_ex.argtypes = [vp, i32, i32, i64, i32, vp, vp]
    L.hyena_spectrum_export_ex.restype = i32
    L.hyena_forward_workspace_bytes_ex.argtypes = [i64, i32, i32, i64, i32, i32]
    L.hyena_forward_workspace_bytes_ex.restype = i64
    L.hyena_forward_ex.argtypes = [vp, ctypes.POINTER(vp), vp, vp, i64, i32, i32, i64, i32, i32, vp, i64, vp]
    L.hyena_forward_ex.restype = i32
    L.hyena_backward_workspace_bytes_ex.argtypes = [i64, i32, i32, i64, i32, i32]
    L.hyena_backward_workspace_bytes_ex.restype = i64
    L.hyena_backward_ex.argtypes = [vp, ctypes.POINTER(vp), vp, vp, vp, ctypes.POINTER(vp), vp, i64, i32, i32, i64,
                                    i32, i32, vp, i64, vp]
    L.hyena_backward_ex.restype = i32
    i64p = ctypes.POINTER(i64)
    L.hyena_nd_plan.argtypes = [i32, i64p, i32, i64p]
    L.hyena_nd_plan.restype = i32
    L.hyena_nd_spectrum_bytes.argtypes = [i32, i32, i64p, i32]
    L.hyena_nd_spectrum_bytes.restype = i64
    L.hyena_nd_workspace_bytes.argtypes = [i64, i32, i64p, i32]
    L.hyena_nd_workspace_bytes.restype = i64
    L.hyena_nd_filter_spectrum.argtypes = [vp, i32, i32, i64p, i32, vp, vp, i64, vp]
    L.hyena_nd_filter_spectrum.restype = i32
    L.hyena_nd_forward.argtypes = [vp, ctypes.POINTER(vp), vp, vp, i64, i32, i32, i32, i64p, i32, i32, i32, vp, i64,
                                   vp]
    L.hyena_nd_forward.restype = i32
    L.hyena_status_str.argtypes = [i32]
    L.hyena_status_str.restype = ctypes.c_char_p
    _lib = L
    return L


def header_functions() -> list[str]:
    """Names of the functions include/hyena.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hyena_[a-z_]+)\s*\(", text)))


def _check(code: int, what: str):
    if code != 0:
        raise HyenaError(code, what)


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need_cuda(t, name, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (ROCm) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


HYENA_CONV_LINEAR, HYENA_CONV_CIRCULAR = 0, 1


def _mode(circular: bool) -> int:
    return HYENA_CONV_CIRCULAR if circular else HYENA_CONV_LINEAR


def plan(L: int, circular: bool = False) -> dict:
    info = PlanInfo()
    _check(lib().hyena_plan_ex(int(L), _mode(circular), ctypes.byref(info)), "hyena_plan")
    return dict(L=info.L, M=info.M, path=("single" if info.path == 1 else "fourstep"),
                n1=info.n1, n2=info.n2, spec_stride=info.spec_stride)


def spectrum_bytes(D: int, N: int, L: int, circular: bool = False) -> int:
    return int(lib().hyena_spectrum_bytes_ex(D, N, L, _mode(circular)))


def spectrum_workspace_bytes(D: int, N: int, L: int, circular: bool = False) -> int:
    return int(lib().hyena_spectrum_workspace_bytes_ex(D, N, L, _mode(circular)))


def forward_workspace_bytes(B: int, D: int, N: int, L: int, io: str = "fp32", circular: bool = False) -> int:
    return int(lib().hyena_forward_workspace_bytes_ex(B, D, N, L, HYENA_FP32 if io == "fp32" else HYENA_BF16,
                                                      _mode(circular)))


def filter_gen(params: dict, L: int, out=None):
    """h[n, d, t] from the implicit-filter weights (torch CUDA fp32 tensors
    W1, W2, W3, alpha and optional b1, b2, b3; ints D, N, K, H)."""
    import torch
    W1 = params["W1"]
    _need_cuda(W1, "W1", torch.float32)
    D, N, K, H = int(params["D"]), int(params["N"]), int(params["K"]), int(params["H"])
    keep = {}
    for k in ("W1", "b1", "W2", "b2", "W3", "b3", "alpha"):
        t = params.get(k)
        if t is not None:
            _need_cuda(t, k, torch.float32)
        keep[k] = t
    p = FilterParams(D, N, K, H, *[_ptr(keep[k]).value for k in ("W1", "b1", "W2", "b2", "W3", "b3", "alpha")])
    h = out if out is not None else _empty((N, D, L), dtype=torch.float32, device=W1.device)
    _need_cuda(h, "h", torch.float32)
    _check(lib().hyena_filter_gen(ctypes.byref(p), int(L), _ptr(h), _stream(h)), "hyena_filter_gen")
    return h


def filter_spectrum(h, out=None, workspace=None, circular: bool = False):
    """Spectrum of the filters h [N, D, L] (fp32), as an opaque uint8 buffer
    (for the linear, zero-padded convolution, or the circular one)."""
    import torch
    _need_cuda(h, "h", torch.float32)
    N, D, L = h.shape
    nbytes = spectrum_bytes(D, N, L, circular)
    if nbytes < 0:
        raise HyenaError(3 if circular else 2, "hyena_spectrum_bytes")
    spec = out if out is not None else _empty(nbytes, dtype=torch.uint8, device=h.device)
    wsb = spectrum_workspace_bytes(D, N, L, circular)
    if workspace is None and wsb > 0:
        workspace = _empty(wsb, dtype=torch.uint8, device=h.device)
    _check(lib().hyena_filter_spectrum_ex(_ptr(h), D, N, L, _mode(circular), _ptr(spec), _ptr(workspace),
                                          workspace.numel() if workspace is not None else 0, _stream(h)),
           "hyena_filter_spectrum")
    spec._hyena_shape = (D, N, L)
    spec._hyena_circular = bool(circular)
    return spec


def spectrum_export(spec, D: int, N: int, L: int, circular: bool | None = None):
    """Natural-order spectrum [N, D, M/2+1] complex64 (unscaled DFT of each
    filter zero-padded to M points; M = L in circular mode)."""
    import torch
    if circular is None:
        circular = getattr(spec, "_hyena_circular", False)
    M = plan(L, circular)["M"]
    out = _empty((N, D, M // 2 + 1, 2), dtype=torch.float32, device=spec.device)
    _check(lib().hyena_spectrum_export_ex(_ptr(spec), D, N, L, _mode(circular), _ptr(out), _stream(out)),
           "hyena_spectrum_export")
    return torch.view_as_complex(out)


class PreparedForward:
    """hyena_forward with its arguments checked and marshalled once: each
    call() is a single C-ABI call on the stream that was current at
    preparation (for loops over fixed buffers, where the per-call Python
    checks would otherwise cost as much as a short kernel)."""

    def __init__(self, v, xs, spec, out=None, workspace=None, circular: bool | None = None):
        import torch
        if circular is None:
            circular = getattr(spec, "_hyena_circular", False)
        if v.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("v must be float32 or bfloat16")
        _need_cuda(v, "v", v.dtype)
        B, D, L = v.shape
        N = len(xs)
        for i, x in enumerate(xs):
            _need_cuda(x, f"x[{i}]", v.dtype)
            if tuple(x.shape) != (B, D, L):
                raise ValueError(f"x[{i}] shape {tuple(x.shape)} != {(B, D, L)}")
        io = HYENA_FP32 if v.dtype == torch.float32 else HYENA_BF16
        y = out if out is not None else _empty_like(v)
        _need_cuda(y, "y", v.dtype)
        wsb = int(lib().hyena_forward_workspace_bytes_ex(B, D, N, L, io, _mode(circular)))
        if workspace is None and wsb > 0:
            workspace = _empty(wsb, dtype=torch.uint8, device=v.device)
        self.y = y
        self._keep = (v, tuple(xs), spec, y, workspace)     # the buffers stay alive while prepared
        self._fn = lib().hyena_forward_ex
        self._args = (_ptr(v), (ctypes.c_void_p * N)(*[x.data_ptr() for x in xs]), _ptr(spec), _ptr(y),
                      B, D, N, L, io, _mode(circular), _ptr(workspace),
                      workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(v))

    def __call__(self):
        code = self._fn(*self._args)
        if code != 0:
            raise HyenaError(code, "hyena_forward")
        return self.y


def forward(v, xs, spec, out=None, workspace=None, circular: bool | None = None):
    """y = z_{N+1} of the order-N Hyena recurrence (v, x_n: [B, D, L] fp32 or bf16).
    The convolution mode defaults to the one the spectrum was built for."""
    return PreparedForward(v, xs, spec, out, workspace, circular)()


def forward_static(v, xs, spec, out):
    """hyena_forward_static: the forward with its four-step intermediate in the
    library's static device scratch (no workspace, no device allocation by the
    library or here: the caller passes the output).  Calls on one GPU share
    that scratch; serialise them (one stream)."""
    import torch
    if v.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("v must be float32 or bfloat16")
    _need_cuda(v, "v", v.dtype)
    _need_cuda(out, "out", v.dtype)
    B, D, L = v.shape
    N = len(xs)
    for i, x in enumerate(xs):
        _need_cuda(x, f"x[{i}]", v.dtype)
        if tuple(x.shape) != (B, D, L):
            raise ValueError(f"x[{i}] shape {tuple(x.shape)} != {(B, D, L)}")
    io = HYENA_FP32 if v.dtype == torch.float32 else HYENA_BF16
    xp = (ctypes.c_void_p * N)(*[x.data_ptr() for x in xs])
    _check(lib().hyena_forward_static(_ptr(v), xp, _ptr(spec), _ptr(out), B, D, N, L, io, _stream(v)),
           "hyena_forward_static")
    return out


# ---------------------------------------------------------------- the block

def _block_struct(bp: dict, io_dtype):
    """BlockParams from a dict of torch CUDA tensors (W_in, W_out in the I/O
    dtype; w_short and optional b_in, b_out fp32) and ints D, N, T."""
    import torch
    for k in ("W_in", "W_out"):
        _need_cuda(bp[k], k, io_dtype)
    _need_cuda(bp["w_short"], "w_short", torch.float32)
    for k in ("b_in", "b_out"):
        if bp.get(k) is not None:
            _need_cuda(bp[k], k, torch.float32)
    return BlockParams(int(bp["D"]), int(bp["N"]), int(bp["T"]), 0, _ptr(bp["W_in"]).value,
                       _ptr(bp.get("b_in")).value, _ptr(bp["w_short"]).value, _ptr(bp["W_out"]).value,
                       _ptr(bp.get("b_out")).value)


def _io_of(t):
    import torch
    if t.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("activations must be float32 or bfloat16")
    return HYENA_FP32 if t.dtype == torch.float32 else HYENA_BF16


def in_projection(u, bp: dict, out=None):
    """u [B, L, D] -> (v, [x_1..x_N]), each [B, D, L] in u's dtype."""
    import torch
    io = _io_of(u)
    _need_cuda(u, "u", u.dtype)
    B, L, D = u.shape
    N = int(bp["N"])
    p = _block_struct(bp, u.dtype)
    streams = out if out is not None else [_empty((B, D, L), dtype=u.dtype, device=u.device)
                                           for _ in range(N + 1)]
    for i, t in enumerate(streams):
        _need_cuda(t, f"stream[{i}]", u.dtype)
    sp = (ctypes.c_void_p * (N + 1))(*[t.data_ptr() for t in streams])
    _check(lib().hyena_in_projection(_ptr(u), ctypes.byref(p), sp, B, L, io, _stream(u)), "hyena_in_projection")
    return streams[0], list(streams[1:])


def out_projection(y, bp: dict, out=None):
    """y [B, D, L] -> [B, L, D] in y's dtype."""
    import torch
    io = _io_of(y)
    _need_cuda(y, "y", y.dtype)
    B, D, L = y.shape
    p = _block_struct(bp, y.dtype)
    o = out if out is not None else _empty((B, L, D), dtype=y.dtype, device=y.device)
    _need_cuda(o, "out", y.dtype)
    _check(lib().hyena_out_projection(_ptr(y), ctypes.byref(p), _ptr(o), B, L, io, _stream(y)),
           "hyena_out_projection")
    return o


def block_workspace_bytes(B: int, D: int, N: int, L: int, io: str = "fp32") -> int:
    return int(lib().hyena_block_workspace_bytes(B, D, N, L, HYENA_FP32 if io == "fp32" else HYENA_BF16))


def block_forward(u, bp: dict, spec, out=None, workspace=None):
    """u [B, L, D] -> [B, L, D]: in-projection, the order-N operator with the
    filters whose spectrum is `spec`, out-projection (one C-ABI call)."""
    import torch
    io = _io_of(u)
    _need_cuda(u, "u", u.dtype)
    B, L, D = u.shape
    N = int(bp["N"])
    p = _block_struct(bp, u.dtype)
    o = out if out is not None else _empty_like(u)
    _need_cuda(o, "out", u.dtype)
    wsb = block_workspace_bytes(B, D, N, L, "fp32" if io == HYENA_FP32 else "bf16")
    if wsb < 0:
        raise HyenaError(2, "hyena_block_workspace_bytes")
    if workspace is None:
        workspace = _empty(wsb, dtype=torch.uint8, device=u.device)
    _check(lib().hyena_block_forward(_ptr(u), ctypes.byref(p), _ptr(spec), _ptr(o), B, L, io, _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(u)),
           "hyena_block_forward")
    return o


class PreparedCall:
    """One C-ABI call with its arguments checked and marshalled once (for
    loops over fixed buffers); keeps the tensors and structs it points to
    alive.  call() returns `result`."""

    def __init__(self, fn, args, keep, result, name):
        self._fn, self._args, self._keep, self.result, self._name = fn, args, keep, result, name

    def __call__(self):
        code = self._fn(*self._args)
        if code != 0:
            raise HyenaError(code, self._name)
        return self.result


def prepare_in_projection(u, bp: dict, streams):
    io = _io_of(u)
    _need_cuda(u, "u", u.dtype)
    B, L, D = u.shape
    p = _block_struct(bp, u.dtype)
    for i, t in enumerate(streams):
        _need_cuda(t, f"stream[{i}]", u.dtype)
    sp = (ctypes.c_void_p * len(streams))(*[t.data_ptr() for t in streams])
    return PreparedCall(lib().hyena_in_projection, (_ptr(u), ctypes.byref(p), sp, B, L, io, _stream(u)),
                        (u, bp, p, sp, tuple(streams)), tuple(streams), "hyena_in_projection")


def prepare_out_projection(y, bp: dict, out):
    io = _io_of(y)
    _need_cuda(y, "y", y.dtype)
    _need_cuda(out, "out", y.dtype)
    B, D, L = y.shape
    p = _block_struct(bp, y.dtype)
    return PreparedCall(lib().hyena_out_projection, (_ptr(y), ctypes.byref(p), _ptr(out), B, L, io, _stream(y)),
                        (y, bp, p, out), out, "hyena_out_projection")


def prepare_block_forward(u, bp: dict, spec, out, workspace):
    io = _io_of(u)
    _need_cuda(u, "u", u.dtype)
    _need_cuda(out, "out", u.dtype)
    B, L, D = u.shape
    p = _block_struct(bp, u.dtype)
    return PreparedCall(lib().hyena_block_forward,
                        (_ptr(u), ctypes.byref(p), _ptr(spec), _ptr(out), B, L, io, _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _stream(u)),
                        (u, bp, p, spec, out, workspace), out, "hyena_block_forward")


# ---------------------------------------------------------------- backward

def backward_workspace_bytes(B: int, D: int, N: int, L: int, io: str = "fp32", circular: bool = False) -> int:
    return int(lib().hyena_backward_workspace_bytes_ex(B, D, N, L, HYENA_FP32 if io == "fp32" else HYENA_BF16,
                                                       _mode(circular)))


def backward(v, xs, spec, gy, workspace=None, circular: bool | None = None):
    """Gradients (gv, [gx_1..gx_N], gh) of a loss with dloss/dy = gy through
    y = forward(v, xs, spec); gh [N, D, L] fp32 summed over the batch.  The
    convolution mode defaults to the one the spectrum was built for."""
    import torch
    if circular is None:
        circular = getattr(spec, "_hyena_circular", False)
    io = _io_of(v)
    _need_cuda(v, "v", v.dtype)
    _need_cuda(gy, "gy", v.dtype)
    B, D, L = v.shape
    N = len(xs)
    for i, t in enumerate(xs):
        _need_cuda(t, f"x[{i}]", v.dtype)
    gv = _empty_like(v)
    gxs = [_empty_like(v) for _ in range(N)]
    gh = _empty((N, D, L), dtype=torch.float32, device=v.device)
    wsb = backward_workspace_bytes(B, D, N, L, "fp32" if io == HYENA_FP32 else "bf16", circular)
    if wsb < 0:
        raise HyenaError(3, "hyena_backward_workspace_bytes")
    if workspace is None:
        workspace = _empty(wsb, dtype=torch.uint8, device=v.device)
    xp = (ctypes.c_void_p * N)(*[t.data_ptr() for t in xs])
    gp = (ctypes.c_void_p * N)(*[t.data_ptr() for t in gxs])
    _check(lib().hyena_backward_ex(_ptr(v), xp, _ptr(spec), _ptr(gy), _ptr(gv), gp, _ptr(gh), B, D, N, L, io,
                                   _mode(circular), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(v)), "hyena_backward")
    return gv, gxs, gh


# ---------------------------------------------------------- filter families

def filter_gen_li(R, lam, D: int, N: int, L: int):
    """Hyena-LI filters h [N, D, L] from R, lam [N*D, S] (fp32 CUDA tensors)."""
    import torch
    _need_cuda(R, "R", torch.float32)
    _need_cuda(lam, "lambda", torch.float32)
    S = R.shape[-1]
    h = _empty((N, D, L), dtype=torch.float32, device=R.device)
    _check(lib().hyena_filter_gen_li(_ptr(R), _ptr(lam), D, N, S, L, _ptr(h), _stream(R)), "hyena_filter_gen_li")
    return h


def filter_gen_mr(hhat, alpha):
    """Hyena-MR filters: hhat [N, D, Lh] damped by exp(-alpha[d] t)."""
    import torch
    _need_cuda(hhat, "hhat", torch.float32)
    _need_cuda(alpha, "alpha", torch.float32)
    N, D, Lh = hhat.shape
    h = _empty_like(hhat)
    _check(lib().hyena_filter_gen_mr(_ptr(hhat), _ptr(alpha), D, N, Lh, _ptr(h), _stream(hhat)),
           "hyena_filter_gen_mr")
    return h


def forward_fir(v, xs, h, out=None):
    """The recurrence with explicit short filters h [N, D, Lh] (fp32), evaluated directly."""
    import torch
    io = _io_of(v)
    _need_cuda(v, "v", v.dtype)
    _need_cuda(h, "h", torch.float32)
    B, D, L = v.shape
    N = len(xs)
    for i, t in enumerate(xs):
        _need_cuda(t, f"x[{i}]", v.dtype)
    y = out if out is not None else _empty_like(v)
    xp = (ctypes.c_void_p * N)(*[t.data_ptr() for t in xs])
    _check(lib().hyena_forward_fir(_ptr(v), xp, _ptr(h), h.shape[-1], _ptr(y), B, D, N, L, io, _stream(v)),
           "hyena_forward_fir")
    return y


# ------------------------------------------------------- grid convolutions

def _dims(dims):
    dims = tuple(int(d) for d in dims)
    return dims, (ctypes.c_int64 * len(dims))(*dims)


def nd_plan(dims, circular: bool = False) -> int:
    """Padded FFT side P of a 2-D or 3-D grid (a cube of side P)."""
    dims, cd = _dims(dims)
    side = ctypes.c_int64(0)
    _check(lib().hyena_nd_plan(len(dims), cd, int(bool(circular)), ctypes.byref(side)), "hyena_nd_plan")
    return int(side.value)


def nd_spectrum_bytes(rows: int, dims, circular: bool = False) -> int:
    dims, cd = _dims(dims)
    return int(lib().hyena_nd_spectrum_bytes(int(rows), len(dims), cd, int(bool(circular))))


def nd_workspace_bytes(rows: int, dims, circular: bool = False) -> int:
    dims, cd = _dims(dims)
    return int(lib().hyena_nd_workspace_bytes(int(rows), len(dims), cd, int(bool(circular))))


def _nd_workspace(rows, dims, circular, device, workspace):
    import torch
    wsb = nd_workspace_bytes(rows, dims, circular)
    if wsb < 0:
        raise HyenaError(3, "hyena_nd_workspace_bytes")
    if workspace is None and wsb > 0:
        workspace = _empty(wsb, dtype=torch.uint8, device=device)
    return workspace, (workspace.numel() * workspace.element_size() if workspace is not None else 0)


def nd_filter_spectrum(kernel, dims, circular: bool = False, out=None, workspace=None):
    """Spectrum of grid kernels [..rows.., extent...] fp32: the extent is
    2*dims-1 per axis (non-circular, index offset + dims - 1) or dims
    (circular).  Leading axes are flattened into kernel rows."""
    import torch
    _need_cuda(kernel, "kernel", torch.float32)
    dims, cd = _dims(dims)
    k = len(dims)
    ext = tuple(dims) if circular else tuple(2 * d - 1 for d in dims)
    if tuple(kernel.shape[-k:]) != ext:
        raise ValueError(f"kernel extent {tuple(kernel.shape[-k:])} != {ext}")
    rows = 1
    for s_ in kernel.shape[:-k]:
        rows *= int(s_)
    nbytes = nd_spectrum_bytes(rows, dims, circular)
    if nbytes < 0:
        raise HyenaError(3, "hyena_nd_spectrum_bytes")
    spec = out if out is not None else _empty(nbytes, dtype=torch.uint8, device=kernel.device)
    workspace, wsb = _nd_workspace(rows, dims, circular, kernel.device, workspace)
    _check(lib().hyena_nd_filter_spectrum(_ptr(kernel), rows, k, cd, int(bool(circular)), _ptr(spec),
                                          _ptr(workspace), wsb, _stream(kernel)), "hyena_nd_filter_spectrum")
    spec._hyena_nd = (dims, bool(circular), rows)
    return spec


def prepare_nd_forward(v, xs, spec, circular: bool | None = None, per_sample: bool = False, out=None,
                       workspace=None):
    """hyena_nd_forward marshalled once (v, x_n: [B, D, dims...] fp32 or bf16)."""
    io = _io_of(v)
    _need_cuda(v, "v", v.dtype)
    if circular is None:
        circular = getattr(spec, "_hyena_nd", (None, False))[1]
    B, D = int(v.shape[0]), int(v.shape[1])
    dims, cd = _dims(v.shape[2:])
    N = len(xs)
    for i, t in enumerate(xs):
        _need_cuda(t, f"x[{i}]", v.dtype)
        if tuple(t.shape) != tuple(v.shape):
            raise ValueError(f"x[{i}] shape {tuple(t.shape)} != {tuple(v.shape)}")
    import torch
    y = out if out is not None else _empty_like(v)
    _need_cuda(y, "y", v.dtype)
    xp = (ctypes.c_void_p * N)(*[t.data_ptr() for t in xs])
    workspace, wsb = _nd_workspace(B * D, dims, circular, v.device, workspace)
    args = (_ptr(v), xp, _ptr(spec), _ptr(y), B, D, N, len(dims), cd, int(bool(circular)), int(bool(per_sample)),
            io, _ptr(workspace), wsb, _stream(v))
    return PreparedCall(lib().hyena_nd_forward, args, (v, tuple(xs), spec, y, xp, cd, workspace), y,
                        "hyena_nd_forward")


def nd_forward(v, xs, spec, circular: bool | None = None, per_sample: bool = False, out=None, workspace=None):
    """y = z_{N+1} of the order-N recurrence with grid convolutions."""
    return prepare_nd_forward(v, xs, spec, circular, per_sample, out, workspace)()
