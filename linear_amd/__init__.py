"""MI355X (gfx950) FP16 linear layer: y = FP16(FP16(x @ weight.T) + b).

Also its bfloat16 form, the unrounded FP32 sums, multi-step epilogue programs,
and the grouped and indexed (per-row expert) contractions.  A thin ctypes
binding over the C ABI of ``liblinear_amd.so`` (declared in
``include/linear_amd.h``).  The functions carry the C entry points' names and
only marshal arguments: every step of the computation runs in the library's
HIP kernels.  PyTorch supplies device memory and the stream.  If the library
is missing the calls raise; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblinear_amd.so")

LINEAR_OK = 0
LINEAR_E_NULL = 1
LINEAR_E_SHAPE = 2
LINEAR_E_STRIDE = 3
LINEAR_E_ALIAS = 4
LINEAR_E_PATH = 5
LINEAR_E_DEVICE = 6
LINEAR_E_LAUNCH = 7
LINEAR_E_EPILOGUE = 8
LINEAR_E_CAPTURE = 9
LINEAR_E_WORKSPACE = 10
LINEAR_E_SCRATCH = 11

# scratch the no-allocation indexed call holds per GPU (include/linear_amd.h)
NOALLOC_SCRATCH_BYTES = 1 << 20

# Epilogue steps (include/linear_amd.h, LINEAR_EPI_*)
EPI_MAX_STEPS = 8
EPI_BIAS = 1
EPI_RESIDUAL = 2
EPI_MUL = 3
EPI_SILU = 4
EPI_GELU_TANH = 5
EPI_GELU_ERF = 6

PATH_AUTO = 0
PATH_GEMM = 1
PATH_SKINNY = 2

ENTRY_POINTS = ("linear_f16", "linear_f16_nobias", "linear_f16_ex", "linear_f16_f32out",
                "linear_bf16", "linear_bf16_nobias", "linear_bf16_ex", "linear_bf16_f32out",
                "linear_f16_epilogue", "linear_bf16_epilogue",
                "linear_f16_grouped", "linear_bf16_grouped", "linear_f16_grouped_f32out", "linear_bf16_grouped_f32out",
                "linear_indexed_workspace_bytes",
                "linear_f16_indexed", "linear_bf16_indexed", "linear_f16_indexed_f32out", "linear_bf16_indexed_f32out",
                "linear_f16_indexed_noalloc",
                "linear_f16_plan", "linear_status_string", "linear_last_hip_error")


class LinearError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__("%s failed: %s (status %d%s)" % (
            what, linear_status_string(code), code,
            ", hip error %d" % _lib().linear_last_hip_error()
            if code in (LINEAR_E_DEVICE, LINEAR_E_LAUNCH) else ""))


class LinearArgumentError(LinearError, ValueError):
    pass


class _Plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("tile_k", ctypes.c_int32), ("threads", ctypes.c_int32), ("vector_io", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("split_n", ctypes.c_int64), ("tile_m2", ctypes.c_int32),
                ("tile_n2", ctypes.c_int32), ("grid2", ctypes.c_int64), ("stages", ctypes.c_int32)]


class _Epilogue(ctypes.Structure):
    _fields_ = [("nsteps", ctypes.c_int32), ("op", ctypes.c_int32 * EPI_MAX_STEPS),
                ("bias", ctypes.c_void_p), ("residual", ctypes.c_void_p), ("ldr", ctypes.c_int64),
                ("mul", ctypes.c_void_p), ("ldm", ctypes.c_int64)]


_LIB = None


def _lib():
    """Load liblinear_amd.so (after torch, so both share one HIP runtime)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("liblinear_amd.so is not built (run `python -m linear_amd.build` or "
                           "__graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.linear_f16.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i64, i64, vp]
    lib.linear_f16.restype = i32
    lib.linear_f16_nobias.argtypes = [vp, i64, vp, i64, vp, i64, i64, i64, i64, vp]
    lib.linear_f16_nobias.restype = i32
    lib.linear_f16_ex.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i64, i64, i32, vp]
    lib.linear_f16_ex.restype = i32
    for name in ("linear_bf16",):
        getattr(lib, name).argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i64, i64, vp]
        getattr(lib, name).restype = i32
    lib.linear_bf16_nobias.argtypes = [vp, i64, vp, i64, vp, i64, i64, i64, i64, vp]
    lib.linear_bf16_nobias.restype = i32
    lib.linear_bf16_ex.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i64, i64, i32, vp]
    lib.linear_bf16_ex.restype = i32
    for name in ("linear_f16_f32out", "linear_bf16_f32out"):
        getattr(lib, name).argtypes = [vp, i64, vp, i64, vp, i64, i64, i64, i64, i32, vp]
        getattr(lib, name).restype = i32
    for name in ("linear_f16_epilogue", "linear_bf16_epilogue"):
        getattr(lib, name).argtypes = [vp, i64, vp, i64, ctypes.POINTER(_Epilogue), vp, i64, i64, i64, i64, i32, vp]
        getattr(lib, name).restype = i32
    for name in ("linear_f16_grouped", "linear_bf16_grouped"):
        getattr(lib, name).argtypes = [vp, i64, i64, vp, i64, vp, vp, i64, i64, i64, i64, i64, i64, i32, vp]
        getattr(lib, name).restype = i32
    for name in ("linear_f16_grouped_f32out", "linear_bf16_grouped_f32out"):
        getattr(lib, name).argtypes = [vp, i64, i64, vp, i64, vp, i64, i64, i64, i64, i64, i64, i32, vp]
        getattr(lib, name).restype = i32
    for name in ("linear_f16_indexed", "linear_bf16_indexed", "linear_f16_indexed_f32out",
                 "linear_bf16_indexed_f32out"):
        getattr(lib, name).argtypes = [vp, i64, vp, i64, i64, vp, vp, i64, i64, i64, i64, i64, vp, i64, vp]
        getattr(lib, name).restype = i32
    lib.linear_f16_indexed_noalloc.argtypes = [vp, i64, vp, i64, i64, vp, vp, i64, i64, i64, i64, i64, vp]
    lib.linear_f16_indexed_noalloc.restype = i32
    lib.linear_indexed_workspace_bytes.argtypes = [i64, i64]
    lib.linear_indexed_workspace_bytes.restype = i64
    lib.linear_f16_plan.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i64, i64, i32,
                                    ctypes.POINTER(_Plan)]
    lib.linear_f16_plan.restype = i32
    lib.linear_status_string.argtypes = [i32]
    lib.linear_status_string.restype = ctypes.c_char_p
    lib.linear_last_hip_error.argtypes = []
    lib.linear_last_hip_error.restype = i32
    _LIB = lib
    return lib


def library_path() -> str:
    return LIB_PATH


def linear_status_string(code: int) -> str:
    return _lib().linear_status_string(int(code)).decode()


def _check(code: int, what: str):
    if code == LINEAR_OK:
        return
    if code in (LINEAR_E_DEVICE, LINEAR_E_LAUNCH):
        raise LinearError(code, what)
    raise LinearArgumentError(code, what)


def _mat(t: torch.Tensor, name: str, dtype=torch.float16):
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.dim() != 2:
        raise ValueError("%s must be 2-D, got shape %s" % (name, tuple(t.shape)))
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("%s must have unit inner stride" % name)
    ld = t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0), 1)
    return t.data_ptr(), ld


def _stream_handle(stream, *tensors):
    """The stream a launch goes to, after checking its tensor arguments: every one
    must be a GPU ('cuda') tensor on the current device, where the library
    launches (a host address handed to a kernel would fault the GPU, so it is
    refused here instead).  stream: a torch stream, a raw handle or None (the
    current stream of that device)."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError("every tensor argument must be on the GPU (a 'cuda' device); got one on %s" % t.device)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensor arguments on two devices: %s and %s" % (dev, t.device))
    if dev is not None and dev.index is not None and dev.index != torch.cuda.current_device():
        raise ValueError("the tensors are on %s but the current device is cuda:%d (the library launches on the "
                         "current device; call under torch.cuda.device(%s))" % (dev, torch.cuda.current_device(), dev))
    if stream is not None:
        sdev = getattr(stream, "device", None)
        if sdev is not None and dev is not None and torch.device(sdev) != dev:
            raise ValueError("the stream belongs to %s but the tensors are on %s" % (sdev, dev))
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    if dev is not None:
        return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    return ctypes.c_void_p(0)


def _prepare(x, weight, b, out, dtype=torch.float16, out_dtype=None):
    out_dtype = out_dtype or dtype
    xp, ldx = _mat(x, "x", dtype)
    wp, ldw = _mat(weight, "weight", dtype)
    M, K = x.shape
    N, K2 = weight.shape
    if K != K2:
        raise ValueError("x is [%d, %d] but weight is [%d, %d]" % (M, K, N, K2))
    bp = None
    if b is not None:
        if b.dtype != dtype or b.dim() != 1 or b.shape[0] != N or (N > 1 and b.stride(0) != 1):
            raise ValueError("b must be a contiguous %s [N] tensor" % dtype)
        bp = b.data_ptr()
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    yp, ldy = _mat(out, "out", out_dtype)
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [%d, %d]" % (M, N))
    return xp, ldx, wp, ldw, bp, out, yp, ldy, M, N, K


def linear_f16(x: torch.Tensor, weight: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """y = FP16(FP16(x @ weight.T) + b) on the GPU (x [M,K], weight [N,K], b [N], float16)."""
    if b is None:
        raise ValueError("linear_f16 needs a bias; use linear_f16_nobias")
    xp, ldx, wp, ldw, bp, out, yp, ldy, M, N, K = _prepare(x, weight, b, out)
    rc = _lib().linear_f16(xp, ldx, wp, ldw, bp, yp, ldy, M, N, K, _stream_handle(stream, x, weight, b, out))
    _check(rc, "linear_f16")
    return out


def linear_f16_nobias(x: torch.Tensor, weight: torch.Tensor, out: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """proj = FP16(x @ weight.T) on the GPU."""
    xp, ldx, wp, ldw, _, out, yp, ldy, M, N, K = _prepare(x, weight, None, out)
    rc = _lib().linear_f16_nobias(xp, ldx, wp, ldw, yp, ldy, M, N, K, _stream_handle(stream, x, weight, out))
    _check(rc, "linear_f16_nobias")
    return out


def linear_f16_ex(x: torch.Tensor, weight: torch.Tensor, b: torch.Tensor | None,
                  out: torch.Tensor | None = None, path: int = PATH_AUTO, stream=None) -> torch.Tensor:
    """linear_f16 with a forced path (PATH_AUTO / PATH_GEMM / PATH_SKINNY) and optional bias."""
    xp, ldx, wp, ldw, bp, out, yp, ldy, M, N, K = _prepare(x, weight, b, out)
    rc = _lib().linear_f16_ex(xp, ldx, wp, ldw, bp, yp, ldy, M, N, K, int(path),
                              _stream_handle(stream, x, weight, b, out))
    _check(rc, "linear_f16_ex")
    return out


def linear_f16_f32out(x: torch.Tensor, weight: torch.Tensor, out: torch.Tensor | None = None,
                      path: int = PATH_AUTO, stream=None) -> torch.Tensor:
    """The unrounded FP32 sums x @ weight.T (float16 operands, float32 output)."""
    xp, ldx, wp, ldw, _, out, yp, ldy, M, N, K = _prepare(x, weight, None, out, torch.float16, torch.float32)
    rc = _lib().linear_f16_f32out(xp, ldx, wp, ldw, yp, ldy, M, N, K, int(path),
                                  _stream_handle(stream, x, weight, out))
    _check(rc, "linear_f16_f32out")
    return out


def linear_bf16(x: torch.Tensor, weight: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
    """y = BF16(BF16(x @ weight.T) + b) (bfloat16 x [M,K], weight [N,K], b [N])."""
    if b is None:
        raise ValueError("linear_bf16 needs a bias; use linear_bf16_nobias")
    xp, ldx, wp, ldw, bp, out, yp, ldy, M, N, K = _prepare(x, weight, b, out, torch.bfloat16)
    rc = _lib().linear_bf16(xp, ldx, wp, ldw, bp, yp, ldy, M, N, K, _stream_handle(stream, x, weight, b, out))
    _check(rc, "linear_bf16")
    return out


def linear_bf16_nobias(x: torch.Tensor, weight: torch.Tensor, out: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """proj = BF16(x @ weight.T)."""
    xp, ldx, wp, ldw, _, out, yp, ldy, M, N, K = _prepare(x, weight, None, out, torch.bfloat16)
    rc = _lib().linear_bf16_nobias(xp, ldx, wp, ldw, yp, ldy, M, N, K, _stream_handle(stream, x, weight, out))
    _check(rc, "linear_bf16_nobias")
    return out


def linear_bf16_ex(x: torch.Tensor, weight: torch.Tensor, b: torch.Tensor | None,
                   out: torch.Tensor | None = None, path: int = PATH_AUTO, stream=None) -> torch.Tensor:
    """linear_bf16 with a forced path and optional bias."""
    xp, ldx, wp, ldw, bp, out, yp, ldy, M, N, K = _prepare(x, weight, b, out, torch.bfloat16)
    rc = _lib().linear_bf16_ex(xp, ldx, wp, ldw, bp, yp, ldy, M, N, K, int(path),
                               _stream_handle(stream, x, weight, b, out))
    _check(rc, "linear_bf16_ex")
    return out


def linear_bf16_f32out(x: torch.Tensor, weight: torch.Tensor, out: torch.Tensor | None = None,
                       path: int = PATH_AUTO, stream=None) -> torch.Tensor:
    """The unrounded FP32 sums x @ weight.T (bfloat16 operands, float32 output)."""
    xp, ldx, wp, ldw, _, out, yp, ldy, M, N, K = _prepare(x, weight, None, out, torch.bfloat16, torch.float32)
    rc = _lib().linear_bf16_f32out(xp, ldx, wp, ldw, yp, ldy, M, N, K, int(path),
                                   _stream_handle(stream, x, weight, out))
    _check(rc, "linear_bf16_f32out")
    return out


def _epilogue_call(fn_name, dtype, x, weight, ops, bias, residual, mul, out, path, stream):
    ops = [int(o) for o in ops]
    if len(ops) > EPI_MAX_STEPS:
        raise ValueError("at most %d epilogue steps" % EPI_MAX_STEPS)
    xp, ldx, wp, ldw, _, out, yp, ldy, M, N, K = _prepare(x, weight, None, out, dtype)
    ep = _Epilogue()
    ep.nsteps = len(ops)
    for i, o in enumerate(ops):
        ep.op[i] = o
    if bias is not None:
        if bias.dtype != dtype or bias.dim() != 1 or bias.shape[0] != N or (N > 1 and bias.stride(0) != 1):
            raise ValueError("bias must be a contiguous %s [N] tensor" % dtype)
        ep.bias = bias.data_ptr()
    for name, t in (("residual", residual), ("mul", mul)):
        if t is None:
            continue
        tp, ld = _mat(t, name, dtype)
        if tuple(t.shape) != (M, N):
            raise ValueError("%s must be [%d, %d]" % (name, M, N))
        setattr(ep, name, tp)
        setattr(ep, "ldr" if name == "residual" else "ldm", ld)
    rc = getattr(_lib(), fn_name)(xp, ldx, wp, ldw, ctypes.byref(ep), yp, ldy, M, N, K, int(path),
                                  _stream_handle(stream, x, weight, bias, residual, mul, out))
    _check(rc, fn_name)
    return out


def linear_f16_epilogue(x: torch.Tensor, weight: torch.Tensor, ops, bias=None, residual=None, mul=None,
                        out: torch.Tensor | None = None, path: int = PATH_AUTO, stream=None) -> torch.Tensor:
    """The projection followed by the epilogue steps `ops` (EPI_*), each rounded to binary16.
    bias [N], residual and mul [M, N] as the steps need them; out may be the residual itself."""
    return _epilogue_call("linear_f16_epilogue", torch.float16, x, weight, ops, bias, residual, mul, out, path,
                          stream)


def linear_bf16_epilogue(x: torch.Tensor, weight: torch.Tensor, ops, bias=None, residual=None, mul=None,
                         out: torch.Tensor | None = None, path: int = PATH_AUTO, stream=None) -> torch.Tensor:
    """linear_f16_epilogue on bfloat16 operands, inputs and output."""
    return _epilogue_call("linear_bf16_epilogue", torch.bfloat16, x, weight, ops, bias, residual, mul, out, path,
                          stream)


def _grouped_call(dtype, x, weight, b, out, f32, path, stream):
    """x [G, M, K] (inner two dims row-major), weight [G*N, K], b [G*N] or None."""
    if x.dtype != dtype or weight.dtype != dtype:
        raise TypeError("x and weight must be %s" % dtype)
    if x.dim() != 3 or weight.dim() != 2:
        raise ValueError("x must be [G, M, K] and weight [G*N, K]")
    G, M, K = x.shape
    if G == 0 or weight.shape[0] % max(G, 1) != 0 or weight.shape[1] != K:
        raise ValueError("weight must be [G*N, %d] for G = %d" % (K, G))
    N = weight.shape[0] // G
    if (K > 1 and x.stride(2) != 1) or (K > 1 and weight.stride(1) != 1):
        raise ValueError("x and weight need unit inner stride")
    ldx = x.stride(1) if M > 1 else max(K, x.stride(1), 1)
    sx = x.stride(0)
    ldw = weight.stride(0) if weight.shape[0] > 1 else max(K, 1)
    out_dtype = torch.float32 if f32 else dtype
    if out is None:
        out = torch.empty((G, M, N), dtype=out_dtype, device=x.device)
    if out.dtype != out_dtype or tuple(out.shape) != (G, M, N) or (N > 1 and out.stride(2) != 1):
        raise ValueError("out must be a %s [%d, %d, %d] tensor with unit inner stride" % (out_dtype, G, M, N))
    ldy = out.stride(1) if M > 1 else max(N, out.stride(1), 1)
    sy = out.stride(0)
    bp = None
    if b is not None:
        if f32:
            raise ValueError("the FP32-output grouped call takes no bias")
        if b.dtype != dtype or b.dim() != 1 or b.shape[0] != G * N or (G * N > 1 and b.stride(0) != 1):
            raise ValueError("b must be a contiguous %s [G*N] tensor" % dtype)
        bp = b.data_ptr()
    tag = "bf16" if dtype == torch.bfloat16 else "f16"
    if f32:
        name = "linear_%s_grouped_f32out" % tag
        rc = getattr(_lib(), name)(x.data_ptr(), ldx, sx, weight.data_ptr(), ldw, out.data_ptr(), ldy, sy, G, M, N,
                                   K, int(path), _stream_handle(stream, x, weight, out))
    else:
        name = "linear_%s_grouped" % tag
        rc = getattr(_lib(), name)(x.data_ptr(), ldx, sx, weight.data_ptr(), ldw, bp, out.data_ptr(), ldy, sy, G, M,
                                   N, K, int(path), _stream_handle(stream, x, weight, b, out))
    _check(rc, name)
    return out


def linear_f16_grouped(x, weight, b=None, out=None, path: int = PATH_AUTO, stream=None):
    """Grouped contraction: x [G, M, K] against weight [G*N, K] read as G blocks of N rows."""
    return _grouped_call(torch.float16, x, weight, b, out, False, path, stream)


def linear_bf16_grouped(x, weight, b=None, out=None, path: int = PATH_AUTO, stream=None):
    return _grouped_call(torch.bfloat16, x, weight, b, out, False, path, stream)


def linear_f16_grouped_f32out(x, weight, out=None, path: int = PATH_AUTO, stream=None):
    return _grouped_call(torch.float16, x, weight, None, out, True, path, stream)


def linear_bf16_grouped_f32out(x, weight, out=None, path: int = PATH_AUTO, stream=None):
    return _grouped_call(torch.bfloat16, x, weight, None, out, True, path, stream)


def indexed_workspace_bytes(E: int, M: int) -> int:
    """Bytes of device workspace an indexed call with E experts and M rows needs."""
    n = _lib().linear_indexed_workspace_bytes(E, M)
    if n < 0:
        raise ValueError("E=%d, M=%d out of range" % (E, M))
    return n


def _indexed_args(dtype, x, w, idx, out, f32):
    """Checks and marshalling shared by the indexed calls: x [M, K], w [E, K, N]
    (inner two dims row-major), idx [M] int32.  Returns (out, pointer/stride/shape
    arguments of the C call up to K)."""
    if x.dtype != dtype or w.dtype != dtype:
        raise TypeError("x and w must be %s" % dtype)
    if idx.dtype != torch.int32 or idx.dim() != 1 or (idx.shape[0] > 1 and idx.stride(0) != 1):
        raise TypeError("idx must be a contiguous int32 [M] tensor")
    xp, ldx = _mat(x, "x", dtype)
    if w.dim() != 3:
        raise ValueError("w must be [E, K, N]")
    E, K, N = w.shape
    M = x.shape[0]
    if x.shape[1] != K or idx.shape[0] != M:
        raise ValueError("x is %s, w is %s, idx is %s" % (tuple(x.shape), tuple(w.shape), tuple(idx.shape)))
    if N > 1 and w.stride(2) != 1:
        raise ValueError("w needs unit inner stride")
    ldw = w.stride(1) if K > 1 else max(N, w.stride(1), 1)
    sw = w.stride(0) if E > 1 else max(K * ldw, w.stride(0), 1)
    out_dtype = torch.float32 if f32 else dtype
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    yp, ldy = _mat(out, "out", out_dtype)
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [%d, %d]" % (M, N))
    return out, (xp, ldx, w.data_ptr(), ldw, sw, idx.data_ptr(), yp, ldy, E, M, N, K)


def _indexed_call(dtype, x, w, idx, out, f32, stream, workspace):
    out, args = _indexed_args(dtype, x, w, idx, out, f32)
    E, M = args[8], args[9]
    need = indexed_workspace_bytes(E, M)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    elif workspace.dtype != torch.uint8 or workspace.dim() != 1 or workspace.numel() < need:
        raise ValueError("workspace must be a uint8 tensor of at least %d bytes" % need)
    tag = "bf16" if dtype == torch.bfloat16 else "f16"
    name = "linear_%s_indexed%s" % (tag, "_f32out" if f32 else "")
    rc = getattr(_lib(), name)(*args, workspace.data_ptr(), workspace.numel(),
                               _stream_handle(stream, x, w, idx, out, workspace))
    _check(rc, name)
    return out


def linear_f16_indexed_noalloc(x, w, idx, out, stream=None):
    """linear_f16_indexed without a workspace, for callers that cannot allocate: the
    library's per-GPU scratch array (NOALLOC_SCRATCH_BYTES) holds the routing.
    out must be given (a [M, N] binary16 tensor; this call allocates nothing).
    Calls in flight at once on one GPU share that array and race."""
    if out is None:
        raise ValueError("out is required: the no-allocation call creates no tensor")
    out, args = _indexed_args(torch.float16, x, w, idx, out, False)
    rc = _lib().linear_f16_indexed_noalloc(*args, _stream_handle(stream, x, w, idx, out))
    _check(rc, "linear_f16_indexed_noalloc")
    return out


def linear_f16_indexed(x, w, idx, out=None, stream=None, workspace=None):
    """Indexed contraction: row m of x against expert table w[idx[m]] ([K, N]); rows whose
    idx has no expert keep out's contents.  workspace: a uint8 device tensor of at least
    indexed_workspace_bytes(E, M) bytes (allocated per call when None)."""
    return _indexed_call(torch.float16, x, w, idx, out, False, stream, workspace)


def linear_bf16_indexed(x, w, idx, out=None, stream=None, workspace=None):
    return _indexed_call(torch.bfloat16, x, w, idx, out, False, stream, workspace)


def linear_f16_indexed_f32out(x, w, idx, out=None, stream=None, workspace=None):
    return _indexed_call(torch.float16, x, w, idx, out, True, stream, workspace)


def linear_bf16_indexed_f32out(x, w, idx, out=None, stream=None, workspace=None):
    return _indexed_call(torch.bfloat16, x, w, idx, out, True, stream, workspace)


def linear_f16_plan(x: torch.Tensor, weight: torch.Tensor, b: torch.Tensor | None = None,
                    out: torch.Tensor | None = None, path: int = PATH_AUTO) -> dict:
    """The kernel and tile a call would use (host only): path, tile_m/tile_n/tile_k,
    threads, vector_io, grid; for a GEMM split by columns into two launches also
    split_n (the second launch's first column), tile_m2/tile_n2 and grid2."""
    if out is None:
        out = torch.empty((x.shape[0], weight.shape[0]), dtype=torch.float16, device="meta")
        yp, ldy = 0x100000000, max(weight.shape[0], 1)
    else:
        yp, ldy = _mat(out, "out", out.dtype)
    xp, ldx = _mat(x, "x", x.dtype)
    wp, ldw = _mat(weight, "weight", weight.dtype)
    p = _Plan()
    rc = _lib().linear_f16_plan(xp, ldx, wp, ldw, None if b is None else b.data_ptr(), yp, ldy,
                                x.shape[0], weight.shape[0], x.shape[1], int(path), ctypes.byref(p))
    _check(rc, "linear_f16_plan")
    return {f: getattr(p, f) for f, _ in _Plan._fields_}


def linear(x: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor | None = None,
           out: torch.Tensor | None = None) -> torch.Tensor:
    """Convenience: the bias call when a bias is given, the projection alone otherwise;
    float16 or bfloat16 by x's dtype."""
    if x.dtype == torch.bfloat16:
        if bias is None:
            return linear_bf16_nobias(x, weight, out=out)
        return linear_bf16(x, weight, bias, out=out)
    if bias is None:
        return linear_f16_nobias(x, weight, out=out)
    return linear_f16(x, weight, bias, out=out)
