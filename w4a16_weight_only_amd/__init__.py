"""W4A16 weight-only-quantized linear layer for MI355X (gfx950).

Thin Python binding over the C ABI in ``include/w4a16.h`` (``libw4a16.so``,
built in-tree by ``python -m w4a16_weight_only_amd.build``).  The functions here
only check and marshal arguments -- dtype, shape, contiguity, device -- and pass
raw device pointers plus torch's current HIP stream to the library; every step
of the computation runs in the library's HIP kernels.  There is no fallback: if
the library is missing or the tensors are not on the GPU, the call raises.

    out = w4a16_gemm(a, b_packed, scales, qzeros, G, zp_bias=8)
    dst = w4a16_repack(src_nk8, K)
    y   = w4a16_decode_step(stack, x)
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "W4A16Error", "lib", "w4a16_gemm", "w4a16_gemm_noalloc", "w4a16_repack", "w4a16_repack_scales", "w4a16_decode_step",
    "w4a16_decode_workspace_bytes", "w4a16_gemm_glue", "w4a16_gemm_glue_workspace_bytes", "w4a16_rownorm",
    "w4a16_gemm_plan", "w4a16_set_tuning", "w4a16_release", "Linear", "STATUS",
    "GLUE_NONE", "GLUE_RMSNORM", "GLUE_SWIGLU",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16.so")

STATUS = {0: "W4A16_OK", 1: "W4A16_ERR_INVALID_ARG", 2: "W4A16_ERR_UNSUPPORTED",
          3: "W4A16_ERR_HIP", 4: "W4A16_ERR_WORKSPACE"}
GLUE_NONE, GLUE_RMSNORM, GLUE_SWIGLU = 0, 1, 2


class W4A16Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status


class Linear(ctypes.Structure):
    """Mirror of ``w4a16_linear`` (host struct holding device pointers)."""
    _fields_ = [("b_packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("qzeros", ctypes.c_void_p), ("K", ctypes.c_int64), ("N", ctypes.c_int64),
                ("G", ctypes.c_int64), ("zp_bias", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libw4a16.so with argument types declared (raises if unbuilt)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libw4a16.so is not built; run `python -m w4a16_weight_only_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    L.w4a16_status_string.restype = ctypes.c_char_p
    L.w4a16_status_string.argtypes = [ctypes.c_int]
    L.w4a16_last_error.restype = ctypes.c_char_p
    L.w4a16_last_error.argtypes = []
    L.w4a16_repack.restype = ctypes.c_int
    L.w4a16_repack.argtypes = [P, P, I64, I64, P]
    L.w4a16_repack_scales.restype = ctypes.c_int
    L.w4a16_repack_scales.argtypes = [P, P, I64, I64, P]
    L.w4a16_gemm.restype = ctypes.c_int
    L.w4a16_gemm.argtypes = [P, P, P, P, I64, I64, I64, I64, I32, P, P]
    L.w4a16_gemm_noalloc.restype = ctypes.c_int
    L.w4a16_gemm_noalloc.argtypes = [P, P, P, P, I64, I64, I64, I64, I32, P, P]
    L.w4a16_decode_workspace_bytes.restype = SZ
    L.w4a16_decode_workspace_bytes.argtypes = [I64, P, I64]
    L.w4a16_decode_step.restype = ctypes.c_int
    L.w4a16_decode_step.argtypes = [P, I64, P, P, I64, P, SZ, P]
    L.w4a16_gemm_glue_workspace_bytes.restype = SZ
    L.w4a16_gemm_glue_workspace_bytes.argtypes = [ctypes.c_int, I64, P]
    L.w4a16_gemm_glue.restype = ctypes.c_int
    L.w4a16_gemm_glue.argtypes = [ctypes.c_int, P, I64, P, I64, P, P, SZ, P]
    L.w4a16_rownorm.restype = ctypes.c_int
    L.w4a16_rownorm.argtypes = [P, I64, I64, I64, P, P]
    L.w4a16_gemm_plan.restype = ctypes.c_int
    L.w4a16_gemm_plan.argtypes = [I64, I64, I64, I64, ctypes.POINTER(ctypes.c_int32),
                                  ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]
    L.w4a16_release.restype = ctypes.c_int
    L.w4a16_release.argtypes = []
    L.w4a16_set_tuning.restype = ctypes.c_int
    L.w4a16_set_tuning.argtypes = [ctypes.c_char_p]
    _lib = L
    return L


def _check(rc: int) -> None:
    if rc != 0:
        raise W4A16Error(rc, lib().w4a16_last_error().decode())


def _torch():
    import torch
    return torch


def _stream_ptr(dev):
    torch = _torch()
    return torch.cuda.current_stream(dev).cuda_stream


def _dev_tensor(t, name, dtype, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.dim() != ndim:
        raise ValueError("%s must be %d-D, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def w4a16_gemm(a, b_packed, scales, qzeros=None, G=128, zp_bias=8, out=None):
    """out[M, N] fp16 = a[M, K] . ((q - z) * s) with b_packed int32 [K, N/8],
    scales fp16 [K/G, N], qzeros int32 [K/G, N/8] or None (z = zp_bias)."""
    torch = _torch()
    _dev_tensor(a, "a", torch.float16, 2)
    _dev_tensor(b_packed, "b_packed", torch.int32, 2)
    _dev_tensor(scales, "scales", torch.float16, 2)
    M, K = a.shape
    N = b_packed.shape[1] * 8
    if b_packed.shape[0] != K:
        raise ValueError("b_packed must be [K, N/8] = [%d, *], got %s" % (K, tuple(b_packed.shape)))
    if G <= 0 or K % G != 0 or tuple(scales.shape) != (K // G, N):
        raise ValueError("scales must be [K/G, N] = [%d, %d], got %s" % (K // max(G, 1), N, tuple(scales.shape)))
    if qzeros is not None:
        _dev_tensor(qzeros, "qzeros", torch.int32, 2)
        if tuple(qzeros.shape) != (K // G, N // 8):
            raise ValueError("qzeros must be [K/G, N/8] = [%d, %d]" % (K // G, N // 8))
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=a.device)
    else:
        _dev_tensor(out, "out", torch.float16, 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out must be [M, N] = [%d, %d]" % (M, N))
    _check(lib().w4a16_gemm(a.data_ptr(), b_packed.data_ptr(), scales.data_ptr(),
                            None if qzeros is None else qzeros.data_ptr(), M, K, N, G, zp_bias,
                            out.data_ptr(), _stream_ptr(a.device)))
    return out


def w4a16_gemm_noalloc(a, b_packed, scales, qzeros, G, zp_bias, out):
    """w4a16_gemm into a caller-allocated `out`, with the library's split-K
    scratch in its fixed per-GPU array: no allocation at all."""
    torch = _torch()
    _dev_tensor(a, "a", torch.float16, 2)
    _dev_tensor(b_packed, "b_packed", torch.int32, 2)
    _dev_tensor(scales, "scales", torch.float16, 2)
    _dev_tensor(out, "out", torch.float16, 2)
    M, K = a.shape
    N = b_packed.shape[1] * 8
    if b_packed.shape[0] != K or tuple(scales.shape) != (K // G, N) or tuple(out.shape) != (M, N):
        raise ValueError("shapes do not match a [M, K], b_packed [K, N/8], scales [K/G, N], out [M, N]")
    if qzeros is not None:
        _dev_tensor(qzeros, "qzeros", torch.int32, 2)
        if tuple(qzeros.shape) != (K // G, N // 8):
            raise ValueError("qzeros must be [K/G, N/8]")
    _check(lib().w4a16_gemm_noalloc(a.data_ptr(), b_packed.data_ptr(), scales.data_ptr(),
                                    None if qzeros is None else qzeros.data_ptr(), M, K, N, G, zp_bias,
                                    out.data_ptr(), _stream_ptr(a.device)))
    return out


def w4a16_repack(src_nk8, K, out=None):
    """Checkpoint int32 [N, K/8] -> kernel layout int32 [K, N/8] (bit-exact)."""
    torch = _torch()
    _dev_tensor(src_nk8, "src_nk8", torch.int32, 2)
    N = src_nk8.shape[0]
    if src_nk8.shape[1] * 8 != K:
        raise ValueError("src_nk8 must be [N, K/8] with K = %d" % K)
    if out is None:
        out = torch.empty((K, N // 8), dtype=torch.int32, device=src_nk8.device)
    else:
        _dev_tensor(out, "out", torch.int32, 2)
    _check(lib().w4a16_repack(src_nk8.data_ptr(), out.data_ptr(), K, N, _stream_ptr(src_nk8.device)))
    return out


def w4a16_repack_scales(src_ng, out=None):
    """Checkpoint group scales fp16 [N, K/G] -> kernel layout fp16 [K/G, N]
    (bit-exact transpose)."""
    torch = _torch()
    _dev_tensor(src_ng, "src_ng", torch.float16, 2)
    N, Gn = src_ng.shape
    if out is None:
        out = torch.empty((Gn, N), dtype=torch.float16, device=src_ng.device)
    else:
        _dev_tensor(out, "out", torch.float16, 2)
        if tuple(out.shape) != (Gn, N):
            raise ValueError("out must be [K/G, N] = [%d, %d]" % (Gn, N))
    _check(lib().w4a16_repack_scales(src_ng.data_ptr(), out.data_ptr(), Gn, N, _stream_ptr(src_ng.device)))
    return out


def _linear_array(stack):
    """stack: list of dicts with b_packed, scales, qzeros (or None), G, zp_bias."""
    torch = _torch()
    arr = (Linear * len(stack))()
    for i, L in enumerate(stack):
        b, s, qz = L["b_packed"], L["scales"], L.get("qzeros")
        _dev_tensor(b, "b_packed", torch.int32, 2)
        _dev_tensor(s, "scales", torch.float16, 2)
        if qz is not None:
            _dev_tensor(qz, "qzeros", torch.int32, 2)
        arr[i] = Linear(b.data_ptr(), s.data_ptr(), None if qz is None else qz.data_ptr(),
                        b.shape[0], b.shape[1] * 8, L["G"], L.get("zp_bias", 8))
    return arr


def w4a16_decode_workspace_bytes(M, stack):
    if len(stack) % 4 != 0 or not stack:
        raise ValueError("stack must hold 4 linears per layer")
    arr = _linear_array(stack)
    return int(lib().w4a16_decode_workspace_bytes(M, ctypes.cast(arr, ctypes.c_void_p), len(stack) // 4))


def w4a16_decode_step(stack, x, out=None, workspace=None):
    """One decode step through len(stack)//4 layers; x fp16 [M, H] on the GPU."""
    torch = _torch()
    _dev_tensor(x, "x", torch.float16, 2)
    if len(stack) % 4 != 0 or not stack:
        raise ValueError("stack must hold 4 linears per layer")
    M = x.shape[0]
    arr = _linear_array(stack)
    nl = len(stack) // 4
    need = int(lib().w4a16_decode_workspace_bytes(M, ctypes.cast(arr, ctypes.c_void_p), nl))
    if need == 0:
        raise ValueError("malformed stack (shapes do not chain)")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty_like(x)
    _check(lib().w4a16_decode_step(ctypes.cast(arr, ctypes.c_void_p), nl, x.data_ptr(), out.data_ptr(), M,
                                   workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   _stream_ptr(x.device)))
    return out


def _one_linear(linear):
    arr = _linear_array([linear])
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def w4a16_gemm_glue_workspace_bytes(glue, M, linear):
    _keep, ptr = _one_linear(linear)
    return int(lib().w4a16_gemm_glue_workspace_bytes(glue, M, ptr))


def w4a16_gemm_glue(glue, x, linear, ldx=None, out=None, workspace=None):
    """One linear on glue-transformed rows of x (fp16 [M, ldx] on the GPU):
    GLUE_NONE out = x . W, GLUE_RMSNORM out = rn(x[:, :K]) . W, GLUE_SWIGLU
    out = rn(silu(x[:, :K]) * x[:, K:2K]) . W; `linear` is a dict like the
    decode stack's entries."""
    torch = _torch()
    _dev_tensor(x, "x", torch.float16, 2)
    M = x.shape[0]
    ldx = x.shape[1] if ldx is None else ldx
    keep, ptr = _one_linear(linear)
    N = keep[0].N
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _dev_tensor(out, "out", torch.float16, 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out must be [M, N] = [%d, %d]" % (M, N))
    need = int(lib().w4a16_gemm_glue_workspace_bytes(glue, M, ptr))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wptr = None if workspace is None else workspace.data_ptr()
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().w4a16_gemm_glue(glue, x.data_ptr(), ldx, ptr, M, out.data_ptr(), wptr, wbytes,
                                 _stream_ptr(x.device)))
    return out


def w4a16_rownorm(x, width=None, out=None):
    """y = rn(x[:, :width]) (fp16 [M, width]) for fp16 rows x on the GPU."""
    torch = _torch()
    _dev_tensor(x, "x", torch.float16, 2)
    M, ldx = x.shape
    width = ldx if width is None else width
    if out is None:
        out = torch.empty((M, width), dtype=torch.float16, device=x.device)
    else:
        _dev_tensor(out, "out", torch.float16, 2)
    _check(lib().w4a16_rownorm(x.data_ptr(), ldx, M, width, out.data_ptr(), _stream_ptr(x.device)))
    return out


def w4a16_gemm_plan(M, K, N, G):
    """(path, splits, grid) the library would use: path 1 = GEMV, 2 = MFMA."""
    path, splits, grid = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _check(lib().w4a16_gemm_plan(M, K, N, G, ctypes.byref(path), ctypes.byref(splits), ctypes.byref(grid)))
    return path.value, splits.value, grid.value


def w4a16_set_tuning(spec=None):
    """Replace the planner's tuning overrides ("key=value,..."; None restores
    the defaults)."""
    _check(lib().w4a16_set_tuning(spec.encode() if spec else None))


def w4a16_release():
    _check(lib().w4a16_release())
