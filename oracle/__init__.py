"""CPU oracle for the W4A16 weight-only linear layer -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library
(``w4a16_weight_only_amd``) never imports, links or calls it, and the two share
no code: this wrapper loads ``liboracle.so`` built from ``w4a16_oracle.c``
(plain C, fp64 accumulation) with gcc.

Sources: the vLLM PR #37352 write-up (Triton W4A16 kernel for ROCm), section
"Code analysis" item 1 (the dequantize-then-matmul reference formula) and item 2
(checkpoint [N, K/8] -> kernel [K, N/8] repack).  Every function below maps to
one C function whose comment gives the definition it evaluates.

Pins: every function here is pinned by a ``-m "not gpu"`` test against closed
forms, hand-derived cases (``tests/golden``), brute force on tiny inputs,
invariants and numpy reductions -- see ``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4a16_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C99, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
            "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I32 = ctypes.c_int32
        lib.w4o_f16_to_f64.restype = ctypes.c_double
        lib.w4o_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.w4o_f64_to_f16.restype = ctypes.c_uint16
        lib.w4o_f64_to_f16.argtypes = [ctypes.c_double]
        for name in ("w4o_gemm", "w4o_gemm_nk8"):
            f = getattr(lib, name)
            f.restype = ctypes.c_int
            f.argtypes = [P, P, P, P, I64, I64, I64, I64, I32, P, P]
        lib.w4o_gemm_sample.restype = ctypes.c_int
        lib.w4o_gemm_sample.argtypes = [P, P, P, P, I64, I64, I64, I64, I32, P, P, I64, P, P]
        lib.w4o_repack.restype = ctypes.c_int
        lib.w4o_repack.argtypes = [P, P, I64, I64]
        lib.w4o_repack_scales.restype = ctypes.c_int
        lib.w4o_repack_scales.argtypes = [P, P, I64, I64]
        lib.w4o_rownorm.restype = ctypes.c_int
        lib.w4o_rownorm.argtypes = [P, I64, I64, I64, P]
        lib.w4o_swiglu_rownorm.restype = ctypes.c_int
        lib.w4o_swiglu_rownorm.argtypes = [P, I64, I64, P]
        lib.w4o_decode_step.restype = ctypes.c_int
        lib.w4o_decode_step.argtypes = [P, I64, P, P, I64]
        _lib = lib
    return _lib


class _Linear(ctypes.Structure):
    _fields_ = [("b_packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("qzeros", ctypes.c_void_p), ("K", ctypes.c_int64), ("N", ctypes.c_int64),
                ("G", ctypes.c_int64), ("zp_bias", ctypes.c_int32)]


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _u16(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    assert x.dtype == np.uint16, x.dtype
    return x


def _i32(x):
    if x is None:
        return None
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint32:
        x = x.view(np.int32)
    assert x.dtype == np.int32, x.dtype
    return x


def f16_to_f64(h: int) -> float:
    return _load().w4o_f16_to_f64(int(h) & 0xFFFF)


def f64_to_f16(x: float) -> int:
    return int(_load().w4o_f64_to_f16(float(x)))


def gemm(a, b_kn8, scales, qzeros, G, zp_bias=8, want_acc=False):
    """out = a . ((q - z) * s); numpy in/out, fp16 output returned as np.float16."""
    a = _u16(a); b = _i32(b_kn8); s = _u16(scales); qz = _i32(qzeros)
    M, K = a.shape
    N = b.shape[1] * 8
    assert b.shape[0] == K and s.shape == (K // G, N)
    out = np.zeros((M, N), np.uint16)
    acc = np.zeros((M, N), np.float64) if want_acc else None
    rc = _load().w4o_gemm(_ptr(a), _ptr(b), _ptr(s), _ptr(qz), M, K, N, G, zp_bias,
                          _ptr(out), _ptr(acc))
    if rc != 0:
        raise ValueError("oracle gemm rejected the shapes (rc=%d)" % rc)
    out = out.view(np.float16)
    return (out, acc) if want_acc else out


def gemm_nk8(a, b_nk8, scales, qzeros, G, zp_bias=8, want_acc=False):
    """The same product read from the checkpoint layout [N, K/8]."""
    a = _u16(a); b = _i32(b_nk8); s = _u16(scales); qz = _i32(qzeros)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape[1] * 8 == K
    out = np.zeros((M, N), np.uint16)
    acc = np.zeros((M, N), np.float64) if want_acc else None
    rc = _load().w4o_gemm_nk8(_ptr(a), _ptr(b), _ptr(s), _ptr(qz), M, K, N, G, zp_bias,
                              _ptr(out), _ptr(acc))
    if rc != 0:
        raise ValueError("oracle gemm_nk8 rejected the shapes (rc=%d)" % rc)
    out = out.view(np.float16)
    return (out, acc) if want_acc else out


def gemm_sample(a, b_kn8, scales, qzeros, G, zp_bias, m_idx, n_idx):
    """Selected elements of gemm(): returns (fp16 values, fp64 unrounded sums)."""
    a = _u16(a); b = _i32(b_kn8); s = _u16(scales); qz = _i32(qzeros)
    M, K = a.shape
    N = b.shape[1] * 8
    mi = np.ascontiguousarray(m_idx, dtype=np.int64)
    ni = np.ascontiguousarray(n_idx, dtype=np.int64)
    out = np.zeros(mi.shape[0], np.uint16)
    acc = np.zeros(mi.shape[0], np.float64)
    rc = _load().w4o_gemm_sample(_ptr(a), _ptr(b), _ptr(s), _ptr(qz), M, K, N, G, zp_bias,
                                 _ptr(mi), _ptr(ni), mi.shape[0], _ptr(out), _ptr(acc))
    if rc != 0:
        raise ValueError("oracle gemm_sample rejected the arguments (rc=%d)" % rc)
    return out.view(np.float16), acc


def repack(src_nk8, K):
    """Checkpoint [N, K/8] -> kernel [K, N/8], bit-exact (returns int32)."""
    src = _i32(src_nk8)
    N = src.shape[0]
    assert src.shape[1] * 8 == K
    dst = np.zeros((K, N // 8), np.int32)
    rc = _load().w4o_repack(_ptr(src), _ptr(dst), K, N)
    if rc != 0:
        raise ValueError("oracle repack rejected the shapes (rc=%d)" % rc)
    return dst


def repack_scales(src_ng):
    """Checkpoint group scales fp16 [N, K/G] -> kernel layout fp16 [K/G, N]
    (the 16-bit patterns unchanged)."""
    src = _u16(src_ng)
    N, Gn = src.shape
    dst = np.zeros((Gn, N), np.uint16)
    rc = _load().w4o_repack_scales(_ptr(src), _ptr(dst), Gn, N)
    if rc != 0:
        raise ValueError("oracle repack_scales rejected the shapes (rc=%d)" % rc)
    return dst.view(np.float16)


def rownorm(x, width=None):
    x = _u16(x)
    M, ld = x.shape
    width = ld if width is None else width
    y = np.zeros((M, width), np.uint16)
    rc = _load().w4o_rownorm(_ptr(x), M, ld, width, _ptr(y))
    if rc != 0:
        raise ValueError("oracle rownorm rejected the shapes")
    return y.view(np.float16)


def swiglu_rownorm(gu):
    gu = _u16(gu)
    M, two_i = gu.shape
    y = np.zeros((M, two_i // 2), np.uint16)
    rc = _load().w4o_swiglu_rownorm(_ptr(gu), M, two_i // 2, _ptr(y))
    if rc != 0:
        raise ValueError("oracle swiglu_rownorm rejected the shapes")
    return y.view(np.float16)


def decode_step(layers, x, n_layers):
    """layers: list of 4*n_layers dicts with b_packed, scales, qzeros, G, zp_bias."""
    x = _u16(x)
    M, H = x.shape
    keep = []
    arr = (_Linear * (4 * n_layers))()
    for i, L in enumerate(layers):
        b = _i32(L["b_packed"]); s = _u16(L["scales"]); qz = _i32(L.get("qzeros"))
        keep += [b, s, qz]
        arr[i] = _Linear(_ptr(b), _ptr(s), _ptr(qz), b.shape[0], b.shape[1] * 8,
                         L["G"], L.get("zp_bias", 8))
    y = np.zeros((M, H), np.uint16)
    rc = _load().w4o_decode_step(arr, n_layers, _ptr(x), _ptr(y), M)
    if rc != 0:
        raise ValueError("oracle decode_step rejected the stack")
    return y.view(np.float16)


def host_workers():
    """Threads for the parallel helpers: the host's cores, at most 16 (the CPU
    share of one GPU on the test machines)."""
    return max(1, min(16, os.cpu_count() or 1))


def split_columns(b_kn8, scales, qzeros, cols=512):
    """Column slices (each a multiple of 8 columns, the last possibly shorter)
    of the weights, scales and zero points, as contiguous arrays."""
    b = _i32(b_kn8); s = _u16(scales); qz = _i32(qzeros)
    N = b.shape[1] * 8
    edges = list(range(0, N, cols)) + [N]
    return [(np.ascontiguousarray(b[:, c0 // 8:c1 // 8]), np.ascontiguousarray(s[:, c0:c1]),
             None if qz is None else np.ascontiguousarray(qz[:, c0 // 8:c1 // 8]))
            for c0, c1 in zip(edges[:-1], edges[1:])]


def gemm_split(a, parts, G, zp_bias=8, workers=None):
    """gemm() over prepared column slices (split_columns), one thread per
    slice at a time, the slices' outputs side by side.  Each output element is
    computed by the same C function from the same inputs (a column slice is a
    smaller instance of the same definition), so the result is identical to
    one gemm() call; the library releases the GIL while it runs."""
    a = _u16(a)
    with ThreadPoolExecutor(max_workers=workers or host_workers()) as ex:
        outs = list(ex.map(lambda t: gemm(a, t[0], t[1], t[2], G, zp_bias), parts))
    return np.concatenate(outs, axis=1)


def gemm_columns(a, b_kn8, scales, qzeros, G, zp_bias=8, workers=None, cols=512):
    """gemm() evaluated over column slices in parallel threads (identical to
    one gemm() call)."""
    return gemm_split(a, split_columns(b_kn8, scales, qzeros, cols), G, zp_bias, workers)


def decode_layer_columns(layers, x, workers=None):
    """One decode-stack layer (the four linears of decode_step with its glue,
    in the same order and roundings) with each product evaluated by
    gemm_columns.  Equal bit for bit to decode_step(layers, x, 1)."""
    L = layers
    H = x.shape[1]
    q = gemm_columns(x, L[0]["b_packed"], L[0]["scales"], L[0].get("qzeros"), L[0]["G"], L[0].get("zp_bias", 8),
                     workers)
    h = rownorm(q, H)
    o = gemm_columns(h, L[1]["b_packed"], L[1]["scales"], L[1].get("qzeros"), L[1]["G"], L[1].get("zp_bias", 8),
                     workers)
    h = rownorm(o)
    gu = gemm_columns(h, L[2]["b_packed"], L[2]["scales"], L[2].get("qzeros"), L[2]["G"], L[2].get("zp_bias", 8),
                      workers)
    h = swiglu_rownorm(gu)
    d = gemm_columns(h, L[3]["b_packed"], L[3]["scales"], L[3].get("qzeros"), L[3]["G"], L[3].get("zp_bias", 8),
                     workers)
    return rownorm(d)
