"""C-ABI boundary tests that need no GPU.

Every call here is rejected by host-side validation before any HIP call, so it
is safe with or without a device: fake pointers are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import w4a16_weight_only_amd as w4
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "w4a16.h")
OK, INVALID, UNSUPPORTED = 0, 1, 2

# Distinct, 16-byte-aligned fake device addresses (never dereferenced).
A, B, S, Z, O = (ctypes.c_void_p(0x10_0000_0000 + i * 0x1_0000_0000) for i in range(5))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(w4.LIB_PATH):
        import w4a16_weight_only_amd.build as bld
        bld.build()
    return w4.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z_]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("w4a16_repack", "w4a16_gemm", "w4a16_decode_step"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", w4.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (w4a16_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        assert hasattr(lib, n)


def test_set_tuning_changes_the_plan_and_rejects_bad_specs(lib):
    default = w4.w4a16_gemm_plan(1, 4096, 12800, 128)
    try:
        w4.w4a16_set_tuning("gemv_splits=2")
        assert w4.w4a16_gemm_plan(1, 4096, 12800, 128)[1] == 2
        w4.w4a16_set_tuning("gemv_mma=0")
        assert w4.w4a16_gemm_plan(1, 4096, 12800, 128)[0] == 1
        w4.w4a16_set_tuning("gemv_mma=0")
        assert w4.w4a16_gemm_plan(4, 4096, 12800, 128)[0] == 1
        w4.w4a16_set_tuning("gemv_waves=4")  # the matrix-core GEMV runs 8-wave workgroups only
        assert w4.w4a16_gemm_plan(4, 4096, 12800, 128)[0] == 1
        w4.w4a16_set_tuning("gemv_max_m=0")
        assert w4.w4a16_gemm_plan(1, 4096, 12800, 128)[0] == 2
        for bad in ("bogus=1", "gemv_splits", "gemv_splits=x", "gemv_splits=3q"):
            with pytest.raises(RuntimeError):
                w4.w4a16_set_tuning(bad)
            assert w4.w4a16_gemm_plan(1, 4096, 12800, 128)[0] == 2  # unchanged
    finally:
        w4.w4a16_set_tuning(None)
    assert w4.w4a16_gemm_plan(1, 4096, 12800, 128) == default


def test_status_strings(lib):
    for code, name in w4.STATUS.items():
        assert lib.w4a16_status_string(code).decode() == name
    assert lib.w4a16_status_string(99).decode() == "W4A16_ERR_UNKNOWN"


def gemm(lib, a=A, b=B, s=S, z=None, M=1, K=256, N=256, G=64, zp=8, o=O):
    return lib.w4a16_gemm(a, b, s, z, M, K, N, G, zp, o, None)


@pytest.mark.parametrize("kw,status", [
    (dict(a=None), INVALID), (dict(b=None), INVALID), (dict(s=None), INVALID), (dict(o=None), INVALID),
    (dict(M=-1), INVALID), (dict(K=0), INVALID), (dict(N=0), INVALID), (dict(G=0), INVALID),
    (dict(N=260), INVALID),                      # N % 8 != 0
    (dict(K=250, G=64), INVALID),                # K % G != 0
    (dict(G=48, K=240), UNSUPPORTED),            # G % 32 != 0
    (dict(zp=16), INVALID), (dict(zp=-1), INVALID),
    (dict(a=ctypes.c_void_p(A.value + 8)), UNSUPPORTED),   # misaligned
    (dict(z=ctypes.c_void_p(Z.value + 4)), UNSUPPORTED),
    (dict(o=ctypes.c_void_p(A.value + 64)), INVALID),      # out overlaps a
    (dict(o=ctypes.c_void_p(B.value)), INVALID),           # out overlaps b_packed
    (dict(o=ctypes.c_void_p(S.value + 16)), INVALID),      # out overlaps scales
    (dict(z=Z, o=ctypes.c_void_p(Z.value)), INVALID),      # out overlaps qzeros
    (dict(M=1 << 21), UNSUPPORTED),
    (dict(K=1 << 16, N=1 << 17, G=64), UNSUPPORTED),        # packed weights >= 4 GiB
])
def test_gemm_rejects(lib, kw, status):
    assert gemm(lib, **kw) == status
    assert lib.w4a16_last_error().decode() != ""


def test_gemm_m0_is_a_noop(lib):
    # M == 0 returns before any HIP call; a and out may then be NULL.
    assert gemm(lib, M=0) == OK
    assert gemm(lib, M=0, a=None, o=None) == OK
    assert gemm(lib, M=0, b=None) == INVALID


def test_gemm_zp_ignored_with_qzeros(lib):
    # zp_bias out of range is only an error in the symmetric case; with qzeros
    # the call gets past that check (and is then rejected for overlap here).
    assert gemm(lib, z=Z, zp=99, o=ctypes.c_void_p(A.value)) == INVALID
    assert "overlap" in lib.w4a16_last_error().decode()


@pytest.mark.parametrize("K,N,status", [(0, 8, INVALID), (8, 0, INVALID), (12, 8, INVALID),
                                        (8, 12, INVALID), (-8, 8, INVALID)])
def test_repack_rejects_sizes(lib, K, N, status):
    assert lib.w4a16_repack(A, B, K, N, None) == status


def test_repack_rejects_null_and_overlap(lib):
    assert lib.w4a16_repack(None, B, 8, 8, None) == INVALID
    assert lib.w4a16_repack(A, None, 8, 8, None) == INVALID
    assert lib.w4a16_repack(A, ctypes.c_void_p(A.value + 4), 64, 64, None) == INVALID


@pytest.mark.parametrize("Gn,N,status", [(0, 8, INVALID), (4, 0, INVALID), (4, 12, INVALID), (-1, 8, INVALID),
                                          (1 << 22, 1 << 10, UNSUPPORTED)])
def test_repack_scales_rejects_sizes(lib, Gn, N, status):
    assert lib.w4a16_repack_scales(A, B, Gn, N, None) == status


def test_repack_scales_rejects_null_and_overlap(lib):
    assert lib.w4a16_repack_scales(None, B, 4, 8, None) == INVALID
    assert lib.w4a16_repack_scales(A, None, 4, 8, None) == INVALID
    assert lib.w4a16_repack_scales(A, ctypes.c_void_p(A.value + 2), 4, 8, None) == INVALID


def test_gemm_plan_paths(lib):
    # decode GEMV (matrix cores; the dot2 form on request), batched and prefill shapes
    for M in range(1, 9):
        assert w4.w4a16_gemm_plan(M, 4096, 12800, 128)[0] == 3
    assert w4.w4a16_gemm_plan(1, 4096, 12800, 128)[1] == 5  # one round: 50 tiles x 5 splits
    assert w4.w4a16_gemm_plan(9, 4096, 12800, 128)[0] == 2
    assert w4.w4a16_gemm_plan(32, 4096, 12800, 128)[0] == 2
    assert w4.w4a16_gemm_plan(256, 12800, 4096, 128)[0] == 2
    # prefill sizes take the 128 x 128 strip kernel: two K-groups where their grid fits one
    # round of the chip (256 workgroups), else one group at two workgroups per CU (512)
    assert w4.w4a16_gemm_plan(256, 12800, 4096, 128) == (2, 4, 256)
    assert w4.w4a16_gemm_plan(256, 4096, 12800, 128) == (2, 1, 200)
    assert w4.w4a16_gemm_plan(384, 12800, 4096, 128) == (2, 5, 480)
    assert w4.w4a16_gemm_plan(512, 4096, 12800, 128) == (2, 1, 400)
    # below M = 161 the register-direct kernel (32-row wave tiles, 8 K-waves)
    assert w4.w4a16_gemm_plan(160, 12800, 4096, 128) == (2, 3, 240)
    # N % 32 != 0 at small M goes to the MFMA kernel (word-granular loads)
    assert w4.w4a16_gemm_plan(1, 256, 264, 64)[0] == 2
    for shape in [(1, 4096, 12800, 128), (32, 4096, 12800, 128), (256, 12800, 4096, 128),
                  (1, 256, 256, 64), (5, 12800, 4096, 128)]:
        path, splits, grid = w4.w4a16_gemm_plan(*shape)
        assert splits >= 1 and grid >= splits
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_gemm_plan(1, 100, 64, 30)
    assert e.value.status == INVALID


def _stack(K=64, NQ=96, I=128, G=32, layers=1, bad=False):
    arr = (w4.Linear * (4 * layers))()
    shapes = [(K, NQ), (K, K), (K, 2 * I), (I, K)]
    for l in range(layers):
        for j, (k, n) in enumerate(shapes):
            if bad and j == 3:
                k = I + 32
            arr[4 * l + j] = w4.Linear(B.value + 0x100_0000 * (4 * l + j), S.value + 0x100_0000 * (4 * l + j),
                                       None, k, n, G, 8)
    return arr


def test_decode_workspace_bytes(lib):
    arr = _stack()
    nb = lib.w4a16_decode_workspace_bytes(3, ctypes.cast(arr, ctypes.c_void_p), 1)
    # three buffers of 3 x max N (256) fp16, each 256-aligned
    assert nb == 3 * 1536
    assert lib.w4a16_decode_workspace_bytes(3, ctypes.cast(_stack(bad=True), ctypes.c_void_p), 1) == 0
    assert lib.w4a16_decode_workspace_bytes(0, ctypes.cast(arr, ctypes.c_void_p), 1) == 0


def test_decode_step_rejects(lib):
    arr = ctypes.cast(_stack(), ctypes.c_void_p)
    W = ctypes.c_void_p(0x20_0000_0000)
    call = lib.w4a16_decode_step
    assert call(arr, 1, None, O, 3, W, 1 << 20, None) == INVALID
    assert call(arr, 1, A, O, 0, W, 1 << 20, None) == INVALID           # M out of range
    assert call(arr, 1, A, O, 3, W, 100, None) == INVALID               # workspace too small
    assert call(ctypes.cast(_stack(bad=True), ctypes.c_void_p), 1, A, O, 3, W, 1 << 20, None) == INVALID
    assert call(arr, 1, A, O, 3, ctypes.c_void_p(A.value), 1 << 20, None) == INVALID  # overlap
    # glue rows live in registers: H and I at most 32768
    wide = ctypes.cast(_stack(I=32800), ctypes.c_void_p)
    assert lib.w4a16_decode_workspace_bytes(3, wide, 1) == 0
    assert call(wide, 1, A, O, 3, W, 1 << 30, None) == UNSUPPORTED
    assert "32768" in lib.w4a16_last_error().decode()


def test_python_binding_rejects_host_tensors_and_bad_dtypes(lib):
    a = torch.zeros(1, 256, dtype=torch.float16)
    b = torch.zeros(256, 32, dtype=torch.int32)
    s = torch.zeros(4, 256, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        w4.w4a16_gemm(a, b, s, None, 64)
    with pytest.raises(TypeError):
        w4.w4a16_gemm(a.float(), b, s, None, 64)
    with pytest.raises(TypeError):
        w4.w4a16_repack(b.to(torch.int64), 256)


def _linear(K=4096, N=12800, G=128):
    return w4.Linear(B.value, S.value, None, K, N, G, 8)


def test_gemm_glue_workspace_bytes(lib):
    """Glue inside the GEMM needs no scratch: the row-norm in every GEMM path,
    SwiGLU in the GEMV below 3 rows; otherwise M x K fp16 values, 256-aligned."""
    down = _linear(12800, 4096)
    ptr = ctypes.cast(ctypes.pointer(down), ctypes.c_void_p)
    ws = lib.w4a16_gemm_glue_workspace_bytes
    assert ws(w4.GLUE_NONE, 1, ptr) == 0
    assert ws(w4.GLUE_RMSNORM, 1, ptr) == 0 and ws(w4.GLUE_RMSNORM, 32, ptr) == 32 * 12800 * 2
    assert ws(w4.GLUE_SWIGLU, 1, ptr) == 0 and ws(w4.GLUE_SWIGLU, 2, ptr) == 0
    assert ws(w4.GLUE_SWIGLU, 3, ptr) == 3 * 12800 * 2
    assert ws(w4.GLUE_SWIGLU, 32, ptr) == 32 * 12800 * 2
    assert ws(3, 1, ptr) == 0 and ws(w4.GLUE_RMSNORM, 0, ptr) == 0
    try:
        w4.w4a16_set_tuning("decode_fuse=0")  # every glue step a kernel of its own
        assert ws(w4.GLUE_RMSNORM, 1, ptr) == 12800 * 2
        w4.w4a16_set_tuning("decode_rn_mfma=1")  # the MFMA GEMM folds the row-norm
        assert ws(w4.GLUE_RMSNORM, 32, ptr) == 0
    finally:
        w4.w4a16_set_tuning(None)


def test_gemm_glue_rejects(lib):
    lin = _linear(4096, 12800)
    ptr = ctypes.cast(ctypes.pointer(lin), ctypes.c_void_p)
    W = ctypes.c_void_p(0x20_0000_0000)
    call = lib.w4a16_gemm_glue
    assert call(3, A, 4096, ptr, 1, O, None, 0, None) == INVALID                   # bad glue value
    assert call(w4.GLUE_NONE, A, 4104, ptr, 1, O, None, 0, None) == INVALID        # NONE needs ldx == K
    assert call(w4.GLUE_SWIGLU, A, 4096, ptr, 1, O, None, 0, None) == INVALID      # SwiGLU reads 2K
    assert call(w4.GLUE_RMSNORM, A, 4100, ptr, 1, O, None, 0, None) == INVALID     # ldx % 8
    assert call(w4.GLUE_RMSNORM, None, 4096, ptr, 1, O, None, 0, None) == INVALID
    assert call(w4.GLUE_RMSNORM, A, 4096, None, 1, O, None, 0, None) == INVALID
    assert call(w4.GLUE_RMSNORM, A, 4096, ptr, 1, ctypes.c_void_p(A.value + 16), None, 0, None) == INVALID
    assert call(w4.GLUE_SWIGLU, A, 8192, ptr, 32, O, None, 0, None) == INVALID     # needs workspace
    assert call(w4.GLUE_SWIGLU, A, 8192, ptr, 32, O, ctypes.c_void_p(A.value), 1 << 24, None) == INVALID
    assert call(w4.GLUE_RMSNORM, A, 4096, ptr, 32, O, None, 0, None) == INVALID    # M >= 9: row-norm kernel
    assert call(w4.GLUE_RMSNORM, A, 4096, ptr, 0, None, None, 0, None) == OK      # M == 0
    wide = _linear(32800, 4096, 32)
    assert call(w4.GLUE_RMSNORM, A, 32800, ctypes.cast(ctypes.pointer(wide), ctypes.c_void_p), 1, O, W, 1 << 30,
                None) == UNSUPPORTED


def test_rownorm_rejects(lib):
    call = lib.w4a16_rownorm
    assert call(A, 64, 2, 60, O, None) == INVALID              # width % 8
    assert call(A, 56, 2, 64, O, None) == INVALID              # ldx < width
    assert call(None, 64, 2, 64, O, None) == INVALID
    assert call(A, 64, 2, 64, ctypes.c_void_p(A.value + 64), None) == INVALID   # y overlaps x
    assert call(A, 32776, 2, 32776, O, None) == UNSUPPORTED    # wider than the glue kernels take
    assert call(A, 64, 0, 64, None, None) == OK
