"""The allocation-free GEMM entry point (w4a16_gemm_noalloc) through the C ABI.

It runs the same plans and kernels as w4a16_gemm with the split-K scratch in
the library's fixed per-GPU array, so its output must equal w4a16_gemm's bit
for bit (and the oracle's within the per-element bound), on consecutive calls
of different sizes that share the array, and under graph capture of shapes
the stream has never run.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import w4a16_weight_only_amd as w4
from w4a16_weight_only_amd import synth

pytestmark = pytest.mark.gpu

TOL = 1e-2


def note(msg):
    print(msg, file=sys.stderr, flush=True)


def dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


def check_close(got, want, what):
    g, r = got.astype(np.float64), want.astype(np.float64)
    err = np.abs(g - r)
    note("%s max|err|=%.3g" % (what, err.max()))
    assert np.all(err <= TOL * np.maximum(1.0, np.abs(r))), what


def inputs(M, K, N, G, asym, seed):
    p = synth.problem(M, K, N, G, asym, seed)
    return p, [dev(p["a"]), dev(p["b_packed"]), dev(p["scales"]), dev(p["qzeros"])]


# (first call, second smaller call): the GEMV with K-splits (fixed-point slots
# in the array), the MFMA GEMM with K-splits (fp32 partials and counters), and
# a change of path between the two calls
PAIRS = [((1, 4096, 12800, 128, False), (1, 1024, 2048, 128, False)),
         ((32, 4096, 12800, 128, True), (20, 2048, 4096, 128, True)),
         ((8, 4096, 6144, 128, True), (3, 512, 1024, 64, False)),
         ((64, 4096, 4096, 128, False), (2, 2048, 1024, 128, True)),
         ((256, 2048, 1024, 128, True), (200, 1024, 512, 64, False))]  # the 128 x 128 strip kernel


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_gemm(first, second):
    for i, (M, K, N, G, asym) in enumerate((first, second)):
        path, splits, grid = w4.w4a16_gemm_plan(M, K, N, G)
        note("noalloc call %d M=%d K=%d N=%d G=%d asym=%s path=%d splits=%d" % (i, M, K, N, G, asym, path, splits))
        p, (a, b, s, z) = inputs(M, K, N, G, asym, seed=600 + M + K)
        ref = w4.w4a16_gemm(a, b, s, z, G, 8).cpu().numpy()
        out = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        w4.w4a16_gemm_noalloc(a, b, s, z, G, 8, out)
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16)), "call %d differs from w4a16_gemm" % i
        want = oracle.gemm_columns(p["a"], p["b_packed"], p["scales"], p["qzeros"], G, 8)
        check_close(got, want, "noalloc call %d M=%d" % (i, M))


def test_noalloc_under_capture_of_new_shapes():
    """Shapes this stream has never run, captured: w4a16_gemm would have to
    allocate and refuses; the allocation-free entry point records its kernels,
    and every replay (with eager work between) equals the eager result."""
    M, K, N, G = 48, 4096, 8192, 128
    assert w4.w4a16_gemm_plan(M, K, N, G)[1] > 1
    p, (a, b, s, z) = inputs(M, K, N, G, True, seed=611)
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    w4.w4a16_gemm_noalloc(a, b, s, z, G, 8, out)  # the array's set-up on this device
    eager = out.cpu().numpy()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        w4.w4a16_gemm_noalloc(a, b, s, z, G, 8, out)
    p2, (a2, b2, s2, z2) = inputs(4, 2048, 4096, 128, False, seed=612)
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint16), eager.view(np.uint16)), "replay %d" % rep
        o2 = torch.empty((4, 4096), dtype=torch.float16, device="cuda")
        w4.w4a16_gemm_noalloc(a2, b2, s2, z2, 128, 8, o2)  # eager work sharing the array between replays
        torch.cuda.synchronize()
        assert np.array_equal(o2.cpu().numpy().view(np.uint16),
                              w4.w4a16_gemm(a2, b2, s2, z2, 128, 8).cpu().numpy().view(np.uint16))
    del g
    want = oracle.gemm_columns(p["a"], p["b_packed"], p["scales"], p["qzeros"], G, 8)
    check_close(eager, want, "noalloc captured M=%d" % M)


def test_noalloc_rejects_oversized_scratch():
    """A plan whose scratch exceeds the array (eight K-splits of 32 x 16384
    fp32 partials: 16 MiB) is refused with UNSUPPORTED, naming the sizes;
    w4a16_gemm runs it.  Real tensors, so nothing could go astray even if a
    launch happened."""
    M, K, N, G = 32, 8192, 16384, 128
    p, (a, b, s, z) = inputs(M, K, N, G, False, seed=613)
    out = torch.zeros((M, N), dtype=torch.float16, device="cuda")
    try:
        w4.w4a16_set_tuning("mfma_splits=8")
        assert w4.w4a16_gemm_plan(M, K, N, G)[1] == 8
        with pytest.raises(w4.W4A16Error) as err:
            w4.w4a16_gemm_noalloc(a, b, s, None, G, 8, out)
        assert err.value.status == 2 and "exceeds" in str(err.value)
        ref = w4.w4a16_gemm(a, b, s, None, G, 8).cpu().numpy()
    finally:
        w4.w4a16_set_tuning(None)
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == 0)  # nothing was written
    assert np.all(np.isfinite(ref))
