"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Acceptance for fp16 outputs: max |gpu - oracle| <= 1e-2 * max(1, |oracle|) per
element (fp32 accumulation on the GPU, fp64 in the oracle).  Repack is checked
bit for bit.  Inputs come from the seeded generators in
w4a16_weight_only_amd.synth, identical bytes on both sides.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import w4a16_weight_only_amd as w4
from tests._fixtures import pack_rows, unpack_rows
from w4a16_weight_only_amd import synth

pytestmark = pytest.mark.gpu

TOL = 1e-2


def note(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    w4.lib()  # raises if libw4a16.so is missing: no fallback
    yield
    torch.cuda.synchronize()


def dev(x):
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    return t.cpu().numpy()


def check_close(got, want, what="", tol=TOL):
    g = got.astype(np.float64)
    r = want.astype(np.float64)
    err = np.abs(g - r)
    bound = tol * np.maximum(1.0, np.abs(r))
    worst = np.unravel_index(np.argmax(err / bound), err.shape) if err.size else None
    ulp = np.abs(got.view(np.uint16).astype(np.int64) - want.view(np.uint16).astype(np.int64))
    note("%s max|err|=%.3g max ulp=%d" % (what, err.max() if err.size else 0, ulp.max() if ulp.size else 0))
    assert np.all(err <= bound), "%s: worst at %s got %r want %r" % (what, worst, g[worst], r[worst])


def run_gemm(p, qzeros=True, b_key="b_packed"):
    qz = p["qzeros"] if qzeros else None
    out = w4.w4a16_gemm(dev(p["a"]), dev(p[b_key]), dev(p["scales"]), dev(qz), p["G"], p["zp_bias"])
    torch.cuda.synchronize()
    return host(out)


# ----------------------------------------------------------------- repack ---

@pytest.mark.parametrize("K,N", [(8, 8), (64, 32), (256, 1024), (1024, 136), (264, 520), (4096, 12800)])
def test_repack_bit_exact(K, N):
    note("repack K=%d N=%d" % (K, N))
    src = synth.packed_words(synth.rng(K + 3 * N), N, K // 8)
    want = oracle.repack(src, K)
    s = dev(src)
    outs = [host(w4.w4a16_repack(s, K)) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs:
        assert np.array_equal(o, want)


# ------------------------------------------------------ small full-output ---

def small_cases():
    cases = []
    for M in range(1, 9):  # GEMV path: tiles of 256 columns, ragged last tile
        cases.append((M, 512, 544, 128, M % 2 == 0))
    cases += [(1, 256, 256, 64, False), (2, 1024, 256, 1024, True), (3, 4096, 1024, 128, False),
              (1, 512, 544, 32, False), (6, 256, 288, 32, True)]  # smallest group size on the GEMV path
    # N = 18432 and 18464: the matrix-core GEMV takes 512-column tiles at M <= 2 (ragged last tile in the second)
    cases += [(1, 256, 18432, 64, False), (2, 512, 18464, 128, True)]
    for M in (9, 15, 16, 17, 32, 33, 64, 65, 100, 128, 200, 256):  # MFMA path, ragged words/rows
        cases.append((M, 512, 520, 64, M % 2 == 1))
    cases += [(1, 256, 264, 64, True), (7, 384, 8, 128, False),  # N % 32 != 0 at small M
              (40, 2048, 1024, 2048, True), (256, 1280, 512, 128, True),
              (96, 96, 256, 32, True),     # large-M kernel: K-groups with no steps
              (72, 160, 136, 32, False),   # large-M kernel: ragged rows and columns
              (128, 2048, 1024, 128, True), (200, 1024, 392, 64, False)]  # 64-row tiles, 128-column shape
    return cases


@pytest.mark.parametrize("M,K,N,G,asym", small_cases())
def test_gemm_matches_oracle(M, K, N, G, asym):
    path, splits, grid = w4.w4a16_gemm_plan(M, K, N, G)
    note("gemm M=%d K=%d N=%d G=%d asym=%s path=%d splits=%d grid=%d" % (M, K, N, G, asym, path, splits, grid))
    p = synth.problem(M, K, N, G, asym, seed=1000 + M * 7 + K + N)
    got = run_gemm(p)
    want = oracle.gemm(p["a"], p["b_packed"], p["scales"], p["qzeros"], G, 8)
    check_close(got, want, "M=%d K=%d N=%d" % (M, K, N))


@pytest.mark.parametrize("M,K,N,G,asym", [c for c in small_cases() if c[0] <= 8 and c[2] % 32 == 0])
def test_gemm_dot2_gemv_matches_oracle(M, K, N, G, asym):
    """The dot2 GEMV (vector ALUs; the planner's default is the matrix-core
    GEMV) on the small GEMV cases."""
    p = synth.problem(M, K, N, G, asym, seed=1000 + M * 7 + K + N)
    try:
        w4.w4a16_set_tuning("gemv_mma=0")
        assert w4.w4a16_gemm_plan(M, K, N, G)[0] == 1
        got = run_gemm(p)
    finally:
        w4.w4a16_set_tuning(None)
    want = oracle.gemm(p["a"], p["b_packed"], p["scales"], p["qzeros"], G, 8)
    check_close(got, want, "dot2 M=%d K=%d N=%d" % (M, K, N))


TUNED_FORMS = ["gemv_mma=0", "gemv_mma=0,gemv_fold=0", "gemv_mma=0,gemv_fold=1", "gemv_waves=4",
               "gemv_waves=4,gemv_fold=1", "gemv_mma=0,gemv_splits=1", "gemv_mma=0,gemv_splits=7",
               "gemv_mma=1", "gemv_mma=1,gemv_splits=1", "gemv_mma=1,gemv_splits=7",
               "gemv_mma_words=4", "gemv_mma_words=4,gemv_splits=3", "gemv_mma_words=2",
               "gemv_max_m=0", "mfma_cfg=4", "mfma_cfg=5,mfma_splits=3",
               "mfma_cfg=3", "mfma_cfg=6", "mfma_cfg=6,mfma_splits=3", "mfma_mgroup=1", "mfma_mgroup=2",
               "mfma_cfg=4,mfma_mgroup=3", "mfma_cfg=1,mfma_mgroup=4,mfma_splits=2"]


@pytest.mark.parametrize("spec", TUNED_FORMS)
def test_gemm_tuned_forms_match_oracle(spec):
    """Every planner override computes the same product (the dot2 GEMV's exact
    and folded forms, the matrix-core GEMV at every M, 4- and 8-wave
    workgroups, forced split counts (uneven per wave included), the MFMA path
    at small M, the alternative MFMA tile shapes, the workgroup orders over
    row tiles, including a ragged last band)."""
    try:
        w4.w4a16_set_tuning(spec)
        for M, K, N, G, asym in [(1, 1024, 544, 128, False), (2, 2048, 1024, 64, True), (3, 512, 800, 128, True),
                                 (5, 1024, 288, 256, False), (8, 1024, 544, 128, True), (20, 1024, 520, 128, True),
                                 (150, 512, 800, 128, True)]:
            path, splits, grid = w4.w4a16_gemm_plan(M, K, N, G)
            note("tuned %s M=%d K=%d N=%d path=%d splits=%d grid=%d" % (spec, M, K, N, path, splits, grid))
            p = synth.problem(M, K, N, G, asym, seed=300 + M)
            got = run_gemm(p)
            want = oracle.gemm(p["a"], p["b_packed"], p["scales"], p["qzeros"], G, 8)
            check_close(got, want, "%s M=%d" % (spec, M))
    finally:
        w4.w4a16_set_tuning(None)


@pytest.mark.parametrize("M", [1, 4, 8, 16, 32, 256])
def test_gemm_deterministic(M):
    p = synth.problem(M, 4096, 2048, 128, True, seed=77)
    a, b, s, z = dev(p["a"]), dev(p["b_packed"]), dev(p["scales"]), dev(p["qzeros"])
    o1 = host(w4.w4a16_gemm(a, b, s, z, 128))
    o2 = host(w4.w4a16_gemm(a, b, s, z, 128))
    assert np.array_equal(o1.view(np.uint16), o2.view(np.uint16))


def f16_ulp(x):
    """Spacing of fp16 values at |x| (subnormal spacing below 2^-14)."""
    e = np.floor(np.log2(np.maximum(np.abs(x.astype(np.float64)), 2.0 ** -14)))
    return 2.0 ** (e - 10)


@pytest.mark.parametrize("M", [1, 2, 5, 8, 12, 32, 256])
def test_gemm_identities(M):
    """All-8 nibbles with zero point 8 give exactly 0 on the dot2 GEMV (also
    in its folded form, whose zero correction runs the same dot chain) and the
    MFMA GEMM, and 0 within the tolerance on the matrix-core GEMV (its zero
    correction runs on separately rounded activation sums); qzeros all 8 equal
    the symmetric call bit for bit where both take the same arithmetic form
    (the default folds only symmetric dot2 GEMVs at M <= 2: there, within the
    tolerance, and bit for bit with the exact form forced); doubling every
    scale doubles the output -- exactly where the K-splits meet in fp32, and
    to within one fp16 step where the GEMVs' K-splits meet in 2^-26 fixed point
    (each split's partial is rounded to that grid, which does not commute with
    doubling)."""
    K, N, G = 1024, 512, 128
    path, splits, _ = w4.w4a16_gemm_plan(M, K, N, G)
    p = synth.problem(M, K, N, G, False, seed=55 + M)
    a, b, s = dev(p["a"]), dev(p["b_packed"]), dev(p["scales"])
    eights = torch.full_like(b, np.uint32(0x88888888).view(np.int32).item())
    zero = host(w4.w4a16_gemm(a, eights, s, None, G, 8))
    if path == 3:
        check_close(zero, np.zeros_like(zero), "all-zp columns, matrix-core GEMV")
    else:
        assert np.all(zero == 0)
    qz8 = torch.full((K // G, N // 8), np.uint32(0x88888888).view(np.int32).item(), dtype=torch.int32, device="cuda")
    sym = host(w4.w4a16_gemm(a, b, s, None, G, 8))
    asym = host(w4.w4a16_gemm(a, b, s, qz8, G, 3))
    if path == 1 and M <= 2:
        check_close(asym, sym, "asym vs folded sym")
        try:
            w4.w4a16_set_tuning("gemv_fold=0")
            sym0 = host(w4.w4a16_gemm(a, b, s, None, G, 8))
            asym0 = host(w4.w4a16_gemm(a, b, s, qz8, G, 3))
        finally:
            w4.w4a16_set_tuning(None)
        assert np.array_equal(sym0.view(np.uint16), asym0.view(np.uint16))
    else:
        assert np.array_equal(sym.view(np.uint16), asym.view(np.uint16))
    dbl = host(w4.w4a16_gemm(a, b, s * 2, None, G, 8)).astype(np.float64)
    two = 2 * sym.astype(np.float64)
    if path in (1, 3) and splits > 1:
        assert np.all(np.abs(dbl - two) <= f16_ulp(two))
    else:
        assert np.array_equal(dbl, two)


@pytest.mark.parametrize("M,K,N", [(1, 4096, 12800), (4, 4096, 2048), (1, 256, 256), (32, 1024, 512)])
def test_gemm_nonfinite_and_overflow(M, K, N):
    """An inf activation makes exactly the oracle's non-finite outputs
    non-finite (the GEMV's fixed-point K-split hand-off reports them as NaN);
    activations of +-60000 against all-15 nibbles overflow fp16 to inf of the
    oracle's sign, also where K-split partials saturate."""
    G = 128 if K >= 128 else K
    path, splits, _ = w4.w4a16_gemm_plan(M, K, N, G)
    note("nonfinite M=%d K=%d N=%d path=%d splits=%d" % (M, K, N, path, splits))
    p = synth.problem(M, K, N, G, False, seed=4242 + M)
    a = p["a"].copy()
    a[0, K // 3] = np.float16(np.inf)
    got = run_gemm(dict(p, a=a), qzeros=False)
    want = oracle.gemm(a, p["b_packed"], p["scales"], None, G, 8)
    assert np.array_equal(np.isfinite(got), np.isfinite(want))
    fin = np.isfinite(want)
    check_close(np.where(fin, got, 0).astype(np.float16), np.where(fin, want, 0).astype(np.float16), "finite part")

    big = np.full((M, K), 60000.0, dtype=np.float16)
    big[M // 2:] = -60000.0
    fifteens = np.full_like(p["b_packed"], np.uint32(0xFFFFFFFF).view(np.int32))
    ones = np.ones_like(p["scales"])
    got = run_gemm(dict(p, a=big, b_packed=fifteens, scales=ones), qzeros=False)
    want = oracle.gemm(big, fifteens, ones, None, G, 8)
    assert np.all(np.isinf(want))
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_gemm_m0_and_into_out():
    p = synth.problem(4, 256, 256, 64, False, seed=5)
    a, b, s = dev(p["a"]), dev(p["b_packed"]), dev(p["scales"])
    empty = w4.w4a16_gemm(a[:0], b, s, None, 64)
    assert empty.shape == (0, 256)
    out = torch.full((4, 256), 7.0, dtype=torch.float16, device="cuda")
    w4.w4a16_gemm(a, b, s, None, 64, out=out)
    want = oracle.gemm(p["a"], p["b_packed"], p["scales"], None, 64)
    check_close(host(out), want, "into out")


def test_gemm_after_repack_matches_checkpoint_layout():
    p = synth.problem(32, 1024, 768, 128, True, seed=31, from_checkpoint=True)
    bk = w4.w4a16_repack(dev(p["b_nk8"]), 1024)
    out = host(w4.w4a16_gemm(dev(p["a"]), bk, dev(p["scales"]), dev(p["qzeros"]), 128))
    want = oracle.gemm_nk8(p["a"], p["b_nk8"], p["scales"], p["qzeros"], 128)
    check_close(out, want, "repack+gemm")


@pytest.mark.parametrize("N,Gn", [(8, 1), (136, 3), (4096, 100), (12800, 32), (256, 200)])
def test_repack_scales_bit_exact(N, Gn):
    note("repack_scales N=%d Gn=%d" % (N, Gn))
    src = synth.rng(N + 7 * Gn).integers(0, 1 << 16, size=(N, Gn), dtype=np.uint16).view(np.float16)
    want = oracle.repack_scales(src)
    got = host(w4.w4a16_repack_scales(dev(src)))
    torch.cuda.synchronize()
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("M,K,N,G", [(1, 4096, 1024, 128), (5, 2048, 768, 64), (32, 1024, 512, 128)])
def test_gemm_after_full_checkpoint_load(M, K, N, G):
    """The whole load path from a checkpoint layout: weights [N, K/8], group
    scales [N, K/G] and zero points packed along the group axis [N, (K/G)/8]
    go through w4a16_repack, w4a16_repack_scales and w4a16_repack (K := K/G);
    the product matches the oracle's on the kernel-layout tensors."""
    p = synth.problem(M, K, N, G, True, seed=4000 + M)
    Gn = K // G
    b_nk8 = pack_rows(unpack_rows(p["b_packed"]).T)               # [N, K/8]
    s_ng = np.ascontiguousarray(p["scales"].T)                     # [N, K/G]
    qz_nk8 = pack_rows(unpack_rows(p["qzeros"]).T)                 # [N, (K/G)/8]
    note("checkpoint load M=%d K=%d N=%d G=%d" % (M, K, N, G))
    b = w4.w4a16_repack(dev(b_nk8), K)
    s = w4.w4a16_repack_scales(dev(s_ng))
    qz = w4.w4a16_repack(dev(qz_nk8), Gn)
    assert np.array_equal(host(b), p["b_packed"])
    assert np.array_equal(host(s).view(np.uint16), p["scales"].view(np.uint16))
    assert np.array_equal(host(qz), p["qzeros"])
    out = host(w4.w4a16_gemm(dev(p["a"]), b, s, qz, G))
    want = oracle.gemm(p["a"], p["b_packed"], p["scales"], p["qzeros"], G, 8)
    check_close(out, want, "checkpoint load M=%d" % M)


# ------------------------------------------- full workload sizes, sampled ---

def sample_idx(M, N, count, seed):
    g = np.random.default_rng(seed)
    mi = g.integers(0, M, count)
    ni = g.integers(0, N, count)
    # always include the corners and the last column (ragged tails)
    mi = np.concatenate([mi, [0, M - 1, 0, M - 1]])
    ni = np.concatenate([ni, [0, 0, N - 1, N - 1]])
    return mi, ni


@pytest.mark.parametrize("name", ["tiny", "gemv"])
def test_workload_full_output(name):
    p = synth.workload(name)
    note("workload %s (full output)" % name)
    got = run_gemm(p)
    want = oracle.gemm(p["a"], p["b_packed"], p["scales"], p["qzeros"], p["G"], 8)
    check_close(got, want, name)


@pytest.mark.parametrize("name,count", [("batched", 3000), ("prefill", 1500)])
def test_workload_sampled(name, count):
    p = synth.workload(name)
    note("workload %s (sampled %d)" % (name, count))
    if "b_nk8" in p:
        b = w4.w4a16_repack(dev(p["b_nk8"]), p["K"])
        want_b = oracle.repack(p["b_nk8"], p["K"])
        assert np.array_equal(host(b), want_b)
        p["b_packed"] = want_b
    else:
        b = dev(p["b_packed"])
    out = host(w4.w4a16_gemm(dev(p["a"]), b, dev(p["scales"]), dev(p["qzeros"]), p["G"], 8))
    mi, ni = sample_idx(p["M"], p["N"], count, seed=9)
    want, _ = oracle.gemm_sample(p["a"], p["b_packed"], p["scales"], p["qzeros"], p["G"], 8, mi, ni)
    check_close(out[mi, ni], want, name)


# ------------------------------------------------------------ decode step ---

def dev_stack(layers):
    return [dict(b_packed=dev(L["b_packed"]), scales=dev(L["scales"]), qzeros=None, G=L["G"], zp_bias=8)
            for L in layers]


@pytest.mark.parametrize("M", [1, 3, 20])
def test_decode_step_small_stack(M):
    """Teacher-forced per layer: the oracle's layer l is fed the GPU's own input
    to layer l, so each comparison covers one layer (four chained linears) at
    the per-element bound.  The multi-layer call matches the chained
    single-layer calls to relative L2 <= 1e-2 (at M <= 8 it applies each
    layer's output row-norm inside the next layer's QKV, one fp16 rounding
    fewer, and rounding differences compound over layers), and so does the
    end-to-end drift against the oracle's own chain."""
    H, NQ, I, G, nl = 256, 384, 512, 64, 3
    layers = []
    for l in range(nl):
        layers += synth.stack_layer(l, H=H, NQ=NQ, I=I, G=G, seed_base=900)
    x = synth.stack_input(M, H, seed=M)
    dstack = dev_stack(layers)
    full = host(w4.w4a16_decode_step(dstack, dev(x)))
    cur = dev(x)
    for l in range(nl):
        y = w4.w4a16_decode_step(dstack[4 * l: 4 * l + 4], cur)
        want = oracle.decode_step(layers[4 * l: 4 * l + 4], host(cur), 1)
        check_close(host(y), want, "decode small M=%d layer %d" % (M, l), tol=FUSED_LAYER_TOL)
        cur = y
    chained = host(cur).astype(np.float64)
    rel = np.linalg.norm(full.astype(np.float64) - chained) / np.linalg.norm(chained)
    note("decode small M=%d n-layer vs chained relative L2 %.3g" % (M, rel))
    assert rel < 1e-2
    e2e = oracle.decode_step(layers, x, nl).astype(np.float64)
    rel = np.linalg.norm(full.astype(np.float64) - e2e) / np.linalg.norm(e2e)
    note("decode small M=%d end-to-end relative L2 drift %.3g" % (M, rel))
    assert rel < 1e-2


def tuned(spec, fn):
    try:
        w4.w4a16_set_tuning(spec)
        return fn()
    finally:
        w4.w4a16_set_tuning(None)


@pytest.mark.parametrize("gemv", ["", "gemv_mma=0", "decode_swiglu_m=9"])
@pytest.mark.parametrize("M", [1, 2, 5, 12, 24])
@pytest.mark.parametrize("H,NQ,I", [(256, 384, 512), (512, 768, 9216), (512, 512, 17408)])
def test_decode_step_fused_matches_unfused(M, H, NQ, I, gemv):
    """At M <= 8 the row-norms run inside the consuming GEMVs (the row scale
    applied to the products; the matrix-core GEMV by default, the dot2 GEMV
    with gemv_mma=0) and a layer's output row-norm inside the next layer's
    QKV; SwiGLU + row-norm runs inside the down GEMV at M <= 2 (at every
    M <= 8 with decode_swiglu_m=9) and as a kernel of its own above; at
    M >= 9 the row-norms run inside the consuming MFMA GEMMs the same way
    (SwiGLU a kernel).  One layer matches the unfused
    step (separate glue kernels, forced with decode_fuse=0) and the oracle at
    the per-element bound; two layers (the cross-layer fold) match the unfused
    step to relative L2 <= 1e-2.  Row widths up to 17408 cover one, two and
    four 8-element vectors per virtual thread of the row sums."""
    if gemv and M > 8:
        pytest.skip("these GEMV-route forms apply at M <= 8 only")
    G, nl = 128, 2
    layers = []
    for l in range(nl):
        layers += synth.stack_layer(l, H=H, NQ=NQ, I=I, G=G, seed_base=1700)
    x = dev(synth.stack_input(M, H, seed=40 + M))
    dstack = dev_stack(layers)
    note("decode fused vs unfused M=%d H=%d I=%d %s" % (M, H, I, gemv))
    fused = tuned(gemv, lambda: host(w4.w4a16_decode_step(dstack, x)))
    unfused = tuned("decode_fuse=0", lambda: host(w4.w4a16_decode_step(dstack, x)))
    rel = np.linalg.norm(fused.astype(np.float64) - unfused) / np.linalg.norm(unfused.astype(np.float64))
    note("decode fused vs unfused M=%d I=%d two layers relative L2 %.3g" % (M, I, rel))
    assert rel < 1e-2
    first = tuned(gemv, lambda: host(w4.w4a16_decode_step(dstack[:4], x)))
    first_unfused = tuned("decode_fuse=0", lambda: host(w4.w4a16_decode_step(dstack[:4], x)))
    check_close(first, first_unfused, "fused vs unfused layer 0 M=%d I=%d" % (M, I), tol=FUSED_LAYER_TOL)
    want = oracle.decode_step(layers[:4], host(x), 1)
    check_close(first, want, "fused layer 0 M=%d I=%d" % (M, I), tol=FUSED_LAYER_TOL)


# A decode layer chains four linears and the glue.  With every glue step a
# kernel of its own, the GPU takes the oracle's roundings (fp16 after each GEMM
# and each glue step) and one layer stays within the single-GEMM bound.  The
# fused routes apply each row-norm to the products and so skip the fp16
# rounding of the normalised activations that the oracle takes; that adds up
# to about 0.004 per element on the 8B-class layer (measured), where the MFMA
# path's fp16 weight operands already use about 0.007 of the 0.01.  The bound
# for a fused layer is twice the single-GEMM bound.
FUSED_LAYER_TOL = 2 * TOL


@pytest.mark.parametrize("M", [1, 16, 32])
def test_decode_step_one_real_layer(M):
    """One layer at the 8B-class shapes (QKV 4096->6144, O, gate+up
    4096->25600, down 12800->4096), same launch plans as the full stack: the
    separate-kernel route within the single-GEMM bound, the fused route (the
    default) within the fused-layer bound."""
    layers = synth.stack_layer(0)
    x = synth.stack_input(M)
    note("decode real layer M=%d" % M)
    want = oracle.decode_step(layers, x, 1)
    got = host(w4.w4a16_decode_step(dev_stack(layers), dev(x)))
    check_close(got, want, "decode real fused M=%d" % M, tol=FUSED_LAYER_TOL)
    try:
        w4.w4a16_set_tuning("decode_fuse=0")
        sep = host(w4.w4a16_decode_step(dev_stack(layers), dev(x)))
    finally:
        w4.w4a16_set_tuning(None)
    check_close(sep, want, "decode real separate M=%d" % M)


def test_decode_step_in_place_and_rms():
    H, NQ, I, G = 256, 256, 384, 128
    layers = synth.stack_layer(0, H=H, NQ=NQ, I=I, G=G) + synth.stack_layer(1, H=H, NQ=NQ, I=I, G=G)
    x = dev(synth.stack_input(5, H))
    ref = host(w4.w4a16_decode_step(dev_stack(layers), x))
    w4.w4a16_decode_step(dev_stack(layers), x, out=x)  # x_out may equal x_in
    got = host(x)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
    rms = np.sqrt((got.astype(np.float64) ** 2).mean(1))
    assert np.allclose(rms, 1.0, atol=5e-3)


@pytest.mark.parametrize("gemv", ["", "gemv_mma=0", "decode_swiglu_m=9"])
@pytest.mark.parametrize("M", [1, 2, 5, 12, 24])
@pytest.mark.parametrize("I", [9216, 12800])
def test_decode_step_down_projection_intermediate(M, I, gemv):
    """White box: the step's output is row-normed, which hides a wrong row
    scale in any linear before it.  After a one-layer step the workspace holds
    the down projection's output and its input: where SwiGLU + row-norm runs
    inside the down GEMV (M <= 2; every M <= 8 with decode_swiglu_m=9) the
    first buffer holds the gate+up output and the second the down output,
    which must be the oracle's down projection of fp16(rn(silu(g) * u));
    elsewhere the second buffer holds the SwiGLU + row-norm kernel's output
    (rows of unit rms) and the first the down GEMV's or GEMM's, which must be
    the oracle's product of the two.  MLP widths 9216 and 12800
    give GEMV K-splits with fewer 16-row chunks than row lanes, where a row-sum
    reduction run on only the lanes that hold a chunk lost part of a wave's
    sum."""
    H, NQ, G = 512, 640, 128
    layers = synth.stack_layer(0, H=H, NQ=NQ, I=I, G=G, seed_base=2300)
    x = dev(synth.stack_input(M, H, seed=90 + M))
    buf = (M * max(L["N"] for L in layers) * 2 + 255) // 256 * 256
    ws = torch.zeros(2 * buf, dtype=torch.uint8, device="cuda")
    if gemv and M > 8:
        pytest.skip("these GEMV-route forms apply at M <= 8 only")
    note("decode down intermediate M=%d I=%d %s" % (M, I, gemv))
    tuned(gemv, lambda: w4.w4a16_decode_step(dev_stack(layers), x, workspace=ws))
    w = host(ws)
    D = layers[3]
    if M <= (8 if gemv == "decode_swiglu_m=9" else 2):
        gu = w[:buf].view(np.float16)[:M * 2 * I].reshape(M, 2 * I)
        down = w[buf:].view(np.float16)[:M * H].reshape(M, H)
        h3 = oracle.swiglu_rownorm(gu)
    else:
        h3 = w[buf:].view(np.float16)[:M * I].reshape(M, I)
        down = w[:buf].view(np.float16)[:M * H].reshape(M, H)
        rms = np.sqrt((h3.astype(np.float64) ** 2).mean(1))
        assert np.allclose(rms, 1.0, atol=5e-3), rms
    want = oracle.gemm(h3, D["b_packed"], D["scales"], None, G, 8)
    check_close(down, want, "down projection M=%d I=%d" % (M, I), tol=FUSED_LAYER_TOL)
