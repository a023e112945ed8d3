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
from tests._fixtures import oracle_gemm_columns, pack_rows, unpack_rows
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
    note("%s max|err|=%.3g max err/bound=%.3g max ulp=%d" % (what, err.max() if err.size else 0,
                                                            (err / bound).max() if err.size else 0,
                                                            ulp.max() if ulp.size else 0))
    assert np.all(err <= bound), "%s: worst at %s got %r want %r" % (what, worst, g[worst], r[worst])


def run_gemm(p, qzeros=True, b_key="b_packed"):
    qz = p["qzeros"] if qzeros else None
    out = w4.w4a16_gemm(dev(p["a"]), dev(p[b_key]), dev(p["scales"]), dev(qz), p["G"], p["zp_bias"])
    torch.cuda.synchronize()
    return host(out)


def tuned(spec, fn):
    """fn() under the planner overrides `spec` ("" = defaults)."""
    try:
        w4.w4a16_set_tuning(spec)
        return fn()
    finally:
        w4.w4a16_set_tuning(None)


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
               "gemv_mma=1", "gemv_mma=1,gemv_splits=1", "gemv_mma=1,gemv_splits=7", "gemv_mma=1,gemv_splits=16",
               "gemv_mma_exact=0", "gemv_mma_exact=0,gemv_mma_words=4",
               "gemv_mma_words=4", "gemv_mma_words=4,gemv_splits=3", "gemv_mma_words=2",
               "gemv_max_m=0", "mfma_cfg=3", "mfma_cfg=2,mfma_splits=3",
               "mfma_cfg=1", "mfma_cfg=2", "mfma_cfg=3,mfma_splits=3", "mfma_cfg=3,mfma_splits=8",
               "mfma_mgroup=1", "mfma_mgroup=2",
               "mfma_cfg=3,mfma_mgroup=3", "mfma_cfg=1,mfma_mgroup=4,mfma_splits=2",
               "mfma_shared_m=0", "mfma_shared_m=0,mfma_cfg=2", "mfma_shared_m=9", "mfma_shared_m=9,mfma_wm=4",
               "mfma_shared_m=9,mfma_splits=2", "mfma_wm=2,mfma_mgroup=2", "mfma_wm=4,mfma_mgroup=1",
               "mfma_tile_m=9", "mfma_tile_m=9,mfma_splits=3", "mfma_tall_m=9", "mfma_tall_m=9,mfma_splits=5"]


@pytest.mark.parametrize("spec", TUNED_FORMS)
def test_gemm_tuned_forms_match_oracle(spec):
    """Every planner override computes the same product (the dot2 GEMV's exact
    and folded forms, the matrix-core GEMV at every M in its folded and exact
    forms, 4- and 8-wave workgroups, forced split counts (uneven per wave, and
    the 16-split maximum, included), the MFMA path at small M, the
    alternative MFMA tile shapes, the workgroup orders over row tiles,
    including a ragged last band)."""
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


SHARED_CASES = [(64, 4096, 1000, 32, True), (129, 4096, 1000, 64, False), (256, 4096, 1032, 128, True),
                (100, 3072, 520, 256, True), (256, 12800, 512, 128, True), (33, 2048, 4104, 128, False),
                (96, 12800, 264, 32, True)]  # 400 groups: at least 4 splits (128 staged groups per split)
SHARED_FORMS = ["", "mfma_wm=2", "mfma_wm=4", "mfma_splits=1", "mfma_splits=3", "mfma_splits=8",
                "mfma_wm=4,mfma_splits=7,mfma_mgroup=1", "mfma_wm=2,mfma_splits=5,mfma_mgroup=3",
                "mfma_shared_kw=1", "mfma_shared_kw=1,mfma_wm=2", "mfma_shared_kw=1,mfma_splits=3",
                "mfma_shared_kw=1,mfma_wm=2,mfma_splits=8,mfma_mgroup=2",
                "mfma_tile_m=1", "mfma_tile_m=1,mfma_splits=1", "mfma_tile_m=1,mfma_splits=3",
                "mfma_tile_m=1,mfma_splits=8,mfma_mgroup=2"]


@pytest.mark.parametrize("M,K,N,G,asym", SHARED_CASES)
def test_gemm_shared_kernel_matches_oracle(M, K, N, G, asym):
    """The MFMA kernels that share dequantised weights through LDS: the
    row-wave kernel in both row-wave shapes and its single-K-wave form, and the
    128 x 256 kernel that also shares the activations, at every group size they
    take, with ragged rows and column tiles, K-waves of unequal group counts
    and forced K-split counts (one to eight, uneven)."""
    p = synth.problem(M, K, N, G, asym, seed=900 + M + K + N)
    want = oracle_gemm_columns(p["a"], p["b_packed"], p["scales"], p["qzeros"], G, 8)
    for spec in SHARED_FORMS:
        full = "mfma_shared_m=1," + spec if spec else "mfma_shared_m=1"
        path, splits, grid = tuned(full, lambda: w4.w4a16_gemm_plan(M, K, N, G))
        note("shared %s M=%d K=%d N=%d G=%d path=%d splits=%d grid=%d" % (full, M, K, N, G, path, splits, grid))
        assert path == 2
        got = tuned(full, lambda: run_gemm(p))
        check_close(got, want, "shared %s M=%d" % (full, M))


TALL_CASES = [(129, 4096, 1024, 64, False), (256, 4096, 1056, 128, True), (256, 12800, 512, 128, True),
              (200, 3072, 544, 256, True), (130, 1024, 320, 32, False), (384, 1056, 288, 96, True),
              (96, 12800, 256, 32, True), (17, 544, 64, 32, False),
              (160, 2048, 512, 2048, False),  # G = K: one group per row
              (513, 1024, 256, 64, False), (1024, 1024, 512, 128, True)]  # many row tiles, a last tile of one row
TALL_FORMS = ["", "mfma_splits=1", "mfma_splits=2", "mfma_splits=3", "mfma_splits=8", "mfma_tall_kg=2",
              "mfma_tall_kg=2,mfma_splits=1", "mfma_tall_kg=2,mfma_splits=3", "mfma_tall_kg=2,mfma_splits=8",
              "mfma_tall_rt=2", "mfma_tall_rt=2,mfma_tall_kg=2,mfma_splits=3", "mfma_tall_rt=4,mfma_splits=5",
              "mfma_tall_rt=4,mfma_tall_kg=2"]


@pytest.mark.parametrize("M,K,N,G,asym", TALL_CASES)
def test_gemm_tall_kernel_matches_oracle(M, K, N, G, asym):
    """The MFMA kernel whose waves convert a 32-column strip of weights for
    all 128 rows of the workgroup tile (activations staged in LDS): ragged row
    tiles (rows past M), ragged column tiles (words past N), group sizes from
    32 to 256 and one (96) that does not divide the two-step LDS stages, odd
    step counts per split, and K-split counts from one to eight; with one and
    with two K-groups of waves per workgroup (the second group's share of a
    split shorter than the first's, or empty)."""
    p = synth.problem(M, K, N, G, asym, seed=700 + M + K + N)
    want = oracle_gemm_columns(p["a"], p["b_packed"], p["scales"], p["qzeros"], G, 8)
    for spec in TALL_FORMS:
        full = "mfma_tall_m=1," + spec if spec else "mfma_tall_m=1"
        path, splits, grid = tuned(full, lambda: w4.w4a16_gemm_plan(M, K, N, G))
        note("tall %s M=%d K=%d N=%d G=%d path=%d splits=%d grid=%d" % (full, M, K, N, G, path, splits, grid))
        assert path == 2
        got = tuned(full, lambda: run_gemm(p))
        check_close(got, want, "tall %s M=%d" % (full, M))


@pytest.mark.parametrize("spec", ["mfma_shared_m=0,mfma_splits=2", "mfma_shared_m=1,mfma_splits=2",
                                  "mfma_tall_m=1,mfma_splits=2", "mfma_tall_m=1,mfma_splits=8",
                                  "mfma_tall_m=1,mfma_tall_kg=2,mfma_splits=4",
                                  "mfma_shared_m=1,mfma_wm=2,mfma_splits=4", "mfma_tile_m=1,mfma_splits=2",
                                  "mfma_tile_m=1,mfma_splits=8"])
def test_gemm_split_partials_repeated(spec):
    """The MFMA kernels' fp32 split partials, ten calls in a row on one
    problem: every call matches the oracle and the first bit for bit.  (A
    partial's wide store once let the next value written into its data
    registers reach memory instead, in some calls only: one split's column c
    summed with its column c + 4.)"""
    M, K, N, G = 128, 1024, 512, 128
    p = synth.problem(M, K, N, G, True, seed=515)
    want = oracle.gemm(p["a"], p["b_packed"], p["scales"], p["qzeros"], G, 8)
    a, b, s, z = dev(p["a"]), dev(p["b_packed"]), dev(p["scales"]), dev(p["qzeros"])
    path, splits, grid = tuned(spec, lambda: w4.w4a16_gemm_plan(M, K, N, G))
    note("partials %s path=%d splits=%d grid=%d" % (spec, path, splits, grid))
    assert splits > 1
    outs = tuned(spec, lambda: [host(w4.w4a16_gemm(a, b, s, z, G, 8)) for _ in range(10)])
    for i, o in enumerate(outs):
        check_close(o, want, "%s call %d" % (spec, i))
        assert np.array_equal(o.view(np.uint16), outs[0].view(np.uint16)), "call %d differs" % i


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
    """All-8 nibbles with zero point 8 give exactly 0 on every path and form
    (exact (q - z) operands on the matrix-core GEMV and the MFMA GEMM; in the
    folded forms the zero term runs the same MFMA or dot chain as the
    products).  qzeros all 8 equal the symmetric call bit for bit where both
    take the same arithmetic form: everywhere by default except the dot2 GEMV
    at M <= 2 (gemv_mma=0), which folds a symmetric zero point per chunk while
    packed zeros take exact (q - z) weights; there, and for the matrix-core
    GEMV's folded form (gemv_mma_exact=0), the two agree within the tolerance,
    and bit for bit with the exact form forced.  Doubling every scale doubles the output: exactly where the
    K-splits meet in fp32 (the MFMA GEMM scales each group's fp32 sums), and to
    within one fp16 step where the GEMVs' K-splits meet in 2^-28 fixed point
    (each split's partial is rounded to that grid, which does not commute with
    doubling)."""
    K, N, G = 1024, 512, 128
    path, splits, _ = w4.w4a16_gemm_plan(M, K, N, G)
    p = synth.problem(M, K, N, G, False, seed=55 + M)
    a, b, s = dev(p["a"]), dev(p["b_packed"]), dev(p["scales"])
    eights = torch.full_like(b, np.uint32(0x88888888).view(np.int32).item())
    for spec in ("", "gemv_mma=0", "gemv_mma_exact=0", "gemv_mma=0,gemv_fold=0"):
        zero = tuned(spec, lambda: host(w4.w4a16_gemm(a, eights, s, None, G, 8)))
        assert np.all(zero == 0), spec
    qz8 = torch.full((K // G, N // 8), np.uint32(0x88888888).view(np.int32).item(), dtype=torch.int32, device="cuda")
    sym = host(w4.w4a16_gemm(a, b, s, None, G, 8))
    asym = host(w4.w4a16_gemm(a, b, s, qz8, G, 3))
    assert np.array_equal(sym.view(np.uint16), asym.view(np.uint16))
    for folded, exact in (("gemv_mma_exact=0", ""), ("gemv_mma=0", "gemv_mma=0,gemv_fold=0")):
        fpath = tuned(folded, lambda: w4.w4a16_gemm_plan(M, K, N, G))[0]
        sym_f = tuned(folded, lambda: host(w4.w4a16_gemm(a, b, s, None, G, 8)))
        asym_f = tuned(folded, lambda: host(w4.w4a16_gemm(a, b, s, qz8, G, 3)))
        check_close(asym_f, sym_f, "asym vs sym, %s" % folded)
        if fpath == 1 and M <= 2 or folded == "gemv_mma_exact=0" and fpath == 3:  # folded: agree within tolerance
            sym_e = tuned(exact, lambda: host(w4.w4a16_gemm(a, b, s, None, G, 8)))
            assert np.array_equal(sym_e.view(np.uint16), asym_f.view(np.uint16))  # packed zeros: exact form
        else:
            assert np.array_equal(sym_f.view(np.uint16), asym_f.view(np.uint16))
    dbl = host(w4.w4a16_gemm(a, b, s * 2, None, G, 8)).astype(np.float64)
    two = 2 * sym.astype(np.float64)
    if path in (1, 3) and splits > 1:
        assert np.all(np.abs(dbl - two) <= f16_ulp(two))
    else:
        assert np.array_equal(dbl, two)


def same_fp16(got, want):
    """Bitwise equal, except that any NaN matches any NaN."""
    g, r = got.view(np.uint16), want.view(np.uint16)
    gn, rn = np.isnan(got), np.isnan(want)
    return np.array_equal(gn, rn) and np.array_equal(g[~gn], r[~rn])


NONFINITE_FORMS = ["", "gemv_mma_exact=0", "gemv_mma=0,gemv_fold=0", "gemv_max_m=0", "gemv_max_m=0,mfma_shared_m=1",
                   "gemv_max_m=0,mfma_tile_m=1", "gemv_max_m=0,mfma_tall_m=1",
                   "gemv_max_m=0,mfma_tall_m=1,mfma_tall_kg=2"]


@pytest.mark.parametrize("spec", NONFINITE_FORMS)
@pytest.mark.parametrize("M,K,N", [(1, 4096, 12800), (4, 4096, 2048), (1, 256, 256), (32, 1024, 512)])
def test_gemm_nonfinite_and_overflow(M, K, N, spec):
    """Non-finite activations follow the definition on the default paths and
    the exact forms: an infinity times a nonzero (q - z) gives an infinity of
    the product's sign, times zero NaN, and infinities of both signs in one
    sum NaN -- the oracle's classes and signs, element for element (the
    matrix-core GEMV's folded form redoes such chunks with exact weights; the
    GEMVs' K-splits keep +-inf apart in the fixed-point slots).  Activations of +-60000 against
    all-15 nibbles overflow fp16 to inf of the oracle's sign, also where split
    partials exceed the fixed-point range."""
    G = 128 if K >= 128 else K
    p = synth.problem(M, K, N, G, False, seed=4242 + M)
    a = p["a"].copy()
    a[0, K // 3] = np.float16(np.inf)
    a[M - 1, K // 2 + 5] = np.float16(-np.inf)
    path, splits, _ = tuned(spec, lambda: w4.w4a16_gemm_plan(M, K, N, G))
    note("nonfinite %s M=%d K=%d N=%d path=%d splits=%d" % (spec, M, K, N, path, splits))
    got = tuned(spec, lambda: run_gemm(dict(p, a=a), qzeros=False))
    want = oracle.gemm(a, p["b_packed"], p["scales"], None, G, 8)
    assert not np.all(np.isfinite(want))
    fin = np.isfinite(want)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[~fin & ~np.isnan(want)], want[~fin & ~np.isnan(want)])  # +-inf, signs included
    check_close(np.where(fin, got, 0).astype(np.float16), np.where(fin, want, 0).astype(np.float16), "finite part")

    big = np.full((M, K), 60000.0, dtype=np.float16)
    big[M // 2:] = -60000.0
    fifteens = np.full_like(p["b_packed"], np.uint32(0xFFFFFFFF).view(np.int32))
    ones = np.ones_like(p["scales"])
    got = tuned(spec, lambda: run_gemm(dict(p, a=big, b_packed=fifteens, scales=ones), qzeros=False))
    want = oracle.gemm(big, fifteens, ones, None, G, 8)
    assert np.all(np.isinf(want))
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("spec", ["gemv_splits=2", "gemv_splits=2,gemv_mma=0,gemv_fold=0", "gemv_max_m=0",
                                  "gemv_max_m=0,mfma_tall_m=1,mfma_splits=2",
                                  "gemv_max_m=0,mfma_tall_m=1,mfma_tall_kg=2,mfma_splits=2"])
def test_gemm_split_cancellation(spec):
    """Two K-splits whose partials cancel, on the forms whose products are
    exact ((q - z) weights).  Within the fixed-point range of the GEMVs'
    split-K slots (|partial| < 2^17) the sum is exact: +100000 and -99900 give
    100.  Beyond it (+3e6 and -3e6 + 100, true sum 100) the GEMV's result is
    NaN -- loud, never a silently wrong finite value; the MFMA GEMM's fp32
    split sums give 100."""
    M, K, N, G = 1, 256, 256, 128
    q = np.full((K, N), 9, np.int64)              # q - z = 1 with zp 8
    b = pack_rows(q)
    s = np.ones((K // G, N), np.float16)
    path, splits, _ = tuned(spec, lambda: w4.w4a16_gemm_plan(M, K, N, G))
    assert splits == 2 or path == 2
    for scale, expect_nan in ((1000.0, False), (60000.0, True)):
        a = np.zeros((M, K), np.float16)
        n = int(round(100 * 1000.0 / scale)) if scale == 1000.0 else 50
        a[0, :n] = scale                           # split 0: +n * scale
        a[0, K // 2:K // 2 + n] = -scale           # split 1: -n * scale ...
        a[0, K // 2 + n] = 100.0                   # ... + 100
        want = oracle.gemm(a, b, s, None, G, 8)
        assert np.all(want.astype(np.float64) == 100.0)
        got = tuned(spec, lambda: run_gemm(dict(a=a, b_packed=b, scales=s, qzeros=None, G=G, zp_bias=8)))
        note("cancellation %s partials +-%.0f: got %r" % (spec, n * scale, got[0, :4]))
        if expect_nan and path != 2:
            assert np.all(np.isnan(got))
        else:
            assert np.all(got.astype(np.float64) == 100.0)


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

@pytest.mark.parametrize("name", ["tiny", "gemv"])
def test_workload_full_output(name):
    p = synth.workload(name)
    note("workload %s (full output)" % name)
    got = run_gemm(p)
    want = oracle.gemm(p["a"], p["b_packed"], p["scales"], p["qzeros"], p["G"], 8)
    check_close(got, want, name)


@pytest.mark.parametrize("name", ["batched", "prefill"])
def test_workload_full_output_large(name):
    """The M = 32 (weights from the checkpoint layout through w4a16_repack)
    and M = 256 workloads at full size, every output element against the
    oracle (evaluated over column slices on the host's cores)."""
    p = synth.workload(name)
    note("workload %s (full output)" % name)
    if "b_nk8" in p:
        b = w4.w4a16_repack(dev(p["b_nk8"]), p["K"])
        want_b = oracle.repack(p["b_nk8"], p["K"])
        assert np.array_equal(host(b), want_b)
        p["b_packed"] = want_b
    else:
        b = dev(p["b_packed"])
    out = host(w4.w4a16_gemm(dev(p["a"]), b, dev(p["scales"]), dev(p["qzeros"]), p["G"], 8))
    want = oracle_gemm_columns(p["a"], p["b_packed"], p["scales"], p["qzeros"], p["G"], 8)
    ratio = np.max(np.abs(out.astype(np.float64) - want) / np.maximum(1.0, np.abs(want.astype(np.float64))))
    note("workload %s max |err| / max(1, |oracle|) = %.3g (bound %.0e)" % (name, ratio, TOL))
    check_close(out, want, name)


# ------------------------------------------------------------ decode step ---

def dev_stack(layers):
    return [dict(b_packed=dev(L["b_packed"]), scales=dev(L["scales"]), qzeros=None, G=L["G"], zp_bias=8)
            for L in layers]


@pytest.mark.parametrize("M", [1, 3, 20])
def test_decode_step_small_stack(M):
    """Teacher-forced per layer: the oracle's layer l is fed the GPU's own input
    to layer l, so each comparison covers one layer (four chained linears) at
    the per-element bound.  The multi-layer call matches the chained
    single-layer calls to relative L2 <= 1e-2 (it applies each layer's output
    row-norm inside the next layer's QKV, one fp16 rounding fewer, and
    rounding differences compound over layers), and so does the end-to-end
    drift against the oracle's own chain."""
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
        check_close(host(y), want, "decode small M=%d layer %d" % (M, l))
        cur = y
    chained = host(cur).astype(np.float64)
    rel = np.linalg.norm(full.astype(np.float64) - chained) / np.linalg.norm(chained)
    note("decode small M=%d n-layer vs chained relative L2 %.3g" % (M, rel))
    assert rel < 1e-2
    e2e = oracle.decode_step(layers, x, nl).astype(np.float64)
    rel = np.linalg.norm(full.astype(np.float64) - e2e) / np.linalg.norm(e2e)
    note("decode small M=%d end-to-end relative L2 drift %.3g" % (M, rel))
    assert rel < 1e-2


def composed_step(dstack, x):
    """The decode step as the public calls the header lists: per layer
    w4a16_gemm_glue(NONE or RMSNORM) for QKV, RMSNORM for O and gate+up,
    SWIGLU for down, then w4a16_rownorm."""
    d = None
    for l in range(len(dstack) // 4):
        L = dstack[4 * l: 4 * l + 4]
        q = w4.w4a16_gemm_glue(w4.GLUE_NONE, x, L[0]) if l == 0 else w4.w4a16_gemm_glue(w4.GLUE_RMSNORM, d, L[0])
        o = w4.w4a16_gemm_glue(w4.GLUE_RMSNORM, q, L[1])  # rn(q[:, :H]), rows of Nq
        gu = w4.w4a16_gemm_glue(w4.GLUE_RMSNORM, o, L[2])
        d = w4.w4a16_gemm_glue(w4.GLUE_SWIGLU, gu, L[3])
    return w4.w4a16_rownorm(d)


@pytest.mark.parametrize("spec", ["", "gemv_mma=0", "decode_fuse=0", "decode_swiglu_m=9", "gemv_mma_exact=0",
                                  "decode_rn_mfma=1"])
@pytest.mark.parametrize("M", [1, 2, 5, 20, 32])
def test_decode_step_is_the_composition(M, spec):
    """w4a16_decode_step gives bit for bit what the sequence of public calls
    its header lists gives (two layers), on every route: the fused GEMVs, the
    dot2 GEMVs, separate glue kernels, SwiGLU inside the GEMV at M <= 8, the
    MFMA route with the row-norm as a kernel and folded."""
    if spec in ("gemv_mma=0", "decode_swiglu_m=9", "gemv_mma_exact=0") and M > 8:
        pytest.skip("GEMV-route forms apply at M <= 8 only")
    H, NQ, I, G = 256, 384, 512, 64
    layers = synth.stack_layer(0, H=H, NQ=NQ, I=I, G=G, seed_base=2900) + \
        synth.stack_layer(1, H=H, NQ=NQ, I=I, G=G, seed_base=2900)
    dstack = dev_stack(layers)
    x = dev(synth.stack_input(M, H, seed=70 + M))
    note("decode composition M=%d %s" % (M, spec))
    step = tuned(spec, lambda: host(w4.w4a16_decode_step(dstack, x)))
    comp = tuned(spec, lambda: host(composed_step(dstack, x)))
    assert np.array_equal(step.view(np.uint16), comp.view(np.uint16))


@pytest.mark.parametrize("gemv", ["", "gemv_mma=0", "decode_swiglu_m=9", "decode_rn_mfma=1"])
@pytest.mark.parametrize("M", [1, 2, 5, 12, 24])
@pytest.mark.parametrize("H,NQ,I", [(256, 384, 512), (512, 768, 9216), (512, 512, 17408)])
def test_decode_step_fused_matches_unfused(M, H, NQ, I, gemv):
    """At M <= 8 the row-norms run inside the consuming GEMVs (the row scale
    applied to the products; the matrix-core GEMV by default, the dot2 GEMV
    with gemv_mma=0) and a layer's output row-norm inside the next layer's
    QKV; SwiGLU + row-norm runs inside the down GEMV at M <= 2 (at every
    M <= 8 with decode_swiglu_m=9) and as a kernel of its own above; at
    M >= 9 the glue runs as kernels of their own (with decode_rn_mfma=1 the
    row-norms run inside the consuming MFMA GEMMs the same way).  One layer
    matches the unfused step (separate glue kernels, forced with
    decode_fuse=0) and the oracle at the per-element bound; two layers (the cross-layer fold) match the unfused step to
    relative L2 <= 1e-2.  Row widths up to 17408 cover one, two and four
    8-element vectors per virtual thread of the row sums."""
    if gemv and gemv != "decode_rn_mfma=1" and M > 8:
        pytest.skip("these GEMV-route forms apply at M <= 8 only")
    if gemv == "decode_rn_mfma=1" and M <= 8:
        pytest.skip("the MFMA-route form applies at M >= 9 only")
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
    check_close(first, first_unfused, "fused vs unfused layer 0 M=%d I=%d" % (M, I))
    want = oracle.decode_step(layers[:4], host(x), 1)
    check_close(first, want, "fused layer 0 M=%d I=%d" % (M, I))


@pytest.mark.parametrize("M", [1, 2, 8, 16, 32])
def test_decode_step_one_real_layer(M):
    """One layer at the 8B-class shapes (QKV 4096->6144, O, gate+up
    4096->25600, down 12800->4096), same launch plans as the full stack: the
    fused route (the default) and the separate-kernel route, both within the
    per-element bound."""
    layers = synth.stack_layer(0)
    x = synth.stack_input(M)
    note("decode real layer M=%d" % M)
    want = oracle.decode_step(layers, x, 1)
    got = host(w4.w4a16_decode_step(dev_stack(layers), dev(x)))
    check_close(got, want, "decode real fused M=%d" % M)
    sep = tuned("decode_fuse=0", lambda: host(w4.w4a16_decode_step(dev_stack(layers), dev(x))))
    check_close(sep, want, "decode real separate M=%d" % M)


def oracle_glue(glue, x, K):
    """The oracle's glue on the rows the GPU linear reads (teacher forcing)."""
    if glue == w4.GLUE_NONE:
        return x[:, :K]
    if glue == w4.GLUE_RMSNORM:
        return oracle.rownorm(x, K)
    return oracle.swiglu_rownorm(np.ascontiguousarray(x[:, :2 * K]))


@pytest.mark.parametrize("gemv", ["", "gemv_mma=0", "decode_swiglu_m=9", "decode_fuse=0", "decode_rn_mfma=1"])
@pytest.mark.parametrize("M", [1, 2, 5, 12, 24])
@pytest.mark.parametrize("glue,K,N", [(w4.GLUE_RMSNORM, 512, 1024), (w4.GLUE_RMSNORM, 768, 512),
                                      (w4.GLUE_SWIGLU, 9216, 512), (w4.GLUE_SWIGLU, 12800, 512)])
def test_gemm_glue_matches_oracle(M, glue, K, N, gemv):
    """One glue linear, teacher-forced: the oracle applies its own glue to the
    same rows the GPU reads, then its product; the GPU (glue inside the GEMV,
    the MFMA GEMM or a kernel of its own, by route) within the per-element
    bound.  Rows are wider than K (a stride, as the decode step's QKV output
    feeds O).  MLP widths 9216 and 12800 give GEMV K-splits holding fewer
    16-row chunks than a wave has row lanes, where a row-sum reduction run on
    only the lanes that hold a chunk once lost part of a wave's sum."""
    if gemv in ("gemv_mma=0", "decode_swiglu_m=9") and M > 8:
        pytest.skip("GEMV-route forms apply at M <= 8 only")
    if gemv == "decode_rn_mfma=1" and (M <= 8 or glue != w4.GLUE_RMSNORM):
        pytest.skip("the folded MFMA row-norm applies at M >= 9 only")
    G = 128
    L = synth.stack_layer(0, H=K, NQ=N, I=N, G=G, seed_base=3100 + K)[0]  # a [K, N] linear
    width = 2 * K if glue == w4.GLUE_SWIGLU else K
    ld = width + 64
    g = synth.rng(7 * M + K)
    x = (g.standard_normal((M, ld), dtype=np.float32) * 2).astype(np.float16)
    lin = dict(b_packed=dev(L["b_packed"]), scales=dev(L["scales"]), qzeros=None, G=G, zp_bias=8)
    got = tuned(gemv, lambda: host(w4.w4a16_gemm_glue(glue, dev(x), lin, ldx=ld)))
    want = oracle.gemm(oracle_glue(glue, x, K), L["b_packed"], L["scales"], None, G, 8)
    note("gemm_glue %d M=%d K=%d %s" % (glue, M, K, gemv))
    check_close(got, want, "gemm_glue %d M=%d K=%d %s" % (glue, M, K, gemv))


@pytest.mark.parametrize("M", [1, 32])
def test_decode_per_linear_8b_layers(M):
    """Per linear, teacher-forced, at the 8B-class shapes on layers 0, 1 and
    39 of the seeded stack: each GPU linear (w4a16_gemm_glue, the calls the
    decode step makes) against the oracle's glue and product on the GPU's own
    input to that linear, within the per-element bound.  Layer 0 starts from
    the seeded input; layers 1 and 39 take the GPU's previous down output as
    their rows (the layer-39 weights are the stack's own, seed 5000 + 4*39 + j)."""
    H = synth.STACK["H"]
    prev = None  # the previous layer's raw down output (GPU), None at layer 0
    x0 = dev(synth.stack_input(M))
    for layer in (0, 1, 39):
        Ls = synth.stack_layer(layer)
        D = dev_stack(Ls)
        steps = [(w4.GLUE_NONE if prev is None else w4.GLUE_RMSNORM, 0), (w4.GLUE_RMSNORM, 1),
                 (w4.GLUE_RMSNORM, 2), (w4.GLUE_SWIGLU, 3)]
        src = x0 if prev is None else prev
        for glue, j in steps:
            y = w4.w4a16_gemm_glue(glue, src, D[j])
            rows = host(src)
            K = Ls[j]["K"]
            want = oracle_gemm_columns(np.ascontiguousarray(oracle_glue(glue, rows, K)), Ls[j]["b_packed"],
                                       Ls[j]["scales"], None, Ls[j]["G"], 8)
            got = host(y)
            ratio = np.max(np.abs(got.astype(np.float64) - want) / np.maximum(1.0, np.abs(want.astype(np.float64))))
            note("layer %d linear %d M=%d: max |err|/max(1,|o|) = %.3g" % (layer, j, M, ratio))
            check_close(got, want, "layer %d linear %d M=%d" % (layer, j, M))
            src = y
        prev = src
        del D
        torch.cuda.empty_cache()


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


# ---------------------------------------------------------- graph capture ---

@pytest.mark.parametrize("M", [1, 5, 32])
def test_decode_step_graph_capture(M):
    """The decode step captured into a HIP graph after one eager call (which
    sizes the library's scratch): every replay, with eager work and
    synchronisation between replays, equals the eager step bit for bit, and
    a captured one-layer step matches the oracle per element.  Then an eager
    call of a shape that needs more scratch (an M = 256 GEMM) on the same
    stream grows the library's scratch; the graph, which still uses the old
    set, replays bit for bit as before."""
    H, NQ, I, G = 512, 768, 1024, 128
    layers = synth.stack_layer(0, H=H, NQ=NQ, I=I, G=G, seed_base=3300) + \
        synth.stack_layer(1, H=H, NQ=NQ, I=I, G=G, seed_base=3300)
    dstack = dev_stack(layers)
    x = dev(synth.stack_input(M, H, seed=80 + M))
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        out2 = torch.empty_like(x)
        out1 = torch.empty_like(x)
        ws2 = torch.empty(w4.w4a16_decode_workspace_bytes(M, dstack), dtype=torch.uint8, device="cuda")
        ws1 = torch.empty(w4.w4a16_decode_workspace_bytes(M, dstack[:4]), dtype=torch.uint8, device="cuda")
        w4.w4a16_decode_step(dstack, x, out=out2, workspace=ws2)
        w4.w4a16_decode_step(dstack[:4], x, out=out1, workspace=ws1)
    stream.synchronize()
    eager2, eager1 = host(out2), host(out1)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        w4.w4a16_decode_step(dstack, x, out=out2, workspace=ws2)
        w4.w4a16_decode_step(dstack[:4], x, out=out1, workspace=ws1)
    want1 = oracle.decode_step(layers[:4], host(x), 1)
    p = synth.problem(256, 2048, 4096, 128, True, seed=81)
    big = [dev(p[k]) for k in ("a", "b_packed", "scales", "qzeros")]
    for rep in range(4):
        out2.zero_()
        out1.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out2).view(np.uint16), eager2.view(np.uint16)), "replay %d" % rep
        assert np.array_equal(host(out1).view(np.uint16), eager1.view(np.uint16)), "replay %d" % rep
        check_close(host(out1), want1, "captured layer M=%d replay %d" % (M, rep))
        if rep == 1:
            with torch.cuda.stream(stream):  # grows the scratch of this stream
                w4.w4a16_gemm(big[0], big[1], big[2], big[3], 128)
            stream.synchronize()
    del g


def test_capture_needing_scratch_reports_workspace():
    """A call whose scratch has not been sized on this stream, made while the
    stream is capturing, is refused with W4A16_ERR_WORKSPACE (an allocation
    cannot be captured) and records nothing."""
    p = synth.problem(64, 4096, 8192, 128, False, seed=82)  # a plan with K-splits
    assert w4.w4a16_gemm_plan(64, 4096, 8192, 128)[1] > 1
    a, b, s = dev(p["a"]), dev(p["b_packed"]), dev(p["scales"])
    w4.w4a16_release()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(w4.W4A16Error) as err:
        with torch.cuda.graph(g, stream=stream):
            w4.w4a16_gemm(a, b, s, None, 128)
    assert err.value.status == 4
    torch.cuda.synchronize()
    out = host(w4.w4a16_gemm(a, b, s, None, 128))  # outside capture it runs
    want = oracle_gemm_columns(p["a"], p["b_packed"], p["scales"], None, 128, 8)
    check_close(out, want, "after refused capture")
