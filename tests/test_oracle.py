"""Pins for the CPU oracle (no GPU).

The pages print no worked numeric example, so every pin here is something the
mathematics fixes independently of the oracle's code: hand-derived cases
(tests/golden), exhaustive brute force on tiny inputs, closed-form identities,
a special case that reduces to numpy's float64 matmul, an independent
group-factorised formula, invariants of the repack, and numpy's own fp16
conversion.  Each is chosen so that a plausible slip in the oracle (nibble
order, group index, scale transposed, zero sign, a transposed activation,
rounding mode) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from tests._fixtures import GOLDEN, pack_rows, read_cases, unpack_rows, words
from w4a16_weight_only_amd import synth


def f16(vals):
    return np.array(vals, dtype=np.float64).astype(np.float16)


# ----------------------------------------------------------------- fp16 ---

def test_f16_decode_exhaustive_vs_numpy():
    lib = oracle._load()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([lib.w4o_f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert math.copysign(1.0, got[0x8000]) == -1.0


def test_f16_encode_edges_vs_numpy():
    lib = oracle._load()
    edge = [0.0, -0.0, 1.0, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -11 + 2.0 ** -40,
            65504.0, 65519.99, 65520.0, -65520.0, 1e9, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 + 2.0 ** -60,
            3 * 2.0 ** -25, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 2.0 ** -26, 5e-8, -3e-5,
            float("inf"), float("-inf")]
    for x in edge:
        want = np.array([x], np.float64).astype(np.float16).view(np.uint16)[0]
        assert lib.w4o_f64_to_f16(x) == want, x
    assert lib.w4o_f64_to_f16(float("nan")) & 0x7C00 == 0x7C00


def test_f16_encode_random_vs_numpy():
    lib = oracle._load()
    g = np.random.default_rng(7)
    xs = np.concatenate([g.standard_normal(100000) * 10.0 ** g.integers(-9, 6, 100000),
                         g.uniform(-70000, 70000, 20000)])
    want = xs.astype(np.float16).view(np.uint16)
    got = np.array([lib.w4o_f64_to_f16(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, want)


# ------------------------------------------------------- GEMM hand cases ---

@pytest.mark.parametrize("case", read_cases("gemm_hand_cases.txt"), ids=lambda c: c["name"])
def test_gemm_hand_cases(case):
    M, K, N, G = (int(case[k]) for k in ("M", "K", "N", "G"))
    a = f16([float(v) for v in case["a"].split()]).reshape(M, K)
    b = words(case["b_packed"]).reshape(K, N // 8)
    s = f16([float(v) for v in case["scales"].split()]).reshape(K // G, N)
    qz = None if case["qzeros"] == "none" else words(case["qzeros"]).reshape(K // G, N // 8)
    want = f16([float(v) for v in case["out"].split()]).reshape(M, N)
    got = oracle.gemm(a, b, s, qz, G, int(case["zp_bias"]))
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


# ------------------------------------------- exhaustive one-hot brute force ---

@pytest.mark.parametrize("k0", range(16))
def test_gemm_one_hot_all_weight_zero_pairs(k0):
    """K=16 (two groups of 8), N=2048: column n carries nibble position n%8,
    weight value (n//8 + k) % 16 and zero ((n//128) + 3g) % 16, so every
    (weight, zero, nibble position) triple appears.  With a = c * e_k0 the
    product is c * (q[k0][n] - z[g0][n]) * s[g0][n]; with c a power of two it
    needs at most 4 + 7 significant bits, so it is exact in fp16."""
    K, N, G = 16, 2048, 8
    n = np.arange(N)
    q = np.array([((n // 8) + k) % 16 for k in range(K)])
    z = np.array([((n // 128) + 3 * g) % 16 for g in range(K // G)])
    s = np.array([(1.0 + (n % 64) / 64.0) * 2.0 ** g for g in range(K // G)])
    c = -0.5
    a = np.zeros((1, K))
    a[0, k0] = c
    got = oracle.gemm(f16(a), pack_rows(q), f16(s), pack_rows(z), G, zp_bias=5)
    g0 = k0 // G
    want = c * (q[k0] - z[g0]) * s[g0]          # exact in fp16 by construction
    assert np.array_equal(got[0].astype(np.float64), want)


# ----------------------------------------------------- closed-form pins ---

def test_gemm_all_eights_is_zero():
    p = synth.problem(3, 256, 64, 64, False, seed=11)
    b = np.full_like(p["b_packed"], np.uint32(0x88888888).view(np.int32))
    out = oracle.gemm(p["a"], b, p["scales"], None, 64, zp_bias=8)
    assert np.all(out == 0)


def test_gemm_sym_equals_asym_with_eight_zeros():
    p = synth.problem(4, 512, 128, 128, False, seed=12)
    qz = np.full((512 // 128, 128 // 8), np.uint32(0x88888888).view(np.int32), np.int32)
    o1 = oracle.gemm(p["a"], p["b_packed"], p["scales"], None, 128, zp_bias=8)
    o2 = oracle.gemm(p["a"], p["b_packed"], p["scales"], qz, 128, zp_bias=3)  # qzeros wins
    assert np.array_equal(o1.view(np.uint16), o2.view(np.uint16))


def test_gemm_power_of_two_scale_doubles_output():
    p = synth.problem(2, 256, 128, 64, True, seed=13)
    o1 = oracle.gemm(p["a"], p["b_packed"], p["scales"], p["qzeros"], 64)
    s2 = (p["scales"].astype(np.float64) * 2).astype(np.float16)
    o2 = oracle.gemm(p["a"], p["b_packed"], s2, p["qzeros"], 64)
    assert np.array_equal(o2.astype(np.float64), 2 * o1.astype(np.float64))


def test_gemm_reduces_to_numpy_matmul():
    """G = K, unit scales, zero point 0: out = fp16(a @ q) with q the integer
    matrix; numpy's float64 matmul is exact here (products are multiples of
    2^-24 below 2^7), so the fp16 results must be identical."""
    g = np.random.default_rng(3)
    M, K, N = 3, 96, 40
    q = g.integers(0, 16, size=(K, N))
    a = g.standard_normal((M, K)).astype(np.float16)
    out = oracle.gemm(a, pack_rows(q), np.ones((1, N), np.float16), None, K, zp_bias=0)
    want = (a.astype(np.float64) @ q.astype(np.float64)).astype(np.float16)
    assert np.array_equal(out.view(np.uint16), want.view(np.uint16))


def test_gemm_matches_group_factorised_formula():
    """Independent formula: acc[m][n] = sum_g s[g][n] * (sum_{k in g} a[m][k] q[k][n]
    - z[g][n] * sum_{k in g} a[m][k]), evaluated with numpy in float64."""
    p = synth.problem(5, 512, 96, 128, True, seed=14)
    _, acc = oracle.gemm(p["a"], p["b_packed"], p["scales"], p["qzeros"], 128, want_acc=True)
    a = p["a"].astype(np.float64)
    q = unpack_rows(p["b_packed"]).astype(np.float64)
    z = unpack_rows(p["qzeros"]).astype(np.float64)
    s = p["scales"].astype(np.float64)
    ref = np.zeros_like(acc)
    for g in range(512 // 128):
        ks = slice(g * 128, (g + 1) * 128)
        ref += s[g] * (a[:, ks] @ q[ks] - np.outer(a[:, ks].sum(1), z[g]))
    assert np.allclose(acc, ref, rtol=1e-12, atol=1e-12)


def test_gemm_sample_equals_full():
    p = synth.workload("tiny")
    full = oracle.gemm(p["a"], p["b_packed"], p["scales"], None, p["G"])
    mi = np.zeros(50, np.int64)
    ni = np.random.default_rng(0).integers(0, p["N"], 50)
    got, _ = oracle.gemm_sample(p["a"], p["b_packed"], p["scales"], None, p["G"], 8, mi, ni)
    assert np.array_equal(got.view(np.uint16), full[0, ni].view(np.uint16))


def test_gemm_rejects_bad_shapes():
    a = np.zeros((1, 64), np.float16)
    with pytest.raises(ValueError):
        oracle.gemm(a, np.zeros((64, 1), np.int32), np.zeros((1, 8), np.float16), None, 48)


# ---------------------------------------------------------------- repack ---

@pytest.mark.parametrize("case", read_cases("repack_hand_cases.txt"), ids=lambda c: c["name"])
def test_repack_hand_cases(case):
    K, N = int(case["K"]), int(case["N"])
    ck, cn = (int(v) for v in case["rule"].split())
    q = np.array([[(ck * k + cn * n) % 16 for n in range(N)] for k in range(K)])
    src = pack_rows(q.T)                               # [N, K/8]
    if case["src"]:
        assert np.array_equal(src.view(np.uint32), np.array(case["src"], np.uint32))
    dst = oracle.repack(src, K)
    assert np.array_equal(dst.view(np.uint32), np.array(case["dst"], np.uint32))


@pytest.mark.parametrize("K,N", [(8, 8), (64, 32), (256, 1024), (1024, 136)])
def test_repack_invariants(K, N):
    g = synth.rng(K * 7 + N)
    src = synth.packed_words(g, N, K // 8)
    dst = oracle.repack(src, K)
    # element map: q_kn(dst)[k][n] == q_nk(src)[n][k]
    assert np.array_equal(unpack_rows(dst), unpack_rows(src).T)
    # the inverse map is the same operation with K and N exchanged
    assert np.array_equal(oracle.repack(dst, N), src)
    # nibble histogram preserved
    h1 = np.bincount(unpack_rows(src).ravel(), minlength=16)
    h2 = np.bincount(unpack_rows(dst).ravel(), minlength=16)
    assert np.array_equal(h1, h2)


def test_repack_scales_hand_case():
    """Checkpoint scales [N = 2, K/G = 3] -> kernel [3, 2]: the value of
    (column n, group g) moves to row g, column n; 16-bit patterns (-0, inf,
    a NaN payload, a subnormal) pass unchanged."""
    src = np.array([[0x3C00, 0x8000, 0x7C00],
                    [0x7E01, 0x0001, 0xC000]], dtype=np.uint16)
    want = np.array([[0x3C00, 0x7E01],
                     [0x8000, 0x0001],
                     [0x7C00, 0xC000]], dtype=np.uint16)
    assert np.array_equal(oracle.repack_scales(src.view(np.float16)).view(np.uint16), want)


@pytest.mark.parametrize("N,Gn", [(8, 1), (16, 32), (136, 3), (1024, 100)])
def test_repack_scales_invariants(N, Gn):
    g = synth.rng(N * 13 + Gn)
    src = g.integers(0, 1 << 16, size=(N, Gn), dtype=np.uint16)
    dst = oracle.repack_scales(src.view(np.float16)).view(np.uint16)
    assert dst.shape == (Gn, N)
    # applied again (reading [Gn, N] as a checkpoint [N', Gn']) it gives the input back
    assert np.array_equal(oracle.repack_scales(dst.view(np.float16)).view(np.uint16), src)
    # a column of the checkpoint (one group) becomes a row of the kernel layout
    for gi in (0, Gn - 1):
        assert np.array_equal(dst[gi], src[:, gi])


def test_gemm_invariant_under_repack():
    p = synth.problem(3, 256, 128, 64, True, seed=15, from_checkpoint=True)
    dst = oracle.repack(p["b_nk8"], 256)
    o1 = oracle.gemm(p["a"], dst, p["scales"], p["qzeros"], 64)
    o2 = oracle.gemm_nk8(p["a"], p["b_nk8"], p["scales"], p["qzeros"], 64)
    assert np.array_equal(o1.view(np.uint16), o2.view(np.uint16))


# -------------------------------------------------------- decode glue ---

def test_rownorm_properties():
    g = np.random.default_rng(5)
    x = (g.standard_normal((4, 512)) * np.array([[0.1], [1], [10], [300]])).astype(np.float16)
    y = oracle.rownorm(x).astype(np.float64)
    rms = np.sqrt((y ** 2).mean(1))
    assert np.allclose(rms, 1.0, atol=2e-3)            # unit RMS up to fp16 rounding
    assert np.array_equal(np.sign(y), np.sign(x.astype(np.float64)))
    # a constant row v maps to v / sqrt(v^2 + 1e-6), i.e. 1 in fp16 for |v| >= 0.1
    c = np.full((1, 64), 0.5, np.float16)
    assert np.all(oracle.rownorm(c) == 1.0)
    # the strided form reads only the first `width` columns
    wide = np.concatenate([x, g.standard_normal((4, 40)).astype(np.float16)], 1)
    assert np.array_equal(oracle.rownorm(wide, 512).view(np.uint16), oracle.rownorm(x).view(np.uint16))


def test_swiglu_rownorm_against_expit():
    """silu(x) = x * logistic(x) (scipy.special.expit), then unit-RMS rows."""
    g = np.random.default_rng(6)
    gu = (g.standard_normal((3, 2 * 300)) * 3).astype(np.float16)
    y = oracle.swiglu_rownorm(gu).astype(np.float64)
    gate = gu[:, :300].astype(np.float64)
    up = gu[:, 300:].astype(np.float64)
    t = gate * scipy.special.expit(gate) * up
    want = t / np.sqrt((t ** 2).mean(1, keepdims=True) + 1e-6)
    assert np.allclose(y, want, rtol=1e-3, atol=1e-3)
    # silu(x) - silu(-x) = x: the difference of mirrored gates with unit up
    xs = np.linspace(-6, 6, 64)
    pair = np.concatenate([xs, -xs])[None, :].astype(np.float16)
    upo = np.ones_like(pair)
    yy = oracle.swiglu_rownorm(np.concatenate([pair, upo], 1)).astype(np.float64)[0]
    t2 = (yy[:64] - yy[64:])
    ratio = t2[np.abs(xs) > 0.5] / pair[0, :64].astype(np.float64)[np.abs(xs) > 0.5]
    assert np.allclose(ratio, ratio.mean(), rtol=2e-3)   # proportional to x


def _tiny_stack(n_layers, H=64, NQ=96, I=128, G=32, seed=40):
    layers = []
    for l in range(n_layers):
        layers += synth.stack_layer(l, H=H, NQ=NQ, I=I, G=G, seed_base=seed)
    return layers


def test_decode_step_is_the_composition():
    H, NQ, I, G, M = 64, 96, 128, 32, 3
    layers = _tiny_stack(2, H, NQ, I, G)
    x = synth.stack_input(M, H)
    got = oracle.decode_step(layers, x, 2)
    h = x
    for l in range(2):
        L = layers[4 * l: 4 * l + 4]
        q = oracle.gemm(h, L[0]["b_packed"], L[0]["scales"], None, G)
        h1 = oracle.rownorm(q, H)
        h2 = oracle.rownorm(oracle.gemm(h1, L[1]["b_packed"], L[1]["scales"], None, G))
        h3 = oracle.swiglu_rownorm(oracle.gemm(h2, L[2]["b_packed"], L[2]["scales"], None, G))
        h = oracle.rownorm(oracle.gemm(h3, L[3]["b_packed"], L[3]["scales"], None, G))
    assert np.array_equal(got.view(np.uint16), h.view(np.uint16))


def test_decode_step_identity_weights():
    """Identity linears (q = 8 + delta, z = 8, s = 1, G = K): every renorm sees
    the previous renorm's output, so the step equals
    rn(swiglu_rn([rn(rn(x)), rn(rn(x))])) built from the pinned pieces."""
    H, I, M = 32, 32, 2
    eye = np.eye(H, dtype=np.int64)
    ident = pack_rows(8 + eye)
    one = np.ones((1, H), np.float16)
    gate_up = pack_rows(np.concatenate([8 + eye, 8 + eye], 1))
    layers = [dict(b_packed=ident, scales=one, G=H),
              dict(b_packed=ident, scales=one, G=H),
              dict(b_packed=gate_up, scales=np.ones((1, 2 * I), np.float16), G=H),
              dict(b_packed=ident, scales=one, G=I)]
    x = synth.stack_input(M, H, seed=9)
    got = oracle.decode_step(layers, x, 1)
    r = oracle.rownorm(oracle.rownorm(x))
    want = oracle.rownorm(oracle.swiglu_rownorm(np.concatenate([r, r], 1)))
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def _glue_eps_cases():
    cases = []
    with open(os.path.join(GOLDEN, "glue_eps_cases.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            lhs, want = line.split("->")
            kind, width, pattern = lhs.split(None, 2)
            cases.append((kind, int(width), pattern.strip(), [int(w, 16) for w in want.split()]))
    return cases


@pytest.mark.parametrize("kind,width,pattern,want", _glue_eps_cases(),
                         ids=lambda v: v if isinstance(v, str) else None)
def test_glue_closed_form_with_epsilon(kind, width, pattern, want):
    """Rows whose mean square is comparable to the glue's 1e-6 term
    (tests/golden/glue_eps_cases.txt, worked out by hand): a different
    epsilon, none, or a sum in place of the mean each give other fp16 bits."""
    if kind == "rownorm":
        pat = np.array([int(w, 16) for w in pattern.split()], np.uint16)
        row = np.tile(pat, width // len(pat))[None, :]
        got = oracle.rownorm(row.view(np.float16)).view(np.uint16)[0]
        assert np.array_equal(got, np.tile(np.array(want, np.uint16), width // len(want)))
    else:
        gate, up = (int(w, 16) for w in pattern.split("/"))
        gu = np.concatenate([np.full(width, gate, np.uint16), np.full(width, up, np.uint16)])[None, :]
        got = oracle.swiglu_rownorm(gu.view(np.float16)).view(np.uint16)[0]
        assert np.all(got == want[0])


def test_parallel_helpers_equal_the_plain_calls():
    """gemm_columns (column slices on threads) and decode_layer_columns equal
    gemm and decode_step bit for bit, ragged last slice included."""
    p = synth.problem(3, 256, 1032, 64, True, seed=21)
    full = oracle.gemm(p["a"], p["b_packed"], p["scales"], p["qzeros"], 64)
    par = oracle.gemm_columns(p["a"], p["b_packed"], p["scales"], p["qzeros"], 64, cols=256)
    assert np.array_equal(full.view(np.uint16), par.view(np.uint16))
    layers = _tiny_stack(1)
    x = synth.stack_input(2, 64)
    a = oracle.decode_step(layers, x, 1)
    b = oracle.decode_layer_columns(layers, x)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
