"""Pins for the CPU oracle: it is checked against things other than itself.

Exact rational brute force, hand-derived closed forms, invariants of the
definition, library routines for the special cases, and the values the
pages print for the memory closed forms (tests/golden/table1_memory.json).
A final test plants plausible mistakes in copies of the oracle and checks
that these pins reject each one.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bruteforce as bf
from oracle import dora_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_like(rng, shape, scale):
    """Random values that are exactly representable in bf16 (small integers / 2^k)."""
    return rng.integers(-127, 128, size=shape).astype(np.float64) * scale


def _f32_like(rng, shape, scale):
    return rng.standard_normal(shape).astype(np.float32).astype(np.float64) * scale


# ---------------------------------------------------------------- norm ----

@pytest.mark.parametrize(
    "d_out,d_in,r,s,kind",
    [
        (4, 16, 3, 2.0, "bf16"),
        (8, 64, 8, 0.5, "bf16"),
        (5, 7, 9, -1.25, "f32"),      # r > d_in, negative s
        (3, 33, 1, 0.3, "f32"),       # s not a power of two
        (6, 20, 4, 0.0, "bf16"),
    ],
)
def test_dense_norm_matches_exact_bruteforce(d_out, d_in, r, s, kind):
    rng = np.random.default_rng(1234 + d_out * 7 + r)
    mk = _bf16_like if kind == "bf16" else _f32_like
    W = mk(rng, (d_out, d_in), 2.0 ** -7)
    A = mk(rng, (r, d_in), 2.0 ** -7)
    B = mk(rng, (d_out, r), 2.0 ** -9)
    exact = bf.exact_row_sq_norms(W.tolist(), A.tolist(), B.tolist(), s)
    got = O.dense_row_norm(W, A, B, s)
    got_alg = O.factored_row_norm(W, A, B, s)
    for j in range(d_out):
        ref = float(bf.exact_sqrt(exact[j]))
        assert got[j] == pytest.approx(ref, rel=1e-14, abs=0.0)
        assert got_alg[j] == pytest.approx(ref, rel=1e-12, abs=1e-300)


def test_norm_hand_worked_example():
    # W + s*B@A with s = 1/2:
    #   B@A = [[1,0,0],[0,1,1],[2,-1,-1]]
    #   W + B@A/2 = [[3.5,4,0],[1,2.5,2.5],[1,-0.5,-0.5]]
    #   squared row norms 113/4, 27/2, 3/2.
    W = np.array([[3, 4, 0], [1, 2, 2], [0, 0, 0]], float)
    A = np.array([[1, 0, 0], [0, 1, 1]], float)
    B = np.array([[1, 0], [0, 1], [2, -1]], float)
    expect_sq = [Fraction(113, 4), Fraction(27, 2), Fraction(3, 2)]
    assert bf.exact_row_sq_norms(W.tolist(), A.tolist(), B.tolist(), 0.5) == expect_sq
    got = O.dense_row_norm(W, A, B, 0.5)
    np.testing.assert_allclose(got ** 2, [float(q) for q in expect_sq], rtol=1e-15)
    base, cross, ba, G = O.factored_terms(W, A, B)
    # base = ||W_j||^2; cross = <W_j,(BA)_j>; ba = ||(BA)_j||^2, by hand:
    np.testing.assert_array_equal(base, [25, 9, 0])
    np.testing.assert_array_equal(cross, [3, 4, 0])
    np.testing.assert_array_equal(ba, [1, 2, 6])
    np.testing.assert_array_equal(G, [[1, 0], [0, 2]])


@pytest.mark.parametrize("budget_cols", [64, 128, 192, 10_000])
def test_factored_terms_add_over_any_split_of_d_in(budget_cols):
    """base, cross and G are sums over k, so the terms of the chunks of d_in
    that the pages' chunk rule cuts add up to the whole-matrix terms, and the
    norm assembled from the summed chunk terms equals the dense norm (ragged
    last chunk included)."""
    rng = np.random.default_rng(7)
    d_out, d_in, r, s = 37, 201, 13, 0.75
    W = rng.standard_normal((d_out, d_in)) / np.sqrt(d_in)
    A = rng.standard_normal((r, d_in)) / np.sqrt(d_in)
    B = rng.standard_normal((d_out, r)) * 0.02
    cs = O.chunk_size(d_out, d_in, budget_cols * 4 * d_out)
    assert cs == min(d_in, max(64, budget_cols // 64 * 64))
    base, cross, G = np.zeros(d_out), np.zeros(d_out), np.zeros((r, r))
    for c in range(0, d_in, cs):
        b_c, x_c, _, G_c = O.factored_terms(W[:, c:c + cs], A[:, c:c + cs], B)
        base, cross, G = base + b_c, cross + x_c, G + G_c
    whole = O.factored_terms(W, A, B)
    np.testing.assert_allclose(base, whole[0], rtol=1e-13)
    np.testing.assert_allclose(cross, whole[1], rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(G, whole[3], rtol=1e-13, atol=1e-15)
    ba = np.array([B[j] @ G @ B[j] for j in range(d_out)])
    np.testing.assert_allclose(np.sqrt(base + 2 * s * cross + s * s * ba), O.dense_row_norm(W, A, B, s), rtol=1e-13)
    np.testing.assert_allclose(O.factored_row_norm(W, A, B, s), O.dense_row_norm(W, A, B, s), rtol=1e-13)


def test_s_zero_is_plain_row_norm():
    rng = np.random.default_rng(3)
    W = rng.standard_normal((19, 50))
    A = rng.standard_normal((6, 50))
    B = rng.standard_normal((19, 6))
    ref = np.linalg.norm(W, axis=1)
    np.testing.assert_allclose(O.dense_row_norm(W, A, B, 0.0), ref, rtol=1e-15)
    np.testing.assert_allclose(O.factored_row_norm(W, A, B, 0.0), ref, rtol=1e-15)


@pytest.mark.parametrize("zero", ["A", "B"])
def test_zero_factor_kills_cross_and_gram(zero):
    # LoRA starts with B = 0; then W + sBA = W.
    rng = np.random.default_rng(4)
    W = rng.standard_normal((11, 40))
    A = rng.standard_normal((5, 40))
    B = rng.standard_normal((11, 5))
    if zero == "A":
        A[:] = 0.0
    else:
        B[:] = 0.0
    _, cross, ba, _ = O.factored_terms(W, A, B)
    assert np.all(cross == 0.0) and np.all(ba == 0.0)
    np.testing.assert_allclose(O.dense_row_norm(W, A, B, 1.5), np.linalg.norm(W, axis=1), rtol=1e-15)


def test_identity_A_closed_form():
    # A = [I_r | 0]: (BA)_j = [B_j, 0,...], so ||W+sBA||_j^2 = sum_{k<r}(W_jk+sB_jk)^2 + sum_{k>=r} W_jk^2.
    rng = np.random.default_rng(5)
    d_out, d_in, r, s = 9, 30, 4, -0.5
    W = rng.standard_normal((d_out, d_in))
    B = rng.standard_normal((d_out, r))
    A = np.zeros((r, d_in))
    A[:, :r] = np.eye(r)
    head = W[:, :r] + s * B
    ref = np.sqrt(np.sum(head ** 2, axis=1) + np.sum(W[:, r:] ** 2, axis=1))
    np.testing.assert_allclose(O.dense_row_norm(W, A, B, s), ref, rtol=1e-15)
    np.testing.assert_allclose(O.factored_row_norm(W, A, B, s), ref, rtol=1e-14)


def test_rank_one_and_zero_W_closed_forms():
    rng = np.random.default_rng(6)
    d_out, d_in, s = 8, 25, 1.75
    A = rng.standard_normal((1, d_in))
    B = rng.standard_normal((d_out, 1))
    W = rng.standard_normal((d_out, d_in))
    _, _, ba, G = O.factored_terms(W, A, B)
    nA2 = float(np.dot(A[0], A[0]))
    np.testing.assert_allclose(ba, B[:, 0] ** 2 * nA2, rtol=1e-14)
    np.testing.assert_allclose(G, [[nA2]], rtol=1e-15)
    W0 = np.zeros_like(W)
    ref = abs(s) * np.abs(B[:, 0]) * np.sqrt(nA2)
    np.testing.assert_allclose(O.dense_row_norm(W0, A, B, s), ref, rtol=1e-14)
    np.testing.assert_allclose(O.factored_row_norm(W0, A, B, s), ref, rtol=1e-13)


def test_rotation_invariance_and_row_permutation():
    rng = np.random.default_rng(8)
    d_out, d_in, r, s = 14, 24, 5, 0.9
    W = rng.standard_normal((d_out, d_in))
    A = rng.standard_normal((r, d_in))
    B = rng.standard_normal((d_out, r))
    Q, _ = np.linalg.qr(rng.standard_normal((d_in, d_in)))
    base = O.dense_row_norm(W, A, B, s)
    np.testing.assert_allclose(O.dense_row_norm(W @ Q, A @ Q, B, s), base, rtol=1e-13)
    np.testing.assert_allclose(O.factored_row_norm(W @ Q, A @ Q, B, s), base, rtol=1e-13)
    p = rng.permutation(d_out)
    np.testing.assert_array_equal(O.dense_row_norm(W[p], A, B[p], s), base[p])


def test_factored_terms_are_the_dense_inner_products():
    rng = np.random.default_rng(9)
    W = rng.standard_normal((10, 33))
    A = rng.standard_normal((7, 33))
    B = rng.standard_normal((10, 7))
    base, cross, ba, G = O.factored_terms(W, A, B)
    BA = np.zeros((10, 33))
    for j in range(10):              # BA row by row, as explicit sums
        for l in range(7):
            BA[j] += B[j, l] * A[l]
    np.testing.assert_allclose(base, [np.dot(w, w) for w in W], rtol=1e-14)
    np.testing.assert_allclose(cross, [np.dot(W[j], BA[j]) for j in range(10)], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ba, [np.dot(BA[j], BA[j]) for j in range(10)], rtol=1e-12)
    np.testing.assert_allclose(G, G.T, rtol=0, atol=1e-13)
    assert np.all(np.linalg.eigvalsh(G) > -1e-12)


def test_norm_clamp_and_cancellation_to_zero():
    # W = -s B A exactly: the true norm is 0.
    rng = np.random.default_rng(10)
    A = _bf16_like(rng, (3, 16), 2.0 ** -4)
    B = _bf16_like(rng, (5, 3), 2.0 ** -4)
    s = 0.5
    W = -s * (B @ A)
    assert np.all(O.dense_row_norm(W, A, B, s) == 0.0)
    alg = O.factored_row_norm(W, A, B, s)
    assert np.all(np.isfinite(alg)) and np.all(alg >= 0.0) and np.all(alg < 1e-6)


# ------------------------------------------------------- chunk + memory ----

def test_chunk_size_rule():
    MiB = 1 << 20
    assert O.chunk_size(8192, 8192, 256 * MiB) == 8192          # [d_out,cs] fp32 = 256 MiB
    assert O.chunk_size(28672, 8192, 256 * MiB) == 2304         # floor(2340.57) -> 64-aligned
    assert O.chunk_size(512, 3584, 256 * MiB) == 3584           # capped at d_in
    assert O.chunk_size(4096, 4096, 1 * MiB) == 64              # never below 64
    assert O.chunk_size(100, 40, 256 * MiB) == 40               # d_in below one chunk
    assert O.chunk_size(1000, 8192, 700_000) == 128             # 175 -> 128


def test_table1_memory_matches_printed_values():
    with open(os.path.join(GOLDEN, "table1_memory.json")) as f:
        gold = json.load(f)
    MiB = float(1 << 20)
    for c in gold["cases"]:
        mem = O.table1_memory(c["d_out"], c["d_in"], c["r"], c["elem_bytes"])
        assert mem["dense"] / MiB == c["dense_MiB"]
        assert round(mem["factored"] / MiB, 1) == c["factored_MiB"]
        assert round(mem["dense"] / mem["factored"], c["ratio_digits"]) == c["ratio_printed"]
        assert mem["gram"] / MiB == c["gram_MiB"]
        assert mem["chunk"] / MiB == c["chunk_buffer_near_MiB"]
    ub = gold["gram_upper_bound"]
    g = O.table1_memory(8192, 8192, ub["r"], ub["elem_bytes"])["gram"]
    assert g / 1e6 <= ub["at_most_MB"]


# ------------------------------------------------------------ g = m/... ----

def test_magnitude_scale_cases():
    m = np.array([2.0, 3.0, 5.0, 7.0])
    wn = np.array([4.0, 0.0, 1e-9, np.nan])
    g = O.magnitude_scale(m, wn, 1e-6)
    assert g[0] == 0.5
    assert g[1] == 3.0 / 1e-6 and g[2] == 5.0 / 1e-6
    assert np.isnan(g[3])


# -------------------------------------------------------------- compose ----

def test_compose_hand_worked_example():
    # (g-1)*base + g*s*lora with g = [1.25, 0.75], s = 2:
    #   col 0: 0.25*1 + 1.25*2*0.5 = 1.5;  col 1: -0.25*-2 + 0.75*2*4 = 6.5
    out = O.compose([[1.0, -2.0]], [[0.5, 4.0]], [1.25, 0.75], 2.0)
    np.testing.assert_array_equal(out, [[1.5, 6.5]])


def test_compose_special_cases():
    rng = np.random.default_rng(11)
    base = rng.standard_normal((6, 9))
    lora = rng.standard_normal((6, 9))
    g = 1.0 + 0.01 * rng.standard_normal(9)
    s = 0.5
    np.testing.assert_array_equal(O.compose(base, lora, np.ones(9), s), s * lora)
    np.testing.assert_array_equal(O.compose(base, lora, g, 0.0), (g - 1.0)[None] * base)
    np.testing.assert_array_equal(O.compose(base, np.zeros_like(lora), g, s), (g - 1.0)[None] * base)
    np.testing.assert_array_equal(O.compose(np.zeros_like(base), lora, g, s), g[None] * (s * lora))
    # algebraically equal to the naive form
    np.testing.assert_allclose(O.compose(base, lora, g, s), O.compose_naive(base, lora, g, s),
                               rtol=1e-9, atol=1e-14)


def test_compose_matches_exact_rational_rounding():
    rng = np.random.default_rng(12)
    n = 3000
    base = O.bf16_round(rng.standard_normal(n))
    lora = O.bf16_round(0.1 * rng.standard_normal(n))
    g = O.f32_round(1.0 + 0.0015 * rng.standard_normal(n))
    s = 0.5
    got = O.bf16_round(O.compose(base[None], lora[None], g, s))[0]
    for i in range(n):
        q = bf.exact_compose(base[i], lora[i], g[i], s)
        assert float(bf.round_fraction_bf16(q)) == got[i], i


def test_bf16_round_matches_torch_and_ties():
    rng = np.random.default_rng(13)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    # exact midpoints between neighbouring bf16 values: ties go to even
    hi = (x.view(np.uint32) & np.uint32(0xFFFF0000))
    ties = (hi | np.uint32(0x8000)).view(np.float32)
    allx = np.concatenate([x, ties, np.float32([0.0, -0.0, 1e-40, 3.0e38, -3.0e38])])
    ref = torch.from_numpy(allx).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_round(allx.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    for v in [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.1, 1.0 / 3.0]:
        assert O.bf16_round(v) == float(bf.round_fraction_bf16(Fraction(v)))


def test_f16_round_matches_exact_rounding():
    """The oracle's fp16 rounding against exact rational rounding (ties to
    even, subnormals, overflow to inf)."""
    rng = np.random.default_rng(14)
    vals = list(rng.standard_normal(300) * 3.0) + list(rng.standard_normal(50) * 1e-5)
    vals += [1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, -(1.0 + 2.0 ** -11), 65504.0, 65519.0, 65520.0,
             -65520.0, 2.0 ** -25, 3 * 2.0 ** -25, 2.0 ** -14 + 2.0 ** -25, 0.1, 1.0 / 3.0]
    for v in vals:
        want = bf.round_fraction_f16(Fraction(v))
        got = O.f16_round(v)
        assert (got == want) if isinstance(want, Fraction) else (got == want), (v, got, want)
    assert O.f16_round(1.0 + 2.0 ** -11) == 1.0 and O.f16_round(1.0 + 3 * 2.0 ** -11) == 1.0 + 2.0 ** -9
    assert O.f16_round(65520.0) == np.inf and O.f16_round(3 * 2.0 ** -25) == 2.0 ** -23


def _f32_cases():
    """Values that exercise every branch of binary32 rounding: random normals,
    exact midpoints between neighbouring binary32 values (ties), points just
    off a midpoint, subnormals and their midpoints, the overflow threshold."""
    rng = np.random.default_rng(16)
    x = rng.standard_normal(400) * 3.0
    a = (rng.standard_normal(200) * 5.0).astype(np.float32)
    nxt = np.nextafter(a, np.float32(np.inf), dtype=np.float32)
    mids = (a.astype(np.float64) + nxt.astype(np.float64)) / 2.0          # exact in fp64
    off = mids + np.abs(mids) * 2.0 ** -40
    tiny = 2.0 ** -149
    special = [tiny, 3 * tiny / 2, 5 * tiny / 2, 2.0 ** -126 - tiny / 2, 2.0 ** -150, 1.0 + 2.0 ** -24,
               1.0 + 3 * 2.0 ** -24, -(1.0 + 2.0 ** -24), 1.0 + 2.0 ** -23 + 2.0 ** -24,
               float(np.finfo(np.float32).max), 2.0 ** 128 - 2.0 ** 103, 2.0 ** 128 - 2.0 ** 103 - 2.0 ** 80,
               -(2.0 ** 128), 0.1, 1.0 / 3.0, 0.0]
    return list(x) + list(mids) + list(off) + special


def _exact_f32(v):
    want = bf.round_fraction_f32(Fraction(v))
    return float(want)


def test_f32_round_matches_exact_rounding():
    """The oracle's binary32 rounding against exact rational rounding on
    integers: 24 significant bits, ties to even, subnormal spacing 2^-149,
    overflow to inf at the midpoint above the largest finite value."""
    for v in _f32_cases():
        assert O.f32_round(v) == _exact_f32(v), v
    assert O.f32_round(1.0 + 2.0 ** -24) == 1.0                       # tie to even (down)
    assert O.f32_round(1.0 + 3 * 2.0 ** -24) == 1.0 + 2.0 ** -22       # tie to even (up)
    assert O.f32_round(3 * 2.0 ** -150) == 2.0 ** -148                 # subnormal tie to even
    assert O.f32_round(2.0 ** 128 - 2.0 ** 103) == np.inf              # midpoint past the max
    assert O.f32_round(2.0 ** 128 - 2.0 ** 103 - 2.0 ** 80) == float(np.finfo(np.float32).max)


def _compose_f32_cases():
    rng = np.random.default_rng(17)
    n = 400
    base = O.bf16_round(rng.standard_normal(n))
    lora = O.bf16_round(0.1 * rng.standard_normal(n))
    g = O.f32_round(1.0 + 0.0015 * rng.standard_normal(n))
    # generic fp64 inputs too (they are rounded to binary32 on entry)
    base2 = rng.standard_normal(n) * 3.0
    lora2 = rng.standard_normal(n)
    g2 = 1.0 + 0.3 * rng.standard_normal(n)
    return [(base, lora, g, 0.5), (base2, lora2, g2, 0.3), (base, lora, g, 16.0 / np.sqrt(384.0))]


@pytest.mark.parametrize("form", ["stable", "naive"])
def test_compose_f32_forms_match_exact_per_operation_rounding(form):
    """The binary32 compose forms against exact rational arithmetic with one
    binary32 rounding after each operation (inputs rounded on entry)."""
    fn = O.compose_f32_stable if form == "stable" else O.compose_f32_naive
    ex = bf.exact_compose_f32_stable if form == "stable" else bf.exact_compose_f32_naive
    for base, lora, g, s in _compose_f32_cases():
        got = np.asarray(fn(base[None], lora[None], g, s), dtype=np.float64)[0]
        for i in range(len(base)):
            assert got[i] == float(ex(base[i], lora[i], g[i], s)), (form, i)


def test_f32_pins_reject_planted_mistakes():
    """Plausible mistakes in the binary32 helpers each fail a pin above."""
    cases = _f32_cases()

    def round_ok(fn):
        return all(fn(v) == _exact_f32(v) for v in cases)

    def to16(v):
        with np.errstate(over="ignore"):
            return float(np.float64(v).astype(np.float16))

    round_mutants = {
        "fp16 cast": to16,
        "no rounding": lambda v: float(v),
        "bf16 rounding": lambda v: float(O.bf16_round(v)),
        "toward zero": lambda v: (lambda r: float(np.nextafter(np.float32(r), np.float32(0)))
                                  if abs(r) > abs(v) else r)(float(O.f32_round(v))),
    }
    assert round_ok(lambda v: float(O.f32_round(v)))
    for name, fn in round_mutants.items():
        assert not round_ok(fn), name

    def compose_ok(fn):
        for base, lora, g, s in _compose_f32_cases():
            got = np.asarray(fn(base[None], lora[None], g, s), dtype=np.float64)[0]
            if not all(got[i] == float(bf.exact_compose_f32_stable(base[i], lora[i], g[i], s))
                       for i in range(len(base))):
                return False
        return True

    f = np.float32
    compose_mutants = {
        "fp64 evaluation": lambda b, l, g, s: O.compose(b, l, g, s),
        "fp16 inputs": lambda b, l, g, s: O.compose_f32_stable(O.f16_round(b), O.f16_round(l), g, s),
        "fused g*(s*lora) + (g-1)*base": lambda b, l, g, s: O.f32_round(
            np.asarray(g, f)[None].astype(np.float64) * (f(s) * np.asarray(l, f)).astype(np.float64)
            + ((np.asarray(g, f) - f(1))[None] * np.asarray(b, f)).astype(np.float64)),
        "naive form": O.compose_f32_naive,
    }
    assert compose_ok(O.compose_f32_stable)
    for name, fn in compose_mutants.items():
        assert not compose_ok(fn), name


def test_stable_compose_beats_naive_near_one():
    # Near g = 1 the naive form cancels; the stable form keeps (g-1) explicit.
    rng = np.random.default_rng(14)
    T, d = 512, 1024
    base = O.bf16_round(rng.standard_normal((T, d)))
    lora = O.bf16_round(0.1 * rng.standard_normal((T, d)))
    g = O.f32_round(1.0 + 0.0015 * rng.standard_normal(d))
    s = 0.5
    ref = O.compose(base, lora, g, s)
    e_st = np.max(np.abs(O.compose_f32_stable(base, lora, g, s) - ref))
    e_nv = np.max(np.abs(O.compose_f32_naive(base, lora, g, s) - ref))
    assert e_st < e_nv / 2


# ----------------------------------------------------- compose backward ----

def test_compose_backward_matches_finite_differences():
    """The delta is linear in base, lora and g separately, so central
    differences of L = sum(dy * delta) are exact up to fp64 rounding."""
    rng = np.random.default_rng(21)
    T, d, s = 5, 7, 0.75
    dy, base, lora = (rng.standard_normal((T, d)) for _ in range(3))
    g = 1.0 + 0.1 * rng.standard_normal(d)
    d_base, d_lora, dg = O.compose_backward(dy, base, lora, g, s)

    def loss(b, l, gg):
        return float(np.sum(dy * O.compose(b, l, gg, s)))

    h = 1e-3
    for (t, j) in [(0, 0), (2, 3), (4, 6)]:
        e = np.zeros((T, d))
        e[t, j] = h
        fd_b = (loss(base + e, lora, g) - loss(base - e, lora, g)) / (2 * h)
        fd_l = (loss(base, lora + e, g) - loss(base, lora - e, g)) / (2 * h)
        assert abs(fd_b - d_base[t, j]) <= 1e-9 and abs(fd_l - d_lora[t, j]) <= 1e-9
    for j in range(d):
        e = np.zeros(d)
        e[j] = h
        fd_g = (loss(base, lora, g + e) - loss(base, lora, g - e)) / (2 * h)
        assert abs(fd_g - dg[j]) <= 1e-9 * max(1.0, abs(dg[j]))


def test_compose_backward_exact_and_special_cases():
    rng = np.random.default_rng(22)
    T, d = 6, 5
    dy = O.bf16_round(rng.standard_normal((T, d)))
    base = O.bf16_round(rng.standard_normal((T, d)))
    lora = O.bf16_round(0.1 * rng.standard_normal((T, d)))
    g = O.f32_round(1.0 + 0.0015 * rng.standard_normal(d))
    s = 0.5
    d_base, d_lora, dg = O.compose_backward(dy, base, lora, g, s)
    # exact rational arithmetic on the storage values
    for j in range(d):
        gj = Fraction(float(g[j]))
        acc = Fraction(0)
        for t in range(T):
            y = Fraction(float(dy[t, j]))
            assert Fraction(float(d_base[t, j])) == (gj - 1) * y
            assert Fraction(float(d_lora[t, j])) == gj * Fraction(s) * y
            acc += y * (Fraction(float(base[t, j])) + Fraction(s) * Fraction(float(lora[t, j])))
        assert abs(float(acc) - dg[j]) <= 4 * np.finfo(np.float64).eps * float(sum(
            abs(Fraction(float(dy[t, j]))) * (abs(Fraction(float(base[t, j]))) + abs(Fraction(float(lora[t, j]))))
            for t in range(T)))
    # g = 1: no base gradient, lora gradient s * dy
    d_base1, d_lora1, _ = O.compose_backward(dy, base, lora, np.ones(d), s)
    assert np.all(d_base1 == 0) and np.array_equal(d_lora1, s * dy)
    # s = 0: no lora gradient, dg = sum dy * base
    _, d_lora0, dg0 = O.compose_backward(dy, base, lora, g, 0.0)
    assert np.all(d_lora0 == 0)
    np.testing.assert_allclose(dg0, np.sum(dy * base, axis=0), rtol=1e-15)
    # dm = dg / max(wnorm, eps), and the eps floor
    wn = np.array([2.0, 0.5, 0.0, 1e-9, 4.0])
    *_, dm = O.compose_backward(dy, base, lora, g, s, wnorm=wn, eps=1e-6)
    np.testing.assert_array_equal(dm, dg / np.array([2.0, 0.5, 1e-6, 1e-6, 4.0]))


# ------------------------------------------------------ planted mistakes ----

def test_layer_output_and_linear_hand_worked():
    """Hand-worked: B = 0, W = [3, 4], m = 10: the weight is renormalised to
    10 * [3, 4] / 5 = [6, 8], so x = [1, 2] gives 1*6 + 2*8 = 22. With
    W = [3, 0], A = [0, 1], B = [4], s = 1 the direction is [3, 4], its norm
    5 = m, so g = 1 and x = [1, 1] gives 3 + 4 = 7."""
    y = O.dora_linear(np.array([[1.0, 2.0]]), np.array([[3.0, 4.0]]), np.array([[1.0, 0.0]]),
                      np.array([[0.0]]), np.array([10.0]), 1.0, 1e-6)
    assert y.shape == (1, 1) and y[0, 0] == 22.0
    y = O.dora_linear(np.array([[1.0, 1.0]]), np.array([[3.0, 0.0]]), np.array([[0.0, 1.0]]),
                      np.array([[4.0]]), np.array([5.0]), 1.0, 1e-6)
    assert y[0, 0] == 7.0
    # layer output: base 2, lora 6, g = 1.5, s = 0.5 -> 2 + (0.5 * 2 + 1.5 * 3) = 7.5
    assert O.layer_output(np.array([[2.0]]), np.array([[6.0]]), np.array([1.5]), 0.5)[0, 0] == 7.5


def test_linear_weight_space_equals_activation_space():
    """The weight-space definition (dense V, normalised rows) equals the
    activation-space route base + compose(x W^T, x A^T B^T, g) with g from the
    row norm; and layer_output = g * (base + s * lora) exactly in algebra."""
    rng = np.random.default_rng(3)
    T, d_out, d_in, r, s, eps = 7, 11, 13, 4, 0.75, 1e-6
    x = rng.standard_normal((T, d_in))
    W = rng.standard_normal((d_out, d_in)) / 4
    A = rng.standard_normal((r, d_in)) / 4
    B = rng.standard_normal((d_out, r)) / 4
    m = rng.uniform(0.5, 2.0, d_out)
    y = O.dora_linear(x, W, A, B, m, s, eps)
    g = O.magnitude_scale(m, O.dense_row_norm(W, A, B, s), eps)
    base, lora = x @ W.T, (x @ A.T) @ B.T
    y2 = O.layer_output(base, lora, g, s)
    np.testing.assert_allclose(y, y2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y2, g[None, :] * (base + s * lora), rtol=1e-13, atol=1e-13)
    # m = ||V||: g = 1 and the layer is the plain LoRA layer x W^T + s x A^T B^T
    y1 = O.dora_linear(x, W, A, B, O.dense_row_norm(W, A, B, s), s, eps)
    np.testing.assert_allclose(y1, base + s * lora, rtol=1e-12, atol=1e-12)


def test_linear_without_adapter_is_weight_normalisation():
    """B = 0 (the LoRA initialisation) leaves weight normalisation: each output
    row j is m_j * <x, w_j> / ||w_j||, computed here one row at a time."""
    rng = np.random.default_rng(4)
    T, d_out, d_in, r = 5, 6, 9, 3
    x = rng.standard_normal((T, d_in))
    W = rng.standard_normal((d_out, d_in))
    m = rng.uniform(0.5, 2.0, d_out)
    y = O.dora_linear(x, W, rng.standard_normal((r, d_in)), np.zeros((d_out, r)), m, 2.0, 1e-6)
    for j in range(d_out):
        wj = W[j]
        nrm = np.sqrt(sum(v * v for v in wj))
        for t in range(T):
            assert abs(y[t, j] - m[j] * sum(a * b for a, b in zip(x[t], wj)) / nrm) <= 1e-12 * (1 + abs(y[t, j]))


def test_pins_reject_planted_mistakes():
    """Each mutant of the oracle must fail at least one of the checks above."""
    rng = np.random.default_rng(15)
    W = _bf16_like(rng, (4, 12), 2.0 ** -6)
    A = _bf16_like(rng, (3, 12), 2.0 ** -6)
    B = _bf16_like(rng, (4, 3), 2.0 ** -6)
    s = 0.5
    exact = np.array([float(bf.exact_sqrt(q)) for q in bf.exact_row_sq_norms(W.tolist(), A.tolist(), B.tolist(), s)])

    def norm_ok(fn):
        return np.allclose(fn(W, A, B, s), exact, rtol=1e-12, atol=0)

    norm_mutants = {
        "minus sign": lambda W, A, B, s: O.dense_row_norm(W, A, -B, s),
        "dropped s": lambda W, A, B, s: O.dense_row_norm(W, A, B, 1.0),
        "transposed product": lambda W, A, B, s: np.sqrt(np.sum((W + s * (B @ A)[::-1]) ** 2, 1)),
        "cross without 2": lambda W, A, B, s: np.sqrt(
            (lambda t: t[0] + s * t[1] + s * s * t[2])(O.factored_terms(W, A, B))),
        "no gram term": lambda W, A, B, s: np.sqrt(
            (lambda t: t[0] + 2 * s * t[1])(O.factored_terms(W, A, B))),
        "s instead of s^2": lambda W, A, B, s: np.sqrt(
            (lambda t: t[0] + 2 * s * t[1] + s * t[2])(O.factored_terms(W, A, B))),
    }
    assert norm_ok(O.dense_row_norm) and norm_ok(O.factored_row_norm)
    for name, fn in norm_mutants.items():
        assert not norm_ok(fn), name

    base = np.array([[1.0, -2.0]])
    lora = np.array([[0.5, 4.0]])
    gg = np.array([1.25, 0.75])

    def compose_ok(fn):
        return (np.array_equal(fn(base, lora, gg, 2.0), [[1.5, 6.5]])
                and np.array_equal(fn(base, lora, np.ones(2), 2.0), 2.0 * lora))

    compose_mutants = {
        "g+1": lambda b, l, g, s: (g[None] + 1) * b + g[None] * s * l,
        "dropped s": lambda b, l, g, s: (g[None] - 1) * b + g[None] * l,
        "dropped g on lora": lambda b, l, g, s: (g[None] - 1) * b + s * l,
        "returns output not delta": lambda b, l, g, s: g[None] * (s * l + b),
    }
    assert compose_ok(O.compose)
    for name, fn in compose_mutants.items():
        assert not compose_ok(fn), name

    # The compose backward: finite differences of the forward oracle catch
    # each planted mistake.
    dy = rng.standard_normal((3, 4))
    b3, l3 = rng.standard_normal((3, 4)), rng.standard_normal((3, 4))
    g3 = 1.0 + 0.1 * rng.standard_normal(4)

    def backward_ok(fn):
        d_base, d_lora, dg = fn(dy, b3, l3, g3, 0.75)
        h = 1e-3

        def loss(b, l, g):
            return float(np.sum(dy * O.compose(b, l, g, 0.75)))
        e = np.zeros((3, 4))
        e[1, 2] = h
        ok = abs((loss(b3 + e, l3, g3) - loss(b3 - e, l3, g3)) / (2 * h) - d_base[1, 2]) < 1e-9
        ok &= abs((loss(b3, l3 + e, g3) - loss(b3, l3 - e, g3)) / (2 * h) - d_lora[1, 2]) < 1e-9
        eg = np.zeros(4)
        eg[3] = h
        ok &= abs((loss(b3, l3, g3 + eg) - loss(b3, l3, g3 - eg)) / (2 * h) - dg[3]) < 1e-9
        return bool(ok)

    def mut(kind):
        def fn(dy, b, l, g, s):
            d_base, d_lora, dg = O.compose_backward(dy, b, l, g, s)
            if kind == "g instead of g-1":
                d_base = g[None] * dy
            elif kind == "dropped s on lora":
                d_lora = g[None] * dy
            elif kind == "dg without lora":
                dg = np.sum(dy * b, axis=0)
            elif kind == "s on base in dg":
                dg = np.sum(dy * (l + s * b), axis=0)
            return d_base, d_lora, dg
        return fn

    assert backward_ok(O.compose_backward)
    for kind in ("g instead of g-1", "dropped s on lora", "dg without lora", "s on base in dg"):
        assert not backward_ok(mut(kind)), kind

    # The linear layer: the hand-worked example and the weight-space /
    # activation-space identity catch each planted mistake.
    xs = rng.standard_normal((3, 5))
    Ws, As, Bs = rng.standard_normal((4, 5)), rng.standard_normal((2, 5)), rng.standard_normal((4, 2))
    ms = rng.uniform(0.5, 2.0, 4)

    def linear_ok(fn):
        hand = fn(np.array([[1.0, 2.0]]), np.array([[3.0, 4.0]]), np.array([[1.0, 0.0]]),
                  np.array([[0.0]]), np.array([10.0]), 1.0, 1e-6)[0, 0] == 22.0
        gs = O.magnitude_scale(ms, O.dense_row_norm(Ws, As, Bs, 0.5), 1e-6)
        ref = O.layer_output(xs @ Ws.T, (xs @ As.T) @ Bs.T, gs, 0.5)
        return bool(hand and np.allclose(fn(xs, Ws, As, Bs, ms, 0.5, 1e-6), ref, rtol=1e-12, atol=1e-12))

    def lin_mut(kind):
        def fn(x, W, A, B, m, s, eps):
            V = W + (1.0 if kind == "dropped s" else s) * (B @ A)
            wn = np.sqrt(np.sum((W if kind == "norm of W" else V) ** 2, axis=1))
            scale = (np.ones_like(m) if kind == "dropped magnitude" else m) / wn
            return x @ (scale[:, None] * (W if kind == "product with W" else V)).T
        return fn

    assert linear_ok(O.dora_linear)
    for kind in ("dropped s", "norm of W", "dropped magnitude", "product with W"):
        assert not linear_ok(lin_mut(kind)), kind
