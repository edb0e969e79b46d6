"""Pins of the oracle's GEMM functions (CPU only).

Each test checks an oracle function against something other than itself:
exact rational arithmetic, a library routine, a hand-derived value, or a
property the pages and IEEE arithmetic fix.

Pages: NVIDIA Technical Blog "Unlocking Tensor Core Performance for Machine
Learning Interatomic Potentials" (Fig. 1 caption: three scaled BF16 components,
nine products, five anti-diagonal bands added into an FP32 accumulator; the
TF32x3 equation under Fig. 2; "Limitations and decision criteria": BF16x9
matched or beat native FP32 accuracy against an FP64 reference), and the
discuss.pytorch.kr summary (BF16x9 section: x = x0 + 2^-8 x1 + 2^-16 x2,
bands added smallest first).
"""
from fractions import Fraction
import math

import numpy as np
import pytest

U = 2.0 ** -24  # FP32 unit roundoff


def _rng(seed):
    return np.random.Generator(np.random.Philox(key=seed))


def _exp_range_values(g, shape, emin=-30, emax=30):
    """24-bit integers times 2^e: exactly representable, exact products in double."""
    m = g.integers(-(1 << 24) + 1, 1 << 24, size=shape).astype(np.float64)
    e = g.integers(emin, emax + 1, size=shape)
    return np.ldexp(m, e - 23).astype(np.float32)


# ---------------------------------------------------------------- FP64 reference

def test_gemm_f64_vs_exact_rationals_all_small_shapes(orc):
    """Every shape with M, N, K <= 8 (K >= 1): C_ref within (K-1) 2^-53 G of the
    exact rational sum, and G within the same of the exact sum of |a b|."""
    g = _rng(11)
    for M in range(1, 9):
        for N in range(1, 9):
            for K in range(1, 9):
                A = _exp_range_values(g, (M, K))
                B = _exp_range_values(g, (K, N))
                C, G = orc.gemm_f64(A, B)
                for i in range(M):
                    for j in range(N):
                        ex = sum(Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(K))
                        ga = sum(abs(Fraction(float(A[i, k])) * Fraction(float(B[k, j]))) for k in range(K))
                        tol = (K - 1) * 2.0 ** -53 * float(ga)
                        assert abs(Fraction(C[i, j]) - ex) <= Fraction(tol)
                        assert abs(Fraction(G[i, j]) - ga) <= Fraction(tol)


def test_gemm_f64_small_integers_exact(orc):
    g = _rng(12)
    A = g.integers(-1000, 1000, size=(17, 23)).astype(np.float32)
    B = g.integers(-1000, 1000, size=(23, 9)).astype(np.float32)
    C, G = orc.gemm_f64(A, B)
    exact = A.astype(np.int64) @ B.astype(np.int64)
    assert np.array_equal(C, exact.astype(np.float64))
    assert np.array_equal(G, (np.abs(A.astype(np.int64)) @ np.abs(B.astype(np.int64))).astype(np.float64))


def test_gemm_f64_vs_numpy_float64(orc):
    g = _rng(13)
    A = g.standard_normal((64, 300)).astype(np.float32)
    B = g.standard_normal((300, 70)).astype(np.float32)
    C, G = orc.gemm_f64(A, B)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    assert np.all(np.abs(C - ref) <= 2 * 300 * 2.0 ** -53 * G)


def test_gemm_f64_row_sampling(orc):
    g = _rng(14)
    A = g.standard_normal((40, 33)).astype(np.float32)
    B = g.standard_normal((33, 21)).astype(np.float32)
    full, Gf = orc.gemm_f64(A, B)
    rows = np.array([39, 0, 7, 7])
    part, Gp = orc.gemm_f64(A, B, rows=rows)
    assert np.array_equal(part, full[rows]) and np.array_equal(Gp, Gf[rows])


# ---------------------------------------------------------------- naive FP32

def test_naive_f32_sequential_rounding_order(orc):
    """1 + 2^-24 rounds to 1 (tie to even) before the next 2^-24 arrives."""
    B = np.ones((3, 1), np.float32)
    fwd = orc.sgemm_naive_f32(np.array([[1.0, U, U]], np.float32), B)
    rev = orc.sgemm_naive_f32(np.array([[U, U, 1.0]], np.float32), B)
    assert fwd[0, 0] == np.float32(1.0)
    assert rev[0, 0] == np.float32(1.0 + 2.0 ** -23)


def test_naive_f32_no_fused_multiply_add(orc):
    """(1+2^-12)^2 = 1 + 2^-11 + 2^-24 rounds to 1 + 2^-11 before the add, so the
    sum with -(1 + 2^-11) is 0; a fused multiply-add would give 2^-24."""
    a = np.array([[-(1.0 + 2.0 ** -11), 1.0 + 2.0 ** -12]], np.float32)
    b = np.array([[1.0], [1.0 + 2.0 ** -12]], np.float32)
    assert orc.sgemm_naive_f32(a, b)[0, 0] == 0.0
    assert orc.gemm_f64(a, b)[0][0, 0] == 2.0 ** -24


def test_naive_f32_within_recursive_summation_bound(orc):
    g = _rng(15)
    A = g.standard_normal((50, 513)).astype(np.float32)
    B = g.standard_normal((513, 40)).astype(np.float32)
    C = orc.sgemm_naive_f32(A, B)
    ref, G = orc.gemm_f64(A, B)
    assert np.all(np.abs(C - ref) <= 513 * U * G * 1.0001)
    assert np.array_equal(orc.sgemm_naive_f32(A, B, rows=[3, 1]), C[[3, 1]])


# ---------------------------------------------------------------- emulation

def _full24(g, shape):
    """Values whose significands use all 24 bits (all three components nonzero)."""
    m = g.integers(1 << 23, 1 << 24, size=shape) | 1
    s = np.where(g.integers(0, 2, size=shape) == 1, -1.0, 1.0)
    e = g.integers(-20, 20, size=shape)
    return (s * np.ldexp(m.astype(np.float64), e - 23)).astype(np.float32)


@pytest.mark.parametrize("nbands", [3, 4, 5])
def test_emu_identity_left_and_right(orc, nbands):
    """A = I gives C = B and B = I gives C = A bit for bit: the bands then hold
    the components themselves and the scaled recombination is exact."""
    g = _rng(21)
    X = _full24(g, (24, 24))
    I = np.eye(24, dtype=np.float32)
    assert np.array_equal(orc.gemm_emu(I, X, nbands).view(np.uint32), X.view(np.uint32))
    assert np.array_equal(orc.gemm_emu(X, I, nbands).view(np.uint32), X.view(np.uint32))


@pytest.mark.parametrize("nbands,bound", [(1, 2.0 ** -6), (2, 2.0 ** -15)])
def test_emu_identity_dropped_bands(orc, nbands, bound):
    """With A = I and b < 3 bands, C keeps x0 (and 2^-8 x1): |B - C| < bound |B|,
    C has B's sign and |C| <= |B| (the split truncates)."""
    g = _rng(22)
    X = _full24(g, (16, 16))
    C = orc.gemm_emu(np.eye(16, dtype=np.float32), X, nbands).astype(np.float64)
    Xd = X.astype(np.float64)
    assert np.all(np.abs(Xd - C) < bound * np.abs(Xd))
    assert np.all(np.abs(C) <= np.abs(Xd)) and np.all(np.sign(C) == np.sign(Xd))
    assert np.any(C != Xd)


def test_emu_scaled_permutation_exact(orc):
    """A = P D with D a diagonal of powers of two: C = P D B exactly."""
    g = _rng(23)
    n = 32
    P = np.eye(n, dtype=np.float32)[g.permutation(n)]
    D = np.diag(np.ldexp(1.0, g.integers(-10, 10, size=n))).astype(np.float32)
    A = P @ D
    B = _full24(g, (n, 20))
    assert np.array_equal(orc.gemm_emu(A, B), (A.astype(np.float64) @ B.astype(np.float64)).astype(np.float32))


@pytest.mark.parametrize("nbands", [3, 4, 5])
def test_emu_small_integers_exact(orc, nbands):
    """Integers below 2^10 with K <= 16: every band sum and the recombination are
    exact, so C equals the exact integer product (bands 0-2 are used)."""
    g = _rng(24)
    A = g.integers(-1023, 1024, size=(20, 16)).astype(np.float32)
    B = g.integers(-1023, 1024, size=(16, 12)).astype(np.float32)
    C = orc.gemm_emu(A, B, nbands)
    assert np.array_equal(C, (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float32))


def _lsb_exponent(v: Fraction) -> int:
    """Exponent of the lowest set bit of a dyadic rational."""
    num, den = v.numerator, v.denominator
    e = -(den.bit_length() - 1)
    num = abs(num)
    while num % 2 == 0:
        num //= 2
        e += 1
    return e


@pytest.mark.parametrize("lo,hi,emax,K,min_certified", [
    (1 << 15, 1 << 16, 0, 32, 3.0),      # 16-bit integers: bands 0-2 always certified
    (1, 1 << 20, 3, 32, 1.0),            # up to 20-bit integers times 2^e, e in [-3, 3]
    (1 << 23, 1 << 24, 0, 2, 1.0),       # full 24-bit significands, all five bands used
])
def test_emu_band_sums_exact_class(orc, lo, hi, emax, K, min_certified):
    """Integer significands times 2^e.  Where every term of a band is a multiple
    of one quantum q and the band's absolute sum is below 2^24 q, the band's
    FP32 sum is exact in any order: there the oracle's band sums must equal the
    exact rational band sums computed here term by term from the components."""
    g = _rng(25 + K + emax)
    M, N = 6, 5

    def draw(shape):
        m = g.integers(lo, hi, size=shape).astype(np.float64)
        m *= np.where(g.integers(0, 2, size=shape) == 1, -1.0, 1.0)
        return np.ldexp(m, g.integers(-emax, emax + 1, size=shape)).astype(np.float32)

    A, B = draw((M, K)), draw((K, N))
    C, S = orc.gemm_emu(A, B, 5, want_bands=True)
    Ac = [Fraction_matrix(np.array(c, np.uint32).__lshift__(16).view(np.float32)) for c in orc.split(A)]
    Bc = [Fraction_matrix(np.array(c, np.uint32).__lshift__(16).view(np.float32)) for c in orc.split(B)]
    certified = 0
    for i in range(M):
        for j in range(N):
            for s in range(5):
                terms = [Ac[p][i][k] * Bc[s - p][k][j] for k in range(K) for p in range(3) if 0 <= s - p < 3]
                nz = [t for t in terms if t != 0]
                if not nz:
                    assert S[s, i, j] == 0.0
                    continue
                q = min(_lsb_exponent(t) for t in nz)
                if sum(abs(t) for t in nz) < Fraction(2) ** (24 + q):
                    certified += 1
                    assert Fraction(float(S[s, i, j])) == sum(nz)
    assert certified >= min_certified * M * N


def _bf16_fraction(h):
    return Fraction(float(np.array([h], np.uint32).__lshift__(16).view(np.float32)[0]))


def Fraction_matrix(X):
    return [[Fraction(float(v)) for v in row] for row in X]


def test_emu_recombination_smallest_band_first(orc):
    """Hand-built row whose bands hold S0 = 1 + 2^-7 + 2^-16, S1 = 2^-7 + 2^-16,
    S2 = 2^-8 exactly.  Adding the weighted bands smallest first gives the exact
    1 + 2^-7 + 2^-15 + 2^-16 + 2^-23; adding S0 first would lose two 2^-24 halves
    to ties-to-even and give 1 + 2^-7 + 2^-15 + 2^-16."""
    a = np.array([[1.0, 2.0 ** -16 + 2.0 ** -24, 2.0 ** -7 + 2.0 ** -15 + 2.0 ** -24]], np.float32)
    b = np.ones((3, 1), np.float32)
    C, S = orc.gemm_emu(a, b, 5, want_bands=True)
    assert S[:, 0, 0].tolist() == [1.0 + 2.0 ** -7 + 2.0 ** -16, 2.0 ** -7 + 2.0 ** -16, 2.0 ** -8, 0.0, 0.0]
    assert C[0, 0] == np.float32(1.0 + 2.0 ** -7 + 2.0 ** -15 + 2.0 ** -16 + 2.0 ** -23)


def test_emu_special_values(orc):
    """IEEE rules applied to the components: Inf times a component that is zero
    gives NaN, so Inf * 1.0 (components 1, 0, 0) is NaN while Inf * pi (three
    nonzero positive components) is +Inf; NaN propagates; zeros give zero."""
    inf, nan = np.float32(np.inf), np.float32(np.nan)
    pi = np.float32(np.pi)
    cases = [(inf, pi, "+inf"), (inf, -pi, "-inf"), (-inf, pi, "-inf"), (inf, np.float32(1.0), "nan"),
             (nan, pi, "nan"), (np.float32(0.0), pi, "zero"), (np.float32(2.0), pi, "finite")]
    for a, b, want in cases:
        c = orc.gemm_emu(np.array([[a]], np.float32), np.array([[b]], np.float32))[0, 0]
        got = "nan" if np.isnan(c) else "+inf" if c == np.inf else "-inf" if c == -np.inf else \
              "zero" if c == 0 else "finite"
        assert got == want, (a, b, c)


def test_emu_tolerance_and_normwise_vs_naive(orc):
    """Elementwise |C - C_ref| <= 2 K 2^-24 G and normwise error no worse than
    twice naive FP32 ("Limitations and decision criteria": BF16x9 matched or
    beat native FP32 against an FP64 reference)."""
    g = _rng(26)
    for (M, N, K) in [(33, 47, 129), (64, 64, 1024), (5, 3, 1)]:
        A = g.standard_normal((M, K)).astype(np.float32)
        B = g.standard_normal((K, N)).astype(np.float32)
        C = orc.gemm_emu(A, B).astype(np.float64)
        ref, G = orc.gemm_f64(A, B)
        assert np.all(np.abs(C - ref) <= 2 * K * U * G)
        naive = orc.sgemm_naive_f32(A, B).astype(np.float64)
        e_emu = np.linalg.norm(C - ref) / np.linalg.norm(ref)
        e_nai = np.linalg.norm(naive - ref) / np.linalg.norm(ref)
        assert e_emu <= 2 * e_nai + 1e-300


@pytest.mark.parametrize("nbands,bound", [(1, 2.0 ** -6 + 2.0 ** -13 + 2.0 ** -21 + 2.0 ** -30),
                                          (2, 2.0 ** -13 + 2.0 ** -21 + 2.0 ** -30),
                                          (3, 2.0 ** -21 + 2.0 ** -30), (4, 2.0 ** -30)])
def test_emu_band_drop_bounds(orc, nbands, bound):
    """Keeping bands s < b drops at most bound_b sum|a b| per element (from
    |x1|, |x2| < 2|x|), plus the FP32 accumulation error."""
    g = _rng(27)
    M, N, K = 24, 31, 200
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = orc.gemm_emu(A, B, nbands).astype(np.float64)
    ref, G = orc.gemm_f64(A, B)
    assert np.all(np.abs(C - ref) <= (bound + 2 * K * U) * G)
    T = orc.gemm_trunc_f64(A, B, nbands)
    assert np.all(np.abs(T - ref) <= bound * G)
    assert np.all(np.abs(C - T) <= 2 * K * U * G)


def test_emu_three_product_form_is_tf32x3_shape(orc):
    """nbands = 2 keeps exactly a0 b0 + 2^-8 (a0 b1 + a1 b0): hi*hi + hi*lo + lo*hi
    with hi = x0 and lo = 2^-8 x1 (the TF32x3 equation's form)."""
    g = _rng(28)
    a = _full24(g, (1, 1))
    b = _full24(g, (1, 1))
    T = orc.gemm_trunc_f64(a, b, 2)[0, 0]
    (a0, a1, _), (b0, b1, _) = [[_bf16_fraction(c[0, 0]) for c in orc.split(x)] for x in (a, b)]
    hi_a, lo_a, hi_b, lo_b = a0, a1 / 256, b0, b1 / 256
    assert Fraction(T) == hi_a * hi_b + hi_a * lo_b + lo_a * hi_b


def test_emu_row_sampling_and_empty(orc):
    g = _rng(29)
    A = g.standard_normal((30, 17)).astype(np.float32)
    B = g.standard_normal((17, 11)).astype(np.float32)
    full = orc.gemm_emu(A, B)
    assert np.array_equal(orc.gemm_emu(A, B, rows=[29, 2]), full[[29, 2]])
    z = orc.gemm_emu(np.zeros((4, 0), np.float32), np.zeros((0, 3), np.float32))
    assert z.shape == (4, 3) and np.all(z == 0)


# ---------------------------------------------------------------- GELU

# Standard normal CDF values from tables (Phi(z), z = -10, -6, -3, -1, 1, 2):
# GELU(z) = z Phi(z) exactly, so these pin the oracle independently of how it
# evaluates Phi, including the far tail where 1 + erf(.) cancels to 0.
PHI_TABLE = [(-10.0, 7.61985302416047e-24), (-6.0, 9.865876450376981e-10), (-3.0, 1.3498980316300946e-03),
             (-1.0, 0.15865525393145707), (1.0, 0.8413447460685429), (2.0, 0.9772498680518208)]


def test_gelu_vs_tabulated_normal_cdf():
    import oracle
    z = np.array([v for v, _ in PHI_TABLE])
    y = oracle.gelu_f64_to_f32(z)
    want = np.array([np.float32(v * p) for v, p in PHI_TABLE])
    assert np.all(np.abs(y.astype(np.float64) - want.astype(np.float64)) <= 2.0 ** -23 * np.abs(want))
    x = np.array([-0.5, -1e-3, 0.0, 1e-3, 0.5, 2.5, 7.0, 30.0])
    y = oracle.gelu_f64_to_f32(x)
    assert y[2] == 0.0 and y[-1] == np.float32(30.0)
    # near zero GELU(x) = x/2 + x^2/sqrt(2 pi) + O(x^4)
    assert abs(float(y[1]) - (-5e-4 + 1e-6 / math.sqrt(2 * math.pi))) <= 1e-10
    assert abs(float(y[3]) - (5e-4 + 1e-6 / math.sqrt(2 * math.pi))) <= 1e-10
    # GELU(x) - GELU(-x) = x, since erf is odd
    xs = np.array([0.25, 0.5, 1.0, 2.0, 3.0])
    d = oracle.gelu_f64_to_f32(xs).astype(np.float64) - oracle.gelu_f64_to_f32(-xs).astype(np.float64)
    assert np.allclose(d, xs, rtol=1e-6, atol=0)


# ---------------------------------------------------------------- round-to-nearest split (ablation)

@pytest.mark.parametrize("nbands", [3, 4, 5])
def test_emu_rne_identity_exact(orc, nbands):
    """With the round-to-nearest split, A = I still gives C = B: the components
    may carry opposite signs, but each partial sum of the recombination is a
    prefix of x's own bits and exact."""
    g = _rng(41)
    X = _full24(g, (24, 24))
    I = np.eye(24, dtype=np.float32)
    C = orc.gemm_emu(I, X, nbands, flags=orc.ORC_SPLIT_RNE)
    assert np.array_equal(C.view(np.uint32), X.view(np.uint32))


def test_emu_rne_small_integers_exact(orc):
    g = _rng(42)
    A = g.integers(-1023, 1024, size=(20, 16)).astype(np.float32)
    B = g.integers(-1023, 1024, size=(16, 12)).astype(np.float32)
    C = orc.gemm_emu(A, B, 5, flags=orc.ORC_SPLIT_RNE)
    assert np.array_equal(C, (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float32))


def test_trunc_rne_nine_products_is_the_product(orc):
    """All nine products of the round-to-nearest split sum to a b exactly, so the
    FP64 truncated-band value with nbands = 5 matches the FP64 reference to
    double rounding."""
    g = _rng(43)
    A = g.standard_normal((9, 40)).astype(np.float32)
    B = g.standard_normal((40, 7)).astype(np.float32)
    T = orc.gemm_trunc_f64(A, B, 5, flags=orc.ORC_SPLIT_RNE)
    ref, G = orc.gemm_f64(A, B)
    assert np.all(np.abs(T - ref) <= 64 * 2.0 ** -53 * G)


def test_rne_split_halves_the_dropped_mass(orc):
    """With three products (nbands = 2) the dropped terms start at 2^-16 x1 y1;
    nearest rounding halves the largest possible |x1| and |x2|, so the RMS error
    of the RNE ablation is well below RZ's (about a sixth here)."""
    g = _rng(44)
    A = g.standard_normal((32, 256)).astype(np.float32)
    B = g.standard_normal((256, 32)).astype(np.float32)
    ref, _ = orc.gemm_f64(A, B)
    e_rz = orc.gemm_trunc_f64(A, B, 2) - ref
    e_rne = orc.gemm_trunc_f64(A, B, 2, flags=orc.ORC_SPLIT_RNE) - ref
    assert np.sqrt(np.mean(e_rne ** 2)) < 0.5 * np.sqrt(np.mean(e_rz ** 2))


def test_unknown_emulation_flag_rejected(orc):
    """The emulation has one mode flag (the round-to-nearest split); any other bit
    is an error rather than a silently different emulation."""
    A = np.ones((2, 2), np.float32)
    for bad in (1, 4, 1 << 30):
        with pytest.raises(RuntimeError):
            orc.gemm_emu(A, A, 5, flags=bad)
        with pytest.raises(RuntimeError):
            orc.gemm_trunc_f64(A, A, 5, flags=bad)


def test_chunked_full_check_catches_one_bad_element(orc):
    """The whole-output parity helper of the GPU tests, run on the oracle's own
    emulation (passes) and on a copy with one element pushed just past the
    elementwise bound in a late row chunk (fails)."""
    import gpu_util
    g = np.random.Generator(np.random.Philox(key=77))
    A = g.standard_normal((300, 100)).astype(np.float32)
    B = g.standard_normal((100, 50)).astype(np.float32)
    C = orc.gemm_emu(A, B)
    abl = {nb: orc.gemm_emu(A, B, nb) for nb in (4, 3, 2)}
    seen = []
    gpu_util.check_full("emu", A, B, C, ablations=abl, chunk_elems=50 * 64,
                        keep_ref=lambda r0, r1, ref: seen.append((r0, r1)))
    assert seen[0] == (0, 64) and seen[-1] == (256, 300)
    ref, G = orc.gemm_f64(A, B)
    bad = C.copy()
    bad[290, 7] = np.float32(ref[290, 7] + 1.5 * gpu_util.elementwise_bound(100, G[290, 7]))
    with pytest.raises(AssertionError, match="rows 256..299"):
        gpu_util.check_full("emu", A, B, bad, chunk_elems=50 * 64)
    bad = {**abl, 2: abl[2].copy()}
    bad[2][5, 5] += np.float32(0.5)
    with pytest.raises(AssertionError, match="nbands=2"):
        gpu_util.check_full("emu", A, B, C, ablations=bad, chunk_elems=50 * 64)
