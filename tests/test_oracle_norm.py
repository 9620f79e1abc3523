"""Pins for the RMSNorm prologue of the CPU oracle (tinyinfer post, decode
section: norms folded into the projections; TileInfer.jl post, "Incremental
acceleration": fused norms) against things other than itself: the bf16 grid
built from bit patterns, midpoints between neighbours, 60-digit decimal
arithmetic, exact special cases and invariants of the definition.  CPU only."""
from decimal import Decimal, getcontext

import numpy as np

import oracle

getcontext().prec = 60


def _value(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _bits(values):
    f = np.asarray(values, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def _rand_bits(rng, shape, scale=1.0, loc=0.0):
    f = (loc + rng.standard_normal(shape) * scale).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# ---- rounding to bfloat16 ---------------------------------------------------

def test_bf16_values_round_to_themselves():
    bits = np.arange(0, 0x7F80, dtype=np.uint16)            # +0 .. largest finite
    assert np.array_equal(oracle.bf16_from_f64(_value(bits)), bits)
    neg = bits[1:] | np.uint16(0x8000)
    assert np.array_equal(oracle.bf16_from_f64(_value(neg)), neg)


def test_midpoints_round_to_even_and_neighbours_of_midpoints_do_not():
    """The midpoint of two consecutive bf16 values goes to the one with an even
    pattern; one fp64 step above or below it goes to the nearer one.  Covers
    subnormals, the subnormal/normal edge and every binade."""
    rng = np.random.default_rng(71)
    lo = np.concatenate([np.arange(0, 300), rng.integers(300, 0x7F7F, 3000)]).astype(np.uint16)
    a, b = _value(lo), _value(lo + np.uint16(1))
    mid = (a + b) / 2                                          # exact in fp64
    even = np.where(lo % 2 == 0, lo, lo + np.uint16(1)).astype(np.uint16)
    assert np.array_equal(oracle.bf16_from_f64(mid), even)
    up = np.nextafter(mid, np.inf)
    down = np.nextafter(mid, -np.inf)
    assert np.array_equal(oracle.bf16_from_f64(up), lo + np.uint16(1))
    assert np.array_equal(oracle.bf16_from_f64(down), lo)
    assert np.array_equal(oracle.bf16_from_f64(-up), (lo + np.uint16(1)) | np.uint16(0x8000))


def test_no_double_rounding_through_binary32():
    """1 + 2^-8 + 2^-40 lies above the midpoint of 1 and 1 + 2^-7 by less than a
    binary32 step: rounding it to binary32 first would land on the midpoint and
    then on 1 (even); the nearest bf16 is 1 + 2^-7."""
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert np.float32(v) == np.float32(1.0 + 2.0 ** -8)
    assert oracle.bf16_from_f64([v])[0] == 0x3F81
    assert oracle.bf16_from_f64([-v])[0] == 0xBF81


def test_overflow_and_specials():
    top = _value([0x7F7F])[0]                                  # (2 - 2^-7) 2^127
    half_step = 2.0 ** (127 - 8)
    got = oracle.bf16_from_f64([top, top + half_step * 0.999, top + half_step, 2.0 ** 128,
                                -(top + half_step), np.inf, 0.0, -0.0, 2.0 ** -134,
                                2.0 ** -134 * 1.0001, 3 * 2.0 ** -134])
    assert list(got) == [0x7F7F, 0x7F7F, 0x7F80, 0x7F80, 0xFF80, 0x7F80, 0, 0x8000, 0, 1, 2]
    nan = oracle.bf16_from_f64([np.nan])[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


# ---- RMSNorm ------------------------------------------------------------------

def _nearest_bf16_decimal(x):
    """Nearest bf16 pattern to a Decimal (ties to even), by comparing the two
    grid neighbours of its binary32 approximation."""
    f = np.float32(float(x))
    u = int(np.array([f]).view(np.uint32)[0]) >> 16
    best = None
    for c in (u - 1, u, u + 1, u + 2):
        cv = Decimal(float(_value([c & 0xFFFF])[0]))
        d = abs(cv - x)
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c & 0xFFFF)
    return best[1]


def test_matches_60_digit_decimal_evaluation():
    rng = np.random.default_rng(72)
    for M, K, eps in [(1, 1, 0.0), (2, 7, 1e-6), (3, 16, 1e-5), (1, 64, 0.5)]:
        X = _rand_bits(rng, (M, K))
        g = _rand_bits(rng, (K,), 0.1, 1.0)
        H = oracle.rmsnorm(X, g, eps)
        xv, gv = _value(X), _value(g)
        for m in range(M):
            ss = sum(Decimal(float(v)) ** 2 for v in xv[m])
            inv = 1 / (ss / K + Decimal(eps)).sqrt()
            for k in range(K):
                exact = Decimal(float(xv[m, k])) * Decimal(float(gv[k])) * inv
                assert H[m, k] == _nearest_bf16_decimal(exact), (M, K, m, k)


def test_closed_form_three_four():
    """x = (3, 4), g = 1, eps = 0: mean x^2 = 12.5, h = (3, 4) / sqrt(12.5)."""
    H = oracle.rmsnorm(_bits([[3.0, 4.0]]), _bits([1.0, 1.0]), 0.0)
    assert list(_value(H[0])) == [0.84765625, 1.1328125]      # 0.8485.., 1.1314..


def test_constant_row_gives_the_gain():
    """x[k] = c for every k and eps = 0: the root mean square is |c|, so h = sign(c) g
    exactly (a missing 1/K or square root would scale it)."""
    rng = np.random.default_rng(73)
    for c, K in [(3.0, 5), (-0.375, 64), (1.5, 2048), (2.0 ** -20, 9)]:
        g = _rand_bits(rng, (K,), 0.2, 1.0)
        H = oracle.rmsnorm(_bits(np.full((1, K), c)), g, 0.0)
        expect = g if c > 0 else g ^ np.uint16(0x8000)
        assert np.array_equal(H[0], expect), (c, K)


def test_scale_invariance_and_row_independence():
    rng = np.random.default_rng(74)
    X = _rand_bits(rng, (3, 96))
    g = _rand_bits(rng, (96,), 0.1, 1.0)
    H = oracle.rmsnorm(X, g, 0.0)
    for p in (-3, 5):
        Xs = _bits(_value(X) * 2.0 ** p)
        assert np.array_equal(oracle.rmsnorm(Xs, g, 0.0), H)
    assert np.array_equal(oracle.rmsnorm(X[::-1].copy(), g, 0.0), H[::-1])
    assert np.array_equal(oracle.rmsnorm(X[1:2].copy(), g, 0.0), H[1:2])


def test_eps():
    """A zero row stays zero; with eps much larger than the mean square the
    result is x g / sqrt(eps)."""
    g = _bits([1.0, 2.0, -0.5, 4.0])
    H = oracle.rmsnorm(np.zeros((1, 4), dtype=np.uint16), g, 1e-6)
    assert np.all(_value(H) == 0)
    x = _bits([[2.0 ** -12, -(2.0 ** -11), 2.0 ** -13, 0.0]])
    H = oracle.rmsnorm(x, g, 4.0)                             # mean x^2 ~ 1e-7 << 4
    assert list(_value(H[0])) == [2.0 ** -13, -(2.0 ** -11), -(2.0 ** -15), 0.0]
    H0 = oracle.rmsnorm(x, g, 0.0)
    assert not np.array_equal(H0, H)


def test_normalised_row_has_unit_mean_square():
    rng = np.random.default_rng(75)
    X = _rand_bits(rng, (4, 2048), 3.0)
    H = oracle.rmsnorm(X, _bits(np.ones(2048)), 0.0)
    ms = np.mean(_value(H) ** 2, axis=1)
    assert np.all(np.abs(ms - 1.0) < 4e-3)                    # bf16 rounding of each entry
