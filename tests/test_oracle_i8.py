"""Pins for the INT8 (one fp32 scale per output channel) part of the CPU oracle,
against things other than itself: numpy's IEEE fp32 division, exact rational
arithmetic, hand-derived ties and invariants of the format (TileInfer.jl post,
"Pushing further with cheating: INT8 quantization").  CPU only."""
from fractions import Fraction

import numpy as np

import oracle


def _bf16_bits_of(values):
    f = np.asarray(values, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def _rand_bf16_bits(rng, shape, scale=1.0):
    f = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _value(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_scale_is_fp32_nearest_absmax_over_127_for_every_bf16():
    """Every finite positive bf16 as a one-weight row: the stored scale equals
    numpy's correctly rounded fp32 division a / 127."""
    bits = np.arange(1, 0x7F80, dtype=np.uint16)           # +subnormals .. max finite
    Wq, S = oracle.quantize_i8(bits.reshape(-1, 1))
    expect = np.float32(1.0) * _value(bits).astype(np.float32) / np.float32(127.0)
    assert np.array_equal(S, expect.astype(np.float32))
    assert np.all(Wq[:, 0] == 127)                          # the absmax lands on the edge
    Wq, S = oracle.quantize_i8((bits | 0x8000).reshape(-1, 1))   # negative weights
    assert np.array_equal(S, expect.astype(np.float32))
    assert np.all(Wq[:, 0] == -127)


def test_ties_round_to_even():
    """s = 2^-7 exactly (absmax 127/128): w = 2.5 s -> 2, 3.5 s -> 4, -2.5 s -> -2."""
    s = 2.0 ** -7
    w = np.array([127 * s, 2.5 * s, 3.5 * s, -2.5 * s, -3.5 * s, 0.5 * s, 1.5 * s, 126.5 * s])
    Wq, S = oracle.quantize_i8(_bf16_bits_of(w.astype(np.float32)).reshape(1, -1))
    assert S[0] == np.float32(s)
    assert list(Wq[0]) == [127, 2, 4, -2, -4, 0, 2, 126]


def test_quantizer_invariants_on_workload_like_data():
    rng = np.random.default_rng(41)
    N, K = 48, 700
    W = _rand_bf16_bits(rng, (N, K), 0.02)
    W[5] = 0                                                  # an all-zero row
    Wq, S = oracle.quantize_i8(W)
    w = _value(W)
    s = S.astype(np.float64)
    q = Wq.astype(np.int64)
    assert q.min() >= -127 and q.max() <= 127
    err = np.abs(w - q * s[:, None])
    assert np.all(err <= s[:, None] / 2)                      # nearest multiple of s
    a = np.abs(w).max(axis=1)
    assert np.all(np.abs(q).max(axis=1)[a > 0] == 127)
    assert s[5] == 0 and np.all(q[5] == 0)
    # symmetric: quantising -W gives -q and the same scales
    Wq2, S2 = oracle.quantize_i8(W ^ np.uint16(0x8000))
    assert np.array_equal(S2, S) and np.array_equal(Wq2.astype(np.int64), -q)


def test_round_trip_with_power_of_two_scales():
    rng = np.random.default_rng(42)
    q = rng.integers(-127, 128, (6, 96))
    q[:, 7] = 127
    sexp = rng.integers(-12, -6, 6)
    wd = q * np.ldexp(1.0, sexp)[:, None]                    # exact in bf16: <= 7 bits
    Wq, S = oracle.quantize_i8(_bf16_bits_of(wd.astype(np.float32)))
    assert np.array_equal(Wq.astype(np.int64), q)
    assert np.array_equal(S.astype(np.float64), np.ldexp(1.0, sexp))


def test_product_matches_exact_rationals():
    rng = np.random.default_rng(43)
    for M, N, K in [(1, 1, 1), (2, 3, 7), (3, 5, 64), (1, 4, 130)]:
        Wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
        S = (rng.uniform(0.001, 0.1, N)).astype(np.float32)
        X = _rand_bf16_bits(rng, (M, K))
        Y, B = oracle.gemm_i8(Wq, S, X)
        xv = _value(X)
        for m in range(M):
            for n in range(N):
                exact = Fraction(float(S[n])) * sum(Fraction(int(Wq[n, k])) * Fraction(float(xv[m, k]))
                                                    for k in range(K))
                mag = Fraction(float(S[n])) * sum(abs(Fraction(int(Wq[n, k])) * Fraction(float(xv[m, k])))
                                                  for k in range(K))
                assert abs(Fraction(Y[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 1000)
                assert abs(Fraction(B[m, n]) - mag) <= mag * Fraction(1, 2 ** 50)


def test_one_hot_selects_code_times_scale():
    rng = np.random.default_rng(44)
    N, K = 9, 200
    Wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    Wq[0, :10] = [-127, -128 + 1, -1, 0, 1, 2, 63, 64, 126, 127]
    S = np.ldexp(1.0, rng.integers(-10, -2, N)).astype(np.float32)
    for j in (0, 1, 5, 9, 63, 64, 127, 199):
        X = np.zeros((1, K), dtype=np.uint16)
        X[0, j] = 0x3F80
        Y, _ = oracle.gemm_i8(Wq, S, X)
        assert np.array_equal(Y[0], Wq[:, j].astype(np.float64) * S.astype(np.float64)), j


def test_product_equals_dense_product_on_dequantised_weights():
    """With integer tokens and power-of-two scales every sum is exact, so the
    INT8 product equals the dense oracle on the dequantised weights bit for
    bit; with workload-like data it agrees to fp64 rounding."""
    rng = np.random.default_rng(45)
    Wq = rng.integers(-127, 128, (7, 160)).astype(np.int8)
    S = np.ldexp(1.0, rng.integers(-9, -3, 7)).astype(np.float32)
    xi = rng.integers(-4, 5, (3, 160)).astype(np.float32)
    X = _bf16_bits_of(xi)
    Y8, B8 = oracle.gemm_i8(Wq, S, X)
    Yd, Bd = oracle.gemm_f64w(oracle.dequant_i8(Wq, S), X)
    assert np.array_equal(Y8, Yd) and np.array_equal(B8, Bd)
    W = _rand_bf16_bits(rng, (11, 512), 0.02)
    X = _rand_bf16_bits(rng, (2, 512))
    Wq, S = oracle.quantize_i8(W)
    Y8, B8 = oracle.gemm_i8(Wq, S, X)
    Yd, Bd = oracle.gemm_f64w(oracle.dequant_i8(Wq, S), X)
    assert np.allclose(Y8, Yd, rtol=0, atol=1e-12 * Bd.max())
    assert np.allclose(B8, Bd, rtol=1e-14)

