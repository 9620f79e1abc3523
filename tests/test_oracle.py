"""Pins for the CPU oracle, against things other than itself: library
conversions, exact rational arithmetic, closed forms, hand-derived worked
examples and invariants of the int4-g64 format.  CPU only."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_bits_of(values):
    """bf16 bit patterns for fp32-exact values whose low 16 bits are zero."""
    f = np.asarray(values, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def _rand_bf16_bits(rng, shape, scale=1.0):
    f = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)   # truncation: any bf16 will do


# ---------------------------------------------------------------- number formats

def test_bf16_decoder_exhaustive():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_value(allbits)
    ref = (allbits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_f16_decoder_exhaustive():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_value(allbits)
    ref = allbits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_f16_encoder_roundtrip_all_finite():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = allbits.view(np.float16).astype(np.float64)
    finite = np.isfinite(vals)
    enc = oracle.f16_from_f64(vals[finite])
    assert np.array_equal(enc, allbits[finite])


def test_f16_encoder_midpoints_go_to_even():
    # consecutive positive finite fp16 values (normal and subnormal)
    lo = np.arange(0, 0x7BFF, dtype=np.uint16)
    a = lo.view(np.float16).astype(np.float64)
    b = (lo + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = (a + b) / 2.0                                   # exact in fp64
    enc = oracle.f16_from_f64(mid).astype(np.int64)
    even = np.where(lo % 2 == 0, lo, lo + 1).astype(np.int64)
    assert np.array_equal(enc, even)
    # just off the midpoint picks the nearer neighbour
    up = oracle.f16_from_f64(np.nextafter(mid, np.inf)).astype(np.int64)
    dn = oracle.f16_from_f64(np.nextafter(mid, -np.inf)).astype(np.int64)
    assert np.array_equal(up, lo.astype(np.int64) + 1)
    assert np.array_equal(dn, lo.astype(np.int64))


def test_f16_encoder_matches_numpy_on_random_doubles():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),
                        [65504.0, 65519.99, 65520.0, 1e6, -1e-9, 0.0, -0.0]])
    got = oracle.f16_from_f64(v)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- dense product

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (1, 5, 7), (2, 3, 64), (3, 8, 130), (1, 2, 9)])
def test_dense_matches_exact_rationals(M, N, K):
    rng = np.random.default_rng(1000 + M * 100 + N * 10 + K)
    W = _rand_bf16_bits(rng, (N, K), 0.02)
    X = _rand_bf16_bits(rng, (M, K), 1.0)
    Y, B = oracle.gemm_dense(W, X)
    wv = (W.astype(np.uint32) << 16).view(np.float32)
    xv = (X.astype(np.uint32) << 16).view(np.float32)
    u = 2.0 ** -53
    for m in range(M):
        for n in range(N):
            terms = [Fraction(float(wv[n, k])) * Fraction(float(xv[m, k])) for k in range(K)]
            exact = sum(terms, Fraction(0))
            mag = sum((abs(t) for t in terms), Fraction(0))
            # sequential fp64 summation of exact products: |err| <= (K-1) u sum|p|
            assert abs(Fraction(Y[m, n]) - exact) <= (K - 1) * Fraction(u) * mag
            assert abs(Fraction(B[m, n]) - mag) <= (K - 1) * Fraction(u) * mag


def test_dense_identity_returns_x():
    K = 96
    W = np.zeros((K, K), dtype=np.uint16)
    W[np.arange(K), np.arange(K)] = 0x3F80                  # 1.0
    rng = np.random.default_rng(3)
    X = _rand_bf16_bits(rng, (2, K))
    Y, _ = oracle.gemm_dense(W, X)
    xv = (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(Y, xv)


def test_dense_one_hot_selects_column():
    rng = np.random.default_rng(4)
    N, K = 7, 40                                             # N != K: a transposed operand fails
    W = _rand_bf16_bits(rng, (N, K), 0.02)
    wv = (W.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for j in (0, 13, K - 1):
        X = np.zeros((1, K), dtype=np.uint16)
        X[0, j] = 0x3F80
        Y, B = oracle.gemm_dense(W, X)
        assert np.array_equal(Y[0], wv[:, j])
        assert np.array_equal(B[0], np.abs(wv[:, j]))


def test_dense_integer_closed_form():
    rng = np.random.default_rng(5)
    N, K, M = 6, 50, 3
    wi = rng.integers(-3, 4, (N, K))
    xi = rng.integers(-2, 3, (M, K))
    W = _bf16_bits_of(wi.astype(np.float32))
    X = _bf16_bits_of(xi.astype(np.float32))
    Y, B = oracle.gemm_dense(W, X)
    assert np.array_equal(Y, (xi @ wi.T).astype(np.float64))
    assert np.array_equal(B, (np.abs(xi) @ np.abs(wi).T).astype(np.float64))


def test_dense_rows_of_batch_equal_single_token_products():
    rng = np.random.default_rng(6)
    W = _rand_bf16_bits(rng, (9, 72), 0.02)
    X = _rand_bf16_bits(rng, (4, 72))
    Y, B = oracle.gemm_dense(W, X)
    for m in range(4):
        y1, b1 = oracle.gemm_dense(W, X[m:m + 1])
        assert np.array_equal(Y[m], y1[0]) and np.array_equal(B[m], b1[0])


def test_dense_power_of_two_scaling_is_exact():
    rng = np.random.default_rng(8)
    W = _rand_bf16_bits(rng, (5, 33), 0.02)
    X = _rand_bf16_bits(rng, (1, 33))
    Y, _ = oracle.gemm_dense(W, X)
    X2 = X.copy()
    nz = (X2 & 0x7F80) != 0                                  # normal values: bump the exponent
    X2[nz] = X2[nz] + 0x80
    Y2, _ = oracle.gemm_dense(W, X2)
    xv = (X.astype(np.uint32) << 16).view(np.float32)
    assert np.all((xv == 0) | nz)
    assert np.array_equal(Y2, 2.0 * Y)


def test_dense_empty_k_gives_zero():
    Y, B = oracle.gemm_dense(np.zeros((3, 0), np.uint16), np.zeros((2, 0), np.uint16))
    assert np.array_equal(Y, np.zeros((2, 3))) and np.array_equal(B, np.zeros((2, 3)))


# ---------------------------------------------------------------- int4-g64

def _pack(q):
    """Pack signed codes [N, K] (even k low nibble, two's complement)."""
    q = np.asarray(q, dtype=np.int64)
    lo = q[:, 0::2] & 0xF
    hi = q[:, 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def test_q4_one_hot_pins_nibble_order_sign_and_group():
    N, K = 4, 192
    rng = np.random.default_rng(9)
    q = rng.integers(-8, 8, (N, K))
    q[0, :16] = np.arange(-8, 8)                             # every code, both nibble slots
    q[1, 64:80] = np.arange(7, -9, -1)
    Wq = _pack(q)
    # power-of-two scales: 2^-3, 2^-1, 2^2 per group, different per row
    sexp = rng.integers(-6, 4, (N, K // 64))
    S = oracle.f16_from_f64(np.ldexp(1.0, sexp))
    for j in list(range(0, 20)) + [63, 64, 65, 127, 128, 191]:
        X = np.zeros((1, K), dtype=np.uint16)
        X[0, j] = 0x3F80
        Y, _ = oracle.gemm_q4g64(Wq, S, X)
        expect = q[:, j] * np.ldexp(1.0, sexp[:, j // 64])
        assert np.array_equal(Y[0], expect.astype(np.float64)), j


def test_q4_dequant_is_code_times_scale():
    rng = np.random.default_rng(10)
    N, K = 3, 128
    q = rng.integers(-8, 8, (N, K))
    S = oracle.f16_from_f64(rng.uniform(0.001, 0.01, (N, K // 64)))
    Wd = oracle.dequant_q4g64(_pack(q), S)
    sv = S.view(np.float16).astype(np.float64)
    assert np.array_equal(Wd, q * np.repeat(sv, 64, axis=1))


def test_q4_product_equals_dense_product_on_dequantised_weights():
    rng = np.random.default_rng(11)
    W = _rand_bf16_bits(rng, (10, 256), 0.02)
    X = _rand_bf16_bits(rng, (3, 256))
    Wq, S = oracle.quantize_q4g64(W)
    Y4, B4 = oracle.gemm_q4g64(Wq, S, X)
    Yd, Bd = oracle.gemm_f64w(oracle.dequant_q4g64(Wq, S), X)
    assert np.array_equal(Y4, Yd) and np.array_equal(B4, Bd)


def test_q4_power_of_two_scales_match_bf16_product():
    # with power-of-two scales q*s is exact in bf16, so the int4 product equals the
    # dense product on those bf16 weights, bit for bit
    rng = np.random.default_rng(12)
    N, K = 6, 128
    q = rng.integers(-8, 8, (N, K))
    sexp = rng.integers(-9, -4, (N, K // 64))
    S = oracle.f16_from_f64(np.ldexp(1.0, sexp))
    wd = q * np.ldexp(1.0, np.repeat(sexp, 64, axis=1))
    Wb = _bf16_bits_of(wd.astype(np.float32))
    X = _rand_bf16_bits(rng, (2, K))
    Y4, B4 = oracle.gemm_q4g64(_pack(q), S, X)
    Yb, Bb = oracle.gemm_dense(Wb, X)
    assert np.array_equal(Y4, Yb) and np.array_equal(B4, Bb)


def _load_worked():
    with open(os.path.join(GOLDEN, "q4g64_worked.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _load_worked(), ids=lambda c: c["name"])
def test_quantizer_worked_examples(case):
    n = case["pad_zero_to"]
    w = np.zeros((1, n), dtype=np.uint16)
    vals = [int(h, 16) for h in case["w_bf16"]]
    w[0, :len(vals)] = vals
    Wq, S = oracle.quantize_q4g64(w)
    assert S[0, 0] == int(case["scale_f16"], 16)
    expect = np.zeros(n // 2, dtype=np.uint8)
    b = [int(h, 16) for h in case["bytes"]]
    expect[:len(b)] = b
    assert np.array_equal(Wq[0], expect)
    # decoded codes
    codes = np.empty(n, dtype=np.int64)
    codes[0::2] = ((Wq[0] & 0xF) ^ 8).astype(np.int64) - 8
    codes[1::2] = ((Wq[0] >> 4) ^ 8).astype(np.int64) - 8
    assert list(codes[:len(case["q"])]) == case["q"]


def test_quantizer_invariants_on_workload_like_data():
    rng = np.random.default_rng(13)
    N, K = 64, 1024
    W = _rand_bf16_bits(rng, (N, K), 0.02)
    W[3, 64:128] = 0                                          # an all-zero group
    Wq, S = oracle.quantize_q4g64(W)
    w = (W.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    s = S.view(np.float16).astype(np.float64)
    codes = np.empty((N, K), dtype=np.int64)
    codes[:, 0::2] = ((Wq & 0xF) ^ 8).astype(np.int64) - 8
    codes[:, 1::2] = ((Wq >> 4) ^ 8).astype(np.int64) - 8
    assert codes.min() >= -8 and codes.max() <= 7
    a = np.abs(w).reshape(N, K // 64, 64).max(axis=2)
    # the stored scale is the fp16 nearest to absmax/7 (numpy's own conversion)
    assert np.array_equal(S, (a / 7.0).astype(np.float16).view(np.uint16))
    srep = np.repeat(s, 64, axis=1)
    err = np.abs(w - codes * srep)
    assert np.all(err <= srep / 2)                            # round to nearest, no clamp hit
    cg = np.abs(codes).reshape(N, K // 64, 64).max(axis=2)
    assert np.all(cg[a > 0] == 7)                             # the absmax lands on +-7
    assert np.all(codes[3, 64:128] == 0) and s[3, 1] == 0
    # round trip: re-quantising q*s with power-of-two scales returns q
    q2 = rng.integers(-7, 8, (4, 128))
    q2[:, ::64] = 7
    sexp = rng.integers(-8, -2, (4, 2))
    wd = q2 * np.ldexp(1.0, np.repeat(sexp, 64, axis=1))
    Wq2, S2 = oracle.quantize_q4g64(_bf16_bits_of(wd.astype(np.float32)))
    assert np.array_equal(Wq2, _pack(q2))
