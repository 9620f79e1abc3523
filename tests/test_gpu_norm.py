"""GPU parity of the RMSNorm prologue (lin_gemv_bf16_norm, lin_gemv_q4g64_norm,
lin_gemv_i8_norm)
against the oracle's RMSNorm followed by the oracle's product (and epilogue),
through the C ABI, for every candidate configuration of the prologue kinds.

Bound per output: the product's bound on the oracle's h (1e-3 * sum_k |W h|,
propagated through the epilogue as in the epilogue tests) plus 2^-8 |W[n][k]
h[k]| for every k whose exact value x g / rms lies within 2^-15 (relative) of a
bf16 rounding boundary: only there can the kernel's fp32 evaluation round h[k]
to the other neighbour."""
import numpy as np
import pytest
import torch

import memory_bound_weight_amd as L
import oracle
import synth
from gpu_util import u16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SHAPES = [(5, 192), (130, 3584), (1000, 2048), (64, 4096)]   # (outputs N, K)
EPS = 1e-6


def _bits_value(b):
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _gain(K, seed):
    rng = np.random.default_rng(seed)
    f = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _near_boundary(xb, g, eps):
    """Entries of one token row whose exact normalised value lies within 2^-15
    of a bf16 rounding boundary (relative), from an fp64 evaluation."""
    x = _bits_value(xb)
    v = x * _bits_value(g) / np.sqrt(np.sum(x * x) / x.size + eps)
    low = v.astype(np.float32).view(np.uint32) & 0xFFFF
    return np.abs(low.astype(np.int64) - 0x8000) < 256


def _case(fmt, NW, K, seed):
    W = synth.weight(seed, 0, 0, NW, K)
    x = synth.activation(seed, 0, 0, 1, K)
    g = _gain(K, seed)
    h = oracle.rmsnorm(u16(x), g, EPS)
    hw = np.where(_near_boundary(u16(x)[0], g, EPS), h[0], 0).astype(np.uint16)[None, :]
    if fmt == "bf16":
        Y, B = oracle.gemm_dense(u16(W), h)
        _, Bw = oracle.gemm_dense(u16(W), hw)
        Wt, kind, fn = (W.to(DEV),), L.LIN_KIND_GEMV_BF16_NORM, L.lin_gemv_bf16_norm
    elif fmt == "i8":
        Wq, S = oracle.quantize_i8(u16(W))
        Y, B = oracle.gemm_i8(Wq, S, h)
        _, Bw = oracle.gemm_i8(Wq, S, hw)
        Wt = (torch.from_numpy(Wq).to(DEV), torch.from_numpy(S).to(DEV))
        kind, fn = L.LIN_KIND_GEMV_I8_NORM, L.lin_gemv_i8_norm
    else:
        Wq, S = oracle.quantize_q4g64(u16(W))
        Y, B = oracle.gemm_q4g64(Wq, S, h)
        _, Bw = oracle.gemm_q4g64(Wq, S, hw)
        Wt = (torch.from_numpy(Wq).to(DEV), synth.from_bits(S, torch.float16, DEV))
        kind, fn = L.LIN_KIND_GEMV_Q4G64_NORM, L.lin_gemv_q4g64_norm
    gd = synth.from_bits(g, torch.bfloat16, DEV)
    return Wt, x.to(DEV), gd, Y[0], 1e-3 * B[0] + 2.0 ** -8 * Bw[0], kind, fn


def _configs(kind, NW, K):
    """Every candidate of the prologue kind."""
    return L.lin_candidates(kind, 1, NW, K)


def _check(y, expect, bound, what):
    d = np.abs(y.cpu().numpy()[0].astype(np.float64) - expect)
    assert np.all(d <= bound), "%s: worst |err|/bound = %.3g" % (what, np.max(d / np.maximum(bound, 1e-300)))


@pytest.mark.parametrize("fmt", ["bf16", "q4", "i8"])
@pytest.mark.parametrize("N,K", SHAPES)
def test_norm_every_configuration(fmt, N, K):
    print("case norm %s N=%d K=%d" % (fmt, N, K), flush=True)
    Wt, x, g, Y, bound, kind, fn = _case(fmt, N, K, 12000 + N + K)
    x0 = x.clone()
    for cfg in _configs(kind, N, K):
        L.lin_set_config(kind, 1, N, K, cfg)
        try:
            y = torch.full((1, N), float("nan"), device=DEV)
            fn(*Wt, x, g, EPS, y=y)
            torch.cuda.synchronize()
            _check(y, Y, bound, "norm %s %s" % (fmt, cfg))
            y2 = fn(*Wt, x, g, EPS)
            torch.cuda.synchronize()
            assert torch.equal(y, y2), cfg                   # deterministic
        finally:
            L.lin_set_config(kind, 1, N, K, None)
    assert torch.equal(x, x0)                                # x is not written


@pytest.mark.parametrize("fmt", ["bf16", "q4", "i8"])
@pytest.mark.parametrize("N,K", SHAPES[1:3])
def test_norm_with_epilogues(fmt, N, K):
    print("case norm+epilogues %s N=%d K=%d" % (fmt, N, K), flush=True)
    # residual add
    Wt, x, g, Y, bound, kind, fn = _case(fmt, N, K, 12500 + N + K)
    r = np.random.default_rng(N).standard_normal((1, N)).astype(np.float32)
    expect = oracle.residual_add(Y, r[0])
    rd = torch.from_numpy(r).to(DEV)
    for cfg in _configs(kind, N, K):
        L.lin_set_config(kind, 1, N, K, cfg)
        try:
            acc = rd.clone()
            fn(*Wt, x, g, EPS, L.LIN_EPI_ADD, r=acc, y=acc)
            torch.cuda.synchronize()
            _check(acc, expect, bound + 1e-3 * np.abs(r[0]), "norm+add %s %s" % (fmt, cfg))
        finally:
            L.lin_set_config(kind, 1, N, K, None)
    # gated product over 2N rows
    Wt, x, g, Y, bound, kind, fn = _case(fmt, 2 * N, K, 13000 + N + K)
    gate, up, bg, bu = Y[:N], Y[N:], bound[:N], bound[N:]
    expect = oracle.swiglu(gate, up)
    silu = oracle.swiglu(gate, np.ones_like(gate))
    sbound = 1.1 * np.abs(up) * bg + np.abs(silu) * bu + 1e-6 * np.abs(expect)
    for cfg in _configs(kind, 2 * N, K):
        L.lin_set_config(kind, 1, 2 * N, K, cfg)
        try:
            y = torch.full((1, N), float("nan"), device=DEV)
            fn(*Wt, x, g, EPS, L.LIN_EPI_SWIGLU, y=y)
            torch.cuda.synchronize()
            _check(y, expect, sbound, "norm+swiglu %s %s" % (fmt, cfg))
        finally:
            L.lin_set_config(kind, 1, 2 * N, K, None)


@pytest.mark.parametrize("fmt,N,K", [("bf16", 3, 8), ("bf16", 17, 520), ("bf16", 9, 32768),
                                     ("q4", 7, 64), ("q4", 17, 576), ("q4", 9, 16384),
                                     ("i8", 5, 16), ("i8", 17, 528), ("i8", 9, 32768)])
def test_norm_edge_shapes(fmt, N, K):
    """The smallest K of each format, K not a multiple of the 512 (bf16) or
    2048 (int4) weights a wavefront step covers, and K near the largest whose
    x and gain copies fit in LDS; every candidate, with and without the gated
    epilogue."""
    print("case norm edge %s N=%d K=%d" % (fmt, N, K), flush=True)
    Wt, x, g, Y, bound, kind, fn = _case(fmt, N, K, 14000 + N + K)
    cands = _configs(kind, N, K)
    assert cands
    for cfg in cands:
        L.lin_set_config(kind, 1, N, K, cfg)
        try:
            y = torch.full((1, N), float("nan"), device=DEV)
            fn(*Wt, x, g, EPS, y=y)
            torch.cuda.synchronize()
            _check(y, Y, bound, "norm edge %s %s" % (fmt, cfg))
        finally:
            L.lin_set_config(kind, 1, N, K, None)


def test_identity_weights_return_the_normalised_row():
    """W = I in bf16: y[k] = h[k] exactly (one exact product per output), so the
    kernel's h is compared with the oracle's entry by entry; entries away from a
    rounding boundary must match bit for bit, the others by at most one bf16
    step.  (The int4 kernels read the same normalised staged row.)"""
    K = 2048
    print("case norm identity K=%d" % K, flush=True)
    x = synth.activation(12999, 0, 0, 1, K)
    g = _gain(K, 77)
    h = _bits_value(oracle.rmsnorm(u16(x), g, EPS)[0])
    near = _near_boundary(u16(x)[0], g, EPS)
    W = torch.eye(K, dtype=torch.bfloat16, device=DEV)
    y = L.lin_gemv_bf16_norm(W, x.to(DEV), synth.from_bits(g, torch.bfloat16, DEV), EPS)
    torch.cuda.synchronize()
    got = y.cpu().numpy()[0].astype(np.float64)
    assert np.array_equal(got[~near], h[~near])
    assert np.all(np.abs(got[near] - h[near]) <= np.abs(h[near]) * 2.0 ** -7)


def test_norm_argument_errors():
    K = 64
    W = torch.zeros((8, K), dtype=torch.bfloat16, device=DEV)
    x = torch.zeros((1, K), dtype=torch.bfloat16, device=DEV)
    g = torch.ones((K,), dtype=torch.bfloat16, device=DEV)
    y = torch.zeros((1, 8), dtype=torch.float32, device=DEV)
    f = L._lib.lin_gemv_bf16_norm
    a = (W.data_ptr(), x.data_ptr(), g.data_ptr())
    assert f(*a, 1e-6, y.data_ptr(), 1, 8, K, 7, None, None) == L.LIN_ERR_ARG
    assert f(*a, -1.0, y.data_ptr(), 1, 8, K, 0, None, None) == L.LIN_ERR_ARG
    assert f(*a, float("nan"), y.data_ptr(), 1, 8, K, 0, None, None) == L.LIN_ERR_ARG
    assert f(*a, float("inf"), y.data_ptr(), 1, 8, K, 0, None, None) == L.LIN_ERR_ARG
    assert f(*a, 1e-6, y.data_ptr(), 2, 8, K, 0, None, None) == L.LIN_ERR_SHAPE
    assert f(*a, 1e-6, y.data_ptr(), 1, 8, 0, 0, None, None) == L.LIN_ERR_SHAPE
    assert f(a[0], a[1], None, 1e-6, y.data_ptr(), 1, 8, K, 0, None, None) == L.LIN_ERR_NULL
    assert f(a[0], a[1], g.data_ptr() + 2, 1e-6, y.data_ptr(), 1, 8, K, 0, None, None) == L.LIN_ERR_ALIGN
    assert f(*a, 1e-6, y.data_ptr(), 1, 8, K, L.LIN_EPI_ADD, None, None) == L.LIN_ERR_NULL
    assert f(None, None, None, 1e-6, None, 0, 8, K, 0, None, None) == L.LIN_OK
    zero = L.lin_gemv_bf16_norm(W, x, g, 1e-6)          # x = 0: h = 0, y = 0
    torch.cuda.synchronize()
    assert torch.count_nonzero(zero).item() == 0
