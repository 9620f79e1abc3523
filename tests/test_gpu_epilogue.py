"""GPU parity of the fused epilogues (lin_gemv_bf16_ep, lin_gemv_q4g64_ep, lin_gemv_i8_ep)
against the oracle's product followed by the oracle's epilogue, for every
candidate configuration of the plain product of the same weight matrix.

Bounds per output: ADD, 1e-3 * (sum_k |W x| + |r|); SWIGLU, the GEMV bound of
the gate and up products propagated through silu(g) u, |d/dg silu(g)| <= 1.1:
1e-3 * (1.1 |u| B_g + |silu(g)| B_u), plus 1e-6 |y| for the fp32 epilogue."""
import numpy as np
import pytest
import torch

import memory_bound_weight_amd as L
import oracle
import synth
from gpu_util import u16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SHAPES = [(5, 192), (130, 3584), (1000, 2048)]   # (outputs N, K)


def _weights(fmt, NW, K, seed, M=1):
    W = synth.weight(seed, 0, 0, NW, K)
    x = synth.activation(seed, 0, 0, M, K)
    if fmt == "bf16":
        Y, B = oracle.gemm_dense(u16(W), u16(x))
        return (W.to(DEV),), x.to(DEV), Y, B, L.LIN_KIND_GEMV_BF16, L.lin_gemv_bf16_ep
    if fmt == "i8":
        Wq, S = oracle.quantize_i8(u16(W))
        Y, B = oracle.gemm_i8(Wq, S, u16(x))
        return ((torch.from_numpy(Wq).to(DEV), torch.from_numpy(S).to(DEV)), x.to(DEV),
                Y, B, L.LIN_KIND_GEMV_I8, L.lin_gemv_i8_ep)
    Wq, S = oracle.quantize_q4g64(u16(W))
    Y, B = oracle.gemm_q4g64(Wq, S, u16(x))
    return ((torch.from_numpy(Wq).to(DEV), synth.from_bits(S, torch.float16, DEV)), x.to(DEV),
            Y, B, L.LIN_KIND_GEMV_Q4G64, L.lin_gemv_q4g64_ep)


def _check(y, expect, bound, what):
    d = np.abs(y.cpu().numpy().astype(np.float64) - expect)
    assert np.all(d <= bound), "%s: worst |err|/bound = %.3g" % (what, np.max(d / np.maximum(bound, 1e-300)))


@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("fmt", ["bf16", "q4", "i8"])
@pytest.mark.parametrize("N,K", SHAPES)
def test_residual_add_every_candidate(fmt, N, K, M):
    print("case epilogue add %s M=%d N=%d K=%d" % (fmt, M, N, K), flush=True)
    Wt, x, Y, B, kind, fn = _weights(fmt, N, K, 9000 + N + K, M)
    rng = np.random.default_rng(N + K)
    r = rng.standard_normal((M, N)).astype(np.float32)
    expect = oracle.residual_add(Y, r)
    bound = 1e-3 * (B + np.abs(r).astype(np.float64))
    rd = torch.from_numpy(r).to(DEV)
    for cfg in L.lin_candidates(kind, M, N, K):
        L.lin_set_config(kind, M, N, K, cfg)
        try:
            y = fn(*Wt, x, L.LIN_EPI_ADD, r=rd)              # separate output
            torch.cuda.synchronize()
            _check(y, expect, bound, "add %s %s" % (fmt, cfg))
            acc = rd.clone()
            fn(*Wt, x, L.LIN_EPI_ADD, r=acc, y=acc)           # accumulate in place
            torch.cuda.synchronize()
            _check(acc, expect, bound, "add in place %s %s" % (fmt, cfg))
        finally:
            L.lin_set_config(kind, M, N, K, None)


@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("fmt", ["bf16", "q4", "i8"])
@pytest.mark.parametrize("N,K", SHAPES)
def test_swiglu_every_candidate(fmt, N, K, M):
    print("case epilogue swiglu %s M=%d N=%d K=%d" % (fmt, M, N, K), flush=True)
    Wt, x, Y, B, kind, fn = _weights(fmt, 2 * N, K, 9500 + N + K, M)
    g, u, Bg, Bu = Y[:, :N], Y[:, N:], B[:, :N], B[:, N:]
    expect = oracle.swiglu(g, u)
    silu = oracle.swiglu(g, np.ones_like(g))
    bound = 1e-3 * (1.1 * np.abs(u) * Bg + np.abs(silu) * Bu) + 1e-6 * np.abs(expect)
    for cfg in L.lin_candidates(kind, M, 2 * N, K):
        L.lin_set_config(kind, M, 2 * N, K, cfg)
        try:
            y = torch.full((M, N), float("nan"), device=DEV)
            fn(*Wt, x, L.LIN_EPI_SWIGLU, y=y)
            torch.cuda.synchronize()
            _check(y, expect, bound, "swiglu %s %s" % (fmt, cfg))
        finally:
            L.lin_set_config(kind, M, 2 * N, K, None)


def test_epilogue_argument_errors():
    W = torch.zeros((8, 64), dtype=torch.bfloat16, device=DEV)
    x = torch.zeros((1, 64), dtype=torch.bfloat16, device=DEV)
    y = torch.zeros((1, 8), dtype=torch.float32, device=DEV)
    f = L._lib.lin_gemv_bf16_ep
    assert f(W.data_ptr(), x.data_ptr(), y.data_ptr(), 1, 8, 64, 7, None, None) == L.LIN_ERR_ARG
    assert f(W.data_ptr(), x.data_ptr(), y.data_ptr(), 1, 8, 64, L.LIN_EPI_ADD, None, None) == L.LIN_ERR_NULL
    assert f(W.data_ptr(), x.data_ptr(), y.data_ptr(), 9, 8, 64, L.LIN_EPI_NONE, None, None) == L.LIN_ERR_SHAPE
    assert f(W.data_ptr(), x.data_ptr(), y.data_ptr(), 1, 8, 64, L.LIN_EPI_ADD,
             y.data_ptr() + 2, None) == L.LIN_ERR_ALIGN
    assert f(None, None, None, 0, 8, 64, L.LIN_EPI_SWIGLU, None, None) == L.LIN_OK
