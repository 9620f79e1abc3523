"""GPU parity at the edge of the weight formats: groups dominated by one outlier.

int4-g64 stores one fp16 scale per 64 weights (tinyinfer post, TL;DR).  When a
group holds one weight 30-50 times larger than the rest, its scale is set by
that weight and almost every other code rounds to 0; the kernels multiply the
codes as exact bf16 values 24 + q and remove 24 * sum x in fp32, whose
rounding is then not proportional to sum |q x|.  These tests run every
candidate configuration of every int4 product (the batch-1 GEMV at 1, 3 and 8
tokens, its fused epilogues and RMSNorm prologue, and the batched product on
the tiled layout) on such weights against the oracle:

- weights N(0, 0.02) with one entry per group at +-U(30, 50) * 0.02 (at least
  80 % of the codes are 0), x ~ N(0, 1), K = 3584 and 18944: the product bound
  |y - y_oracle| <= 1e-3 * sum_k |W x| per output;
- the same weights with the outliers at shared positions and x shrunk by 1e-3
  exactly there (an input built against the offset removal): the bound the
  library guarantees for int4, 1e-4 * sum_k |W x| + 4e-4 * sum_g s_g
  sum_{k in g} |x_k|.

INT8 weights (one fp32 scale per row; TileInfer.jl post, INT8 section) get
the analogous inputs: one-hot rows (a single code 127, the rest exactly 0) and
rows dominated by one outlier, with the product bound 1e-3 * sum_k |W x|."""
import numpy as np
import pytest
import torch

import memory_bound_weight_amd as L
import oracle
import synth
from gpu_util import assert_within_bound, pinned, u16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SHAPES = [(96, 3584), (40, 18944)]    # (N, K): a 7B-shaped K and a down-projection K


def _codes(Wq):
    """Signed int4 codes [N][K] of packed bytes (low nibble = even k)."""
    lo = (Wq & 0xF).astype(np.int64)
    hi = (Wq >> 4).astype(np.int64)
    q = np.empty((Wq.shape[0], 2 * Wq.shape[1]), dtype=np.int64)
    q[:, 0::2], q[:, 1::2] = lo, hi
    return np.where(q >= 8, q - 16, q)


def _bf16_values(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _scale_term(S, X):
    """sum_g s[n][g] * sum_{k in g} |x[m][k]| as [M][N] (fp64)."""
    s = oracle.f16_value(S)                                    # [N][G]
    ax = np.abs(_bf16_values(u16(X)))                          # [M][K]
    M, K = ax.shape
    gx = ax.reshape(M, K // 64, 64).sum(axis=2)                # [M][G]
    return gx @ s.T


def _outlier_q4(seed, N, K, shared=False):
    W, pos = synth.outlier_weight(seed, N, K, shared=shared)
    Wq, S = oracle.quantize_q4g64(u16(W))
    zero = float(np.mean(_codes(Wq) == 0))
    assert zero >= 0.8, "outlier weights should quantise to mostly zero codes (%.3f)" % zero
    return Wq, S, pos


def _dev_q4(Wq, S):
    return torch.from_numpy(Wq).to(DEV), synth.from_bits(S, torch.float16, DEV)


def _tiny_at(X, cols, factor=1e-3):
    """x with the entries of the given columns multiplied by `factor` (bf16)."""
    x = X.float().clone()
    x[:, torch.from_numpy(np.unique(cols))] *= factor
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("M", [1, 3, 8])
def test_q4_gemv_outlier_groups_every_candidate(M, N, K):
    print("case q4 gemv outliers M=%d N=%d K=%d" % (M, N, K), flush=True)
    seed = 21000 + M + N + K
    Wq, S, _ = _outlier_q4(seed, N, K)
    X = synth.activation(seed, 0, 1, M, K)
    Y, B = oracle.gemm_q4g64(Wq, S, u16(X))
    Wqd, Sd = _dev_q4(Wq, S)
    Xd = X.to(DEV)
    kind = L.LIN_KIND_GEMV_Q4G64
    cands = L.lin_candidates(kind, M, N, K)
    assert cands
    worst = 0.0
    for cfg in cands:
        with pinned(kind, M, N, K, cfg):
            y = torch.full((M, N), float("nan"), device=DEV)
            L.lin_gemv_q4g64(Wqd, Sd, Xd, y)
            torch.cuda.synchronize()
            worst = max(worst, assert_within_bound(y, Y, B, "q4 outliers %s" % cfg))
    print("worst |err|/bound over %d candidates: %.3g" % (len(cands), worst), flush=True)


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("M", [1, 8, 64, 256])
def test_q4_skinny_outlier_groups_every_candidate(M, N, K):
    print("case q4 skinny outliers M=%d N=%d K=%d" % (M, N, K), flush=True)
    seed = 22000 + M + N + K
    Wq, S, _ = _outlier_q4(seed, N, K)
    X = synth.activation(seed, 0, 1, M, K)
    Y, B = oracle.gemm_q4g64(Wq, S, u16(X))
    Wt = L.lin_q4g64_tile(*_dev_q4(Wq, S))
    Xd = X.to(DEV)
    kind = L.LIN_KIND_SKINNY_Q4G64
    cands = L.lin_candidates(kind, M, N, K)
    assert cands
    for cfg in cands:
        with pinned(kind, M, N, K, cfg):
            y = torch.full((M, N), float("nan"), device=DEV)
            L.lin_gemm_skinny_q4g64(Wt, Xd, y)
            torch.cuda.synchronize()
            assert_within_bound(y, Y, B, "q4 skinny outliers %s" % cfg)


def _check(y, expect, bound, what):
    d = np.abs(y.cpu().numpy().astype(np.float64) - expect)
    assert np.all(d <= bound), "%s: worst |err|/bound = %.3g" % (
        what, np.max(d / np.maximum(bound, 1e-300)))


@pytest.mark.parametrize("N,K", SHAPES)
def test_q4_epilogues_outlier_groups_every_candidate(N, K):
    print("case q4 epilogues outliers N=%d K=%d" % (N, K), flush=True)
    kind = L.LIN_KIND_GEMV_Q4G64
    seed = 23000 + N + K
    # residual add over N rows
    Wq, S, _ = _outlier_q4(seed, N, K)
    X = synth.activation(seed, 0, 1, 1, K)
    Y, B = oracle.gemm_q4g64(Wq, S, u16(X))
    r = np.random.default_rng(seed).standard_normal((1, N)).astype(np.float32)
    expect = oracle.residual_add(Y, r)
    bound = 1e-3 * (B + np.abs(r).astype(np.float64))
    Wqd, Sd = _dev_q4(Wq, S)
    Xd, rd = X.to(DEV), torch.from_numpy(r).to(DEV)
    for cfg in L.lin_candidates(kind, 1, N, K):
        with pinned(kind, 1, N, K, cfg):
            y = L.lin_gemv_q4g64_ep(Wqd, Sd, Xd, L.LIN_EPI_ADD, r=rd)
            torch.cuda.synchronize()
            _check(y, expect, bound, "add %s" % cfg)
    # gated product over gate|up = 2N rows
    Wq, S, _ = _outlier_q4(seed + 1, 2 * N, K)
    Y, B = oracle.gemm_q4g64(Wq, S, u16(X))
    g, u, Bg, Bu = Y[:, :N], Y[:, N:], B[:, :N], B[:, N:]
    expect = oracle.swiglu(g, u)
    silu = oracle.swiglu(g, np.ones_like(g))
    bound = 1e-3 * (1.1 * np.abs(u) * Bg + np.abs(silu) * Bu) + 1e-6 * np.abs(expect)
    Wqd, Sd = _dev_q4(Wq, S)
    for cfg in L.lin_candidates(kind, 1, 2 * N, K):
        with pinned(kind, 1, 2 * N, K, cfg):
            y = torch.full((1, N), float("nan"), device=DEV)
            L.lin_gemv_q4g64_ep(Wqd, Sd, Xd, L.LIN_EPI_SWIGLU, y=y)
            torch.cuda.synchronize()
            _check(y, expect, bound, "swiglu %s" % cfg)


def _gain(K, seed):
    f = (1.0 + 0.1 * np.random.default_rng(seed).standard_normal(K)).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _near_boundary(xb, g, eps):
    """Entries whose exact normalised value lies within 2^-15 (relative) of a
    bf16 rounding boundary (fp64 evaluation): only there may the kernel's fp32
    RMSNorm round h[k] to the other neighbour."""
    x = _bf16_values(xb)
    v = x * _bf16_values(g) / np.sqrt(np.sum(x * x) / x.size + eps)
    low = v.astype(np.float32).view(np.uint32) & 0xFFFF
    return np.abs(low.astype(np.int64) - 0x8000) < 256


@pytest.mark.parametrize("N,K", SHAPES)
def test_q4_norm_outlier_groups_every_candidate(N, K):
    print("case q4 norm outliers N=%d K=%d" % (N, K), flush=True)
    eps = 1e-6
    seed = 24000 + N + K
    Wq, S, _ = _outlier_q4(seed, N, K)
    X = synth.activation(seed, 0, 1, 1, K)
    g = _gain(K, seed)
    h = oracle.rmsnorm(u16(X), g, eps)
    hw = np.where(_near_boundary(u16(X)[0], g, eps), h[0], 0).astype(np.uint16)[None, :]
    Y, B = oracle.gemm_q4g64(Wq, S, h)
    _, Bw = oracle.gemm_q4g64(Wq, S, hw)
    bound = 1e-3 * B + 2.0 ** -8 * Bw
    Wqd, Sd = _dev_q4(Wq, S)
    Xd, gd = X.to(DEV), synth.from_bits(g, torch.bfloat16, DEV)
    kind = L.LIN_KIND_GEMV_Q4G64_NORM
    cands = L.lin_candidates(kind, 1, N, K)
    assert cands
    for cfg in cands:
        with pinned(kind, 1, N, K, cfg):
            y = L.lin_gemv_q4g64_norm(Wqd, Sd, Xd, gd, eps)
            torch.cuda.synchronize()
            _check(y, Y, bound, "norm %s" % cfg)


@pytest.mark.parametrize("N,K", [(64, 128), (96, 3584)])
def test_q4_offset_removal_within_stated_bound_on_adversarial_x(N, K):
    """x shrunk by 1e-3 exactly at the (shared) outlier positions: sum |q x| is
    then tiny against sum |x|, and the result must stay within the bound the
    library states for int4 (every GEMV candidate at M = 1, every batched
    candidate at M = 1 and M = 16)."""
    print("case q4 adversarial N=%d K=%d" % (N, K), flush=True)
    seed = 25000 + N + K
    Wq, S, pos = _outlier_q4(seed, N, K, shared=True)
    Wqd, Sd = _dev_q4(Wq, S)
    Wt = L.lin_q4g64_tile(Wqd, Sd)
    for M, kind in ((1, L.LIN_KIND_GEMV_Q4G64), (1, L.LIN_KIND_SKINNY_Q4G64),
                    (16, L.LIN_KIND_SKINNY_Q4G64)):
        X = _tiny_at(synth.activation(seed, 0, 1, M, K), pos[0])
        Y, B = oracle.gemm_q4g64(Wq, S, u16(X))
        bound = 1e-4 * B + 4e-4 * _scale_term(S, X)
        Xd = X.to(DEV)
        for cfg in L.lin_candidates(kind, M, N, K):
            with pinned(kind, M, N, K, cfg):
                y = torch.full((M, N), float("nan"), device=DEV)
                if kind == L.LIN_KIND_GEMV_Q4G64:
                    L.lin_gemv_q4g64(Wqd, Sd, Xd, y)
                else:
                    L.lin_gemm_skinny_q4g64(Wt, Xd, y)
                torch.cuda.synchronize()
                _check(y, Y, bound, "adversarial kind %d %s" % (kind, cfg))


def _i8_case(seed, N, K, one_hot):
    if one_hot:
        rng = np.random.default_rng(seed)
        W = torch.zeros((N, K), dtype=torch.float32)
        cols = rng.integers(0, K, size=N)
        W[torch.arange(N), torch.from_numpy(cols)] = torch.from_numpy(
            rng.uniform(0.5, 1.0, size=N) * rng.choice([-1.0, 1.0], size=N)).float()
        W = W.to(torch.bfloat16)
    else:
        W, _ = synth.outlier_weight(seed, N, K, group=K)   # one outlier per row
    Wq, S = oracle.quantize_i8(u16(W))
    return Wq, S


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("one_hot", [True, False])
def test_i8_outlier_rows_every_candidate(M, N, K, one_hot):
    print("case i8 %s M=%d N=%d K=%d" % ("one-hot" if one_hot else "outlier", M, N, K), flush=True)
    seed = 26000 + M + N + K + one_hot
    Wq, S = _i8_case(seed, N, K, one_hot)
    if one_hot:
        assert np.all(np.count_nonzero(Wq, axis=1) == 1) and np.all(np.abs(Wq).max(axis=1) == 127)
    X = synth.activation(seed, 0, 1, M, K)
    Y, B = oracle.gemm_i8(Wq, S, u16(X))
    Wqd, Sd, Xd = torch.from_numpy(Wq).to(DEV), torch.from_numpy(S).to(DEV), X.to(DEV)
    kind = L.LIN_KIND_GEMV_I8
    for cfg in L.lin_candidates(kind, M, N, K):
        with pinned(kind, M, N, K, cfg):
            y = torch.full((M, N), float("nan"), device=DEV)
            L.lin_gemv_i8(Wqd, Sd, Xd, y)
            torch.cuda.synchronize()
            assert_within_bound(y, Y, B, "i8 %s" % cfg)
