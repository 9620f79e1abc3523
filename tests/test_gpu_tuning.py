"""Load-time tuning on the GPU, through the C ABI.

lin_autotune (tinyinfer post, v0.2: time the candidate configurations of every
distinct shape when the model loads and keep the fastest) is run for one shape
of every kind: the configuration it returns must be one of the candidates,
carry a positive time, be the one the library then uses (lin_get_config), and
the product in it must match the oracle within the product bound.

The split-K workspace: a graph captured with a split-K configuration must keep
working after a later load-time call grows the workspace (the library never
frees a workspace a launch may have used)."""
import numpy as np
import pytest
import torch

import memory_bound_weight_amd as L
import oracle
import synth
from gpu_util import assert_within_bound, pinned, u16
from test_gpu_norm import EPS, _case as norm_case

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FIELDS = ("algo", "rows", "unroll", "split", "stage_x", "tile_m", "waves")


def _same(a, b):
    return all(a[f] == b[f] for f in FIELDS)


def _plain_case(kind, M, N, K, seed):
    """Device operands, the call, and the oracle's (Y, B) for one product kind."""
    W = synth.weight(seed, 0, 0, N, K)
    X = synth.activation(seed, 0, 1, M, K)
    Xd = X.to(DEV)
    if kind in (L.LIN_KIND_GEMV_BF16, L.LIN_KIND_SKINNY_BF16):
        Y, B = oracle.gemm_dense(u16(W), u16(X))
        Wd = W.to(DEV)
        fn = L.lin_gemv_bf16 if kind == L.LIN_KIND_GEMV_BF16 else L.lin_gemm_skinny_bf16
        return (Wd, None), Xd, lambda y: fn(Wd, Xd, y), Y, B
    if kind == L.LIN_KIND_GEMV_I8:
        Wq, S = oracle.quantize_i8(u16(W))
        Y, B = oracle.gemm_i8(Wq, S, u16(X))
        Wqd, Sd = torch.from_numpy(Wq).to(DEV), torch.from_numpy(S).to(DEV)
        return (Wqd, Sd), Xd, lambda y: L.lin_gemv_i8(Wqd, Sd, Xd, y), Y, B
    Wq, S = oracle.quantize_q4g64(u16(W))
    Y, B = oracle.gemm_q4g64(Wq, S, u16(X))
    Wqd, Sd = torch.from_numpy(Wq).to(DEV), synth.from_bits(S, torch.float16, DEV)
    if kind == L.LIN_KIND_GEMV_Q4G64:
        return (Wqd, Sd), Xd, lambda y: L.lin_gemv_q4g64(Wqd, Sd, Xd, y), Y, B
    Wt = L.lin_q4g64_tile(Wqd, Sd)
    return (Wt, None), Xd, lambda y: L.lin_gemm_skinny_q4g64(Wt, Xd, y), Y, B


PLAIN = [(L.LIN_KIND_GEMV_BF16, 1, 300, 2048), (L.LIN_KIND_GEMV_Q4G64, 1, 300, 2048),
         (L.LIN_KIND_GEMV_I8, 1, 300, 2048), (L.LIN_KIND_SKINNY_BF16, 64, 300, 2048),
         (L.LIN_KIND_SKINNY_Q4G64, 64, 300, 2048), (L.LIN_KIND_GEMV_Q4G64, 3, 300, 2048)]


@pytest.mark.parametrize("kind,M,N,K", PLAIN)
def test_lin_autotune_keeps_a_candidate_and_the_product_matches(kind, M, N, K):
    print("case lin_autotune kind=%d M=%d N=%d K=%d" % (kind, M, N, K), flush=True)
    (W, S), Xd, call, Y, B = _plain_case(kind, M, N, K, 31000 + kind)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    try:
        cfg = L.lin_autotune(kind, W, Xd, y, S)
        assert cfg["us"] > 0
        assert any(_same(cfg, c) for c in L.lin_candidates(kind, M, N, K))
        assert _same(L.lin_get_config(kind, M, N, K), cfg)
        y = torch.full((M, N), float("nan"), device=DEV)
        call(y)
        torch.cuda.synchronize()
        assert_within_bound(y, Y, B, "after lin_autotune %s" % cfg)
    finally:
        L.lin_set_config(kind, M, N, K, None)


@pytest.mark.parametrize("fmt", ["bf16", "q4", "i8"])
def test_lin_autotune_prologue_kinds(fmt):
    N, K = 300, 2048
    print("case lin_autotune norm %s N=%d K=%d" % (fmt, N, K), flush=True)
    Wt, x, g, Y, bound, kind, fn = norm_case(fmt, N, K, 32000)
    W, S = (Wt[0], None) if len(Wt) == 1 else Wt
    y = torch.empty((1, N), dtype=torch.float32, device=DEV)
    try:
        cfg = L.lin_autotune(kind, W, x, y, S)   # x stands in for the gain while timing
        assert cfg["us"] > 0
        assert any(_same(cfg, c) for c in L.lin_candidates(kind, 1, N, K))
        assert _same(L.lin_get_config(kind, 1, N, K), cfg)
        y = fn(*Wt, x, g, EPS)
        torch.cuda.synchronize()
        d = np.abs(y.cpu().numpy()[0].astype(np.float64) - Y)
        assert np.all(d <= bound), "norm %s %s: worst %.3g" % (fmt, cfg, np.max(d / bound))
    finally:
        L.lin_set_config(kind, 1, N, K, None)


def _split_cfg(kind, M, N, K, split):
    for c in L.lin_candidates(kind, M, N, K):
        if c["algo"] == L.LIN_ALGO_MFMA and c["split"] == split:
            return c
    raise AssertionError("no split-K %d candidate for %dx%dx%d" % (split, M, N, K))


def test_captured_split_k_graph_survives_workspace_growth():
    kind = L.LIN_KIND_SKINNY_BF16
    M, N, K = 64, 256, 4096
    print("case workspace growth M=%d N=%d K=%d" % (M, N, K), flush=True)
    W = synth.weight(33000, 0, 0, N, K)
    X = synth.activation(33000, 0, 1, M, K)
    Y, B = oracle.gemm_dense(u16(W), u16(X))
    Wd, Xd = W.to(DEV), X.to(DEV)
    big = (256, 2048, 8192)   # split 8: about 32 times the partial-tile bytes of the small shape
    with pinned(kind, M, N, K, _split_cfg(kind, M, N, K, 8)):
        y = torch.full((M, N), float("nan"), device=DEV)
        L.lin_gemm_skinny_bf16(Wd, Xd, y)            # eager call (loads the code)
        torch.cuda.synchronize()
        assert_within_bound(y, Y, B, "split-K before capture")
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            L.lin_gemm_skinny_bf16(Wd, Xd, y)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            L.lin_gemm_skinny_bf16(Wd, Xd, y)
        torch.cuda.synchronize()
        # a load-time call that grows the workspace, then a product in it
        Mb, Nb, Kb = big
        Wb = synth.weight(33001, 0, 0, Nb, Kb)
        Xb = synth.activation(33001, 0, 1, Mb, Kb)
        with pinned(kind, Mb, Nb, Kb, _split_cfg(kind, Mb, Nb, Kb, 8)):
            yb = torch.full((Mb, Nb), float("nan"), device=DEV)
            L.lin_gemm_skinny_bf16(Wb.to(DEV), Xb.to(DEV), yb)
            torch.cuda.synchronize()
            Yb, Bb = oracle.gemm_dense(u16(Wb), u16(Xb[:4]))
            assert_within_bound(yb[:4], Yb, Bb, "split-K on the grown workspace")
        for rep in range(3):                          # replays on the captured workspace
            y.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert_within_bound(y, Y, B, "graph replay %d after growth" % rep)
