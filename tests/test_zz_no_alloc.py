"""The allocation-free batched product (lin_gemm_skinny_bf16_noalloc), through
the C ABI, against the entry point it varies (lin_gemm_skinny_bf16) and the
oracle.  Split-K configurations are forced, so the static scratch array holds
the partial tiles and tile counters: two calls in a row, the second on a
smaller input, must each give the same bits as lin_gemm_skinny_bf16 in the same
configuration (which uses the library-owned workspace) and stay within the
product bound |y - y_oracle| <= 1e-3 * sum_k |W x|."""
import pytest
import torch

import memory_bound_weight_amd as L
import oracle
import synth
from gpu_util import assert_within_bound, pinned, u16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
KIND = L.LIN_KIND_SKINNY_BF16


def _split_cfg(M, N, K, split):
    for c in L.lin_candidates(KIND, M, N, K):
        if c["algo"] == L.LIN_ALGO_MFMA and c["split"] == split:
            return c
    raise AssertionError("no split-K %d candidate for %dx%dx%d" % (split, M, N, K))


def _case(seed, M, N, K):
    W = synth.weight(seed, 0, 0, N, K)
    X = synth.activation(seed, 0, 1, M, K)
    Y, B = oracle.gemm_dense(u16(W), u16(X))
    return W.to(DEV), X.to(DEV), Y, B


def test_noalloc_matches_the_workspace_entry_point_twice_in_a_row():
    cases = [(64, 1024, 4096, 8), (32, 256, 2048, 4)]   # the second call is smaller
    for i, (M, N, K, split) in enumerate(cases):
        print("case noalloc call %d M=%d N=%d K=%d split=%d" % (i, M, N, K, split), flush=True)
        Wd, Xd, Y, B = _case(40000 + i, M, N, K)
        cfg = _split_cfg(M, N, K, split)
        y_static = torch.full((M, N), float("nan"), device=DEV)
        L.lin_gemm_skinny_bf16_noalloc(Wd, Xd, y_static, cfg)
        torch.cuda.synchronize()
        assert_within_bound(y_static, Y, B, "noalloc %s" % cfg)
        with pinned(KIND, M, N, K, cfg):
            y_ws = torch.full((M, N), float("nan"), device=DEV)
            L.lin_gemm_skinny_bf16(Wd, Xd, y_ws)
            torch.cuda.synchronize()
        assert torch.equal(y_static, y_ws), "noalloc and workspace results differ (%s)" % cfg


def test_noalloc_repeated_calls_and_table_configuration():
    M, N, K = 48, 512, 2048
    print("case noalloc repeat M=%d N=%d K=%d" % (M, N, K), flush=True)
    Wd, Xd, Y, B = _case(40100, M, N, K)
    cfg = _split_cfg(M, N, K, 2)
    first = torch.empty((M, N), device=DEV)
    L.lin_gemm_skinny_bf16_noalloc(Wd, Xd, first, cfg)
    for _ in range(3):                                  # counters are left cleared
        y = torch.full((M, N), float("nan"), device=DEV)
        L.lin_gemm_skinny_bf16_noalloc(Wd, Xd, y, cfg)
        torch.cuda.synchronize()
        assert torch.equal(y, first)
    assert_within_bound(first, Y, B, "noalloc repeated")
    # no configuration given: the table's (here the built-in default)
    y = torch.full((M, N), float("nan"), device=DEV)
    L.lin_gemm_skinny_bf16_noalloc(Wd, Xd, y)
    ref = L.lin_gemm_skinny_bf16(Wd, Xd)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)


def test_noalloc_refuses_configurations_beyond_the_scratch():
    M, N, K = 256, 32000, 4096
    cfg = _split_cfg(M, N, K, 8)
    W = torch.zeros((N, K), dtype=torch.bfloat16, device=DEV)
    X = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    Y = torch.zeros((M, N), dtype=torch.float32, device=DEV)
    c = L.LinConfig.from_dict(cfg)
    import ctypes
    rc = L._lib.lin_gemm_skinny_bf16_noalloc(W.data_ptr(), X.data_ptr(), Y.data_ptr(), M, N, K,
                                             ctypes.byref(c), None)
    assert rc == L.LIN_ERR_SCRATCH
    bad = dict(cfg, rows=3)
    rc = L._lib.lin_gemm_skinny_bf16_noalloc(W.data_ptr(), X.data_ptr(), Y.data_ptr(), M, N, K,
                                             ctypes.byref(L.LinConfig.from_dict(bad)), None)
    assert rc == L.LIN_ERR_UNSUPPORTED
