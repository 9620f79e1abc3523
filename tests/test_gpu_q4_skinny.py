"""GPU parity of the int4-g64 batched-token product (lin_gemm_skinny_q4g64 on
weights rearranged by lin_q4g64_tile) against the CPU oracle, through the C ABI.

Every candidate configuration of every case is checked against the oracle's
product on the plain int4-g64 layout (the rearrangement is a byte permutation
and is checked bit for bit on its own).  Bound: |y_gpu - y_oracle| <= 1e-3 *
sum_k |w x| per output."""
import numpy as np
import pytest
import torch

import memory_bound_weight_amd as L
import oracle
import synth
from gpu_util import assert_within_bound, pinned, u16
from tiled_layout import tile_codes, tile_scales

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
KIND = L.LIN_KIND_SKINNY_Q4G64


def _quantized(seed, M, N, K):
    W = synth.weight(seed, 0, 0, N, K)
    X = synth.activation(seed, 0, 0, M, K)
    Wq, S = oracle.quantize_q4g64(u16(W))
    return Wq, S, X


def _tiled(Wq, S):
    return L.lin_q4g64_tile(torch.from_numpy(Wq).to(DEV), synth.from_bits(S, torch.float16, DEV))


# ragged N (not a multiple of 16), K % 128 == 64, M around the token tiles
CASES = [(1, 64, 2048), (8, 130, 1088), (16, 257, 576), (17, 100, 4096), (33, 64, 192),
         (64, 300, 1024), (100, 257, 640), (128, 48, 2112), (200, 130, 1024), (256, 130, 2048),
         (256, 64, 4160)]


@pytest.mark.parametrize("M,N,K", CASES)
def test_skinny_q4g64_every_candidate(M, N, K):
    print("case skinny_q4 M=%d N=%d K=%d" % (M, N, K), flush=True)
    Wq, S, X = _quantized(5000 + M + N + K, M, N, K)
    Y, B = oracle.gemm_q4g64(Wq, S, u16(X))
    Wt = _tiled(Wq, S)
    Xd = X.to(DEV)
    cands = L.lin_candidates(KIND, M, N, K)
    assert cands
    for cfg in cands:
        with pinned(KIND, M, N, K, cfg):
            y = torch.full((M, N), float("nan"), device=DEV)
            L.lin_gemm_skinny_q4g64(Wt, Xd, y)
            torch.cuda.synchronize()
            assert_within_bound(y, Y, B, "skinny q4 %s" % cfg)


def test_tile_matches_layout_bit_for_bit():
    for N, K in [(1, 64), (17, 192), (130, 1088), (64, 4096)]:
        print("case tile N=%d K=%d" % (N, K), flush=True)
        Wq, S, _ = _quantized(6000 + N + K, 1, N, K)
        t = _tiled(Wq, S)
        torch.cuda.synchronize()
        assert np.array_equal(t.Wt.cpu().numpy(), tile_codes(Wq, N, K))
        assert np.array_equal(t.St.cpu().numpy().view(np.uint16), tile_scales(S, N, K))


def _pack(q):
    q = np.asarray(q, dtype=np.int64)
    return ((q[:, 0::2] & 0xF) | ((q[:, 1::2] & 0xF) << 4)).astype(np.uint8)


def test_one_hot_tokens_exact():
    """Integer codes, power-of-two scales, token m one-hot at column j_m:
    Y[m][n] = q[n][j_m] * s[n][j_m / 64] exactly, every code from -8 to 7
    (pins nibble order, sign, the k order of the tiles and the scale groups)."""
    N, K = 40, 384
    rng = np.random.default_rng(31)
    q = rng.integers(-8, 8, (N, K))
    q[0, :16] = np.arange(-8, 8)
    q[1, 16:32] = np.arange(7, -9, -1)
    sexp = rng.integers(-6, 3, (N, K // 64))
    S = oracle.f16_from_f64(np.ldexp(1.0, sexp))
    Wt = L.lin_q4g64_tile(torch.from_numpy(_pack(q)).to(DEV), synth.from_bits(S, torch.float16, DEV))
    cols = np.array([0, 1, 2, 3, 4, 7, 8, 15, 16, 31, 32, 63, 64, 65, 100, 127, 128, 129, 200,
                     255, 256, 300, 383])
    M = len(cols)
    X = torch.zeros((M, K), dtype=torch.bfloat16)
    X[np.arange(M), cols] = 1.0
    Xd = X.to(DEV)
    expect = (q[:, cols] * np.ldexp(1.0, sexp[:, cols // 64])).T
    for cfg in L.lin_candidates(KIND, M, N, K):
        with pinned(KIND, M, N, K, cfg):
            y = L.lin_gemm_skinny_q4g64(Wt, Xd)
            torch.cuda.synchronize()
            assert np.array_equal(y.cpu().numpy().astype(np.float64), expect), cfg


def test_deterministic_and_degenerate():
    M, N, K = 64, 300, 1024
    Wq, S, X = _quantized(7000, M, N, K)
    Wt = _tiled(Wq, S)
    Xd = X.to(DEV)
    for cfg in L.lin_candidates(KIND, M, N, K):
        if cfg["split"] == 1:
            continue
        with pinned(KIND, M, N, K, cfg):
            a = L.lin_gemm_skinny_q4g64(Wt, Xd)
            b = L.lin_gemm_skinny_q4g64(Wt, Xd)
            torch.cuda.synchronize()
            assert torch.equal(a, b), cfg
    # K == 0 writes zeros; M == 0 and N == 0 are empty calls
    z = L.lin_q4g64_tile(torch.zeros((5, 0), dtype=torch.uint8, device=DEV),
                         torch.zeros((5, 0), dtype=torch.float16, device=DEV))
    y = torch.full((3, 5), float("nan"), device=DEV)
    L.lin_gemm_skinny_q4g64(z, torch.zeros((3, 0), dtype=torch.bfloat16, device=DEV), y)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0
    assert L._lib.lin_gemm_skinny_q4g64(None, None, None, None, 0, 5, 64, None) == L.LIN_OK
