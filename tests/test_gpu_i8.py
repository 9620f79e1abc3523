"""GPU parity of the INT8 product (lin_gemv_i8) and quantiser (lin_quantize_i8)
against the CPU oracle, through the C ABI.  Every candidate configuration is
checked; the quantiser must match bit for bit.  Bound: |y_gpu - y_oracle| <=
1e-3 * sum_k |w x| per output."""
import numpy as np
import pytest
import torch

import memory_bound_weight_amd as L
import oracle
import synth
from gpu_util import assert_within_bound, pinned, u16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
KIND = L.LIN_KIND_GEMV_I8

# ragged N, K not a multiple of the 1 KiB wavefront row (K % 1024 != 0), long K
SHAPES = [(1, 16), (5, 48), (33, 528), (64, 2048), (130, 3584), (2048, 2048), (37, 18944)]


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("M", [1, 2, 3, 8])
def test_gemv_i8_every_candidate(M, N, K):
    print("case gemv_i8 M=%d N=%d K=%d" % (M, N, K), flush=True)
    W = synth.weight(8000 + N + K, 0, 0, N, K)
    X = synth.activation(8000 + N + K, 0, 0, M, K)
    Wq, S = oracle.quantize_i8(u16(W))
    Y, B = oracle.gemm_i8(Wq, S, u16(X))
    Wqd = torch.from_numpy(Wq).to(DEV)
    Sd = torch.from_numpy(S).to(DEV)
    Xd = X.to(DEV)
    cands = L.lin_candidates(KIND, M, N, K)
    assert cands
    for cfg in cands:
        with pinned(KIND, M, N, K, cfg):
            y = torch.full((M, N), float("nan"), device=DEV)
            L.lin_gemv_i8(Wqd, Sd, Xd, y)
            torch.cuda.synchronize()
            assert_within_bound(y, Y, B, "i8 %s" % cfg)


def test_quantizer_bit_exact():
    """Workload-like rows, a zero row, tiny (subnormal-range) and huge rows, and
    exact ties: codes and scales equal the oracle's bit for bit."""
    rng = np.random.default_rng(51)
    N, K = 70, 1040
    W = synth.bits(synth.weight(51, 0, 0, N, K))
    W[3] = 0
    W[4] = (rng.integers(0, 0x0080, K) | (rng.integers(0, 2, K) << 15)).astype(np.uint16)   # subnormal bf16
    W[5] = (rng.integers(0x7E00, 0x7F7F, K) | (rng.integers(0, 2, K) << 15)).astype(np.uint16)   # huge
    s = 2.0 ** -7                                                         # ties at half multiples
    ties = np.array([127 * s] + [(j + 0.5) * s * (1 if j % 2 else -1) for j in range(15)], dtype=np.float32)
    W[6, :16] = (ties.view(np.uint32) >> 16).astype(np.uint16)
    W[6, 16:] = 0
    Wq, S = oracle.quantize_i8(W)
    Wd = synth.from_bits(W, torch.bfloat16, DEV)
    q, sc = L.lin_quantize_i8(Wd)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), Wq)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), S.view(np.uint32))


def test_one_hot_exact():
    N, K = 40, 272
    rng = np.random.default_rng(52)
    Wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    Wq[0, :5] = [-127, -1, 0, 1, 127]
    S = np.ldexp(1.0, rng.integers(-10, -2, N)).astype(np.float32)
    Wqd, Sd = torch.from_numpy(Wq).to(DEV), torch.from_numpy(S).to(DEV)
    for cfg in L.lin_candidates(KIND, 1, N, K):
        with pinned(KIND, 1, N, K, cfg):
            for j in (0, 1, 4, 15, 16, 17, 128, 271):
                x = torch.zeros((1, K), dtype=torch.bfloat16)
                x[0, j] = 1.0
                y = L.lin_gemv_i8(Wqd, Sd, x.to(DEV))
                torch.cuda.synchronize()
                expect = Wq[:, j].astype(np.float64) * S.astype(np.float64)
                assert np.array_equal(y.cpu().numpy()[0].astype(np.float64), expect), (cfg, j)


def test_degenerate_shapes():
    y = torch.full((2, 5), float("nan"), device=DEV)
    L.lin_gemv_i8(torch.zeros((5, 0), dtype=torch.int8, device=DEV),
                  torch.zeros((5,), dtype=torch.float32, device=DEV),
                  torch.zeros((2, 0), dtype=torch.bfloat16, device=DEV), y)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0
    assert L._lib.lin_gemv_i8(None, None, None, None, 0, 5, 32, None) == L.LIN_OK
    assert L._lib.lin_gemv_i8(None, None, None, y.data_ptr(), 2, 5, 0, None) == L.LIN_OK
