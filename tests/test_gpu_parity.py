"""GPU parity: the HIP products against the CPU oracle, through the C ABI.

Every candidate configuration of every shape is checked: a tuned library may
pick any of them.  Bound: |y_gpu - y_oracle| <= 1e-3 * sum_k |W x| per output.
Integer work (the quantiser) must match bit for bit."""
import json
import os

import numpy as np
import pytest
import torch

import memory_bound_weight_amd as L
import oracle
import synth
from gpu_util import assert_within_bound, pinned, u16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _inputs(seed, M, N, K):
    W = synth.weight(seed, 0, 0, N, K)
    X = synth.activation(seed, 0, 0, M, K)
    return W, X


# shapes: one wave-load rows, ragged K tails (K % 512 != 0), ragged N, several tiles
# (37, 18944): x staged in more than 64 KB of LDS
BF16_SHAPES = [(1, 8), (3, 24), (7, 520), (64, 2048), (129, 1032), (257, 4104), (2048, 2048),
               (37, 18944)]
BF16_M = [1, 2, 3, 5, 8]


@pytest.mark.parametrize("N,K", BF16_SHAPES)
@pytest.mark.parametrize("M", BF16_M)
def test_gemv_bf16_every_candidate(M, N, K):
    print("case gemv_bf16 M=%d N=%d K=%d" % (M, N, K), flush=True)
    W, X = _inputs(2000 + N + K, M, N, K)
    Y, B = oracle.gemm_dense(u16(W), u16(X))
    Wd, Xd = W.to(DEV), X.to(DEV)
    cands = L.lin_candidates(L.LIN_KIND_GEMV_BF16, M, N, K)
    assert cands
    for cfg in cands:
        with pinned(L.LIN_KIND_GEMV_BF16, M, N, K, cfg):
            y = torch.full((M, N), float("nan"), device=DEV)
            L.lin_gemv_bf16(Wd, Xd, y)
            torch.cuda.synchronize()
            assert_within_bound(y, Y, B, "bf16 %s" % cfg)


Q4_SHAPES = [(1, 64), (5, 192), (33, 576), (64, 2048), (130, 3584), (2048, 2048), (37, 18944)]
Q4_M = [1, 2, 3, 8]


@pytest.mark.parametrize("N,K", Q4_SHAPES)
@pytest.mark.parametrize("M", Q4_M)
def test_gemv_q4g64_every_candidate(M, N, K):
    print("case gemv_q4g64 M=%d N=%d K=%d" % (M, N, K), flush=True)
    W, X = _inputs(3000 + N + K, M, N, K)
    Wq, S = oracle.quantize_q4g64(u16(W))
    Y, B = oracle.gemm_q4g64(Wq, S, u16(X))
    Wqd = torch.from_numpy(Wq).to(DEV)
    Sd = synth.from_bits(S, torch.float16, DEV)
    Xd = X.to(DEV)
    for cfg in L.lin_candidates(L.LIN_KIND_GEMV_Q4G64, M, N, K):
        with pinned(L.LIN_KIND_GEMV_Q4G64, M, N, K, cfg):
            y = torch.full((M, N), float("nan"), device=DEV)
            L.lin_gemv_q4g64(Wqd, Sd, Xd, y)
            torch.cuda.synchronize()
            assert_within_bound(y, Y, B, "q4 %s" % cfg)


# VALU path (M <= 32) and matrix-core path (M > 16): ragged M, N and K tails
SKINNY_CASES = [(1, 64, 2048), (9, 130, 1032), (16, 257, 520), (17, 64, 2048), (31, 100, 4096),
                (33, 100, 4096), (48, 1000, 576), (64, 130, 1032), (100, 257, 520),
                (256, 64, 2048), (256, 300, 4104)]


@pytest.mark.parametrize("M,N,K", SKINNY_CASES)
def test_skinny_bf16_every_candidate(M, N, K):
    print("case skinny M=%d N=%d K=%d" % (M, N, K), flush=True)
    W, X = _inputs(4000 + M + N + K, M, N, K)
    Y, B = oracle.gemm_dense(u16(W), u16(X))
    Wd, Xd = W.to(DEV), X.to(DEV)
    for cfg in L.lin_candidates(L.LIN_KIND_SKINNY_BF16, M, N, K):
        with pinned(L.LIN_KIND_SKINNY_BF16, M, N, K, cfg):
            y = torch.full((M, N), float("nan"), device=DEV)
            L.lin_gemm_skinny_bf16(Wd, Xd, y)
            torch.cuda.synchronize()
            assert_within_bound(y, Y, B, "skinny %s" % cfg)


def _pack(q):
    q = np.asarray(q, dtype=np.int64)
    return ((q[:, 0::2] & 0xF) | ((q[:, 1::2] & 0xF) << 4)).astype(np.uint8)


def test_q4_one_hot_exact_on_gpu():
    """Integer codes, power-of-two scales and one-hot x: y = q[n][j] * s[n][j/64]
    exactly, for every code including -8 and 7 (pins nibble order and sign)."""
    N, K = 40, 256
    rng = np.random.default_rng(21)
    q = rng.integers(-8, 8, (N, K))
    q[0, :16] = np.arange(-8, 8)
    q[1, 16:32] = np.arange(7, -9, -1)
    sexp = rng.integers(-6, 3, (N, K // 64))
    S = oracle.f16_from_f64(np.ldexp(1.0, sexp))
    Wqd = torch.from_numpy(_pack(q)).to(DEV)
    Sd = synth.from_bits(S, torch.float16, DEV)
    cols = [0, 1, 2, 3, 15, 16, 31, 63, 64, 65, 127, 128, 200, 255]
    for cfg in L.lin_candidates(L.LIN_KIND_GEMV_Q4G64, 1, N, K):
        with pinned(L.LIN_KIND_GEMV_Q4G64, 1, N, K, cfg):
            for j in cols:
                x = torch.zeros((1, K), dtype=torch.bfloat16)
                x[0, j] = 1.0
                y = L.lin_gemv_q4g64(Wqd, Sd, x.to(DEV))
                torch.cuda.synchronize()
                expect = q[:, j] * np.ldexp(1.0, sexp[:, j // 64])
                assert np.array_equal(y.cpu().numpy()[0].astype(np.float64), expect), (cfg, j)


def test_bf16_integer_closed_form_exact():
    """Small integers: every partial sum is exact in fp32, so y is exact."""
    rng = np.random.default_rng(22)
    N, K, M = 50, 1032, 3
    wi = rng.integers(-3, 4, (N, K)).astype(np.float32)
    xi = rng.integers(-2, 3, (M, K)).astype(np.float32)
    Wd = torch.from_numpy(wi).to(torch.bfloat16).to(DEV)
    Xd = torch.from_numpy(xi).to(torch.bfloat16).to(DEV)
    for cfg in L.lin_candidates(L.LIN_KIND_GEMV_BF16, M, N, K):
        with pinned(L.LIN_KIND_GEMV_BF16, M, N, K, cfg):
            y = L.lin_gemv_bf16(Wd, Xd)
            torch.cuda.synchronize()
            assert np.array_equal(y.cpu().numpy(), xi @ wi.T), cfg


def test_quantizer_bit_exact():
    shapes = [(1, 64), (7, 192), (130, 3584), (512, 2048)]
    for N, K in shapes:
        W = synth.weight(5000 + N, 0, 0, N, K)
        Wb = u16(W).copy()
        if N >= 7:
            Wb[2, 64:128] = 0                         # all-zero group
            Wb[3, 0:64] = 0x3520                      # tiny group, subnormal scale
            Wb[3, 1] = 0xB520                         # clamps to -8
            Wb[4, 0:64] = 0x4900                      # scale saturates
            Wb[5, :] = 0x3F80                         # ties of w/s
        Wq_o, S_o = oracle.quantize_q4g64(Wb)
        Wq, S = L.lin_quantize_q4g64(synth.from_bits(Wb, torch.bfloat16, DEV))
        torch.cuda.synchronize()
        assert np.array_equal(Wq.cpu().numpy(), Wq_o), (N, K)
        assert np.array_equal(u16(S), S_o), (N, K)
        # the products on these weights, special groups included
        X = synth.activation(5100 + N, 0, 0, 2, K)
        Y, B = oracle.gemm_q4g64(Wq_o, S_o, u16(X))
        y = L.lin_gemv_q4g64(Wq, S, X.to(DEV))
        torch.cuda.synchronize()
        assert_within_bound(y, Y, B, "q4 special groups %dx%d" % (N, K))


def test_quantizer_worked_examples_on_gpu():
    with open(os.path.join(GOLDEN, "q4g64_worked.json")) as f:
        cases = json.load(f)["cases"]
    w = np.zeros((len(cases), 64), dtype=np.uint16)
    for i, c in enumerate(cases):
        vals = [int(h, 16) for h in c["w_bf16"]]
        w[i, :len(vals)] = vals
    Wq, S = L.lin_quantize_q4g64(synth.from_bits(w, torch.bfloat16, DEV))
    torch.cuda.synchronize()
    Wq, S = Wq.cpu().numpy(), u16(S)
    for i, c in enumerate(cases):
        assert S[i, 0] == int(c["scale_f16"], 16), c["name"]
        b = [int(h, 16) for h in c["bytes"]]
        assert list(Wq[i, :len(b)]) == b and not Wq[i, len(b):].any(), c["name"]


def test_quantizer_scale_exhaustive_over_bf16_absmax():
    """Every positive finite bf16 as a group's absmax: the fp16 scale a/7 and the
    code of a itself match the oracle bit for bit."""
    a = np.arange(1, 0x7F80, dtype=np.uint16)
    w = np.zeros((a.size, 64), dtype=np.uint16)
    w[:, 0] = a
    w[:, 1] = a | 0x8000
    w[:, 2] = a >> 1
    Wq_o, S_o = oracle.quantize_q4g64(w)
    Wq, S = L.lin_quantize_q4g64(synth.from_bits(w, torch.bfloat16, DEV))
    torch.cuda.synchronize()
    assert np.array_equal(u16(S), S_o)
    assert np.array_equal(Wq.cpu().numpy(), Wq_o)


def test_results_are_deterministic():
    N, K = 3000, 4096
    W, X = _inputs(6000, 1, N, K)
    Wd, Xd = W.to(DEV), X.to(DEV)
    Wq, S = L.lin_quantize_q4g64(Wd)
    for cfg in L.lin_candidates(L.LIN_KIND_GEMV_BF16, 1, N, K)[:6]:
        with pinned(L.LIN_KIND_GEMV_BF16, 1, N, K, cfg):
            a = L.lin_gemv_bf16(Wd, Xd)
            b = L.lin_gemv_bf16(Wd, Xd)
            torch.cuda.synchronize()
            assert torch.equal(a, b)
    for cfg in L.lin_candidates(L.LIN_KIND_GEMV_Q4G64, 1, N, K)[::3]:
        with pinned(L.LIN_KIND_GEMV_Q4G64, 1, N, K, cfg):
            a = L.lin_gemv_q4g64(Wq, S, Xd)
            b = L.lin_gemv_q4g64(Wq, S, Xd)
            torch.cuda.synchronize()
            assert torch.equal(a, b), cfg


def test_empty_and_degenerate_shapes():
    # K = 0: y is zeroed
    y = torch.full((2, 5), 7.0, device=DEV)
    e = torch.empty((5, 0), dtype=torch.bfloat16, device=DEV)
    x = torch.empty((2, 0), dtype=torch.bfloat16, device=DEV)
    L.lin_gemv_bf16(e, x, y)
    L.lin_gemm_skinny_bf16(e, x, y)
    torch.cuda.synchronize()
    assert torch.equal(y, torch.zeros_like(y))
    y = torch.full((1, 3), 7.0, device=DEV)
    L.lin_gemv_q4g64(torch.empty((3, 0), dtype=torch.uint8, device=DEV),
                     torch.empty((3, 0), dtype=torch.float16, device=DEV),
                     torch.empty((1, 0), dtype=torch.bfloat16, device=DEV), y)
    torch.cuda.synchronize()
    assert torch.equal(y, torch.zeros_like(y))
    # N = 0 / M = 0: nothing written, no error
    L.lin_gemv_bf16(torch.empty((0, 8), dtype=torch.bfloat16, device=DEV),
                    torch.ones((1, 8), dtype=torch.bfloat16, device=DEV))
    # misaligned view is rejected before any launch
    W = torch.zeros((4, 16), dtype=torch.bfloat16, device=DEV)
    flat = torch.zeros(80, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(L.LinError) as ei:
        L.lin_gemv_bf16(W, flat[4:20].view(1, 16))
    assert ei.value.status == L.LIN_ERR_ALIGN
    torch.cuda.synchronize()


def test_output_rows_past_n_untouched():
    """The kernels never write outside y: a guard band after y keeps its values."""
    for kind, N, K, M in [(L.LIN_KIND_GEMV_BF16, 37, 1032, 3), (L.LIN_KIND_GEMV_Q4G64, 37, 1088, 3),
                          (L.LIN_KIND_GEMV_Q4G64, 37, 1088, 1), (L.LIN_KIND_GEMV_Q4G64, 300, 3584, 1)]:
        W, X = _inputs(7000 + N, M, N, K)
        buf = torch.full((M * N + 256,), 12345.0, device=DEV)
        y = buf[:M * N].view(M, N)
        for cfg in L.lin_candidates(kind, M, N, K):
            with pinned(kind, M, N, K, cfg):
                if kind == L.LIN_KIND_GEMV_BF16:
                    L.lin_gemv_bf16(W.to(DEV), X.to(DEV), y)
                else:
                    Wq, S = L.lin_quantize_q4g64(W.to(DEV))
                    L.lin_gemv_q4g64(Wq, S, X.to(DEV), y)
                torch.cuda.synchronize()
                assert torch.all(buf[M * N:] == 12345.0), cfg


def test_split_k_workspace_shared_across_shapes():
    """Split-K configurations of shapes with few and with many output tiles run
    one after another on the shared workspace; each must stay exact to the
    bound (the tile counters live in a region partial tiles never touch)."""
    cases = [(64, 130, 4096), (64, 4096, 4096), (40, 200, 2048), (64, 2000, 4096)]
    data = []
    for M, N, K in cases:
        W, X = _inputs(9300 + N, M, N, K)
        data.append((M, N, K, W.to(DEV), X.to(DEV), oracle.gemm_dense(u16(W), u16(X))))
    for rep in range(2):
        for M, N, K, Wd, Xd, (Y, B) in data:
            splits = [c for c in L.lin_candidates(L.LIN_KIND_SKINNY_BF16, M, N, K)
                      if c["algo"] == L.LIN_ALGO_MFMA and (c["split"] != 1 or c["stage_x"] == 2)]
            assert splits
            for cfg in splits:
                with pinned(L.LIN_KIND_SKINNY_BF16, M, N, K, cfg):
                    y = L.lin_gemm_skinny_bf16(Wd, Xd)
                    torch.cuda.synchronize()
                    assert_within_bound(y, Y, B, "split-K %dx%dx%d %s" % (M, N, K, cfg))


@pytest.mark.parametrize("kind,M,N,K", [(0, 1, 300, 2048), (1, 1, 300, 2048), (2, 64, 300, 1024)])
def test_autotune_set_keeps_results_exact(kind, M, N, K):
    """Tuning over a set of same-shaped matrices picks a candidate that the
    later calls use, and that candidate still matches the oracle."""
    print("case autotune_set kind=%d M=%d N=%d K=%d" % (kind, M, N, K), flush=True)
    mats = [synth.weight(9700 + i, 0, 0, N, K) for i in range(3)]
    X = synth.activation(9700, 0, 0, M, K)
    Xd = X.to(DEV)
    y = torch.empty((M, N), device=DEV)
    if kind == L.LIN_KIND_GEMV_Q4G64:
        qs = [oracle.quantize_q4g64(u16(W)) for W in mats]
        Wqs = [torch.from_numpy(q).to(DEV) for q, _ in qs]
        Ss = [synth.from_bits(sc, torch.float16, DEV) for _, sc in qs]
        cfg = L.lin_autotune_set(kind, Wqs, Xd, y, Ss=Ss)
    else:
        Wds = [W.to(DEV) for W in mats]
        cfg = L.lin_autotune_set(kind, Wds, Xd, y)
    try:
        assert cfg["us"] > 0
        assert L.lin_get_config(kind, M, N, K) == dict(cfg, us=0.0)
        for i in range(3):
            y = torch.full((M, N), float("nan"), device=DEV)
            if kind == L.LIN_KIND_GEMV_Q4G64:
                Y, B = oracle.gemm_q4g64(qs[i][0], qs[i][1], u16(X))
                L.lin_gemv_q4g64(Wqs[i], Ss[i], Xd, y)
            else:
                Y, B = oracle.gemm_dense(u16(mats[i]), u16(X))
                if kind == L.LIN_KIND_GEMV_BF16:
                    L.lin_gemv_bf16(Wds[i], Xd, y)
                else:
                    L.lin_gemm_skinny_bf16(Wds[i], Xd, y)
            torch.cuda.synchronize()
            assert_within_bound(y, Y, B, "autotune_set %s" % cfg)
    finally:
        L.lin_set_config(kind, M, N, K, None)


def test_large_lds_configuration_pinned_then_captured_in_a_graph():
    """A staged-x configuration above 64 KB of LDS, pinned at load time, runs
    correctly when its first launch is inside a graph capture; every replay
    (with eager work in between) matches the oracle."""
    N, K, M = 37, 18944, 1
    print("case large-LDS graph N=%d K=%d" % (N, K), flush=True)
    W, X = _inputs(9800, M, N, K)
    Wq, S = oracle.quantize_q4g64(u16(W))
    Y, B = oracle.gemm_q4g64(Wq, S, u16(X))
    Wqd = torch.from_numpy(Wq).to(DEV)
    Sd = synth.from_bits(S, torch.float16, DEV)
    Xd = X.to(DEV)
    staged = [c for c in L.lin_candidates(L.LIN_KIND_GEMV_Q4G64, M, N, K) if c["stage_x"] == 1]
    assert staged
    cfg = staged[0]
    y = torch.full((M, N), float("nan"), device=DEV)
    try:
        L.lin_set_config(L.LIN_KIND_GEMV_Q4G64, M, N, K, cfg)
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                L.lin_gemv_q4g64(Wqd, Sd, Xd, y)
        for rep in range(3):
            y.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert_within_bound(y, Y, B, "graph replay %d %s" % (rep, cfg))
            torch.empty(1 << 20, device=DEV).normal_()   # eager work between replays
    finally:
        L.lin_set_config(L.LIN_KIND_GEMV_Q4G64, M, N, K, None)


def test_stream_read_runs_on_ragged_sizes():
    """The read-only pass used as the bandwidth ceiling: any multiple of 16
    bytes, including sizes that leave a partial workgroup, completes without
    error and leaves the buffer unchanged."""
    for nbytes in (16, 4096 + 16, (1 << 20) + 48, 3 << 20):
        buf = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV)
        ref = buf.clone()
        L.lin_stream_read(buf)
        torch.cuda.synchronize()
        assert torch.equal(buf, ref)
