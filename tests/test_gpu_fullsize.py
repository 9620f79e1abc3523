"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (its tuning tables), on sampled outputs the oracle computes one by one.

Weights are drawn on the GPU by the seeded generator; the sampled rows (and x)
are copied back and handed to the oracle, so both sides see the same inputs.
int4 weights come from the GPU quantiser; the sampled rows of its output must
equal the oracle quantiser's output for the same bf16 rows, bit for bit."""
import os

import numpy as np
import pytest
import torch

import memory_bound_weight_amd as L
import oracle
import synth
from gpu_util import assert_within_bound, u16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _sample_rows(N, k=40, seed=0):
    rng = np.random.default_rng(seed + N)
    rows = set([0, 1, N // 2, N - 2, N - 1]) | set(rng.integers(0, N, k).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < N))


def _tuned(model_name):
    path = os.path.join(L.TUNING_DIR, "%s.json" % model_name)
    if os.path.exists(path):
        L.load_tuning(path)


def _shapes(model):
    seen = []
    for layer, parts in synth.decode_groups(model, fused=True):
        N = sum(p[2] for p in parts)
        K = parts[0][3]
        if (N, K) not in seen:
            seen.append((N, K))
    return seen


@pytest.mark.parametrize("model", [synth.TINYLLAMA, synth.QWEN7B], ids=lambda m: m["name"])
def test_decode_shapes_bf16_and_int4_sampled(model):
    _tuned(model["name"])
    for N, K in _shapes(model):
        print("case fullsize %s %dx%d" % (model["name"], N, K), flush=True)
        W = synth.weight(model["seed"], 0, 99, N, K, device=DEV)
        x = synth.activation(model["seed"], 0, 99, 1, K, device=DEV)
        rows = _sample_rows(N)
        Wr = u16(W[torch.from_numpy(rows).to(DEV)])
        xb = u16(x)
        # bf16
        y = L.lin_gemv_bf16(W, x)
        torch.cuda.synchronize()
        Y, B = oracle.gemm_dense(Wr, xb)
        assert_within_bound(y[:, torch.from_numpy(rows).to(DEV)], Y, B, "bf16 %dx%d" % (N, K))
        # int4-g64: GPU quantiser, checked against the oracle's on the sampled rows
        Wq, S = L.lin_quantize_q4g64(W)
        y4 = L.lin_gemv_q4g64(Wq, S, x)
        torch.cuda.synchronize()
        idx = torch.from_numpy(rows).to(DEV)
        Wq_o, S_o = oracle.quantize_q4g64(Wr)
        assert np.array_equal(Wq[idx].cpu().numpy(), Wq_o)
        assert np.array_equal(u16(S[idx]), S_o)
        Y4, B4 = oracle.gemm_q4g64(Wq_o, S_o, xb)
        assert_within_bound(y4[:, idx], Y4, B4, "int4 %dx%d" % (N, K))
        del W, Wq, S



@pytest.mark.parametrize("M", [3, 8])
def test_decode_shapes_few_tokens_sampled(M):
    """The batch-1 products at 2-8 tokens (no table entry: default
    configurations) on every Qwen2.5-7B shape, bf16, int4-g64 and INT8,
    sampled rows against the oracle."""
    model = synth.QWEN7B
    _tuned(model["name"])
    for N, K in _shapes(model):
        print("case fullsize few tokens M=%d %dx%d" % (M, N, K), flush=True)
        W = synth.weight(model["seed"] + 3, 0, 98, N, K, device=DEV)
        x = synth.activation(model["seed"] + 3, 0, 98, M, K, device=DEV)
        rows = _sample_rows(N, k=12)
        idx = torch.from_numpy(rows).to(DEV)
        Wr = u16(W[idx])
        xb = u16(x)
        y = L.lin_gemv_bf16(W, x)
        torch.cuda.synchronize()
        Y, B = oracle.gemm_dense(Wr, xb)
        assert_within_bound(y[:, idx], Y, B, "bf16 M=%d %dx%d" % (M, N, K))
        Wq, S = L.lin_quantize_q4g64(W)
        y4 = L.lin_gemv_q4g64(Wq, S, x)
        torch.cuda.synchronize()
        Y4, B4 = oracle.gemm_q4g64(*oracle.quantize_q4g64(Wr), xb)
        assert_within_bound(y4[:, idx], Y4, B4, "int4 M=%d %dx%d" % (M, N, K))
        W8, S8 = L.lin_quantize_i8(W)
        y8 = L.lin_gemv_i8(W8, S8, x)
        torch.cuda.synchronize()
        Y8, B8 = oracle.gemm_i8(*oracle.quantize_i8(Wr), xb)
        assert_within_bound(y8[:, idx], Y8, B8, "i8 M=%d %dx%d" % (M, N, K))
        del W, Wq, S, W8, S8


def test_single_gemv_full_oracle():
    N, K = synth.SINGLE_SHAPE
    W = synth.weight(synth.SINGLE_SEED, 0, 0, N, K, device=DEV)
    x = synth.activation(synth.SINGLE_SEED, 0, 0, 1, K, device=DEV)
    y = L.lin_gemv_bf16(W, x)
    torch.cuda.synchronize()
    Y, B = oracle.gemm_dense(u16(W), u16(x))
    assert_within_bound(y, Y, B, "single 2048x2048")


@pytest.mark.parametrize("model", [synth.TINYLLAMA, synth.QWEN7B], ids=lambda m: m["name"])
def test_decode_shapes_int8_sampled(model):
    _tuned(model["name"] + "-i8")
    for N, K in _shapes(model):
        print("case fullsize i8 %s %dx%d" % (model["name"], N, K), flush=True)
        W = synth.weight(model["seed"], 0, 98, N, K, device=DEV)
        x = synth.activation(model["seed"], 0, 98, 1, K, device=DEV)
        rows = _sample_rows(N)
        idx = torch.from_numpy(rows).to(DEV)
        Wr = u16(W[idx])
        Wq, S = L.lin_quantize_i8(W)
        y = L.lin_gemv_i8(Wq, S, x)
        torch.cuda.synchronize()
        Wq_o, S_o = oracle.quantize_i8(Wr)
        assert np.array_equal(Wq[idx].cpu().numpy(), Wq_o)
        assert np.array_equal(S[idx].cpu().numpy().view(np.uint32), S_o.view(np.uint32))
        Y, B = oracle.gemm_i8(Wq_o, S_o, u16(x))
        assert_within_bound(y[:, idx], Y, B, "i8 %dx%d" % (N, K))
        del W, Wq, S


@pytest.mark.parametrize("M", list(synth.MISTRAL_M))
def test_mistral_skinny_q4_sampled(M):
    _tuned("mistral-7b-skinny-q4")
    for N, K in synth.MISTRAL_SHAPES:
        print("case skinny q4 full M=%d %dx%d" % (M, N, K), flush=True)
        W = synth.weight(synth.MISTRAL_SEED, 0, N, N, K, device=DEV)
        X = synth.activation(synth.MISTRAL_SEED, 0, N, M, K, device=DEV)
        Wq, S = L.lin_quantize_q4g64(W)
        T = L.lin_q4g64_tile(Wq, S)
        Y = L.lin_gemm_skinny_q4g64(T, X)
        torch.cuda.synchronize()
        rows = _sample_rows(N, k=12 if M == 256 else 24)
        idx = torch.from_numpy(rows).to(DEV)
        Wq_o, S_o = oracle.quantize_q4g64(u16(W[idx]))
        assert np.array_equal(Wq[idx].cpu().numpy(), Wq_o)
        Yo, Bo = oracle.gemm_q4g64(Wq_o, S_o, u16(X))
        assert_within_bound(Y[:, idx], Yo, Bo, "skinny q4 M=%d %dx%d" % (M, N, K))
        del W, Wq, S, T


@pytest.mark.parametrize("M", list(synth.MISTRAL_M))
def test_mistral_skinny_sampled(M):
    _tuned("mistral-7b-skinny")
    for N, K in synth.MISTRAL_SHAPES:
        print("case skinny full M=%d %dx%d" % (M, N, K), flush=True)
        W = synth.weight(synth.MISTRAL_SEED, 0, N, N, K, device=DEV)
        X = synth.activation(synth.MISTRAL_SEED, 0, N, M, K, device=DEV)
        Y = L.lin_gemm_skinny_bf16(W, X)
        torch.cuda.synchronize()
        rows = _sample_rows(N, k=12 if M == 256 else 24)
        idx = torch.from_numpy(rows).to(DEV)
        Yo, Bo = oracle.gemm_dense(u16(W[idx]), u16(X))
        assert_within_bound(Y[:, idx], Yo, Bo, "skinny M=%d %dx%d" % (M, N, K))



@pytest.mark.parametrize("M", [1, 33, 200])
def test_mistral_skinny_default_configs_sampled(M):
    """Token counts the tables hold no entry for run in the library's default
    configurations (no tuning at this M): full Mistral shapes, bf16 and tiled
    int4-g64, sampled rows against the oracle."""
    _tuned("mistral-7b-skinny")
    _tuned("mistral-7b-skinny-q4")
    for N, K in synth.MISTRAL_SHAPES:
        print("case skinny default full M=%d %dx%d" % (M, N, K), flush=True)
        W = synth.weight(synth.MISTRAL_SEED + 7, 0, N, N, K, device=DEV)
        X = synth.activation(synth.MISTRAL_SEED + 7, 0, N, M, K, device=DEV)
        rows = _sample_rows(N, k=12)
        idx = torch.from_numpy(rows).to(DEV)
        Y = L.lin_gemm_skinny_bf16(W, X)
        torch.cuda.synchronize()
        Yo, Bo = oracle.gemm_dense(u16(W[idx]), u16(X))
        assert_within_bound(Y[:, idx], Yo, Bo, "skinny default M=%d %dx%d" % (M, N, K))
        Wq, S = L.lin_quantize_q4g64(W)
        T = L.lin_q4g64_tile(Wq, S)
        Yq = L.lin_gemm_skinny_q4g64(T, X)
        torch.cuda.synchronize()
        Wq_o, S_o = oracle.quantize_q4g64(u16(W[idx]))
        Yqo, Bqo = oracle.gemm_q4g64(Wq_o, S_o, u16(X))
        assert_within_bound(Yq[:, idx], Yqo, Bqo, "skinny q4 default M=%d %dx%d" % (M, N, K))
        del W, Wq, S, T


def test_maximum_k():
    K = 1 << 22   # LIN_MAX_K
    for N in (3,):
        W = synth.weight(8000, 0, 0, N, K, device=DEV)
        x = synth.activation(8000, 0, 0, 2, K, device=DEV)
        y = L.lin_gemv_bf16(W, x)
        Wq, S = L.lin_quantize_q4g64(W)
        y4 = L.lin_gemv_q4g64(Wq, S, x)
        torch.cuda.synchronize()
        Y, B = oracle.gemm_dense(u16(W), u16(x))
        assert_within_bound(y, Y, B, "bf16 K=2^22")
        Wq_o, S_o = oracle.quantize_q4g64(u16(W))
        Y4, B4 = oracle.gemm_q4g64(Wq_o, S_o, u16(x))
        assert_within_bound(y4, Y4, B4, "int4 K=2^22")
        # INT8 and the tiled int4 batched product at the same K
        Wi, Si = L.lin_quantize_i8(W)
        yi = L.lin_gemv_i8(Wi, Si, x)
        T = L.lin_q4g64_tile(Wq, S)
        yt = L.lin_gemm_skinny_q4g64(T, x)
        torch.cuda.synchronize()
        Wi_o, Si_o = oracle.quantize_i8(u16(W))
        Yi, Bi = oracle.gemm_i8(Wi_o, Si_o, u16(x))
        assert_within_bound(yi, Yi, Bi, "i8 K=2^22")
        assert_within_bound(yt, Y4, B4, "skinny q4 K=2^22")


@pytest.mark.parametrize("model", [synth.TINYLLAMA, synth.QWEN7B], ids=lambda m: m["name"])
def test_norm_prologue_sampled(model):
    """RMSNorm folded into the normalised projections (q|k|v, gate|up with the
    gated epilogue, head) at full size, bf16, int4-g64 and INT8, in the tuned
    configurations; bound as in test_gpu_norm."""
    from test_gpu_norm import _gain, _near_boundary
    _tuned(model["name"])
    _tuned(model["name"] + "-i8")
    eps = 1e-6
    shapes = _shapes(model)
    named = {"q|k|v": shapes[0], "gate|up": shapes[2], "head": shapes[-1]}
    for name, (NW, K) in named.items():
        print("case fullsize norm %s %s %dx%d" % (model["name"], name, NW, K), flush=True)
        W = synth.weight(model["seed"], 0, 98, NW, K, device=DEV)
        x = synth.activation(model["seed"], 0, 98, 1, K, device=DEV)
        g = _gain(K, NW)
        gd = synth.from_bits(g, torch.bfloat16, DEV)
        h = oracle.rmsnorm(u16(x), g, eps)
        hw = np.where(_near_boundary(u16(x)[0], g, eps), h[0], 0).astype(np.uint16)[None, :]
        swiglu = name == "gate|up"
        N = NW // 2 if swiglu else NW
        out = _sample_rows(N)
        rows = np.concatenate([out, out + N]) if swiglu else out
        Wr = u16(W[torch.from_numpy(rows).to(DEV)])
        Wq, S = L.lin_quantize_q4g64(W)
        Wi, Si = L.lin_quantize_i8(W)
        idx = torch.from_numpy(rows).to(DEV)
        Wq_o, S_o = oracle.quantize_q4g64(Wr)
        Wi_o, Si_o = oracle.quantize_i8(Wr)
        assert np.array_equal(Wi[idx].cpu().numpy(), Wi_o)
        assert np.array_equal(Si[idx].cpu().numpy().view(np.uint32), Si_o.view(np.uint32))
        for fmt in ("bf16", "q4", "i8"):
            if fmt == "bf16":
                Y, B = oracle.gemm_dense(Wr, h)
                _, Bw = oracle.gemm_dense(Wr, hw)
                y = L.lin_gemv_bf16_norm(W, x, gd, eps, L.LIN_EPI_SWIGLU if swiglu else L.LIN_EPI_NONE)
            elif fmt == "i8":
                Y, B = oracle.gemm_i8(Wi_o, Si_o, h)
                _, Bw = oracle.gemm_i8(Wi_o, Si_o, hw)
                y = L.lin_gemv_i8_norm(Wi, Si, x, gd, eps, L.LIN_EPI_SWIGLU if swiglu else L.LIN_EPI_NONE)
            else:
                Y, B = oracle.gemm_q4g64(Wq_o, S_o, h)
                _, Bw = oracle.gemm_q4g64(Wq_o, S_o, hw)
                y = L.lin_gemv_q4g64_norm(Wq, S, x, gd, eps, L.LIN_EPI_SWIGLU if swiglu else L.LIN_EPI_NONE)
            torch.cuda.synchronize()
            got = y[0, torch.from_numpy(out).to(DEV)].cpu().numpy().astype(np.float64)
            bound = 1e-3 * B[0] + 2.0 ** -8 * Bw[0]
            if swiglu:
                n = len(out)
                gate, up, bg, bu = Y[0, :n], Y[0, n:], bound[:n], bound[n:]
                expect = oracle.swiglu(gate, up)
                silu = oracle.swiglu(gate, np.ones_like(gate))
                bound = 1.1 * np.abs(up) * bg + np.abs(silu) * bu + 1e-6 * np.abs(expect)
            else:
                expect = Y[0]
            d = np.abs(got - expect)
            assert np.all(d <= bound), "%s %s: worst %.3g" % (fmt, name, np.max(d / bound))
        del W, Wq, S, Wi, Si
