"""The byte accounting behind every GB/s and tok/s figure, pinned to the
numbers the pages print (tests/golden/pages_figures.json):

- tinyinfer post, TL;DR: a TinyLlama-1.1B decode step reads about 2.07 GB of
  bf16 weights and about 0.55 GB in int4 with one fp16 scale per 64 weights,
  so at 168 GB/s the ceilings are about 81 and 305 tokens/s;
- llm-rs benchmark post, section 2: Qwen2.5-7B in bf16 is about 15 GB, which
  at 768 GB/s gives a floor of 19.6 ms per token (at most about 51 tokens/s).

The figures are computed with the benchmark's own formulas (bench.bytes_bf16,
bench.bytes_q4) over the shape tables of synth, so a change to either formula
or table fails here.  The pages count weights only; the benchmark's x and y
terms are pinned separately by their closed form."""
import json
import os

import pytest

import bench
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


@pytest.fixture(scope="module")
def pages():
    with open(GOLDEN) as f:
        return json.load(f)


def _weight_bytes(model, fn):
    """Weight bytes of one decode step: every matrix once, M = 0 tokens (no x, no y)."""
    return sum(fn(N, K, 0) for _, _, _, N, K in synth.decode_matrices(model))


def test_tinyllama_step_bytes_match_the_pages(pages):
    p = pages["tinyllama"]
    bf16 = _weight_bytes(synth.TINYLLAMA, bench.bytes_bf16)
    q4 = _weight_bytes(synth.TINYLLAMA, bench.bytes_q4)
    assert bf16 == 2_068_840_448
    assert q4 == 549_535_744
    assert round(bf16 / 1e9, 2) == p["bf16_gb_per_token"]
    assert round(q4 / 1e9, 2) == p["int4g64_gb_per_token"]
    bw = p["bandwidth_gb_s"] * 1e9
    # "about": within one token/s of the printed figure
    assert abs(bw / bf16 - p["bf16_ceiling_tok_s_about"]) < 1.0
    assert abs(bw / q4 - p["int4g64_ceiling_tok_s_about"]) < 1.0
    # 4.25 bits per weight: 4-bit codes plus one fp16 scale per 64
    n_weights = bf16 // 2
    assert q4 * 8 == n_weights * 4 + n_weights // 64 * 16


def test_qwen7b_step_bytes_match_the_pages(pages):
    p = pages["qwen7b"]
    linear = _weight_bytes(synth.QWEN7B, bench.bytes_bf16)
    assert linear == 14_140_571_648
    vocab, hidden = synth.QWEN7B["head"][1], synth.QWEN7B["head"][2]
    total = linear + 2 * vocab * hidden        # plus the input embedding table
    assert abs(total / 1e9 - p["bf16_gb_about"]) < 0.5
    floor_ms = total / (p["bandwidth_gb_s"] * 1e9) * 1e3
    assert abs(floor_ms - p["floor_ms"]) / p["floor_ms"] < 0.02
    assert abs(1e3 / floor_ms - p["max_tok_s_about"]) < 1.0


@pytest.mark.parametrize("N,K,M", [(2048, 2048, 1), (37888, 3584, 1), (4096, 14336, 64), (1, 64, 256)])
def test_activation_terms_are_one_read_of_x_and_one_write_of_y(N, K, M):
    for fn in (bench.bytes_bf16, bench.bytes_q4, bench.bytes_i8):
        assert fn(N, K, M) - fn(N, K, 0) == 2 * M * K + 4 * M * N


def test_weight_terms_per_format():
    N, K = 4608, 3584
    assert bench.bytes_bf16(N, K, 0) == 2 * N * K
    assert bench.bytes_q4(N, K, 0) == N * K // 2 + N * K // 32
    assert bench.bytes_i8(N, K, 0) == N * K + 4 * N
