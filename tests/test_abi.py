"""The C-ABI library loads, exports every symbol include/lin.h declares, and
rejects invalid arguments before touching the GPU.  CPU only: every call here
returns from argument validation, no kernel is launched."""
import ctypes
import json
import os
import re

import pytest

import memory_bound_weight_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "lin.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(lin_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = _header_functions()
    assert len(names) >= 10
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(L.EXPORTS) == names


def test_version_and_status_strings():
    assert L.lin_version() >> 16 == 1
    for st in (L.LIN_OK, L.LIN_ERR_NULL, L.LIN_ERR_SHAPE, L.LIN_ERR_ALIGN,
               L.LIN_ERR_UNSUPPORTED, L.LIN_ERR_HIP, L.LIN_ERR_ARG, L.LIN_ERR_SCRATCH):
        assert L.status_string(st) != "unknown status"
    assert L.status_string(12345) == "unknown status"


P = 1 << 20   # a 16-byte aligned fake address; never dereferenced


@pytest.mark.parametrize("fn,args,expect", [
    # shape checks come first
    ("lin_gemv_bf16", (P, P, P, -1, 8, 8, None), L.LIN_ERR_SHAPE),
    ("lin_gemv_bf16", (P, P, P, 9, 8, 8, None), L.LIN_ERR_SHAPE),
    ("lin_gemv_bf16", (P, P, P, 1, 8, 12, None), L.LIN_ERR_SHAPE),
    ("lin_gemv_bf16", (P, P, P, 1, 1 << 31, 8, None), L.LIN_ERR_SHAPE),
    ("lin_gemv_bf16", (P, P, P, 1, 8, (1 << 22) + 8, None), L.LIN_ERR_SHAPE),
    ("lin_gemv_q4g64", (P, P, P, P, 1, 8, 96, None), L.LIN_ERR_SHAPE),
    ("lin_gemv_i8", (P, P, P, P, 1, 8, 24, None), L.LIN_ERR_SHAPE),
    ("lin_gemv_i8", (P, P, P, P, 9, 8, 32, None), L.LIN_ERR_SHAPE),
    ("lin_gemm_skinny_bf16", (P, P, P, 257, 8, 8, None), L.LIN_ERR_SHAPE),
    ("lin_gemm_skinny_bf16_noalloc", (P, P, P, 257, 8, 8, None, None), L.LIN_ERR_SHAPE),
    ("lin_gemm_skinny_bf16_noalloc", (P, P, P, 4, 8, 12, None, None), L.LIN_ERR_SHAPE),
    ("lin_gemm_skinny_q4g64", (P, P, P, P, 257, 8, 64, None), L.LIN_ERR_SHAPE),
    ("lin_gemm_skinny_q4g64", (P, P, P, P, 4, 8, 96, None), L.LIN_ERR_SHAPE),
    # empty calls succeed without pointers
    ("lin_gemv_bf16", (None, None, None, 0, 8, 8, None), L.LIN_OK),
    ("lin_gemv_bf16", (None, None, None, 1, 0, 8, None), L.LIN_OK),
    ("lin_gemv_q4g64", (None, None, None, None, 0, 0, 64, None), L.LIN_OK),
    ("lin_gemv_i8", (None, None, None, None, 0, 8, 32, None), L.LIN_OK),
    ("lin_gemm_skinny_bf16", (None, None, None, 0, 0, 0, None), L.LIN_OK),
    ("lin_gemm_skinny_bf16_noalloc", (None, None, None, 0, 8, 8, None, None), L.LIN_OK),
    ("lin_gemm_skinny_q4g64", (None, None, None, None, 0, 8, 64, None), L.LIN_OK),
    # null pointers
    ("lin_gemv_bf16", (P, P, None, 1, 8, 8, None), L.LIN_ERR_NULL),
    ("lin_gemv_bf16", (None, P, P, 1, 8, 8, None), L.LIN_ERR_NULL),
    ("lin_gemv_bf16", (P, None, P, 1, 8, 8, None), L.LIN_ERR_NULL),
    ("lin_gemv_q4g64", (P, None, P, P, 1, 8, 64, None), L.LIN_ERR_NULL),
    ("lin_gemv_i8", (P, None, P, P, 1, 8, 32, None), L.LIN_ERR_NULL),
    ("lin_gemm_skinny_bf16", (P, P, None, 4, 8, 8, None), L.LIN_ERR_NULL),
    ("lin_gemm_skinny_bf16_noalloc", (P, P, None, 4, 8, 8, None, None), L.LIN_ERR_NULL),
    ("lin_gemm_skinny_q4g64", (P, None, P, P, 4, 8, 64, None), L.LIN_ERR_NULL),
    # alignment
    ("lin_gemv_bf16", (P + 8, P, P, 1, 8, 8, None), L.LIN_ERR_ALIGN),
    ("lin_gemv_bf16", (P, P + 2, P, 1, 8, 8, None), L.LIN_ERR_ALIGN),
    ("lin_gemv_bf16", (P, P, P + 2, 1, 8, 8, None), L.LIN_ERR_ALIGN),
    ("lin_gemv_q4g64", (P, P + 1, P, P, 1, 8, 64, None), L.LIN_ERR_ALIGN),
    ("lin_gemv_i8", (P, P + 2, P, P, 1, 8, 32, None), L.LIN_ERR_ALIGN),
    ("lin_gemv_i8", (P + 8, P, P, P, 1, 8, 32, None), L.LIN_ERR_ALIGN),
    ("lin_gemm_skinny_bf16", (P + 4, P, P, 4, 8, 8, None), L.LIN_ERR_ALIGN),
    ("lin_gemm_skinny_bf16_noalloc", (P, P + 4, P, 4, 8, 8, None, None), L.LIN_ERR_ALIGN),
    ("lin_gemm_skinny_q4g64", (P, P + 2, P, P, 4, 8, 64, None), L.LIN_ERR_ALIGN),
    ("lin_gemm_skinny_q4g64", (P + 8, P, P, P, 4, 8, 64, None), L.LIN_ERR_ALIGN),
])
def test_argument_validation(fn, args, expect):
    assert getattr(L._lib, fn)(*args) == expect


def test_quantizer_validation():
    q = L._lib.lin_quantize_q4g64
    assert q(P, P, P, 4, 96, None) == L.LIN_ERR_SHAPE
    assert q(P, P, P, -1, 64, None) == L.LIN_ERR_SHAPE
    assert q(None, None, None, 0, 64, None) == L.LIN_OK
    assert q(None, P, P, 4, 64, None) == L.LIN_ERR_NULL
    assert q(P + 8, P, P, 4, 64, None) == L.LIN_ERR_ALIGN
    assert q(P, P, P + 1, 4, 64, None) == L.LIN_ERR_ALIGN


def test_tile_validation_and_sizes():
    t = L._lib.lin_q4g64_tile
    assert t(P, P, P, P, 4, 96, None) == L.LIN_ERR_SHAPE
    assert t(P, P, P, P, -1, 64, None) == L.LIN_ERR_SHAPE
    assert t(None, None, None, None, 0, 64, None) == L.LIN_OK
    assert t(None, None, None, None, 4, 0, None) == L.LIN_OK
    assert t(P, P, None, P, 4, 64, None) == L.LIN_ERR_NULL
    assert t(P, P, P, P + 8, 4, 64, None) == L.LIN_ERR_ALIGN
    assert t(P, P + 1, P, P, 4, 64, None) == L.LIN_ERR_ALIGN
    # ceil(N/16) * ceil(K/128) units of 1024 and 64 bytes
    assert L.lin_q4g64_tiled_size(1, 64) == (1024, 64)
    assert L.lin_q4g64_tiled_size(16, 128) == (1024, 64)
    assert L.lin_q4g64_tiled_size(17, 192) == (4 * 1024, 4 * 64)
    assert L.lin_q4g64_tiled_size(14336, 4096) == (896 * 32 * 1024, 896 * 32 * 64)
    assert L.lin_q4g64_tiled_size(0, 0) == (0, 0)
    with pytest.raises(L.LinError):
        L.lin_q4g64_tiled_size(8, 100)


def test_quantize_i8_validation():
    q = L._lib.lin_quantize_i8
    assert q(P, P, P, 4, 24, None) == L.LIN_ERR_SHAPE
    assert q(P, P, P, -1, 16, None) == L.LIN_ERR_SHAPE
    assert q(None, None, None, 0, 16, None) == L.LIN_OK
    assert q(None, P, P, 4, 16, None) == L.LIN_ERR_NULL
    assert q(P + 8, P, P, 4, 16, None) == L.LIN_ERR_ALIGN
    assert q(P, P + 8, P, 4, 16, None) == L.LIN_ERR_ALIGN
    assert q(P, P, P + 2, 4, 16, None) == L.LIN_ERR_ALIGN


def test_epilogue_validation():
    for f, extra in ((L._lib.lin_gemv_bf16_ep, ()), (L._lib.lin_gemv_q4g64_ep, (P,)),
                     (L._lib.lin_gemv_i8_ep, (P,))):
        assert f(P, *extra, P, P, 1, 8, 64, 3, None, None) == L.LIN_ERR_ARG
        assert f(P, *extra, P, P, 1, 8, 64, L.LIN_EPI_ADD, None, None) == L.LIN_ERR_NULL
        assert f(P, *extra, P, P, 9, 8, 64, L.LIN_EPI_NONE, None, None) == L.LIN_ERR_SHAPE
        assert f(P, *extra, P, P, 1, 1 << 30, 64, L.LIN_EPI_SWIGLU, None, None) == L.LIN_ERR_SHAPE
        assert f(P, *extra, P, P, 1, 8, 64, L.LIN_EPI_ADD, P + 2, None) == L.LIN_ERR_ALIGN
        assert f(None, *((None,) if extra else ()), None, None, 0, 8, 64, L.LIN_EPI_SWIGLU, None, None) == L.LIN_OK


def test_norm_validation():
    for f, extra in ((L._lib.lin_gemv_bf16_norm, ()), (L._lib.lin_gemv_q4g64_norm, (P,)),
                     (L._lib.lin_gemv_i8_norm, (P,))):
        assert f(P, *extra, P, P, 1e-6, P, 1, 8, 64, 3, None, None) == L.LIN_ERR_ARG
        assert f(P, *extra, P, P, -1.0, P, 1, 8, 64, 0, None, None) == L.LIN_ERR_ARG
        assert f(P, *extra, P, P, float("nan"), P, 1, 8, 64, 0, None, None) == L.LIN_ERR_ARG
        assert f(P, *extra, P, P, float("inf"), P, 1, 8, 64, 0, None, None) == L.LIN_ERR_ARG
        assert f(P, *extra, P, None, 1e-6, P, 1, 8, 64, 0, None, None) == L.LIN_ERR_NULL
        assert f(P, *extra, P, P + 8, 1e-6, P, 1, 8, 64, 0, None, None) == L.LIN_ERR_ALIGN
        assert f(P, *extra, P, P, 1e-6, P, 1, 8, 64, L.LIN_EPI_ADD, None, None) == L.LIN_ERR_NULL
        assert f(P, *extra, P, P, 1e-6, P, 2, 8, 64, 0, None, None) == L.LIN_ERR_SHAPE
        assert f(P, *extra, P, P, 1e-6, P, 1, 8, 0, 0, None, None) == L.LIN_ERR_SHAPE
        assert f(P, *extra, P, P, 1e-6, P, 1, 8, 60, 0, None, None) == L.LIN_ERR_SHAPE
        assert f(None, *((None,) if extra else ()), None, None, 1e-6, None, 0, 8, 64, 0, None,
                 None) == L.LIN_OK


def test_stream_read_validation():
    r = L._lib.lin_stream_read
    assert r(None, 0, None) == L.LIN_OK
    assert r(P, -16, None) == L.LIN_ERR_SHAPE
    assert r(P, 24, None) == L.LIN_ERR_SHAPE
    assert r(None, 16, None) == L.LIN_ERR_NULL
    assert r(P + 8, 16, None) == L.LIN_ERR_ALIGN


def test_autotune_validation():
    cfg = L.LinConfig()
    t = L._lib.lin_autotune
    assert t(8, P, P, P, P, 1, 8, 8, None, ctypes.byref(cfg)) == L.LIN_ERR_ARG
    assert t(0, P, None, P, P, 9, 8, 8, None, ctypes.byref(cfg)) == L.LIN_ERR_SHAPE
    assert t(1, P, None, P, P, 1, 8, 64, None, ctypes.byref(cfg)) == L.LIN_ERR_NULL
    assert t(0, None, None, None, None, 0, 8, 8, None, ctypes.byref(cfg)) == L.LIN_OK


def test_autotune_set_validation():
    cfg = L.LinConfig()
    t = L._lib.lin_autotune_set
    two = (ctypes.c_void_p * 2)(P, P)
    null2 = (ctypes.c_void_p * 2)(None, None)
    assert t(8, two, None, 2, P, P, 1, 8, 8, None, ctypes.byref(cfg)) == L.LIN_ERR_ARG
    assert t(0, two, None, 0, P, P, 1, 8, 8, None, ctypes.byref(cfg)) == L.LIN_ERR_ARG
    assert t(0, None, None, 2, P, P, 1, 8, 8, None, ctypes.byref(cfg)) == L.LIN_ERR_NULL
    assert t(1, two, None, 2, P, P, 1, 8, 64, None, ctypes.byref(cfg)) == L.LIN_ERR_NULL
    assert t(0, null2, None, 2, P, P, 1, 8, 8, None, ctypes.byref(cfg)) == L.LIN_ERR_NULL
    assert t(0, two, None, 2, P, P, 9, 8, 8, None, ctypes.byref(cfg)) == L.LIN_ERR_SHAPE
    assert t(0, two, None, 2, P, P, 1, 8, 12, None, ctypes.byref(cfg)) == L.LIN_ERR_SHAPE
    misaligned = (ctypes.c_void_p * 2)(P, P + 8)
    assert t(0, misaligned, None, 2, P, P, 1, 8, 8, None, ctypes.byref(cfg)) == L.LIN_ERR_ALIGN
    assert t(0, two, None, 2, None, None, 0, 8, 8, None, ctypes.byref(cfg)) == L.LIN_OK


def test_candidate_enumeration():
    for kind, M, N, K in [(0, 1, 2048, 2048), (0, 8, 512, 3584), (1, 1, 2048, 2048),
                          (1, 3, 512, 18944), (2, 8, 4096, 4096), (2, 17, 1024, 4096),
                          (3, 1, 4096, 4096), (3, 64, 14336, 4096), (3, 256, 300, 4160),
                          (4, 1, 2048, 2048), (4, 8, 300, 4112), (5, 1, 4608, 3584),
                          (6, 1, 37888, 3584)]:
        n = L.lin_num_candidates(kind, M, N, K)
        assert n > 0
        cands = L.lin_candidates(kind, M, N, K)
        assert len(cands) == n
        keys = {tuple(sorted((k, v) for k, v in c.items() if k != "us")) for c in cands}
        assert len(keys) == n                       # no duplicates
        for c in cands:
            assert c["algo"] in (L.LIN_ALGO_VALU, L.LIN_ALGO_MFMA)
            if c["algo"] == L.LIN_ALGO_VALU:
                assert c["tile_m"] >= M and c["tile_m"] < 2 * M or (M == 1 and c["tile_m"] == 1)
        assert L.lin_get_config(kind, M, N, K) in [dict(c, us=0.0) for c in cands]
    # staged x in LDS is only offered while it fits
    big = L.lin_candidates(0, 8, 4096, 14336)
    assert not any(c["stage_x"] for c in big)
    with pytest.raises(L.LinError):
        L.lin_candidate(0, 1, 8, 8, 10 ** 6)
    assert L._lib.lin_num_candidates(0, 1, 8, 12) == L.LIN_ERR_SHAPE
    assert L._lib.lin_num_candidates(8, 1, 8, 8) == L.LIN_ERR_ARG
    assert L._lib.lin_num_candidates(-1, 1, 8, 8) == L.LIN_ERR_ARG


def test_norm_kind_candidates():
    """The RMSNorm kinds offer only staged-x batch-1 configurations, refuse
    M > 1 and K == 0, and drop configurations whose x + gain copies do not fit
    in LDS."""
    for kind, base in ((L.LIN_KIND_GEMV_BF16_NORM, L.LIN_KIND_GEMV_BF16),
                       (L.LIN_KIND_GEMV_Q4G64_NORM, L.LIN_KIND_GEMV_Q4G64),
                       (L.LIN_KIND_GEMV_I8_NORM, L.LIN_KIND_GEMV_I8)):
        for N, K in ((2560, 2048), (37888, 3584), (152064, 3584)):
            cands = L.lin_candidates(kind, 1, N, K)
            assert cands and all(c["stage_x"] == 1 and c["tile_m"] == 1 for c in cands)
            staged = [c for c in L.lin_candidates(base, 1, N, K) if c["stage_x"] == 1]
            assert len(cands) == len(staged)
            assert L.lin_get_config(kind, 1, N, K)["stage_x"] == 1
        assert L._lib.lin_num_candidates(kind, 2, 2048, 2048) == L.LIN_ERR_SHAPE
        assert L._lib.lin_num_candidates(kind, 1, 2048, 0) == L.LIN_ERR_SHAPE
        big = L.lin_candidates(kind, 1, 64, 65536)
        assert len(big) < len(L.lin_candidates(kind, 1, 64, 4096))
    # x and gain copies beyond LDS: no configuration, the call is refused
    assert L.lin_candidates(L.LIN_KIND_GEMV_Q4G64_NORM, 1, 9, 32768) == []
    assert L._lib.lin_gemv_q4g64_norm(P, P, P, P, 1e-6, P, 1, 9, 32768, 0, None, None) == \
        L.LIN_ERR_UNSUPPORTED
    assert L._lib.lin_gemv_bf16_norm(P, P, P, 1e-6, P, 1, 9, 65536, 0, None, None) == \
        L.LIN_ERR_UNSUPPORTED


def test_default_skinny_config_needs_no_workspace():
    """Without tuning or pinning, a product call must never need the split-K
    workspace (it is only created by the load-time calls)."""
    for M in (17, 32, 33, 64, 100, 128, 200, 256):
        for N, K in ((1024, 4096), (14336, 4096), (4096, 14336), (300, 4104)):
            c = L.lin_get_config(L.LIN_KIND_SKINNY_BF16, M, N, K)
            if c["algo"] == L.LIN_ALGO_MFMA:
                assert c["split"] == 1 and c["stage_x"] == 4 and c["waves"] == 0, (M, N, K, c)


def test_default_q4_skinny_config_needs_no_workspace():
    for M in (1, 8, 16, 17, 32, 33, 64, 100, 128, 200, 256):
        for N, K in ((1024, 4096), (14336, 4096), (4096, 14336), (300, 4160)):
            c = L.lin_get_config(L.LIN_KIND_SKINNY_Q4G64, M, N, K)
            assert c["algo"] == L.LIN_ALGO_MFMA and c["split"] == 1, (M, N, K, c)
            assert c["tile_m"] >= min(M, 128) or c["tile_m"] == 16, (M, N, K, c)


def test_loader_wavefront_rings_are_candidates():
    """Both batched products offer the ring with four loader wavefronts
    (stage_x 5) at every split, beside the rings whose product wavefronts
    issue their own loads; the tables pick them by shape."""
    for kind in (L.LIN_KIND_SKINNY_BF16, L.LIN_KIND_SKINNY_Q4G64):
        for M in (8, 64, 256):
            cands = L.lin_candidates(kind, M, 14336, 4096)
            ld = [c for c in cands if c["algo"] == L.LIN_ALGO_MFMA and c["stage_x"] == 5]
            own = [c for c in cands if c["algo"] == L.LIN_ALGO_MFMA and c["stage_x"] == 4]
            assert ld and own, (kind, M)
            assert {c["split"] for c in ld} == {1, 2, 4, 8}, (kind, M)
    for name, kind in (("mistral-7b-skinny.json", L.LIN_KIND_SKINNY_BF16),
                       ("mistral-7b-skinny-q4.json", L.LIN_KIND_SKINNY_Q4G64)):
        table = json.load(open(os.path.join(os.path.dirname(L.__file__), "tuning", name)))
        picked = [e["cfg"]["stage_x"] for e in table["entries"] if e["kind"] == kind]
        assert 5 in picked, name


def test_candidate_configs_are_unique():
    """A configuration names one kernel: no two candidates of a kind and shape
    share every public field, so a tuning-table entry is unambiguous."""
    fields = ("algo", "rows", "unroll", "split", "stage_x", "tile_m", "waves")
    kinds = [getattr(L, k) for k in dir(L) if k.startswith("LIN_KIND_")]
    for kind in kinds:
        for M, N, K in ((1, 4096, 4096), (3, 37888, 3584), (8, 4096, 4096), (64, 14336, 4096),
                        (256, 14336, 4096), (256, 300, 4104)):
            try:
                cands = L.lin_candidates(kind, M, N, K)
            except L.LinError:
                continue
            keys = [tuple(c[f] for f in fields) for c in cands]
            assert len(keys) == len(set(keys)), (kind, M, N, K)
