"""The Python binding rejects what the C ABI cannot take, before any GPU call:
wrong types and dtypes, and tensors that are not on a GPU.  CPU only (the
GPU-side battery, non-contiguous and misaligned tensors, is in
test_gpu_binding.py)."""
import pytest
import torch

import memory_bound_weight_amd as L


def _bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


CALLS = [
    ("lin_gemv_bf16", lambda: L.lin_gemv_bf16(_bf16(8, 64), _bf16(1, 64))),
    ("lin_gemv_q4g64", lambda: L.lin_gemv_q4g64(torch.zeros((8, 32), dtype=torch.uint8),
                                                torch.zeros((8, 1), dtype=torch.float16), _bf16(1, 64))),
    ("lin_gemv_i8", lambda: L.lin_gemv_i8(torch.zeros((8, 64), dtype=torch.int8),
                                          torch.zeros((8,), dtype=torch.float32), _bf16(1, 64))),
    ("lin_gemm_skinny_bf16", lambda: L.lin_gemm_skinny_bf16(_bf16(8, 64), _bf16(4, 64))),
    ("lin_gemv_bf16_ep", lambda: L.lin_gemv_bf16_ep(_bf16(8, 64), _bf16(1, 64), L.LIN_EPI_SWIGLU)),
    ("lin_gemv_bf16_norm", lambda: L.lin_gemv_bf16_norm(_bf16(8, 64), _bf16(1, 64), _bf16(64), 1e-6)),
    ("lin_quantize_q4g64", lambda: L.lin_quantize_q4g64(_bf16(8, 64))),
    ("lin_quantize_i8", lambda: L.lin_quantize_i8(_bf16(8, 64))),
]


@pytest.mark.parametrize("name,call", CALLS, ids=[c[0] for c in CALLS])
def test_host_tensors_are_refused(name, call):
    with pytest.raises(ValueError, match="GPU device"):
        call()


def test_wrong_types_and_dtypes_are_refused():
    with pytest.raises(TypeError, match="torch.Tensor"):
        L.lin_gemv_bf16([[0.0]], _bf16(1, 1))
    with pytest.raises(TypeError, match="bfloat16"):
        L.lin_gemv_bf16(torch.zeros((8, 64), dtype=torch.float32), _bf16(1, 64))
    with pytest.raises(TypeError, match="uint8"):
        L.lin_gemv_q4g64(torch.zeros((8, 32), dtype=torch.int8), torch.zeros((8, 1), dtype=torch.float16),
                         _bf16(1, 64))
