"""GPU side of the binding's input battery: tensors the C ABI cannot take are
refused before launch (non-contiguous views, wrong shapes and dtypes), and a
misaligned view reaches the C ABI, which refuses it with LIN_ERR_ALIGN."""
import pytest
import torch

import memory_bound_weight_amd as L

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16, device=DEV)


def test_non_contiguous_views_are_refused():
    print("case binding non-contiguous", flush=True)
    W = _bf16(64, 128)
    with pytest.raises(ValueError, match="contiguous"):
        L.lin_gemv_bf16(W[:, ::2], _bf16(1, 64))
    with pytest.raises(ValueError, match="contiguous"):
        L.lin_gemv_bf16(_bf16(64, 64).t(), _bf16(1, 64))
    with pytest.raises(ValueError, match="contiguous"):
        L.lin_gemm_skinny_bf16(_bf16(64, 64), _bf16(64, 8).t())
    with pytest.raises(ValueError, match="contiguous"):
        L.lin_gemv_bf16_norm(_bf16(8, 64), _bf16(1, 64), _bf16(128)[::2], 1e-6)


def test_shapes_and_dtypes_are_refused():
    print("case binding shapes", flush=True)
    W, x = _bf16(8, 64), _bf16(1, 64)
    with pytest.raises(ValueError):
        L.lin_gemv_bf16(W, _bf16(1, 32))                       # K mismatch
    with pytest.raises(ValueError):
        L.lin_gemv_bf16(W, x, y=torch.zeros((1, 7), device=DEV))
    with pytest.raises(TypeError):
        L.lin_gemv_bf16(W, x, y=torch.zeros((1, 8), dtype=torch.float16, device=DEV))
    with pytest.raises(TypeError, match="float16"):
        L.lin_gemv_q4g64(torch.zeros((8, 32), dtype=torch.uint8, device=DEV),
                         torch.zeros((8, 1), dtype=torch.bfloat16, device=DEV), x)
    with pytest.raises(ValueError):
        L.lin_gemv_q4g64(torch.zeros((8, 32), dtype=torch.uint8, device=DEV),
                         torch.zeros((8, 2), dtype=torch.float16, device=DEV), x)   # scales per 64
    with pytest.raises(ValueError):
        L.lin_gemv_bf16_norm(W, x, _bf16(32), 1e-6)             # gain length
    with pytest.raises(TypeError):
        L.lin_gemv_bf16_norm(W, x, torch.ones(64, device=DEV), 1e-6)
    with pytest.raises(ValueError):
        L.lin_gemv_bf16_ep(_bf16(7, 64), x, L.LIN_EPI_SWIGLU)   # odd gate|up rows
    with pytest.raises(ValueError):
        L.lin_gemv_bf16_ep(W, x, 5)
    with pytest.raises(L.LinError) as e:
        L.lin_gemm_skinny_bf16(W, _bf16(257, 64))               # M beyond the batched product
    assert e.value.status == L.LIN_ERR_SHAPE
    with pytest.raises(L.LinError) as e:
        L.lin_gemv_bf16(W, _bf16(9, 64))                        # M beyond the GEMV
    assert e.value.status == L.LIN_ERR_SHAPE


def test_misaligned_view_reaches_the_abi_and_is_refused():
    print("case binding misaligned", flush=True)
    flat = _bf16(8 * 64 + 1)
    W = flat[1:].view(8, 64)                                    # contiguous, 2 bytes off
    assert W.is_contiguous() and W.data_ptr() % 16 == 2
    with pytest.raises(L.LinError) as e:
        L.lin_gemv_bf16(W, _bf16(1, 64))
    assert e.value.status == L.LIN_ERR_ALIGN
    xf = _bf16(65)
    with pytest.raises(L.LinError) as e:
        L.lin_gemv_bf16_norm(_bf16(8, 64), _bf16(1, 64), xf[1:], 1e-6)
    assert e.value.status == L.LIN_ERR_ALIGN
    torch.cuda.synchronize()
