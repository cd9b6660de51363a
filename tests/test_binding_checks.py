"""The Python binding refuses buffers the kernels could overrun, before anything reaches the
library: wrong element types, wrong ranks, and buffers shorter than the call reads or writes.
CPU tensors are enough here, since these checks come before the device check (no GPU needed)."""
import os

import pytest
import torch

from int8_quantized_projections_amd import q8lib

ROW, PLANE = q8lib.LAYOUT_ROW, q8lib.LAYOUT_PLANE64


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(q8lib.LIB_PATH):
        from int8_quantized_projections_amd import _build
        _build.build()


def f32(*shape):
    return torch.zeros(*shape, dtype=torch.float32)


def test_activation_rank_and_dtype():
    with pytest.raises(ValueError, match="rows, K"):
        q8lib.q8_quantize(f32(2, 3, 32))
    with pytest.raises(TypeError, match="float32"):
        q8lib.q8_quantize(torch.zeros(2, 32, dtype=torch.float16))
    with pytest.raises(TypeError, match="float32"):
        q8lib.rmsnorm_quant(f32(2, 64), torch.zeros(64, dtype=torch.bfloat16), 1e-6)
    with pytest.raises(ValueError, match="differ"):
        q8lib.swiglu_quant(f32(2, 64), f32(64, 2))


def test_short_or_mistyped_quantized_buffers():
    qs, sd = torch.zeros(128, dtype=torch.int8), torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="qs: 128 elements, at least 192"):
        q8lib.q8_quantize(f32(3, 64), ROW, qs, sd)
    with pytest.raises(ValueError, match="sd: 4 elements, at least 6"):
        q8lib.q8_quantize(f32(3, 64), ROW, torch.zeros(192, dtype=torch.int8), sd)
    # PLANE64 pads the tokens to 64: 3 rows of K=64 take 64 x 64 bytes
    with pytest.raises(ValueError, match="at least 4096"):
        q8lib.q8_quantize(f32(3, 64), PLANE, torch.zeros(192, dtype=torch.int8), torch.zeros(6, dtype=torch.int32))
    with pytest.raises(TypeError, match="int8"):
        q8lib.q8_quantize(f32(3, 64), ROW, torch.zeros(192, dtype=torch.int32), torch.zeros(6, dtype=torch.int32))
    with pytest.raises(TypeError, match="int32"):
        q8lib.q8_quantize(f32(3, 64), ROW, torch.zeros(192, dtype=torch.int8), torch.zeros(6, dtype=torch.int16))
    with pytest.raises(ValueError, match="y: 100 elements"):
        q8lib.rmsnorm_quant(f32(2, 64), f32(64), 1e-6, ROW, f32(100))
    with pytest.raises(ValueError, match="w: 32 elements"):
        q8lib.rmsnorm_quant(f32(2, 64), f32(32), 1e-6)


def _weights(n, k):
    return q8lib.Q8Weights(torch.zeros(n, k, dtype=torch.int8), torch.zeros(n, k // 32, dtype=torch.int16))


def test_gemv_and_gemm_buffers():
    W = _weights(16, 64)
    aq, asd = torch.zeros(64, dtype=torch.int8), torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="y: 15 elements"):
        q8lib.q8_gemv(W, aq, asd, f32(15))
    with pytest.raises(ValueError, match="a_qs: 32 elements"):
        q8lib.q8_gemv(W, aq[:32], asd, f32(16))
    with pytest.raises(ValueError, match="x: 32 elements"):
        q8lib.q8_gemv_f32(W, f32(32), f32(16))
    with pytest.raises(ValueError, match="2 weight matrices and 1 outputs"):
        q8lib.q8_gemv_shared_multi([W, W], aq, asd, [f32(16)])
    with pytest.raises(ValueError, match=r"y\[1\]: 8 elements"):
        q8lib.q8_gemv_shared_multi([W, W], aq, asd, [f32(16), f32(8)])
    # a T=3 plane of K=64 is 64 tokens x 64 bytes; C must hold (T-1)*ldc + N floats
    pq, ps = torch.zeros(4096, dtype=torch.int8), torch.zeros(128, dtype=torch.int32)
    with pytest.raises(ValueError, match="at least 4096"):
        q8lib.q8_gemm(W, pq[:2048], ps, 3, f32(3, 16))
    with pytest.raises(ValueError, match="C: 47 elements, at least 48"):
        q8lib.q8_gemm(W, pq, ps, 3, f32(47))
    with pytest.raises(ValueError, match="C: 40 elements, at least 48"):
        q8lib.q8_gemm(W, pq, ps, 3, f32(40), ldc=16)


def test_weight_descriptors():
    with pytest.raises(ValueError, match="d is"):
        q8lib.Q8Weights(torch.zeros(4, 64, dtype=torch.int8), torch.zeros(4, 3, dtype=torch.int16)).struct()
    with pytest.raises(TypeError, match="int16"):
        q8lib.Q8Weights(torch.zeros(4, 64, dtype=torch.int8), torch.zeros(4, 2, dtype=torch.float16)).struct()
    with pytest.raises(ValueError, match="super-blocks"):
        q8lib.Q4KWeights(torch.zeros(4, 144, dtype=torch.uint8), 512).struct()
    with pytest.raises(ValueError, match="blocks: 100 elements"):
        q8lib.q8_weights_repack(torch.zeros(100, dtype=torch.uint8), 2, 64)
