"""The Python binding refuses tensors whose shape does not match what the
kernels will index, before anything is launched (CPU: no GPU needed, the
checks run before the device check).  A tensor of the right shape on the CPU
is refused for its device instead."""
import pytest
import torch

from fp8_fine_grained_token_amd import binding as B


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def test_quant_act_outputs():
    x = bf16(4, 256)
    with pytest.raises(ValueError, match="q must have shape"):
        B.fp8_quant_act_1x128(x, q=u8(4, 128), scales=f32(4, 2))
    with pytest.raises(ValueError, match="scales must have shape"):
        B.fp8_quant_act_1x128(x, q=u8(4, 256), scales=f32(4, 1))
    with pytest.raises(ValueError, match="must be 2-dimensional"):
        B.fp8_quant_act_1x128(bf16(1024))
    with pytest.raises(ValueError, match="on the GPU"):
        B.fp8_quant_act_1x128_pow2(x, q=u8(4, 256), scales=f32(4, 2))


def test_quant_weight_outputs():
    w = bf16(200, 130)
    with pytest.raises(ValueError, match="scales must have shape"):
        B.fp8_quant_weight_128x128(w, q=u8(200, 130), scales=f32(1, 2))
    with pytest.raises(ValueError, match="q must have shape"):
        B.fp8_quant_weight_128x128_pow2(w, q=u8(130, 200), scales=f32(2, 2))


def test_block_gemm_operands_and_output():
    a, sa = u8(64, 256), f32(64, 2)
    w, sw = u8(384, 256), f32(3, 2)
    with pytest.raises(ValueError, match="w must have shape"):
        B.fp8_block_gemm(a, sa, u8(384, 384), f32(3, 3))          # K differs
    with pytest.raises(ValueError, match="sa must have shape"):
        B.fp8_block_gemm(a, f32(64, 1), w, sw)
    with pytest.raises(ValueError, match="sw must have shape"):
        B.fp8_block_gemm(a, sa, w, f32(2, 2))
    with pytest.raises(ValueError, match="c must have shape"):
        B.fp8_block_gemm(a, sa, w, sw, out_dtype="f32", c=f32(64, 256))
    with pytest.raises(ValueError, match="on the GPU"):
        B.fp8_block_gemm_pow2(a, sa, w, sw, out_dtype="bf16", c=bf16(64, 384))


def test_grouped_gemm_operands_and_output():
    a, sa = u8(70, 256), f32(70, 2)
    w, sw = u8(4, 128, 256), f32(4, 1, 2)
    off = torch.zeros(5, dtype=torch.int32)
    with pytest.raises(ValueError, match="group_offsets must have shape"):
        B.fp8_block_grouped_gemm(a, sa, w, sw, torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="sw must have shape"):
        B.fp8_block_grouped_gemm(a, sa, w, f32(4, 2, 2), off)
    with pytest.raises(ValueError, match="c must have shape"):
        B.fp8_block_grouped_gemm_pow2(a, sa, w, sw, off, c=bf16(70, 256))
    with pytest.raises(ValueError, match="must be 3-dimensional"):
        B.fp8_block_grouped_gemm(a, sa, u8(512, 256), sw, off)


def test_backward_entry_points():
    x = bf16(300, 200)
    with pytest.raises(ValueError, match="q_t must have shape"):
        B.fp8_quant_act_128x1_t(x, q_t=u8(300, 200), scales_t=f32(200, 3))
    with pytest.raises(ValueError, match="scales_t must have shape"):
        B.fp8_quant_act_128x1_t(x, q_t=u8(200, 300), scales_t=f32(200, 2))
    q, s = u8(256, 384), f32(2, 3)
    with pytest.raises(ValueError, match="scales must have shape"):
        B.fp8_transpose_weight_128x128(q, f32(3, 2))
    with pytest.raises(ValueError, match="q_t must have shape"):
        B.fp8_transpose_weight_128x128(q, s, q_t=u8(256, 384))
    dy, x_t = u8(128, 256), u8(64, 256)
    with pytest.raises(ValueError, match="x_t must have shape"):
        B.fp8_block_gemm_wgrad(dy, f32(128, 2), u8(64, 128), f32(64, 1))
    with pytest.raises(ValueError, match="dy_t_scales must have shape"):
        B.fp8_block_gemm_wgrad(dy, f32(128, 1), x_t, f32(64, 2))
    with pytest.raises(ValueError, match="dw must have shape"):
        B.fp8_block_gemm_wgrad(dy, f32(128, 2), x_t, f32(64, 2), dw=f32(64, 128))
