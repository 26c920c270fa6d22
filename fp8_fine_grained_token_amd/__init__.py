"""fp8blk: fine-grained FP8 (1x128 activation tiles, 128x128 weight blocks)
quantization and block-scaled FP8 GEMM for MI355X (gfx950).

The compute lives in the HIP library built from ``csrc/`` (see ``build.py``);
``binding`` is its Python face.  ``inputs`` is the seeded synthetic input
generator.  Importing this package loads nothing; the library is loaded on
first use and its absence is an error.
"""
from .binding import (  # noqa: F401
    FP8_OUT_BF16, FP8_OUT_F32, Fp8Error, fp8_block_gemm, fp8_block_gemm_pow2,
    fp8_block_grouped_gemm, fp8_block_grouped_gemm_pow2, fp8_gemm_workspace_bytes,
    fp8_quant_act_1x128, fp8_quant_act_1x128_pow2, fp8_quant_weight_128x128,
    fp8_quant_weight_128x128_pow2, lib, status_string, fp8_quant_act_128x1_t,
    fp8_transpose_weight_128x128, fp8_block_gemm_wgrad, fp8_block_gemm_fused_quant,
    fp8_block_gemm_noalloc, fp8_block_gemm_dgrad, fp8_fused_quant_workspace_bytes,
    fp8_fused_quant_kernel_workspace_bytes, fp8_quant_act_128x1_t_pow2,
    fp8_block_gemm_wgrad_pow2, fp8_block_gemm_dgrad_pow2,
)
