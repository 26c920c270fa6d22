"""C-ABI contract checks that need no GPU (CPU only).

The library must load and export every function include/fp8blk.h declares,
and reject bad arguments with the documented status before any launch (every
call here fails validation or is a documented no-op, so nothing reaches the
HIP runtime).
"""
import ctypes
import os
import re

import pytest

from fp8_fine_grained_token_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8blk.h")

# Fake device addresses: only ever passed where validation rejects the call.
A16 = ctypes.c_void_p(0x10000)
A8 = ctypes.c_void_p(0x10008)
NUL = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    method = ["fp8_quant_act_1x128", "fp8_quant_weight_128x128", "fp8_block_gemm",
              "fp8_block_grouped_gemm"]
    assert declared_functions() == sorted(
        method + [m + "_pow2" for m in method]
        + ["fp8_quant_act_128x1_t", "fp8_transpose_weight_128x128", "fp8_block_gemm_wgrad"]
        + ["fp8_gemm_workspace_bytes", "fp8_status_string"])


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(B._SIGNATURES) == set(declared_functions())


def test_status_strings():
    for code in range(7):
        s = B.status_string(code)
        assert s.startswith(["FP8_OK", "FP8_ERR_NULL", "FP8_ERR_SHAPE", "FP8_ERR_ALIGN",
                             "FP8_ERR_DTYPE", "FP8_ERR_WORKSPACE", "FP8_ERR_HIP"][code])
    assert B.status_string(99) == "unknown fp8_status"


SUFFIXES = ["", "_pow2"]


def gemm(lib, a=A16, sa=A16, w=A16, sw=A16, c=A16, dt=B.FP8_OUT_BF16, M=128, N=256, K=512,
         ws=NUL, wsb=0, suffix=""):
    fn = getattr(lib, "fp8_block_gemm" + suffix)
    return fn(a, sa, w, sw, c, dt, M, N, K, ws, wsb, NUL)


def grouped(lib, a=A16, sa=A16, w=A16, sw=A16, off=A16, E=4, T=128, c=A16,
            dt=B.FP8_OUT_BF16, N=256, K=512, ws=NUL, wsb=0, suffix=""):
    fn = getattr(lib, "fp8_block_grouped_gemm" + suffix)
    return fn(a, sa, w, sw, off, E, T, c, dt, N, K, ws, wsb, NUL)


@pytest.mark.parametrize("suffix", SUFFIXES)
def test_quantizer_argument_errors(suffix):
    lib = B.lib()
    for fn in (getattr(lib, "fp8_quant_act_1x128" + suffix),
               getattr(lib, "fp8_quant_weight_128x128" + suffix)):
        assert fn(NUL, 4, 128, NUL, NUL, NUL) == B.FP8_ERR_NULL
        assert fn(A16, 4, 128, NUL, A16, NUL) == B.FP8_ERR_NULL
        assert fn(A16, -1, 128, A16, A16, NUL) == B.FP8_ERR_SHAPE
        assert fn(A16, 4, -128, A16, A16, NUL) == B.FP8_ERR_SHAPE
        assert fn(A16, 1 << 31, 128, A16, A16, NUL) == B.FP8_ERR_SHAPE
        assert fn(A16, 1 << 21, 1 << 20, A16, A16, NUL) == B.FP8_ERR_SHAPE
        # empty problems are no-ops, even with NULL pointers
        assert fn(NUL, 0, 128, NUL, NUL, NUL) == B.FP8_OK
        assert fn(NUL, 5, 0, NUL, NUL, NUL) == B.FP8_OK
        # misaligned bf16 / scale pointers
        assert fn(ctypes.c_void_p(0x10001), 4, 128, A16, A16, NUL) == B.FP8_ERR_ALIGN
        assert fn(A16, 4, 128, A16, ctypes.c_void_p(0x10002), NUL) == B.FP8_ERR_ALIGN


@pytest.mark.parametrize("suffix", SUFFIXES)
def test_gemm_argument_errors(suffix):
    lib = B.lib()

    def gemm_(*a, **k):
        return gemm(*a, suffix=suffix, **k)
    assert gemm_(lib, K=500) == B.FP8_ERR_SHAPE
    assert gemm_(lib, N=200) == B.FP8_ERR_SHAPE
    assert gemm_(lib, M=-1) == B.FP8_ERR_SHAPE
    assert gemm_(lib, dt=7) == B.FP8_ERR_DTYPE
    assert gemm_(lib, a=NUL) == B.FP8_ERR_NULL
    assert gemm_(lib, sw=NUL) == B.FP8_ERR_NULL
    assert gemm_(lib, c=NUL) == B.FP8_ERR_NULL
    assert gemm_(lib, a=A8) == B.FP8_ERR_ALIGN
    assert gemm_(lib, w=A8) == B.FP8_ERR_ALIGN
    assert gemm_(lib, c=A8) == B.FP8_ERR_ALIGN
    assert gemm_(lib, sa=ctypes.c_void_p(0x10002)) == B.FP8_ERR_ALIGN
    assert gemm_(lib, ws=A16, wsb=0) == B.FP8_ERR_WORKSPACE
    assert gemm_(lib, ws=NUL, wsb=1024) == B.FP8_ERR_WORKSPACE
    assert gemm_(lib, ws=ctypes.c_void_p(0x10010), wsb=1024) == B.FP8_ERR_WORKSPACE
    assert gemm_(lib, K=0) == B.FP8_ERR_SHAPE
    # inner dimension at or beyond the 32-bit tile addressing (256 K < 2^32);
    # the largest valid K passes validation (M = 0: a no-op, nothing launches)
    assert gemm_(lib, K=1 << 24) == B.FP8_ERR_SHAPE
    assert gemm_(lib, K=(1 << 24) - 128, M=0) == B.FP8_OK
    # M = 0 is a no-op
    assert gemm_(lib, a=NUL, sa=NUL, c=NUL, M=0) == B.FP8_OK
    # dtype is checked before the empty-problem shortcut
    assert gemm_(lib, M=0, dt=3) == B.FP8_ERR_DTYPE


@pytest.mark.parametrize("suffix", SUFFIXES)
def test_grouped_argument_errors(suffix):
    lib = B.lib()

    def grouped_(*a, **k):
        return grouped(*a, suffix=suffix, **k)
    assert grouped_(lib, off=NUL) == B.FP8_ERR_NULL
    assert grouped_(lib, E=0) == B.FP8_ERR_SHAPE
    assert grouped_(lib, E=-2) == B.FP8_ERR_SHAPE
    assert grouped_(lib, K=384 + 1) == B.FP8_ERR_SHAPE
    assert grouped_(lib, N=100) == B.FP8_ERR_SHAPE
    assert grouped_(lib, dt=2) == B.FP8_ERR_DTYPE
    assert grouped_(lib, off=ctypes.c_void_p(0x10002)) == B.FP8_ERR_ALIGN
    assert grouped_(lib, c=A8) == B.FP8_ERR_ALIGN
    assert grouped_(lib, ws=A16, wsb=0) == B.FP8_ERR_WORKSPACE
    # T = 0 is a no-op (E = 0 allowed then)
    assert grouped_(lib, T=0, E=0, a=NUL, sa=NUL, off=NUL, c=NUL) == B.FP8_OK


def test_backward_argument_errors():
    lib = B.lib()
    q = lib.fp8_quant_act_128x1_t
    assert q(NUL, 4, 128, A16, A16, NUL) == B.FP8_ERR_NULL
    assert q(A16, -1, 128, A16, A16, NUL) == B.FP8_ERR_SHAPE
    assert q(NUL, 0, 128, NUL, NUL, NUL) == B.FP8_OK
    assert q(ctypes.c_void_p(0x10001), 4, 128, A16, A16, NUL) == B.FP8_ERR_ALIGN
    t = lib.fp8_transpose_weight_128x128
    assert t(NUL, A16, 128, 128, A16, A16, NUL) == B.FP8_ERR_NULL
    assert t(A16, A16, -1, 128, A16, A16, NUL) == B.FP8_ERR_SHAPE
    assert t(NUL, NUL, 0, 128, NUL, NUL, NUL) == B.FP8_OK
    assert t(A16, ctypes.c_void_p(0x10002), 128, 128, A16, A16, NUL) == B.FP8_ERR_ALIGN
    w = lib.fp8_block_gemm_wgrad

    def wg(a=A16, sa=A16, b=A16, sb=A16, c=A16, dt=B.FP8_OUT_F32, N=256, K=256, T=512):
        return w(a, sa, b, sb, c, dt, N, K, T, NUL)
    assert wg(T=500) == B.FP8_ERR_SHAPE          # the token axis must be whole 128-blocks
    assert wg(K=200) == B.FP8_ERR_SHAPE
    assert wg(T=0) == B.FP8_ERR_SHAPE
    assert wg(T=1 << 24) == B.FP8_ERR_SHAPE
    assert wg(dt=9) == B.FP8_ERR_DTYPE
    assert wg(a=NUL) == B.FP8_ERR_NULL
    assert wg(c=A8) == B.FP8_ERR_ALIGN
    assert wg(N=0, a=NUL, sa=NUL, c=NUL) == B.FP8_OK


def test_workspace_query():
    lib = B.lib()
    # decode-shaped GEMMs have few output tiles and split K
    ws = lib.fp8_gemm_workspace_bytes(256, 2048, 7168, B.FP8_OUT_BF16)
    assert ws > 0 and ws % (256 * 2048 * 4) == 0
    # prefill-shaped GEMMs fill the GPU without it
    assert lib.fp8_gemm_workspace_bytes(4096, 7168, 7168, B.FP8_OUT_BF16) == 0
    assert lib.fp8_gemm_workspace_bytes(256, 2048, 7000, B.FP8_OUT_BF16) == 0
    assert lib.fp8_gemm_workspace_bytes(256, 2048, 7168, 5) == 0
    assert lib.fp8_gemm_workspace_bytes(0, 2048, 7168, B.FP8_OUT_F32) == 0


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        B.fp8_quant_act_1x128(x, q=torch.zeros((4, 128), dtype=torch.uint8),
                              scales=torch.zeros((4, 1)))
