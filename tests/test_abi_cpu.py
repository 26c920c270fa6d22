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
        + ["fp8_gemm_workspace_bytes", "fp8_status_string", "fp8_block_gemm_noalloc",
           "fp8_block_gemm_fused_quant", "fp8_fused_quant_workspace_bytes",
           "fp8_fused_quant_kernel_workspace_bytes", "fp8_block_gemm_dgrad",
           "fp8_quant_act_128x1_t_pow2", "fp8_block_gemm_wgrad_pow2",
           "fp8_block_gemm_dgrad_pow2"])


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


@pytest.mark.parametrize("suffix", SUFFIXES)
def test_dgrad_argument_errors(suffix):
    lib = B.lib()

    def dg(dy=A16, sdy=A16, w=A16, sw=A16, dx=A16, dt=B.FP8_OUT_BF16, M=128, N=256, K=512,
           ws=NUL, wsb=0):
        return getattr(lib, "fp8_block_gemm_dgrad" + suffix)(dy, sdy, w, sw, dx, dt, M, N, K,
                                                            ws, wsb, NUL)
    assert dg(N=200) == B.FP8_ERR_SHAPE          # inner dimension
    assert dg(K=500) == B.FP8_ERR_SHAPE          # output columns
    assert dg(M=-1) == B.FP8_ERR_SHAPE
    assert dg(N=0) == B.FP8_ERR_SHAPE
    assert dg(N=1 << 24) == B.FP8_ERR_SHAPE
    assert dg(N=1 << 17, K=1 << 15) == B.FP8_ERR_SHAPE   # W of 2^32 bytes
    assert dg(dt=5) == B.FP8_ERR_DTYPE
    assert dg(w=NUL) == B.FP8_ERR_NULL
    assert dg(w=A8) == B.FP8_ERR_ALIGN
    assert dg(dx=A8) == B.FP8_ERR_ALIGN
    assert dg(ws=A16, wsb=0) == B.FP8_ERR_WORKSPACE
    assert dg(M=0, dy=NUL, dx=NUL) == B.FP8_OK


def test_fused_quant_gemm_argument_errors():
    lib = B.lib()

    def fq(x=A16, w=A16, sw=A16, c=A16, dt=B.FP8_OUT_BF16, M=128, N=256, K=512, q=NUL, s=NUL,
           ws=NUL, wsb=0):
        return lib.fp8_block_gemm_fused_quant(x, w, sw, c, dt, M, N, K, q, s, ws, wsb, NUL)
    assert fq(K=500) == B.FP8_ERR_SHAPE
    assert fq(N=200) == B.FP8_ERR_SHAPE
    assert fq(M=-1) == B.FP8_ERR_SHAPE
    assert fq(K=1 << 24) == B.FP8_ERR_SHAPE
    assert fq(dt=7) == B.FP8_ERR_DTYPE
    assert fq(x=NUL) == B.FP8_ERR_NULL
    assert fq(sw=NUL) == B.FP8_ERR_NULL
    assert fq(q=A16) == B.FP8_ERR_NULL           # bytes out without scales out
    assert fq(s=A16) == B.FP8_ERR_NULL
    assert fq(x=A8) == B.FP8_ERR_ALIGN
    assert fq(c=A8) == B.FP8_ERR_ALIGN
    assert fq(q=ctypes.c_void_p(0x10004), s=A16) == B.FP8_ERR_ALIGN
    assert fq(q=A8, s=ctypes.c_void_p(0x10002)) == B.FP8_ERR_ALIGN
    assert fq(K=0) == B.FP8_ERR_SHAPE
    assert fq(ws=A16, wsb=0) == B.FP8_ERR_WORKSPACE      # pointer without a size
    assert fq(ws=NUL, wsb=256) == B.FP8_ERR_WORKSPACE    # size without a pointer
    assert fq(ws=ctypes.c_void_p(0x10010), wsb=256) == B.FP8_ERR_WORKSPACE  # not 256-aligned
    assert fq(M=0, x=NUL, c=NUL) == B.FP8_OK


def test_fused_quant_kernel_workspace_bytes():
    # the fused kernel's 64 x 256 tiles split K while tiles x splits fit in
    # 256 CUs and every split keeps 4 K blocks; its partials are FP32
    # [S][M][N]
    lib = B.lib()
    ws = lib.fp8_fused_quant_kernel_workspace_bytes
    assert ws(4096, 256, 7168, B.FP8_OUT_BF16) == 4 * 4096 * 256 * 4   # 64 tiles -> 4 splits
    assert ws(4096, 512, 7168, B.FP8_OUT_F32) == 2 * 4096 * 512 * 4    # 128 tiles -> 2 splits
    assert ws(4096, 1024, 7168, B.FP8_OUT_BF16) == 0                   # 256 tiles fill the CUs
    assert ws(64, 256, 512, B.FP8_OUT_BF16) == 0                       # K too short to split
    assert ws(64, 256, 1024, B.FP8_OUT_BF16) == 2 * 64 * 256 * 4
    assert ws(0, 256, 1024, B.FP8_OUT_BF16) == 0
    assert ws(64, 200, 1024, B.FP8_OUT_BF16) == 0
    assert ws(64, 256, 1024, 7) == 0


def r256(n):
    return (n + 255) // 256 * 256


@pytest.mark.parametrize("M,N,K,expect", [
    # the fused kernel is the faster plan: C one 256-column tile wide over at
    # least 2048 tokens; its own split-K partials
    (4096, 256, 7168, 4 * 4096 * 256 * 4),  # 64 tiles: 4 splits of 14
    (2048, 128, 7168, 8 * 2048 * 128 * 4),  # 32 tiles: 8 splits of 7 K blocks
    (16384, 256, 7168, 0),                  # 256 tiles of 64 rows fill the CUs
    # elsewhere the staged plan: E4M3 activations, their scales, then the
    # block GEMM's split-K partials, each part rounded up to 256 bytes
    (4096, 512, 7168, 4096 * 7168 + 4096 * 56 * 4),
    (4096, 7168, 7168, 4096 * 7168 + 4096 * 56 * 4),
    (2047, 256, 7168, 2047 * 7168 + r256(2047 * 56 * 4) + 4 * 2047 * 256 * 4),
    (64, 256, 1024, 64 * 1024 + 64 * 8 * 4 + 2 * 64 * 256 * 4),
    (64, 256, 512, 64 * 512 + 64 * 4 * 4),
    (1, 128, 128, 256 + 256),
])
def test_fused_quant_workspace_bytes(M, N, K, expect):
    lib = B.lib()
    assert lib.fp8_fused_quant_workspace_bytes(M, N, K, B.FP8_OUT_BF16) == expect
    assert lib.fp8_fused_quant_workspace_bytes(M, N, K, B.FP8_OUT_F32) == expect


def test_fused_quant_workspace_bytes_invalid():
    ws = B.lib().fp8_fused_quant_workspace_bytes
    assert ws(0, 256, 1024, B.FP8_OUT_BF16) == 0
    assert ws(64, 200, 1024, B.FP8_OUT_BF16) == 0
    assert ws(64, 256, 1000, B.FP8_OUT_BF16) == 0
    assert ws(64, 256, 1024, 7) == 0


def test_noalloc_gemm_argument_errors():
    lib = B.lib()

    def na(a=A16, sa=A16, w=A16, sw=A16, c=A16, dt=B.FP8_OUT_BF16, M=128, N=256, K=512):
        return lib.fp8_block_gemm_noalloc(a, sa, w, sw, c, dt, M, N, K, NUL)
    assert na(K=500) == B.FP8_ERR_SHAPE
    assert na(N=200) == B.FP8_ERR_SHAPE
    assert na(M=-1) == B.FP8_ERR_SHAPE
    assert na(dt=7) == B.FP8_ERR_DTYPE
    assert na(a=NUL) == B.FP8_ERR_NULL
    assert na(c=A8) == B.FP8_ERR_ALIGN
    assert na(K=0) == B.FP8_ERR_SHAPE
    assert na(M=0, a=NUL, sa=NUL, c=NUL) == B.FP8_OK
    # every split-K plan fits the static scratch array: the largest
    # workspace any shape asks for is 256 workgroups of 128 x 64 FP32
    worst = max(lib.fp8_gemm_workspace_bytes(m, n, k, B.FP8_OUT_F32)
                for m in (1, 64, 128, 200, 256, 512, 1024)
                for n in (128, 256, 1024, 2048, 4096, 8192)
                for k in (512, 2048, 7168, 65536))
    assert 0 < worst <= 8 << 20


@pytest.mark.parametrize("suffix", SUFFIXES)
def test_backward_argument_errors(suffix):
    lib = B.lib()
    q = getattr(lib, "fp8_quant_act_128x1_t" + suffix)
    assert q(NUL, 4, 128, A16, A16, NUL) == B.FP8_ERR_NULL
    assert q(A16, -1, 128, A16, A16, NUL) == B.FP8_ERR_SHAPE
    assert q(NUL, 0, 128, NUL, NUL, NUL) == B.FP8_OK
    assert q(ctypes.c_void_p(0x10001), 4, 128, A16, A16, NUL) == B.FP8_ERR_ALIGN
    t = lib.fp8_transpose_weight_128x128
    assert t(NUL, A16, 128, 128, A16, A16, NUL) == B.FP8_ERR_NULL
    assert t(A16, A16, -1, 128, A16, A16, NUL) == B.FP8_ERR_SHAPE
    assert t(NUL, NUL, 0, 128, NUL, NUL, NUL) == B.FP8_OK
    assert t(A16, ctypes.c_void_p(0x10002), 128, 128, A16, A16, NUL) == B.FP8_ERR_ALIGN
    w = getattr(lib, "fp8_block_gemm_wgrad" + suffix)

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


def test_grid_limits_are_refused_as_shape_errors():
    """Shapes whose launch would pass 2^32 work-items are refused with
    FP8_ERR_SHAPE before anything is enqueued; the largest shapes that fit
    pass validation (checked with a NULL output, so nothing launches)."""
    lib = B.lib()
    act, wq = lib.fp8_quant_act_1x128, lib.fp8_quant_weight_128x128
    # 1x128: at most 16 threads per group, so M * ceil(K/128) < 2^28 groups
    assert act(A16, 1 << 20, 1 << 15, A16, A16, NUL) == B.FP8_ERR_SHAPE     # 2^28 groups
    assert act(A16, (1 << 20) - 1, 1 << 15, NUL, A16, NUL) == B.FP8_ERR_NULL
    assert act(A16, (1 << 31) - 1, 1, A16, A16, NUL) == B.FP8_ERR_SHAPE     # tiny K, many rows
    # 128x128: 256 threads per block, so ceil(N/128) ceil(K/128) < 2^24 blocks
    assert wq(A16, 1 << 19, 1 << 19, A16, A16, NUL) == B.FP8_ERR_SHAPE
    assert lib.fp8_transpose_weight_128x128(A16, A16, 1 << 19, 1 << 19, A16, A16,
                                            NUL) == B.FP8_ERR_SHAPE
    # GEMMs: fewer than 2^22 output tiles of 128 x 128 (with one extra row)
    assert gemm(lib, M=(1 << 22) * 128, N=128, K=128) == B.FP8_ERR_SHAPE
    assert gemm(lib, M=1 << 20, N=1 << 16, K=128) == B.FP8_ERR_SHAPE
    assert gemm(lib, M=(1 << 20) - 256, N=1 << 16, K=128, c=NUL) == B.FP8_ERR_NULL
    assert grouped(lib, E=1 << 14, T=128, N=1 << 15) == B.FP8_ERR_SHAPE


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


@pytest.mark.parametrize("M,N,K,splits", [
    # 128 x 64 output tiles; the split count doubles while tiles x splits
    # stay within 256 CUs and every split keeps at least 4 K blocks, then K
    # blocks are dealt evenly (ceil) and empty splits dropped
    (256, 2048, 7168, 4),     # 64 tiles, 56 K blocks -> 4 x 14
    (256, 256, 32768, 32),    # 8 tiles, 256 K blocks -> 32 x 8
    (300, 384, 1280, 2),      # 18 tiles (ragged M), 10 K blocks: 4 would leave 2 each
    (128, 128, 896, 1),       # 7 K blocks cannot give two splits of 4
    (128, 128, 1152, 2),      # 9 K blocks -> 5 + 4
    (128, 128, 2048, 4),      # 16 K blocks -> 4 x 4
    (128, 128, 4224, 7),      # 33 K blocks: 8 splits of ceil(33/8) = 5 need only 7
    (100, 128, 4224, 7),
    (1024, 1024, 1024, 2),    # 128 tiles: doubling reaches exactly 256
    (1032, 1024, 1024, 1),    # 144 tiles
    (4096, 3840, 7168, 1),    # 240 256x256 tiles: too few for the big plan, too many to split
    (4096, 4096, 7168, 1),    # 256 256x256 tiles: the big plan
])
def test_workspace_split_counts(M, N, K, splits):
    ws = B.lib().fp8_gemm_workspace_bytes(M, N, K, B.FP8_OUT_BF16)
    assert ws == (splits * M * N * 4 if splits > 1 else 0)


def test_workspace_fits_noalloc_scratch():
    # every split plan's FP32 partials fit the no-allocation entry point's
    # fixed array, whose size the header states as 8 MiB
    lib = B.lib()
    worst = 0
    for M in (1, 64, 127, 128, 129, 256, 300, 512, 1000, 1024, 2048, 4000):
        for N in (128, 256, 384, 1024, 2048, 4096, 7168):
            for K in (128, 512, 1024, 4224, 7168, 65536):
                worst = max(worst, lib.fp8_gemm_workspace_bytes(M, N, K, B.FP8_OUT_F32))
    assert 0 < worst <= 8 << 20


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        B.fp8_quant_act_1x128(x, q=torch.zeros((4, 128), dtype=torch.uint8),
                              scales=torch.zeros((4, 1)))
