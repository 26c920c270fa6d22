"""CPU oracle for fine-grained FP8 quantization and block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path (the HIP library
and its Python binding) never does.  The arithmetic lives in ``oracle.c``
(plain C99, gcc, binary32/binary64, OpenMP across rows); this module builds it
with gcc and marshals numpy arrays through ctypes.

What each entry computes, with the pages it follows, is documented in
``oracle.c``.  Arrays are numpy: bf16 inputs as ``uint16`` bit patterns, E4M3
codes as ``uint8``, scales as ``float32``, GEMM references as ``float64``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "liboracle.so")

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc into oracle/_build/liboracle.so."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = [
            "gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
            "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
            "-o", tmp, _SRC, "-lm",
        ]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.orc_e4m3_value.argtypes = [ctypes.c_int]
        lib.orc_e4m3_value.restype = ctypes.c_double
        lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
        lib.orc_e4m3_encode.restype = ctypes.c_uint8
        lib.orc_e4m3_encode_array.argtypes = [P, I64, P]
        lib.orc_e4m3_encode_array.restype = None
        lib.orc_quant_act_1x128.argtypes = [P, I64, I64, P, P]
        lib.orc_quant_act_1x128.restype = None
        lib.orc_quant_weight_128x128.argtypes = [P, I64, I64, P, P]
        lib.orc_quant_weight_128x128.restype = None
        lib.orc_quant_act_1x128_pow2.argtypes = [P, I64, I64, P, P]
        lib.orc_quant_act_1x128_pow2.restype = None
        lib.orc_quant_weight_128x128_pow2.argtypes = [P, I64, I64, P, P]
        lib.orc_quant_weight_128x128_pow2.restype = None
        lib.orc_block_gemm_rows.argtypes = [P, P, P, P, I64, I64, I64, P, I64, P]
        lib.orc_block_gemm_rows.restype = None
        lib.orc_rowscaled_gemm_rows.argtypes = [P, P, P, P, I64, I64, I64, P, I64, P]
        lib.orc_rowscaled_gemm_rows.restype = None
        lib.orc_quant_act_128x1_t.argtypes = [P, I64, I64, P, P]
        lib.orc_quant_act_128x1_t.restype = None
        lib.orc_quant_act_128x1_t_pow2.argtypes = [P, I64, I64, P, P]
        lib.orc_quant_act_128x1_t_pow2.restype = None
        lib.orc_grouped_gemm_rows.argtypes = [P, P, P, P, P, I64, I64, I64, I64,
                                              P, I64, P, P]
        lib.orc_grouped_gemm_rows.restype = None
        lib.orc_max_threads.argtypes = []
        lib.orc_max_threads.restype = ctypes.c_int
        lib.orc_set_threads.argtypes = [ctypes.c_int]
        lib.orc_set_threads.restype = None
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def max_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().orc_max_threads())


def set_threads(n: int) -> None:
    """Set the OpenMP thread count of the oracle's parallel loops."""
    _load().orc_set_threads(int(n))


def e4m3_value(code: int) -> float:
    """Value of one E4M3FN code (NaN for 0x7F / 0xFF)."""
    return float(_load().orc_e4m3_value(int(code)))


def e4m3_encode(y) -> np.ndarray:
    """Encode float32 value(s) into E4M3FN codes (RNE, saturating, signed 0)."""
    arr = np.ascontiguousarray(np.asarray(y, dtype=np.float32))
    out = np.empty(arr.shape, dtype=np.uint8)
    _load().orc_e4m3_encode_array(_ptr(arr), arr.size, _ptr(out))
    return out


def quant_act_1x128(x_bf16: np.ndarray):
    """1x128 activation quantization of bf16 bits [M][K] -> (q u8 [M][K],
    scales f32 [M][ceil(K/128)])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    G = (K + 127) // 128
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, G), dtype=np.float32)
    _load().orc_quant_act_1x128(_ptr(x), M, K, _ptr(q), _ptr(s))
    return q, s


def quant_weight_128x128(w_bf16: np.ndarray):
    """128x128 block quantization of bf16 bits [N][K] -> (q u8 [N][K],
    scales f32 [ceil(N/128)][ceil(K/128)])."""
    w = _c(w_bf16, np.uint16)
    N, K = w.shape
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty(((N + 127) // 128, (K + 127) // 128), dtype=np.float32)
    _load().orc_quant_weight_128x128(_ptr(w), N, K, _ptr(q), _ptr(s))
    return q, s


def quant_act_1x128_pow2(x_bf16: np.ndarray):
    """As quant_act_1x128 with power-of-two scales (oracle.c, pow2 reading)."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    G = (K + 127) // 128
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, G), dtype=np.float32)
    _load().orc_quant_act_1x128_pow2(_ptr(x), M, K, _ptr(q), _ptr(s))
    return q, s


def quant_weight_128x128_pow2(w_bf16: np.ndarray):
    """As quant_weight_128x128 with power-of-two scales."""
    w = _c(w_bf16, np.uint16)
    N, K = w.shape
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty(((N + 127) // 128, (K + 127) // 128), dtype=np.float32)
    _load().orc_quant_weight_128x128_pow2(_ptr(w), N, K, _ptr(q), _ptr(s))
    return q, s


def block_gemm(qa, sa, qw, sw, rows=None) -> np.ndarray:
    """Binary64 reference of the block-scaled GEMM for the given activation
    rows (all rows when None): returns float64 [len(rows)][N]."""
    qa = _c(qa, np.uint8)
    sa = _c(sa, np.float32)
    qw = _c(qw, np.uint8)
    sw = _c(sw, np.float32)
    M, K = qa.shape
    N = qw.shape[0]
    if rows is None:
        rows = np.arange(M, dtype=np.int64)
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= M):
        raise IndexError("row index out of range")
    R = np.empty((rows.size, N), dtype=np.float64)
    _load().orc_block_gemm_rows(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K,
                                _ptr(rows), rows.size, _ptr(R))
    return R


def quant_act_128x1_t(x_bf16: np.ndarray):
    """128x1 tiles (128 tokens of one channel) of bf16 bits [M][K], written
    transposed: (q_t u8 [K][M], scales_t f32 [K][ceil(M/128)])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    q = np.empty((K, M), dtype=np.uint8)
    s = np.empty((K, (M + 127) // 128), dtype=np.float32)
    _load().orc_quant_act_128x1_t(_ptr(x), M, K, _ptr(q), _ptr(s))
    return q, s


def quant_act_128x1_t_pow2(x_bf16: np.ndarray):
    """As quant_act_128x1_t with power-of-two scales (oracle.c, pow2
    reading)."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    q = np.empty((K, M), dtype=np.uint8)
    s = np.empty((K, (M + 127) // 128), dtype=np.float32)
    _load().orc_quant_act_128x1_t_pow2(_ptr(x), M, K, _ptr(q), _ptr(s))
    return q, s


def transpose_weight(qw: np.ndarray, sw: np.ndarray):
    """Weights quantized in 128x128 blocks, transposed: q [N][K] -> [K][N],
    scales [N/128][K/128] -> [K/128][N/128] (a block's scale is the same
    whichever way the block is read)."""
    return np.ascontiguousarray(_c(qw, np.uint8).T), np.ascontiguousarray(_c(sw, np.float32).T)


def rowscaled_gemm(qa, sa, qb, sb, rows=None) -> np.ndarray:
    """Binary64 reference of the GEMM with one scale row per row of both
    operands: R[r][n] = sum_k (qa[m][k] sa[m][k/128]) (qb[n][k] sb[n][k/128])
    for m = rows[r] (all rows when None)."""
    qa = _c(qa, np.uint8)
    sa = _c(sa, np.float32)
    qb = _c(qb, np.uint8)
    sb = _c(sb, np.float32)
    M, K = qa.shape
    N = qb.shape[0]
    if sb.shape != (N, (K + 127) // 128):
        raise ValueError("sb must be [N][ceil(K/128)]")
    if rows is None:
        rows = np.arange(M, dtype=np.int64)
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= M):
        raise IndexError("row index out of range")
    R = np.empty((rows.size, N), dtype=np.float64)
    _load().orc_rowscaled_gemm_rows(_ptr(qa), _ptr(sa), _ptr(qb), _ptr(sb), M, N, K,
                                    _ptr(rows), rows.size, _ptr(R))
    return R


def grouped_gemm(qa, sa, qw, sw, offsets, rows=None):
    """Binary64 reference of the grouped GEMM.  qw is [E][N][K], sw is
    [E][ceil(N/128)][ceil(K/128)], offsets int32 [E+1].  Returns (R float64
    [len(rows)][N], found bool [len(rows)]); rows outside every expert are
    NaN in R and False in found."""
    qa = _c(qa, np.uint8)
    sa = _c(sa, np.float32)
    qw = _c(qw, np.uint8)
    sw = _c(sw, np.float32)
    off = _c(np.asarray(offsets, dtype=np.int32), np.int32)
    T, K = qa.shape
    E, N, _ = qw.shape
    if off.size != E + 1:
        raise ValueError("offsets must hold E+1 entries")
    if rows is None:
        rows = np.arange(T, dtype=np.int64)
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    R = np.full((rows.size, N), np.nan, dtype=np.float64)
    found = np.zeros(rows.size, dtype=np.int32)
    _load().orc_grouped_gemm_rows(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw),
                                  _ptr(off), E, T, N, K, _ptr(rows), rows.size,
                                  _ptr(R), _ptr(found))
    return R, found.astype(bool)
