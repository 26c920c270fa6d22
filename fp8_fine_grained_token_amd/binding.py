"""Python binding of the fp8blk C ABI (include/fp8blk.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``_build/libfp8blk.so``.  PyTorch supplies device memory and the
current HIP stream.  If the library is missing, loading raises at once; there
is no fallback of any kind.

Two layers:
  * ``lib()`` returns the ctypes handle with typed signatures of the C
    functions (raw device pointers, sizes, stream handle);
  * ``fp8_quant_act_1x128``, ``fp8_quant_weight_128x128``,
    ``fp8_block_gemm`` and ``fp8_block_grouped_gemm`` (and their ``_pow2``
    forms, power-of-two scales for the block-scaled matrix core), and the
    backward-pass pieces ``fp8_quant_act_128x1_t``,
    ``fp8_transpose_weight_128x128`` and ``fp8_block_gemm_wgrad``, take torch
    tensors on the GPU, allocate outputs when not given, call the C function
    on ``torch.cuda.current_stream()`` and raise ``Fp8Error`` on a nonzero
    status.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
# FP8BLK_LIB may name another build of the same library (the race-check
# build _build/libfp8blk_poison.so); by default the released one loads.
LIB_PATH = os.environ.get("FP8BLK_LIB") or os.path.join(HERE, "_build", "libfp8blk.so")

FP8_OK = 0
FP8_ERR_NULL = 1
FP8_ERR_SHAPE = 2
FP8_ERR_ALIGN = 3
FP8_ERR_DTYPE = 4
FP8_ERR_WORKSPACE = 5
FP8_ERR_HIP = 6
FP8_OUT_F32 = 0
FP8_OUT_BF16 = 1

# Every symbol the header declares, with (argtypes, restype).
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIGNATURES = {
    "fp8_quant_act_1x128": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "fp8_quant_weight_128x128": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "fp8_block_gemm": ([_P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P,
                        ctypes.c_size_t, _P], ctypes.c_int),
    "fp8_block_grouped_gemm": ([_P, _P, _P, _P, _P, _I64, _I64, _P, ctypes.c_int,
                                _I64, _I64, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "fp8_gemm_workspace_bytes": ([_I64, _I64, _I64, ctypes.c_int], ctypes.c_size_t),
    "fp8_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "fp8_quant_act_128x1_t": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "fp8_quant_act_128x1_t_pow2": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "fp8_transpose_weight_128x128": ([_P, _P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "fp8_block_gemm_wgrad": ([_P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P],
                             ctypes.c_int),
    "fp8_block_gemm_wgrad_pow2": ([_P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P],
                                  ctypes.c_int),
    "fp8_block_gemm_dgrad": ([_P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P,
                              ctypes.c_size_t, _P], ctypes.c_int),
    "fp8_block_gemm_dgrad_pow2": ([_P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P,
                                   ctypes.c_size_t, _P], ctypes.c_int),
    "fp8_block_gemm_fused_quant": ([_P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P, _P,
                                    _P, ctypes.c_size_t, _P], ctypes.c_int),
    "fp8_fused_quant_workspace_bytes": ([_I64, _I64, _I64, ctypes.c_int], ctypes.c_size_t),
    "fp8_fused_quant_kernel_workspace_bytes": ([_I64, _I64, _I64, ctypes.c_int],
                                               ctypes.c_size_t),
    "fp8_block_gemm_noalloc": ([_P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P],
                               ctypes.c_int),
    "fp8_quant_act_1x128_pow2": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "fp8_quant_weight_128x128_pow2": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "fp8_block_gemm_pow2": ([_P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P,
                        ctypes.c_size_t, _P], ctypes.c_int),
    "fp8_block_grouped_gemm_pow2": ([_P, _P, _P, _P, _P, _I64, _I64, _P, ctypes.c_int,
                                _I64, _I64, _P, ctypes.c_size_t, _P], ctypes.c_int),
}

_lock = threading.Lock()
_lib = None


class Fp8Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().fp8_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")


def lib():
    """Load libfp8blk.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"fp8blk HIP library not found at {LIB_PATH}; build it with "
                    "`python -m fp8_fine_grained_token_amd.build`")
            h = ctypes.CDLL(LIB_PATH)
            for name, (args, res) in _SIGNATURES.items():
                fn = getattr(h, name)
                fn.argtypes = args
                fn.restype = res
            _lib = h
        return _lib


def status_string(status: int) -> str:
    return lib().fp8_status_string(status).decode()


def _check(status: int, where: str):
    if status != FP8_OK:
        raise Fp8Error(status, where)


# ---- torch-tensor layer -----------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_handle(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _shape(t, name, shape):
    """The kernels index every buffer by the sizes they are given, so a
    tensor of another shape would be read or written out of bounds: refuse
    it here, before anything is launched."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _rank(t, name, n):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != n:
        raise ValueError(f"{name} must be {n}-dimensional, got shape {tuple(t.shape)}")


def _out_code(out_dtype):
    torch = _torch()
    if out_dtype in (torch.float32, "f32", FP8_OUT_F32):
        return FP8_OUT_F32, torch.float32
    if out_dtype in (torch.bfloat16, "bf16", FP8_OUT_BF16):
        return FP8_OUT_BF16, torch.bfloat16
    raise ValueError(f"unsupported out_dtype {out_dtype}")


def _quant_act(fn, x, q, scales, stream):
    torch = _torch()
    _rank(x, "x", 2)
    M, K = x.shape
    G = (K + 127) // 128
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, G), dtype=torch.float32, device=x.device)
    _shape(q, "q", (M, K))
    _shape(scales, "scales", (M, G))
    _check(getattr(lib(), fn)(_dev(x, "x", torch.bfloat16), M, K, _dev(q, "q", torch.uint8),
                              _dev(scales, "scales", torch.float32), _stream_handle(stream)), fn)
    return q, scales


def fp8_quant_act_1x128(x, q=None, scales=None, stream=None):
    """x: bf16 [M][K] -> (q uint8 [M][K] E4M3, scales fp32 [M][ceil(K/128)])."""
    return _quant_act("fp8_quant_act_1x128", x, q, scales, stream)


def fp8_quant_act_1x128_pow2(x, q=None, scales=None, stream=None):
    """As fp8_quant_act_1x128 with power-of-two scales."""
    return _quant_act("fp8_quant_act_1x128_pow2", x, q, scales, stream)


def _quant_weight(fn, w, q, scales, stream):
    torch = _torch()
    _rank(w, "w", 2)
    N, K = w.shape
    if q is None:
        q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(((N + 127) // 128, (K + 127) // 128), dtype=torch.float32,
                             device=w.device)
    _shape(q, "q", (N, K))
    _shape(scales, "scales", ((N + 127) // 128, (K + 127) // 128))
    _check(getattr(lib(), fn)(_dev(w, "w", torch.bfloat16), N, K, _dev(q, "q", torch.uint8),
                              _dev(scales, "scales", torch.float32), _stream_handle(stream)), fn)
    return q, scales


def fp8_quant_weight_128x128(w, q=None, scales=None, stream=None):
    """w: bf16 [N][K] -> (q uint8 [N][K], scales fp32 [ceil(N/128)][ceil(K/128)])."""
    return _quant_weight("fp8_quant_weight_128x128", w, q, scales, stream)


def fp8_quant_weight_128x128_pow2(w, q=None, scales=None, stream=None):
    """As fp8_quant_weight_128x128 with power-of-two scales."""
    return _quant_weight("fp8_quant_weight_128x128_pow2", w, q, scales, stream)


def fp8_gemm_workspace_bytes(M: int, N: int, K: int, out_dtype="bf16") -> int:
    code, _ = _out_code(out_dtype)
    return int(lib().fp8_gemm_workspace_bytes(M, N, K, code))


def fp8_fused_quant_workspace_bytes(M: int, N: int, K: int, out_dtype="bf16") -> int:
    code, _ = _out_code(out_dtype)
    return int(lib().fp8_fused_quant_workspace_bytes(M, N, K, code))


def fp8_fused_quant_kernel_workspace_bytes(M: int, N: int, K: int, out_dtype="bf16") -> int:
    code, _ = _out_code(out_dtype)
    return int(lib().fp8_fused_quant_kernel_workspace_bytes(M, N, K, code))


def _workspace_args(workspace):
    if workspace is None:
        return ctypes.c_void_p(0), 0
    torch = _torch()
    return _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()


def _block_gemm(fn, a, sa, w, sw, out_dtype, c, workspace, stream):
    torch = _torch()
    _rank(a, "a", 2)
    _rank(w, "w", 2)
    M, K = a.shape
    N = w.shape[0]
    code, tdt = _out_code(out_dtype)
    if c is None:
        c = torch.empty((M, N), dtype=tdt, device=a.device)
    _shape(w, "w", (N, K))
    # K and N must be multiples of 128 (the library returns FP8_ERR_SHAPE
    # otherwise); the scale shapes are checked for those that are
    if K % 128 == 0 and N % 128 == 0:
        _shape(sa, "sa", (M, K // 128))
        _shape(sw, "sw", (N // 128, K // 128))
    _shape(c, "c", (M, N))
    wp, wb = _workspace_args(workspace)
    _check(getattr(lib(), fn)(_dev(a, "a", torch.uint8), _dev(sa, "sa", torch.float32),
                              _dev(w, "w", torch.uint8), _dev(sw, "sw", torch.float32),
                              _dev(c, "c", tdt), code, M, N, K, wp, wb, _stream_handle(stream)),
           fn)
    return c


def fp8_block_gemm(a, sa, w, sw, out_dtype="bf16", c=None, workspace=None, stream=None):
    """C[M][N] = block-scaled product of a [M][K] E4M3 (scales [M][K/128]) and
    w [N][K] E4M3 (scales [N/128][K/128]); bf16 or fp32 output."""
    return _block_gemm("fp8_block_gemm", a, sa, w, sw, out_dtype, c, workspace, stream)


def fp8_block_gemm_dgrad(dy, sdy, w, sw, out_dtype="bf16", dx=None, workspace=None,
                         stream=None):
    """dX [M][K] = dY [M][N] W [N][K]: dy E4M3 [M][N] with scales [M][N/128]
    (1x128 along N), w the forward weights E4M3 [N][K] with 128x128 block
    scales [N/128][K/128], read transposed inside the GEMM."""
    return _dgrad("fp8_block_gemm_dgrad", dy, sdy, w, sw, out_dtype, dx, workspace, stream)


def fp8_block_gemm_dgrad_pow2(dy, sdy, w, sw, out_dtype="bf16", dx=None, workspace=None,
                              stream=None):
    """As fp8_block_gemm_dgrad, for power-of-two scales."""
    return _dgrad("fp8_block_gemm_dgrad_pow2", dy, sdy, w, sw, out_dtype, dx, workspace,
                  stream)


def _dgrad(fn, dy, sdy, w, sw, out_dtype, dx, workspace, stream):
    torch = _torch()
    _rank(dy, "dy", 2)
    _rank(w, "w", 2)
    M, N = dy.shape
    K = w.shape[1]
    code, tdt = _out_code(out_dtype)
    if dx is None:
        dx = torch.empty((M, K), dtype=tdt, device=dy.device)
    _shape(w, "w", (N, K))
    if K % 128 == 0 and N % 128 == 0:
        _shape(sdy, "sdy", (M, N // 128))
        _shape(sw, "sw", (N // 128, K // 128))
    _shape(dx, "dx", (M, K))
    wp, wb = _workspace_args(workspace)
    _check(getattr(lib(), fn)(_dev(dy, "dy", torch.uint8), _dev(sdy, "sdy", torch.float32),
                              _dev(w, "w", torch.uint8), _dev(sw, "sw", torch.float32),
                              _dev(dx, "dx", tdt), code, M, N, K, wp, wb, _stream_handle(stream)),
           fn)
    return dx


def fp8_block_gemm_fused_quant(x, w, sw, out_dtype="bf16", c=None, q_out=None, sa_out=None,
                               return_quantized=False, workspace=None, stream=None):
    """C[M][N] = fp8_block_gemm(fp8_quant_act_1x128(x), w, sw) with the 1x128
    quantization of the bf16 activations x [M][K] done inside the GEMM.
    With return_quantized (or q_out / sa_out given) the E4M3 bytes [M][K]
    and scales [M][K/128] are written too and (c, q, sa) is returned.  With a
    workspace of fp8_fused_quant_workspace_bytes(M, N, K) bytes the library
    takes the faster plan for the shape (for wide outputs or few tokens: the
    quantizer, then the block GEMM); with one of
    fp8_fused_quant_kernel_workspace_bytes(M, N, K) bytes the fused kernel
    splits K."""
    torch = _torch()
    _rank(x, "x", 2)
    _rank(w, "w", 2)
    M, K = x.shape
    N = w.shape[0]
    code, tdt = _out_code(out_dtype)
    if c is None:
        c = torch.empty((M, N), dtype=tdt, device=x.device)
    _shape(w, "w", (N, K))
    if K % 128 == 0 and N % 128 == 0:
        _shape(sw, "sw", (N // 128, K // 128))
    _shape(c, "c", (M, N))
    want_q = return_quantized or q_out is not None or sa_out is not None
    if want_q:
        if q_out is None:
            q_out = torch.empty((M, K), dtype=torch.uint8, device=x.device)
        if sa_out is None:
            sa_out = torch.empty((M, (K + 127) // 128), dtype=torch.float32, device=x.device)
        _shape(q_out, "q_out", (M, K))
        _shape(sa_out, "sa_out", (M, (K + 127) // 128))
        qp, sp = _dev(q_out, "q_out", torch.uint8), _dev(sa_out, "sa_out", torch.float32)
    else:
        qp, sp = ctypes.c_void_p(0), ctypes.c_void_p(0)
    wp, wb = _workspace_args(workspace)
    fn = "fp8_block_gemm_fused_quant"
    _check(getattr(lib(), fn)(_dev(x, "x", torch.bfloat16), _dev(w, "w", torch.uint8),
                              _dev(sw, "sw", torch.float32), _dev(c, "c", tdt), code, M, N, K,
                              qp, sp, wp, wb, _stream_handle(stream)), fn)
    return (c, q_out, sa_out) if want_q else c


def fp8_block_gemm_noalloc(a, sa, w, sw, out_dtype="bf16", c=None, stream=None):
    """fp8_block_gemm whose split-K partials live in the library's static
    device scratch array (no workspace, no allocation by the library; c is
    allocated here with torch only when not given).  Calls that overlap on
    one GPU race on that array."""
    torch = _torch()
    _rank(a, "a", 2)
    _rank(w, "w", 2)
    M, K = a.shape
    N = w.shape[0]
    code, tdt = _out_code(out_dtype)
    if c is None:
        c = torch.empty((M, N), dtype=tdt, device=a.device)
    _shape(w, "w", (N, K))
    if K % 128 == 0 and N % 128 == 0:
        _shape(sa, "sa", (M, K // 128))
        _shape(sw, "sw", (N // 128, K // 128))
    _shape(c, "c", (M, N))
    fn = "fp8_block_gemm_noalloc"
    _check(getattr(lib(), fn)(_dev(a, "a", torch.uint8), _dev(sa, "sa", torch.float32),
                              _dev(w, "w", torch.uint8), _dev(sw, "sw", torch.float32),
                              _dev(c, "c", tdt), code, M, N, K, _stream_handle(stream)), fn)
    return c


def fp8_block_gemm_pow2(a, sa, w, sw, out_dtype="bf16", c=None, workspace=None, stream=None):
    """As fp8_block_gemm, for power-of-two scales (the block-scaled MFMA)."""
    return _block_gemm("fp8_block_gemm_pow2", a, sa, w, sw, out_dtype, c, workspace, stream)


def _grouped_gemm(fn, a, sa, w, sw, group_offsets, out_dtype, c, workspace, stream):
    torch = _torch()
    _rank(a, "a", 2)
    _rank(w, "w", 3)
    T, K = a.shape
    E, N, _ = w.shape
    code, tdt = _out_code(out_dtype)
    if c is None:
        c = torch.empty((T, N), dtype=tdt, device=a.device)
    _shape(w, "w", (E, N, K))
    if K % 128 == 0 and N % 128 == 0:
        _shape(sa, "sa", (T, K // 128))
        _shape(sw, "sw", (E, N // 128, K // 128))
    _shape(group_offsets, "group_offsets", (E + 1,))
    _shape(c, "c", (T, N))
    wp, wb = _workspace_args(workspace)
    _check(getattr(lib(), fn)(_dev(a, "a", torch.uint8), _dev(sa, "sa", torch.float32),
                              _dev(w, "w", torch.uint8), _dev(sw, "sw", torch.float32),
                              _dev(group_offsets, "group_offsets", torch.int32), E, T,
                              _dev(c, "c", tdt), code, N, K, wp, wb, _stream_handle(stream)), fn)
    return c


def fp8_block_grouped_gemm(a, sa, w, sw, group_offsets, out_dtype="bf16", c=None,
                           workspace=None, stream=None):
    """Grouped GEMM over expert-sorted rows: a [T][K], w [E][N][K],
    sw [E][N/128][K/128], group_offsets int32 [E+1] on the GPU."""
    return _grouped_gemm("fp8_block_grouped_gemm", a, sa, w, sw, group_offsets, out_dtype, c,
                         workspace, stream)


def fp8_block_grouped_gemm_pow2(a, sa, w, sw, group_offsets, out_dtype="bf16", c=None,
                                workspace=None, stream=None):
    """As fp8_block_grouped_gemm, for power-of-two scales."""
    return _grouped_gemm("fp8_block_grouped_gemm_pow2", a, sa, w, sw, group_offsets, out_dtype,
                         c, workspace, stream)


# ---- backward pass ------------------------------------------------------------

def fp8_quant_act_128x1_t(x, q_t=None, scales_t=None, stream=None):
    """x: bf16 [M][K] -> (q_t uint8 [K][M], scales_t fp32 [K][ceil(M/128)]):
    128x1 tiles (128 rows of one column), written transposed."""
    return _quant_128x1_t("fp8_quant_act_128x1_t", x, q_t, scales_t, stream)


def fp8_quant_act_128x1_t_pow2(x, q_t=None, scales_t=None, stream=None):
    """As fp8_quant_act_128x1_t with power-of-two scales."""
    return _quant_128x1_t("fp8_quant_act_128x1_t_pow2", x, q_t, scales_t, stream)


def _quant_128x1_t(fn, x, q_t, scales_t, stream):
    torch = _torch()
    _rank(x, "x", 2)
    M, K = x.shape
    if q_t is None:
        q_t = torch.empty((K, M), dtype=torch.uint8, device=x.device)
    if scales_t is None:
        scales_t = torch.empty((K, (M + 127) // 128), dtype=torch.float32, device=x.device)
    _shape(q_t, "q_t", (K, M))
    _shape(scales_t, "scales_t", (K, (M + 127) // 128))
    _check(getattr(lib(), fn)(_dev(x, "x", torch.bfloat16), M, K,
                              _dev(q_t, "q_t", torch.uint8),
                              _dev(scales_t, "scales_t", torch.float32),
                              _stream_handle(stream)), fn)
    return q_t, scales_t


def fp8_transpose_weight_128x128(q, scales, q_t=None, scales_t=None, stream=None):
    """q: uint8 [N][K] with scales [ceil(N/128)][ceil(K/128)] -> (q_t [K][N],
    scales_t [ceil(K/128)][ceil(N/128)])."""
    torch = _torch()
    _rank(q, "q", 2)
    N, K = q.shape
    if q_t is None:
        q_t = torch.empty((K, N), dtype=torch.uint8, device=q.device)
    if scales_t is None:
        scales_t = torch.empty(((K + 127) // 128, (N + 127) // 128), dtype=torch.float32,
                               device=q.device)
    _shape(scales, "scales", ((N + 127) // 128, (K + 127) // 128))
    _shape(q_t, "q_t", (K, N))
    _shape(scales_t, "scales_t", ((K + 127) // 128, (N + 127) // 128))
    _check(lib().fp8_transpose_weight_128x128(_dev(q, "q", torch.uint8),
                                              _dev(scales, "scales", torch.float32), N, K,
                                              _dev(q_t, "q_t", torch.uint8),
                                              _dev(scales_t, "scales_t", torch.float32),
                                              _stream_handle(stream)),
           "fp8_transpose_weight_128x128")
    return q_t, scales_t


def fp8_block_gemm_wgrad(dy_t, dy_t_scales, x_t, x_t_scales, out_dtype="f32", dw=None,
                         stream=None):
    """dW [N][K] = dY^T X from 128x1-grouped operands written transposed:
    dy_t [N][T], x_t [K][T] (uint8 E4M3), scales [N][T/128] and [K][T/128]."""
    return _wgrad("fp8_block_gemm_wgrad", dy_t, dy_t_scales, x_t, x_t_scales, out_dtype, dw,
                  stream)


def fp8_block_gemm_wgrad_pow2(dy_t, dy_t_scales, x_t, x_t_scales, out_dtype="f32", dw=None,
                              stream=None):
    """As fp8_block_gemm_wgrad, for power-of-two scales."""
    return _wgrad("fp8_block_gemm_wgrad_pow2", dy_t, dy_t_scales, x_t, x_t_scales, out_dtype,
                  dw, stream)


def _wgrad(fn, dy_t, dy_t_scales, x_t, x_t_scales, out_dtype, dw, stream):
    torch = _torch()
    _rank(dy_t, "dy_t", 2)
    _rank(x_t, "x_t", 2)
    N, T = dy_t.shape
    K = x_t.shape[0]
    code, tdt = _out_code(out_dtype)
    if dw is None:
        dw = torch.empty((N, K), dtype=tdt, device=dy_t.device)
    _shape(x_t, "x_t", (K, T))
    if T % 128 == 0:
        _shape(dy_t_scales, "dy_t_scales", (N, T // 128))
        _shape(x_t_scales, "x_t_scales", (K, T // 128))
    _shape(dw, "dw", (N, K))
    _check(getattr(lib(), fn)(_dev(dy_t, "dy_t", torch.uint8),
                              _dev(dy_t_scales, "dy_t_scales", torch.float32),
                              _dev(x_t, "x_t", torch.uint8),
                              _dev(x_t_scales, "x_t_scales", torch.float32),
                              _dev(dw, "dw", tdt), code, N, K, T,
                              _stream_handle(stream)), fn)
    return dw
