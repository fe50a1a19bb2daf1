"""ctypes binding of libfp8fg.so (include/fp8fg.h), same function names.

Argument marshalling only: these functions check tensor devices, dtypes and
shapes, allocate outputs with torch when none are given, and pass raw device
pointers plus torch's current HIP stream to the C ABI.  Every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is not built, or a call fails, an exception is raised.
"""

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8fg.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "fp8fg.h")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_MISALIGNED, ERR_HIP = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
B_BLOCK_128x128, B_ROW_1x128 = 0, 1
ACCUM_FP8_MFMA, ACCUM_EXACT, ACCUM_SCALED_MFMA = 0, 1, 2

_lib = None

_c = ctypes
_SIGS = {
    "fp8_quant_act_1x128": [_c.c_void_p, _c.c_int, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64,
                            _c.c_void_p, _c.c_void_p, _c.c_void_p],
    "fp8_quant_act_1x128_pow2": [_c.c_void_p, _c.c_int, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64,
                                 _c.c_void_p, _c.c_void_p, _c.c_void_p],
    "fp8_quant_weight_128x128": [_c.c_void_p, _c.c_int, _c.c_int64, _c.c_int64, _c.c_int64,
                                 _c.c_void_p, _c.c_void_p, _c.c_void_p],
    "fp8_quant_weight_128x128_pow2": [_c.c_void_p, _c.c_int, _c.c_int64, _c.c_int64, _c.c_int64,
                                      _c.c_void_p, _c.c_void_p, _c.c_void_p],
    "fp8_quant_per_tensor": [_c.c_void_p, _c.c_int, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_void_p,
                             _c.c_void_p, _c.c_int, _c.c_void_p],
    "fp8_quant_act_weight": [_c.c_void_p, _c.c_int, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_void_p,
                             _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int64, _c.c_int64, _c.c_int64,
                             _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_void_p],
    "fp8_quant_weight_128x128_dual": [_c.c_void_p, _c.c_int, _c.c_int64, _c.c_int64, _c.c_int64,
                                      _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p],
    "fp8_quant_weight_128x128_dual_pow2": [_c.c_void_p, _c.c_int, _c.c_int64, _c.c_int64, _c.c_int64,
                                           _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p],
    "fp8_block_gemm": [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int,
                       _c.c_void_p, _c.c_int, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_void_p],
    "fp8_block_gemm_accum": [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int,
                             _c.c_void_p, _c.c_int, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_void_p],
    "fp8_block_gemm_quant": [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int,
                             _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_void_p],
    "fp8_block_grouped_gemm": [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_void_p,
                               _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int64,
                               _c.c_int64, _c.c_int64, _c.c_void_p],
    "fp8_block_grouped_gemm_accum": [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_void_p,
                                     _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int, _c.c_int64,
                                     _c.c_int64, _c.c_int64, _c.c_void_p],
    "fp8_block_grouped_gemm_gather": [_c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_void_p, _c.c_void_p,
                                      _c.c_int64, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int,
                                      _c.c_int64, _c.c_int64, _c.c_int64, _c.c_void_p],
    "fp8fg_status_string": [_c.c_int],
    "fp8fg_abi_version": [],
}


class Fp8fgError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: status {status}: {lib().fp8fg_status_string(status).decode()}")


def lib():
    """The loaded library (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built: run `python -m fp8_fine_grained_amd.build` "
                "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_char_p if name == "fp8fg_status_string" else ctypes.c_int
        _lib = L
    return _lib


def declared_functions():
    """Names of the functions include/fp8fg.h declares."""
    text = open(HEADER).read()
    return re.findall(r"^(?:int|const char\*)\s+(\w+)\s*\(", text, flags=re.M)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dtype_code(dt):
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {dt} (float32 or bfloat16)")


def _check(fn, status):
    if status != OK:
        raise Fp8fgError(fn, status)


def _on_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def fp8_quant_act_1x128(x, q=None, scales=None, stream=None, pow2=False):
    """1x128 quantisation of the logical matrix ``x`` [M, K] along K.

    ``x`` may be row-contiguous, or a transposed view of a row-major [K, M]
    tensor (e.g. ``dy.t()``: tiles then run along the token axis).
    ``pow2=True`` calls fp8_quant_act_1x128_pow2 (power-of-two scales).
    Returns ``(q uint8 [M, K], scales fp32 [M, K/128])``.
    """
    _on_gpu(x)
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, K // 128 if K % 128 == 0 else 0), dtype=torch.float32, device=x.device)
    _on_gpu(q, scales)
    fn = "fp8_quant_act_1x128_pow2" if pow2 else "fp8_quant_act_1x128"
    st = getattr(lib(), fn)(_ptr(x), _dtype_code(x.dtype), M, K, x.stride(0), x.stride(1),
                            _ptr(q), _ptr(scales), _stream(stream))
    _check(fn, st)
    return q, scales


def fp8_quant_weight_128x128(w, q=None, scales=None, stream=None, pow2=False):
    """128x128 quantisation of ``w`` [N, K].  Returns ``(q [N, K], scales [N/128, K/128])``.
    ``pow2=True`` calls fp8_quant_weight_128x128_pow2 (power-of-two scales)."""
    _on_gpu(w)
    N, K = w.shape
    if w.stride(1) != 1:
        raise ValueError("w must be row-contiguous")
    if q is None:
        q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((N // 128, K // 128), dtype=torch.float32, device=w.device)
    _on_gpu(q, scales)
    fn = "fp8_quant_weight_128x128_pow2" if pow2 else "fp8_quant_weight_128x128"
    st = getattr(lib(), fn)(_ptr(w), _dtype_code(w.dtype), N, K, w.stride(0), _ptr(q),
                            _ptr(scales), _stream(stream))
    _check(fn, st)
    return q, scales


def fp8_quant_act_weight(x, w, q_x=None, s_x=None, q_w=None, s_w=None, stream=None, pow2=False):
    """1x128 quantisation of the row-contiguous ``x`` [M, K_x] and 128x128
    quantisation of ``w`` [N, K_w] in one launch (fp8_quant_act_weight).
    Returns ``(q_x, s_x, q_w, s_w)``, equal to fp8_quant_act_1x128(x) and
    fp8_quant_weight_128x128(w)."""
    _on_gpu(x, w)
    M, Kx = x.shape
    N, Kw = w.shape
    if x.stride(1) != 1 or w.stride(1) != 1:
        raise ValueError("x and w must be row-contiguous")
    dev = x.device
    q_x = torch.empty((M, Kx), dtype=torch.uint8, device=dev) if q_x is None else q_x
    s_x = torch.empty((M, Kx // 128), dtype=torch.float32, device=dev) if s_x is None else s_x
    q_w = torch.empty((N, Kw), dtype=torch.uint8, device=dev) if q_w is None else q_w
    s_w = torch.empty((N // 128, Kw // 128), dtype=torch.float32, device=dev) if s_w is None else s_w
    _on_gpu(q_x, s_x, q_w, s_w)
    st = lib().fp8_quant_act_weight(_ptr(x), _dtype_code(x.dtype), M, Kx, x.stride(0), _ptr(q_x), _ptr(s_x),
                                    _ptr(w), _dtype_code(w.dtype), N, Kw, w.stride(0), _ptr(q_w), _ptr(s_w),
                                    1 if pow2 else 0, _stream(stream))
    _check("fp8_quant_act_weight", st)
    return q_x, s_x, q_w, s_w


def fp8_quant_per_tensor(x, layout="act", q=None, scales=None, stream=None):
    """One scale for the whole row-contiguous ``x`` [M, K] (fp8_quant_per_tensor).

    ``layout="act"`` fills scales [M, K/128] (the GEMM's A operand), ``"weight"``
    scales [M/128, K/128] (its B operand in block mode); every entry is the one
    scale.  Returns ``(q uint8 [M, K], scales)``."""
    _on_gpu(x)
    M, K = x.shape
    if x.stride(1) != 1:
        raise ValueError("x must be row-contiguous")
    mode = {"act": B_ROW_1x128, "weight": B_BLOCK_128x128}[layout]
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        rows = M if layout == "act" else M // 128
        scales = torch.empty((rows, K // 128), dtype=torch.float32, device=x.device)
    _on_gpu(q, scales)
    st = lib().fp8_quant_per_tensor(_ptr(x), _dtype_code(x.dtype), M, K, x.stride(0), _ptr(q), _ptr(scales), mode,
                                    _stream(stream))
    _check("fp8_quant_per_tensor", st)
    return q, scales


def fp8_quant_weight_128x128_dual(w, q=None, scales=None, q_t=None, scales_t=None, stream=None, pow2=False):
    """128x128 quantisation of ``w`` [N, K] plus the transposed operand.

    Returns ``(q [N, K], scales [N/128, K/128], q_t [K, N], scales_t [K/128, N/128])``;
    ``(q_t, scales_t)`` is the B operand of the data-gradient GEMM dX = dY W.
    ``pow2=True`` calls fp8_quant_weight_128x128_dual_pow2 (power-of-two scales)."""
    _on_gpu(w)
    N, K = w.shape
    if w.stride(1) != 1:
        raise ValueError("w must be row-contiguous")
    dev = w.device
    q = torch.empty((N, K), dtype=torch.uint8, device=dev) if q is None else q
    scales = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev) if scales is None else scales
    q_t = torch.empty((K, N), dtype=torch.uint8, device=dev) if q_t is None else q_t
    scales_t = torch.empty((K // 128, N // 128), dtype=torch.float32, device=dev) if scales_t is None else scales_t
    _on_gpu(q, scales, q_t, scales_t)
    fn = "fp8_quant_weight_128x128_dual_pow2" if pow2 else "fp8_quant_weight_128x128_dual"
    st = getattr(lib(), fn)(_ptr(w), _dtype_code(w.dtype), N, K, w.stride(0), _ptr(q), _ptr(scales), _ptr(q_t),
                            _ptr(scales_t), _stream(stream))
    _check(fn, st)
    return q, scales, q_t, scales_t


def _accum_code(accum, out_dtype):
    if accum is None:
        return ACCUM_EXACT if out_dtype == torch.float32 else ACCUM_FP8_MFMA
    return {"fp8": ACCUM_FP8_MFMA, "exact": ACCUM_EXACT, "scaled": ACCUM_SCALED_MFMA,
            ACCUM_FP8_MFMA: ACCUM_FP8_MFMA, ACCUM_EXACT: ACCUM_EXACT, ACCUM_SCALED_MFMA: ACCUM_SCALED_MFMA}[accum]


def _contig(*ts):
    for t in ts:
        if not t.is_contiguous():
            raise ValueError("GEMM operands, scales and outputs must be contiguous")


def fp8_block_gemm(a, sa, b, sb, b_scale_mode="block", accum=None, out_dtype=torch.bfloat16,
                   y=None, stream=None):
    """Y = deq(a) deq(b)^T; ``accum`` "fp8", "exact" (default for fp32 output) or
    "scaled" (power-of-two scales applied by the matrix cores)."""
    _on_gpu(a, sa, b, sb)
    M, K = a.shape
    N = b.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _on_gpu(y)
    _contig(a, sa, b, sb, y)
    mode = {"block": B_BLOCK_128x128, "row": B_ROW_1x128}[b_scale_mode]
    if accum is None:  # the library's default summation for the output type
        st = lib().fp8_block_gemm(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), mode, _ptr(y), _dtype_code(y.dtype),
                                  M, N, K, _stream(stream))
        _check("fp8_block_gemm", st)
    else:
        st = lib().fp8_block_gemm_accum(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), mode, _accum_code(accum, y.dtype),
                                        _ptr(y), _dtype_code(y.dtype), M, N, K, _stream(stream))
        _check("fp8_block_gemm_accum", st)
    return y


def fp8_block_gemm_quant(a, sa, b, sb, accum="fp8", pow2=False, q=None, scales=None, stream=None):
    """Y = deq(a) deq(b)^T leaving the GEMM 1x128-quantised: returns (q uint8 [M, N],
    scales fp32 [M, N/128]); ``accum`` "fp8" or "scaled", ``pow2`` power-of-two scales."""
    _on_gpu(a, sa, b, sb)
    M, K = a.shape
    N = b.shape[0]
    if q is None:
        q = torch.empty((M, N), dtype=torch.uint8, device=a.device)
    if scales is None:
        scales = torch.empty((M, N // 128), dtype=torch.float32, device=a.device)
    _on_gpu(q, scales)
    _contig(a, sa, b, sb, q, scales)
    st = lib().fp8_block_gemm_quant(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _accum_code(accum, torch.bfloat16),
                                    1 if pow2 else 0, _ptr(q), _ptr(scales), M, N, K, _stream(stream))
    _check("fp8_block_gemm_quant", st)
    return q, scales


def fp8_block_grouped_gemm(a, sa, offsets, b, sb, accum=None, out_dtype=torch.bfloat16, y=None,
                           stream=None):
    """Grouped GEMM over expert row segments ``offsets`` (device int32 [G+1])."""
    _on_gpu(a, sa, offsets, b, sb)
    M, K = a.shape
    G, N, _ = b.shape
    if offsets.dtype != torch.int32 or offsets.numel() != G + 1:
        raise ValueError("offsets must be int32 [G+1]")
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _on_gpu(y)
    _contig(a, sa, offsets, b, sb, y)
    if accum is None:  # the library's default summation for the output type
        st = lib().fp8_block_grouped_gemm(_ptr(a), _ptr(sa), _ptr(offsets), G, _ptr(b), _ptr(sb), _ptr(y),
                                          _dtype_code(y.dtype), M, N, K, _stream(stream))
        _check("fp8_block_grouped_gemm", st)
    else:
        st = lib().fp8_block_grouped_gemm_accum(_ptr(a), _ptr(sa), _ptr(offsets), G, _ptr(b), _ptr(sb),
                                                _accum_code(accum, y.dtype), _ptr(y), _dtype_code(y.dtype),
                                                M, N, K, _stream(stream))
        _check("fp8_block_grouped_gemm_accum", st)
    return y


def fp8_block_grouped_gemm_gather(a_tok, sa_tok, row_index, offsets, b, sb, accum=None,
                                  out_dtype=torch.bfloat16, y=None, stream=None):
    """Grouped GEMM whose row r is token ``row_index[r]`` of ``a_tok`` [T, K]
    (``row_index`` device int32 [M_total]); Y stays in routed-row order."""
    _on_gpu(a_tok, sa_tok, row_index, offsets, b, sb)
    T, K = a_tok.shape
    G, N, _ = b.shape
    M = row_index.numel()
    if offsets.dtype != torch.int32 or offsets.numel() != G + 1:
        raise ValueError("offsets must be int32 [G+1]")
    if row_index.dtype != torch.int32:
        raise ValueError("row_index must be int32")
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=a_tok.device)
    _on_gpu(y)
    _contig(a_tok, sa_tok, row_index, offsets, b, sb, y)
    st = lib().fp8_block_grouped_gemm_gather(_ptr(a_tok), _ptr(sa_tok), T, _ptr(row_index), _ptr(offsets), G,
                                             _ptr(b), _ptr(sb), _accum_code(accum, y.dtype), _ptr(y),
                                             _dtype_code(y.dtype), M, N, K, _stream(stream))
    _check("fp8_block_grouped_gemm_gather", st)
    return y
