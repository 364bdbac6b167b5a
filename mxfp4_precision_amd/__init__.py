"""Python binding of libmxfp4 (MXFP4 quantize + block-scaled a4w4 GEMM for gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libmxfp4.so``.  Functions carry the C ABI's names (``include/mxfp4.h``) and
take device pointers as ints or GPU torch tensors (their ``data_ptr()``; host
tensors and arrays are refused before any call), sizes as ints, and a stream
as a ``torch.cuda.Stream``, an int handle, or None (torch's current stream).
A non-zero status raises ``MXError``; if the shared library is missing, the
first call raises: there is no fallback.

Build the library with ``python -m mxfp4_precision_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
# MXFP4_LIB names another build of the same library (the sanitizer build of
# the host code that the CPU tests run); the default is the in-tree build.
LIB_PATH = os.environ.get("MXFP4_LIB") or os.path.join(_HERE, "libmxfp4.so")

MX_SUCCESS = 0
MX_ERR_INVALID_ARGUMENT = 1
MX_ERR_MISALIGNED = 2
MX_ERR_UNSUPPORTED = 3
MX_ERR_DEVICE_UNSUPPORTED = 4
MX_ERR_HIP = 5

MX_LAYOUT_CANONICAL = 0
MX_LAYOUT_TILED = 1
MX_BF16 = 0
MX_F32 = 1
MX_FP6_E2M3 = 2
MX_FP6_E3M2 = 3

EXPORTED = ("mx_blob_bytes", "mx_quantize_rowwise", "mx_quantize_dual", "mx_gemm_a4w4", "mx_gemm_a4w4_bias",
            "mx_layout_convert", "mx_layout_convert_host", "mx_dequantize", "mx_device_supported",
            "mx_fp8_blob_bytes", "mx_quantize_fp8_tw", "mx_gemm_f8_tw",
            "mx_fp6_blob_bytes", "mx_quantize_fp6", "mx_gemm_fp6", "mx_quantize_dual_mul",
            "mx_measure_mfma", "mx_set_device_arch_override", "mx_status_string", "mx_last_error")


class MXError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__("%s: %s" % (_status_name(status), detail))
        self.status = status


class mx_quant_opts(ctypes.Structure):
    _fields_ = [("use_2d_block", ctypes.c_uint32), ("use_sr", ctypes.c_uint32),
                ("seed", ctypes.c_uint64), ("tensor_id", ctypes.c_uint32),
                ("index_base", ctypes.c_uint64), ("rht", ctypes.c_uint32)]


def quant_opts(use_2d_block: bool = False, use_sr: bool = False, seed: int = 0,
               tensor_id: int = 0, index_base: int = 0, rht: int = 0) -> mx_quant_opts:
    return mx_quant_opts(int(use_2d_block), int(use_sr), seed, tensor_id, index_base, rht)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmxfp4.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libmxfp4.so not found at %s: build it with "
                           "`python -m mxfp4_precision_amd.build` (no fallback path exists)" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    optp = ctypes.POINTER(mx_quant_opts)
    L.mx_blob_bytes.argtypes = [i64, i64, i32, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    L.mx_quantize_rowwise.argtypes = [vp, i64, i64, i64, optp, i32, vp, vp, vp]
    L.mx_quantize_dual.argtypes = [vp, i64, i64, i64, optp, optp, i32, vp, vp, vp, vp, vp]
    L.mx_gemm_a4w4.argtypes = [i32, i32, i64, i64, i64, vp, vp, vp, vp, i32, i32, vp, i64, vp]
    L.mx_gemm_a4w4_bias.argtypes = [i32, i32, i64, i64, i64, vp, vp, vp, vp, i32, i32, vp, vp, i64, vp]
    L.mx_layout_convert.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp]
    L.mx_fp8_blob_bytes.argtypes = [i64, i64, i32, ctypes.POINTER(ctypes.c_size_t)]
    L.mx_quantize_fp8_tw.argtypes = [vp, i64, i64, i64, i32, vp, vp, vp, vp]
    L.mx_gemm_f8_tw.argtypes = [i32, i32, i64, i64, i64, vp, vp, vp, vp, i32, i32, vp, i64, vp]
    L.mx_layout_convert_host.argtypes = [i32, i64, i64, vp, vp, vp, vp]
    L.mx_fp6_blob_bytes.argtypes = [i64, i64, i32, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    L.mx_quantize_fp6.argtypes = [vp, i64, i64, i64, i32, optp, i32, optp, i32, vp, vp, vp, vp, vp]
    L.mx_quantize_dual_mul.argtypes = [vp, vp, i64, i64, i64, i64, optp, optp, i32, vp, vp, vp, vp, vp]
    L.mx_gemm_fp6.argtypes = [i32, i32, i64, i64, i64, i32, vp, vp, i32, vp, vp, i32, i32, vp, i64, vp]
    L.mx_dequantize.argtypes = [vp, vp, i64, i64, i32, vp, i64, vp]
    L.mx_measure_mfma.argtypes = [i32, i32, vp, i32, i64, vp, vp]
    L.mx_set_device_arch_override.argtypes = [ctypes.c_char_p]
    L.mx_device_supported.argtypes = [i32]
    L.mx_device_supported.restype = i32
    L.mx_status_string.argtypes = [i32]
    L.mx_status_string.restype = ctypes.c_char_p
    L.mx_last_error.argtypes = []
    L.mx_last_error.restype = ctypes.c_char_p
    for name in EXPORTED:
        if name not in ("mx_device_supported", "mx_status_string", "mx_last_error"):
            getattr(L, name).restype = i32     # mx_status
    _lib = L
    return L


def _status_name(st: int) -> str:
    try:
        return lib().mx_status_string(st).decode()
    except Exception:
        return "status %d" % st


def _check(st: int):
    if st != MX_SUCCESS:
        raise MXError(st, lib().mx_last_error().decode())


def _dptr(p) -> Optional[int]:
    """A device-pointer argument.  Ints pass through (the caller vouches for
    them); a tensor must live on a GPU.  Host tensors and arrays are refused
    here: a kernel that dereferences a host address faults the device."""
    if p is None or isinstance(p, int):
        return p
    if hasattr(p, "data_ptr"):
        if not getattr(p, "is_cuda", False):
            raise TypeError("a device pointer is required, got a tensor on %s" % p.device)
        return p.data_ptr()
    raise TypeError("a device pointer is required, got %r (host arrays are not accepted)" % type(p))


def _hptr(p) -> Optional[int]:
    """A host-pointer argument (the host layout converter): numpy arrays, CPU
    tensors or ints; device tensors are refused."""
    if p is None or isinstance(p, int):
        return p
    if hasattr(p, "data_ptr"):
        if getattr(p, "is_cuda", False):
            raise TypeError("a host pointer is required, got a tensor on %s" % p.device)
        return p.data_ptr()
    if hasattr(p, "ctypes"):          # numpy array
        return p.ctypes.data
    raise TypeError("expected a host array, tensor or int, got %r" % type(p))


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _opts(o):
    return ctypes.byref(o) if o is not None else None


# ------------------------------------------------------------------ C ABI names

def mx_blob_bytes(rows: int, length: int, layout: int) -> Tuple[int, int]:
    d, s = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().mx_blob_bytes(rows, length, layout, ctypes.byref(d), ctypes.byref(s)))
    return d.value, s.value


def mx_quantize_rowwise(x, M: int, N: int, ldx: int, opts, layout: int, q, s, stream=None):
    _check(lib().mx_quantize_rowwise(_dptr(x), M, N, ldx, _opts(opts), layout, _dptr(q), _dptr(s),
                                     _stream(stream)))


def mx_quantize_dual(x, M: int, N: int, ldx: int, row_opts, col_opts, layout: int,
                     q_row, s_row, q_col, s_col, stream=None):
    _check(lib().mx_quantize_dual(_dptr(x), M, N, ldx, _opts(row_opts), _opts(col_opts), layout,
                                  _dptr(q_row), _dptr(s_row), _dptr(q_col), _dptr(s_col), _stream(stream)))


def mx_quantize_dual_mul(x, g, M: int, N: int, ldx: int, ldg: int, row_opts, col_opts, layout: int,
                         q_row, s_row, q_col=None, s_col=None, stream=None):
    _check(lib().mx_quantize_dual_mul(_dptr(x), _dptr(g), M, N, ldx, ldg, _opts(row_opts), _opts(col_opts),
                                      layout, _dptr(q_row), _dptr(s_row), _dptr(q_col), _dptr(s_col),
                                      _stream(stream)))


def mx_fp6_blob_bytes(rows: int, length: int, layout: int) -> Tuple[int, int]:
    d, s = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().mx_fp6_blob_bytes(rows, length, layout, ctypes.byref(d), ctypes.byref(s)))
    return d.value, s.value


def mx_quantize_fp6(x, M: int, N: int, ldx: int, row_fmt: int, row_opts, col_fmt: int, col_opts,
                    layout: int, q_row, s_row, q_col=None, s_col=None, stream=None):
    _check(lib().mx_quantize_fp6(_dptr(x), M, N, ldx, row_fmt, _opts(row_opts), col_fmt, _opts(col_opts),
                                 layout, _dptr(q_row), _dptr(s_row), _dptr(q_col), _dptr(s_col), _stream(stream)))


def mx_gemm_fp6(transA: int, transB: int, M: int, N: int, K: int, fmt_a: int, A, A_scale, fmt_b: int, B, B_scale,
                layout: int, out_dtype: int, C, ldc: int, stream=None):
    _check(lib().mx_gemm_fp6(transA, transB, M, N, K, fmt_a, _dptr(A), _dptr(A_scale), fmt_b, _dptr(B),
                             _dptr(B_scale), layout, out_dtype, _dptr(C), ldc, _stream(stream)))


def mx_gemm_a4w4(transA: int, transB: int, M: int, N: int, K: int, A, A_scale, B, B_scale,
                 layout: int, out_dtype: int, C, ldc: int, stream=None):
    _check(lib().mx_gemm_a4w4(transA, transB, M, N, K, _dptr(A), _dptr(A_scale), _dptr(B), _dptr(B_scale),
                              layout, out_dtype, _dptr(C), ldc, _stream(stream)))


def mx_gemm_a4w4_bias(transA: int, transB: int, M: int, N: int, K: int, A, A_scale, B, B_scale,
                      layout: int, out_dtype: int, bias, C, ldc: int, stream=None):
    _check(lib().mx_gemm_a4w4_bias(transA, transB, M, N, K, _dptr(A), _dptr(A_scale), _dptr(B), _dptr(B_scale),
                                   layout, out_dtype, _dptr(bias), _dptr(C), ldc, _stream(stream)))


def mx_fp8_blob_bytes(rows: int, length: int, layout: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().mx_fp8_blob_bytes(rows, length, layout, ctypes.byref(n)))
    return n.value


def mx_quantize_fp8_tw(x, M: int, N: int, ldx: int, layout: int, q_row, q_col, info, stream=None):
    _check(lib().mx_quantize_fp8_tw(_dptr(x), M, N, ldx, layout, _dptr(q_row), _dptr(q_col), _dptr(info),
                                    _stream(stream)))


def mx_gemm_f8_tw(transA: int, transB: int, M: int, N: int, K: int, A, a_scale_inv, B, b_scale_inv,
                  layout: int, out_dtype: int, C, ldc: int, stream=None):
    _check(lib().mx_gemm_f8_tw(transA, transB, M, N, K, _dptr(A), _dptr(a_scale_inv), _dptr(B),
                               _dptr(b_scale_inv), layout, out_dtype, _dptr(C), ldc, _stream(stream)))


def mx_layout_convert(to_tiled: int, rows: int, length: int, q_src, s_src, q_dst, s_dst, stream=None):
    _check(lib().mx_layout_convert(to_tiled, rows, length, _dptr(q_src), _dptr(s_src), _dptr(q_dst),
                                   _dptr(s_dst), _stream(stream)))


def mx_layout_convert_host(to_tiled: int, rows: int, length: int, q_src, s_src, q_dst, s_dst):
    _check(lib().mx_layout_convert_host(to_tiled, rows, length, _hptr(q_src), _hptr(s_src),
                                        _hptr(q_dst), _hptr(s_dst)))


def mx_dequantize(q, s, rows: int, length: int, layout: int, out_f32, ldo: int, stream=None):
    _check(lib().mx_dequantize(_dptr(q), _dptr(s), rows, length, layout, _dptr(out_f32), ldo,
                               _stream(stream)))


def mx_measure_mfma(fmt_a: int, fmt_b: int, operands, workgroups: int, iters: int, out, stream=None):
    _check(lib().mx_measure_mfma(fmt_a, fmt_b, _dptr(operands), workgroups, iters, _dptr(out), _stream(stream)))


def mx_device_supported(device: int) -> bool:
    return bool(lib().mx_device_supported(device))


def mx_set_device_arch_override(arch: Optional[str]):
    """Test aid: fixed architecture name in place of the device query (None restores it)."""
    _check(lib().mx_set_device_arch_override(None if arch is None else arch.encode()))


def mx_status_string(status: int) -> str:
    return lib().mx_status_string(status).decode()


def mx_last_error() -> str:
    return lib().mx_last_error().decode()


# ------------------------------------------------- allocation helpers (plumbing)

def empty_blob(rows: int, length: int, layout: int, device="cuda"):
    """Allocate (data, scale) uint8 tensors of the right byte sizes on `device`."""
    import torch
    db, sb = mx_blob_bytes(rows, length, layout)
    return (torch.empty(max(db, 1), dtype=torch.uint8, device=device),
            torch.empty(max(sb, 1), dtype=torch.uint8, device=device))
