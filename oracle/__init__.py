"""CPU oracle for the MXFP4 hot path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct definition of MXFP4 block quantization
(OCP Microscaling Formats v1.0, E2M1 elements with an E8M0 scale per 32
elements) and of the block-scaled NT GEMM that consumes the blobs, written in
plain C (``mx_oracle.c``) and wrapped here with ctypes and numpy.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library
(``mxfp4_precision_amd``) never imports, links or calls it, and the two share
no code: only the seeded input generators (``mxfp4_precision_amd.synth``, which
hold none of the method's arithmetic) feed both.

Pins (what checks this oracle against something other than itself) live in
``tests/test_oracle_*.py``.  Every oracle function has at least one pin; the
list is kept in the design notes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mx_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

BLOCK = 32
PAD = 128

_i64 = ctypes.c_int64
_u64 = ctypes.c_uint64
_u32 = ctypes.c_uint32
_int = ctypes.c_int
_vp = ctypes.c_void_p


def build(force: bool = False) -> str:
    """Compile mx_oracle.c with gcc (plain C, OpenMP over independent rows)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        # MX_ORACLE_LIB names another build of mx_oracle.c (the sanitizer build
        # the CPU tests run); the default is the build next to this file.
        path = os.environ.get("MX_ORACLE_LIB")
        if not path:
            build()
            path = _LIB_PATH
        L = ctypes.CDLL(path)
        L.oracle_quantize.argtypes = [_vp, _i64, _i64, _i64, _int, _int, _int, _u64, _u32, _u64, _u32, _vp, _vp]
        L.oracle_quantize.restype = _int
        L.oracle_dequantize.argtypes = [_vp, _vp, _i64, _i64, _vp]
        L.oracle_dequantize.restype = _int
        L.oracle_gemm_entries.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _vp]
        L.oracle_gemm_entries.restype = _int
        L.oracle_gemm_rows.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp]
        L.oracle_gemm_rows.restype = _int
        L.oracle_bf16_from_double_array.argtypes = [_vp, _i64, _vp]
        L.oracle_bf16_from_double_array.restype = None
        L.oracle_philox4x32_10.argtypes = [_vp, _vp, _vp]
        L.oracle_philox4x32_10.restype = None
        L.oracle_sr_byte.argtypes = [_u64, _u32, _u32, _u64]
        L.oracle_sr_byte.restype = ctypes.c_uint
        L.oracle_to_tiled.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp]
        L.oracle_to_tiled.restype = _int
        L.oracle_rht_signs.argtypes = [_u32]
        L.oracle_rht_signs.restype = _u32
        L.oracle_rht32.argtypes = [_vp, _u32, _vp]
        L.oracle_rht32.restype = None
        L.oracle_e5m2_value.argtypes = [ctypes.c_uint8]
        L.oracle_e5m2_value.restype = ctypes.c_double
        L.oracle_e5m2_from_double.argtypes = [ctypes.c_double]
        L.oracle_e5m2_from_double.restype = ctypes.c_uint8
        L.oracle_quantize_fp8_tw.argtypes = [_vp, _i64, _i64, _i64, _int, _vp, _vp, _vp]
        L.oracle_quantize_fp8_tw.restype = _int
        L.oracle_gemm_fp8_entries.argtypes = [_vp, ctypes.c_float, _vp, ctypes.c_float, _i64, _i64, _i64, _i64,
                                              _vp, _vp, _vp]
        L.oracle_gemm_fp8_entries.restype = _int
        L.oracle_fp8_to_tiled.argtypes = [_vp, _i64, _i64, _vp]
        L.oracle_fp8_to_tiled.restype = _int
        L.oracle_fp6_value.argtypes = [ctypes.c_uint, _int]
        L.oracle_fp6_value.restype = ctypes.c_double
        L.oracle_quantize_fp6.argtypes = [_vp, _i64, _i64, _i64, _int, _int, _int, _int, _u64, _u32, _u64, _vp, _vp]
        L.oracle_quantize_fp6.restype = _int
        L.oracle_dequantize_fp6.argtypes = [_vp, _vp, _i64, _i64, _int, _vp]
        L.oracle_dequantize_fp6.restype = _int
        L.oracle_gemm_fp6_entries.argtypes = [_vp, _vp, _int, _vp, _vp, _int, _i64, _i64, _i64, _i64,
                                              _vp, _vp, _vp, _vp]
        L.oracle_gemm_fp6_entries.restype = _int
        L.oracle_fp6_to_tiled.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp]
        L.oracle_fp6_to_tiled.restype = _int
        L.oracle_bf16_mul_array.argtypes = [_vp, _vp, _i64, _vp]
        L.oracle_bf16_mul_array.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def padded(n: int) -> int:
    """Length of a quantized axis after padding to a multiple of 128."""
    return cdiv(n, PAD) * PAD


def blob_shapes(rows: int, length: int) -> Tuple[Tuple[int, int], Tuple[int, int]]:
    """Canonical (data, scale) byte shapes for `rows` blob rows quantized along `length`."""
    lp = padded(length)
    return (rows, lp // 2), (rows, lp // BLOCK)


def quantize(x: np.ndarray, direction: int, use_2d: bool = False, use_sr: bool = False,
             seed: int = 0, tensor_id: int = 0, index_base: int = 0, rht: int = 0):
    """Quantize bf16 bits x (M x N uint16) row-wise (direction 0) or column-wise (1).

    rht != 0: random Hadamard transform of every 32-element block first, with
    the sign pattern of seed `rht` (see rht32).

    Returns canonical (q, s) uint8 arrays: direction 0 -> (M, N_pad/2), (M, N_pad/32);
    direction 1 -> (N, M_pad/2), (N, M_pad/32).
    """
    assert x.dtype == np.uint16 and x.ndim == 2
    x = np.ascontiguousarray(x)
    M, N = x.shape
    rows, length = (M, N) if direction == 0 else (N, M)
    qs, ss = blob_shapes(rows, length)
    q = np.zeros(qs, dtype=np.uint8)
    s = np.zeros(ss, dtype=np.uint8)
    rc = lib().oracle_quantize(_ptr(x), M, N, N, direction, int(use_2d), int(use_sr),
                               seed, tensor_id, index_base, rht, _ptr(q), _ptr(s))
    if rc != 0:
        raise ValueError("oracle_quantize rejected its arguments")
    return q, s


def rht_signs(rht: int) -> int:
    """The 32-bit sign pattern D of seed `rht` (bit p set: negate block position p)."""
    return int(lib().oracle_rht_signs(rht))


def rht32(x: np.ndarray, signs: int) -> np.ndarray:
    """The random Hadamard transform of one 32-element fp32 block (see mx_oracle.c)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape == (32,)
    out = np.empty(32, dtype=np.float32)
    lib().oracle_rht32(_ptr(x), signs, _ptr(out))
    return out


def dequantize(q: np.ndarray, s: np.ndarray, rows: int, length: int) -> np.ndarray:
    """Exact fp64 values of a canonical blob, shape (rows, L_pad)."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    assert q.shape == blob_shapes(rows, length)[0] and s.shape == blob_shapes(rows, length)[1]
    out = np.empty((rows, padded(length)), dtype=np.float64)
    lib().oracle_dequantize(_ptr(q), _ptr(s), rows, length, _ptr(out))
    return out


def gemm_entries(qa, sa, qb, sb, M: int, N: int, K: int, ii, jj) -> np.ndarray:
    """fp64 C[ii[t], jj[t]] of C = deq(A) . deq(B)^T over the padded K."""
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    out = np.empty(ii.shape[0], dtype=np.float64)
    qa, sa, qb, sb = (np.ascontiguousarray(a, dtype=np.uint8) for a in (qa, sa, qb, sb))
    lib().oracle_gemm_entries(_ptr(qa), _ptr(sa), _ptr(qb), _ptr(sb), M, N, K,
                              ii.shape[0], _ptr(ii), _ptr(jj), _ptr(out))
    return out


def gemm_rows(qa, sa, qb, sb, M: int, N: int, K: int, i0: int, i1: int) -> np.ndarray:
    """fp64 rows [i0, i1) of C = deq(A) . deq(B)^T."""
    out = np.empty((i1 - i0, N), dtype=np.float64)
    qa, sa, qb, sb = (np.ascontiguousarray(a, dtype=np.uint8) for a in (qa, sa, qb, sb))
    rc = lib().oracle_gemm_rows(_ptr(qa), _ptr(sa), _ptr(qb), _ptr(sb), M, N, K, i0, i1, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_gemm_rows rejected its arguments")
    return out


def gemm_dense(qa, sa, qb, sb, M: int, N: int, K: int):
    """Whole C = deq(A) . deq(B)^T over the padded K and S = |deq(A)| . |deq(B)|^T
    (the sum of |products| each entry's error bar is scaled by), both fp64 M x N:
    the oracle's exact dequantization, then numpy's float64 matrix product (a
    library routine standing in for the sum; its rounding, ~K 2^-53 S, is far
    below any bar it is used for).  Used where the entry-by-entry sum would
    take too long (full-size products)."""
    da = dequantize(qa, sa, M, K)
    db = dequantize(qb, sb, N, K)
    C = da @ db.T
    np.abs(da, out=da)
    np.abs(db, out=db)
    S = da @ db.T
    return C, S


def e5m2_value(code: int) -> float:
    """Exact value of an FP8 E5M2 code (OFP8)."""
    return float(lib().oracle_e5m2_value(code))


def e5m2_from_double(v: float) -> int:
    """E5M2 code of v: RNE, finite overflow saturates to 57344, Inf kept, NaN -> 0x7F."""
    return int(lib().oracle_e5m2_from_double(float(v)))


def quantize_fp8_tw(x: np.ndarray, direction: int):
    """Tensorwise E5M2 of bf16 bits x (M x N): returns (q, scale_inv, amax); q is
    (M, N_pad) for direction 0, (N, M_pad) for direction 1 (the transpose)."""
    assert x.dtype == np.uint16 and x.ndim == 2
    x = np.ascontiguousarray(x)
    M, N = x.shape
    rows, length = (M, N) if direction == 0 else (N, M)
    q = np.zeros((rows, padded(length)), dtype=np.uint8)
    si = np.zeros(1, np.float32)
    am = np.zeros(1, np.float32)
    if lib().oracle_quantize_fp8_tw(_ptr(x), M, N, N, direction, _ptr(q), _ptr(si), _ptr(am)) != 0:
        raise ValueError("oracle_quantize_fp8_tw rejected its arguments")
    return q, float(si[0]), float(am[0])


def gemm_fp8_entries(qa, sa_inv: float, qb, sb_inv: float, M: int, N: int, K: int, ii, jj) -> np.ndarray:
    """fp64 C[ii, jj] of the tensorwise FP8 NT product (times both inverse scales)."""
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    out = np.empty(ii.shape[0], dtype=np.float64)
    qa = np.ascontiguousarray(qa, dtype=np.uint8)
    qb = np.ascontiguousarray(qb, dtype=np.uint8)
    lib().oracle_gemm_fp8_entries(_ptr(qa), sa_inv, _ptr(qb), sb_inv, M, N, K, ii.shape[0], _ptr(ii), _ptr(jj),
                                  _ptr(out))
    return out


def fp8_to_tiled(q: np.ndarray, rows: int, length: int) -> np.ndarray:
    """Canonical FP8 blob (rows x L_pad) -> the library's FP8 tiled layout (flat uint8)."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.empty(cdiv(rows, 16) * 16 * padded(length), dtype=np.uint8)
    lib().oracle_fp8_to_tiled(_ptr(q), rows, length, _ptr(out))
    return out


def bf16_to_double(bits) -> np.ndarray:
    """bf16 bit patterns -> their exact fp64 values (a bf16 is the top half of an fp32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def gemm_bias_entries(qa, sa, qb, sb, M: int, N: int, K: int, bias_bits, ii, jj) -> np.ndarray:
    """fp64 C[ii[t], jj[t]] + bias[jj[t]]: the NT product plus the linear
    layer's bf16 bias vector (one entry per output column), the sum that the
    parallel linear layers of the page "primus_turbo_mxfp4_local.py" form
    after the FP4 GEMM (``output + bias``).  Taken exactly here; rounding to
    the output type is a separate step (bf16_from_double)."""
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    return gemm_entries(qa, sa, qb, sb, M, N, K, ii, jj) + bf16_to_double(bias_bits)[jj]


def bf16_from_double(a) -> np.ndarray:
    """Correctly rounded (RNE) fp64 -> bf16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().oracle_bf16_from_double_array(_ptr(a), a.size, _ptr(out))
    return out


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    assert c.shape == (4,) and k.shape == (2,)
    out = np.empty(4, dtype=np.uint32)
    lib().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_byte(seed: int, tensor_id: int, direction: int, n: int) -> int:
    return int(lib().oracle_sr_byte(seed, tensor_id, direction, n))


def tiled_shapes(rows: int, length: int) -> Tuple[int, int]:
    """Byte sizes (data, scale) of the tiled layout."""
    lp = padded(length)
    r16 = cdiv(rows, 16) * 16
    return r16 * lp // 2, r16 * cdiv(lp, 512) * 16


def to_tiled(q: np.ndarray, s: np.ndarray, rows: int, length: int):
    """Canonical blob -> the library's tiled layout (flat uint8 arrays)."""
    dq, ds = tiled_shapes(rows, length)
    qt = np.empty(dq, dtype=np.uint8)
    st = np.empty(ds, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    lib().oracle_to_tiled(_ptr(q), _ptr(s), rows, length, _ptr(qt), _ptr(st))
    return qt, st


# ------------------------------------------------------------------ MXFP6
FP6_E2M3 = 2
FP6_E3M2 = 3


def fp6_value(code: int, fmt: int) -> float:
    """Value of a 6-bit code (fmt 2 = E2M3, 3 = E3M2; OCP MX v1.0 sec. 5.3.2)."""
    return float(lib().oracle_fp6_value(code, fmt))


def fp6_blob_shapes(rows: int, length: int) -> Tuple[Tuple[int, int], Tuple[int, int]]:
    """Canonical FP6 (data, scale) byte shapes: 6 bits per element, scales as MXFP4."""
    lp = padded(length)
    return (rows, lp * 3 // 4), (rows, lp // BLOCK)


def quantize_fp6(x: np.ndarray, direction: int, fmt: int, use_2d: bool = False, use_sr: bool = False,
                 seed: int = 0, tensor_id: int = 0, index_base: int = 0):
    """MXFP6 quantization of bf16 bits x (M x N) along rows (0) or columns (1); canonical (q, s)."""
    assert x.dtype == np.uint16 and x.ndim == 2
    x = np.ascontiguousarray(x)
    M, N = x.shape
    rows, length = (M, N) if direction == 0 else (N, M)
    qs, ss = fp6_blob_shapes(rows, length)
    q = np.zeros(qs, dtype=np.uint8)
    s = np.zeros(ss, dtype=np.uint8)
    rc = lib().oracle_quantize_fp6(_ptr(x), M, N, N, direction, fmt, int(use_2d), int(use_sr),
                                   seed, tensor_id, index_base, _ptr(q), _ptr(s))
    if rc != 0:
        raise ValueError("oracle_quantize_fp6 rejected its arguments")
    return q, s


def dequantize_fp6(q: np.ndarray, s: np.ndarray, rows: int, length: int, fmt: int) -> np.ndarray:
    """Exact fp64 values of a canonical FP6 blob, shape (rows, L_pad)."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    assert q.shape == fp6_blob_shapes(rows, length)[0] and s.shape == fp6_blob_shapes(rows, length)[1]
    out = np.empty((rows, padded(length)), dtype=np.float64)
    if lib().oracle_dequantize_fp6(_ptr(q), _ptr(s), rows, length, fmt, _ptr(out)) != 0:
        raise ValueError("oracle_dequantize_fp6 rejected its arguments")
    return out


def gemm_fp6_entries(qa, sa, fmt_a: int, qb, sb, fmt_b: int, M: int, N: int, K: int, ii, jj):
    """fp64 C[ii[t], jj[t]] of deq(A) . deq(B)^T on FP6 blobs, and sum |a b| per entry."""
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    out = np.empty(ii.shape[0], dtype=np.float64)
    aout = np.empty(ii.shape[0], dtype=np.float64)
    qa, sa, qb, sb = (np.ascontiguousarray(a, dtype=np.uint8) for a in (qa, sa, qb, sb))
    if lib().oracle_gemm_fp6_entries(_ptr(qa), _ptr(sa), fmt_a, _ptr(qb), _ptr(sb), fmt_b, M, N, K,
                                     ii.shape[0], _ptr(ii), _ptr(jj), _ptr(out), _ptr(aout)) != 0:
        raise ValueError("oracle_gemm_fp6_entries rejected its arguments")
    return out, aout


def fp6_tiled_shapes(rows: int, length: int) -> Tuple[int, int]:
    """Byte sizes (data, scale) of the tiled FP6 layout."""
    lp = padded(length)
    r16 = cdiv(rows, 16) * 16
    return r16 * lp * 3 // 4, r16 * cdiv(lp, 512) * 16


def fp6_to_tiled(q: np.ndarray, s: np.ndarray, rows: int, length: int):
    """Canonical FP6 blob -> the library's tiled FP6 layout (flat uint8 arrays)."""
    dq, ds = fp6_tiled_shapes(rows, length)
    qt = np.empty(dq, dtype=np.uint8)
    st = np.empty(ds, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    lib().oracle_fp6_to_tiled(_ptr(q), _ptr(s), rows, length, _ptr(qt), _ptr(st))
    return qt, st


# ------------------------------------------------------- multiply prologue
def bf16_mul(x: np.ndarray, g: np.ndarray) -> np.ndarray:
    """bf16(fp32(x * g)) elementwise on bf16 bit arrays of one shape: the tensor the
    multiply prologue quantizes."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    g = np.ascontiguousarray(g, dtype=np.uint16)
    assert x.shape == g.shape
    out = np.empty_like(x)
    lib().oracle_bf16_mul_array(_ptr(x), _ptr(g), x.size, _ptr(out))
    return out
