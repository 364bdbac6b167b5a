"""Host-side checks of the libmxfp4 C ABI that need no GPU: the library loads
and exports every function include/mxfp4.h declares, argument validation
rejects bad calls before any launch, blob sizes match the canonical shapes of
the fake dual-quantize op (page "primus_turbo_mxfp4_local.py") and the tiled
layout's definition, and the host layout converter agrees with the oracle's
independent permutation."""
import ctypes
import os
import re

import numpy as np
import pytest

import mxfp4_precision_amd as mx
from mxfp4_precision_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mx.LIB_PATH):
        from mxfp4_precision_amd import build
        build.build()
    return mx.lib()


def _gpu_present():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.fixture(autouse=True)
def _no_launch_on_a_gpu(L):
    """These tests pass fake (never dereferenced) addresses.  On a machine with
    a GPU, a call whose arguments pass validation would launch a kernel on
    them, so the device query is replaced by a non-gfx950 name there and every
    such call stops at the device check instead.  Without a GPU the real query
    runs (and fails with MX_ERR_HIP)."""
    if _gpu_present():
        mx.mx_set_device_arch_override("gfx000")
        yield
        mx.mx_set_device_arch_override(None)
    else:
        yield


def declared_functions():
    names = []
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            text = open(os.path.join(inc, f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w \*]*?\b(mx_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(mx.EXPORTED) <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for st, name in [(0, "MX_SUCCESS"), (1, "MX_ERR_INVALID_ARGUMENT"), (2, "MX_ERR_MISALIGNED"),
                     (3, "MX_ERR_UNSUPPORTED"), (4, "MX_ERR_DEVICE_UNSUPPORTED"), (5, "MX_ERR_HIP")]:
        assert mx.mx_status_string(st) == name


@pytest.mark.parametrize("rows,length", [(1, 1), (4600, 3072), (3072, 4600), (127, 129), (256, 512),
                                         (18432, 12288), (0, 5), (7, 0)])
def test_blob_bytes(L, oracle_mod, rows, length):
    d, s = mx.mx_blob_bytes(rows, length, mx.MX_LAYOUT_CANONICAL)
    (qr, qc), (sr, sc) = oracle_mod.blob_shapes(rows, length)
    assert d == qr * qc and s == sr * sc
    dt, st = mx.mx_blob_bytes(rows, length, mx.MX_LAYOUT_TILED)
    assert (dt, st) == oracle_mod.tiled_shapes(rows, length)


def test_blob_bytes_errors(L):
    with pytest.raises(mx.MXError) as e:
        mx.mx_blob_bytes(-1, 4, 0)
    assert e.value.status == mx.MX_ERR_INVALID_ARGUMENT
    with pytest.raises(mx.MXError) as e:
        mx.mx_blob_bytes(1, 4, 7)
    assert e.value.status == mx.MX_ERR_UNSUPPORTED


def _status(fn, *args):
    try:
        fn(*args)
        return mx.MX_SUCCESS
    except mx.MXError as e:
        return e.status


def test_quantize_validation_runs_before_any_launch(L):
    """Every bad argument is rejected on the host (no device is touched here)."""
    A16 = 1 << 20          # fake, 16-byte aligned addresses: never dereferenced
    o = mx.quant_opts()
    Q = mx.mx_quantize_rowwise
    assert _status(Q, A16, -1, 8, 8, o, 0, A16, A16, 0) == mx.MX_ERR_INVALID_ARGUMENT
    assert _status(Q, A16, 4, 16, 8, o, 0, A16, A16, 0) == mx.MX_ERR_INVALID_ARGUMENT   # ldx < N
    assert _status(Q, 0, 4, 8, 8, o, 0, A16, A16, 0) == mx.MX_ERR_INVALID_ARGUMENT       # x NULL
    assert _status(Q, A16 + 2, 4, 8, 8, o, 0, A16, A16, 0) == mx.MX_ERR_MISALIGNED
    assert _status(Q, A16, 4, 8, 12, o, 0, A16, A16, 0) == mx.MX_ERR_MISALIGNED           # ldx % 8
    assert _status(Q, A16, 4, 8, 8, o, 5, A16, A16, 0) == mx.MX_ERR_UNSUPPORTED           # layout
    assert _status(Q, A16, 4, 8, 8, o, 0, 0, A16, 0) == mx.MX_ERR_INVALID_ARGUMENT        # q NULL
    assert _status(Q, A16, 4, 8, 8, o, 0, A16, A16 + 4, 0) == mx.MX_ERR_MISALIGNED
    bad = mx.quant_opts(); bad.use_sr = 2
    assert _status(Q, A16, 4, 8, 8, bad, 0, A16, A16, 0) == mx.MX_ERR_INVALID_ARGUMENT
    rht2d = mx.quant_opts(use_2d_block=True, rht=5)
    assert _status(Q, A16, 4, 8, 8, rht2d, 0, A16, A16, 0) == mx.MX_ERR_UNSUPPORTED
    # empty tensors are a no-op success before any device query
    assert _status(Q, A16, 0, 8, 8, o, 0, A16, A16, 0) == mx.MX_SUCCESS
    assert _status(Q, A16, 4, 0, 8, o, 0, A16, A16, 0) == mx.MX_SUCCESS
    D = mx.mx_quantize_dual
    assert _status(D, A16, 4, 8, 8, o, o, 0, A16, A16, 0, A16, 0) == mx.MX_ERR_INVALID_ARGUMENT
    assert _status(D, A16, 4, 8, 8, o, bad, 0, A16, A16, A16, A16, 0) == mx.MX_ERR_INVALID_ARGUMENT
    assert _status(D, A16, 0, 8, 8, o, o, 0, A16, A16, A16, A16, 0) == mx.MX_SUCCESS
    assert mx.mx_last_error() != ""


def test_gemm_validation(L):
    A16 = 1 << 20
    G = mx.mx_gemm_a4w4
    T = mx.MX_LAYOUT_TILED
    for ta, tb in [(0, 0), (1, 1), (1, 0)]:
        assert _status(G, ta, tb, 4, 4, 4, A16, A16, A16, A16, T, 0, A16, 8, 0) == mx.MX_ERR_UNSUPPORTED
    assert "transA" in mx.mx_last_error()
    assert _status(G, 0, 1, -1, 4, 4, A16, A16, A16, A16, T, 0, A16, 8, 0) == mx.MX_ERR_INVALID_ARGUMENT
    assert _status(G, 0, 1, 4, 4, 4, A16, A16, A16, A16, 0, 0, A16, 8, 0) == mx.MX_ERR_UNSUPPORTED   # canonical
    assert _status(G, 0, 1, 4, 4, 4, A16, A16, A16, A16, T, 9, A16, 8, 0) == mx.MX_ERR_UNSUPPORTED   # dtype
    assert _status(G, 0, 1, 4, 16, 4, A16, A16, A16, A16, T, 0, A16, 8, 0) == mx.MX_ERR_INVALID_ARGUMENT  # ldc
    assert _status(G, 0, 1, 4, 4, 4, 0, A16, A16, A16, T, 0, A16, 8, 0) == mx.MX_ERR_INVALID_ARGUMENT
    assert _status(G, 0, 1, 4, 4, 4, A16, A16, A16, A16, T, 0, 0, 8, 0) == mx.MX_ERR_INVALID_ARGUMENT
    assert _status(G, 0, 1, 4, 4, 4, A16 + 8, A16, A16, A16, T, 0, A16, 8, 0) == mx.MX_ERR_MISALIGNED
    assert _status(G, 0, 1, 4, 4, 4, A16, A16, A16, A16, T, 0, A16, 12, 0) == mx.MX_ERR_MISALIGNED
    assert _status(G, 0, 1, 0, 4, 4, A16, A16, A16, A16, T, 0, A16, 8, 0) == mx.MX_SUCCESS


def test_gemm_operand_blob_limit(L):
    """Operand blobs are addressed with 32-bit buffer offsets: a tiled blob of
    2 GiB or more is refused before anything is launched (here with no GPU:
    the check runs ahead of the device query).  2^20 rows x K 4096 is exactly
    2 GiB of E2M1 data (a guard on cdiv(rows, 16) * K_pad / 2 would pass it)."""
    A16 = 1 << 20
    T = mx.MX_LAYOUT_TILED
    G = mx.mx_gemm_a4w4
    big, K = 1 << 20, 4096
    assert _status(G, 0, 1, big, 4, K, A16, A16, A16, A16, T, 0, A16, 8, 0) == mx.MX_ERR_UNSUPPORTED
    assert "2 GiB" in mx.mx_last_error() and "operand A" in mx.mx_last_error()
    assert _status(G, 0, 1, 4, big, K, A16, A16, A16, A16, T, 0, A16, big, 0) == mx.MX_ERR_UNSUPPORTED
    assert "operand B" in mx.mx_last_error()
    # one 16-row group less is below the limit: validation passes and the call
    # reaches the device check (which fails here for want of a GPU)
    assert _status(G, 0, 1, big - 16, 4, K, A16, A16, A16, A16, T, 0, A16, 8, 0) != mx.MX_ERR_UNSUPPORTED
    # FP6: 3/4 byte per element, FP8: one byte per element
    F6 = mx.mx_gemm_fp6
    assert _status(F6, 0, 1, 1 << 19, 4, 8192, mx.MX_FP6_E2M3, A16, A16, mx.MX_FP6_E2M3, A16, A16, T, 0,
                   A16, 8, 0) == mx.MX_ERR_UNSUPPORTED
    F8 = mx.mx_gemm_f8_tw
    assert _status(F8, 0, 1, 1 << 19, 4, 4096, A16, A16, A16, A16, T, 0, A16, 8, 0) == mx.MX_ERR_UNSUPPORTED
    assert _status(F8, 0, 1, (1 << 19) - 16, 4, 4096, A16, A16, A16, A16, T, 0, A16, 8, 0) != mx.MX_ERR_UNSUPPORTED


def test_host_objects_refused_as_device_pointers(L):
    """Device entry points refuse CPU tensors and numpy arrays before calling
    into the library (a kernel given a host address would fault the GPU); the
    host converter takes them."""
    import numpy as np
    torch = pytest.importorskip("torch")
    host_t = torch.zeros(64, dtype=torch.uint8)
    host_a = np.zeros(64, dtype=np.uint8)
    T = mx.MX_LAYOUT_TILED
    for bad in (host_t, host_a):
        with pytest.raises(TypeError, match="device pointer"):
            mx.mx_gemm_a4w4(0, 1, 4, 4, 4, bad, bad, bad, bad, T, 0, bad, 8, 0)
        with pytest.raises(TypeError, match="device pointer"):
            mx.mx_quantize_dual(bad, 4, 8, 8, None, None, T, bad, bad, bad, bad, 0)
    # ints pass through untouched (validation then answers for them)
    with pytest.raises(mx.MXError):
        mx.mx_gemm_a4w4(0, 0, 4, 4, 4, 1 << 20, 1 << 20, 1 << 20, 1 << 20, T, 0, 1 << 20, 8, 0)


def test_measure_mfma_validation(L):
    A16 = 1 << 20
    M = mx.mx_measure_mfma
    assert _status(M, 5, 4, A16, 4, 10, A16, 0) == mx.MX_ERR_UNSUPPORTED
    assert _status(M, 4, -1, A16, 4, 10, A16, 0) == mx.MX_ERR_UNSUPPORTED
    assert _status(M, 4, 4, 0, 4, 10, A16, 0) == mx.MX_ERR_INVALID_ARGUMENT
    assert _status(M, 4, 4, A16, 0, 10, A16, 0) == mx.MX_ERR_INVALID_ARGUMENT
    assert _status(M, 4, 4, A16, 4, 0, A16, 0) == mx.MX_ERR_INVALID_ARGUMENT
    assert _status(M, 4, 4, A16 + 4, 4, 10, A16, 0) == mx.MX_ERR_MISALIGNED


def test_dequantize_validation(L):
    A16 = 1 << 20
    assert _status(mx.mx_dequantize, A16, A16, -1, 4, 0, A16, 4, 0) == mx.MX_ERR_INVALID_ARGUMENT
    assert _status(mx.mx_dequantize, A16, A16, 2, 8, 0, A16, 4, 0) == mx.MX_ERR_INVALID_ARGUMENT
    assert _status(mx.mx_dequantize, A16, A16, 0, 8, 0, A16, 8, 0) == mx.MX_SUCCESS


@pytest.mark.parametrize("rows,length", [(1, 1), (37, 640), (40, 700), (16, 512), (100, 3000)])
def test_host_layout_convert_matches_oracle(L, oracle_mod, rows, length):
    x = synth.random_bf16(rows * 7 + length, (rows, length))
    q, s = oracle_mod.quantize(x, 0)
    qt_ref, st_ref = oracle_mod.to_tiled(q, s, rows, length)
    dt, sz = mx.mx_blob_bytes(rows, length, mx.MX_LAYOUT_TILED)
    qt = np.full(dt, 0xAB, np.uint8)
    st = np.full(sz, 0xCD, np.uint8)
    mx.mx_layout_convert_host(1, rows, length, q, s, qt, st)
    assert (qt == qt_ref).all() and (st == st_ref).all()
    q2 = np.zeros_like(q)
    s2 = np.zeros_like(s)
    mx.mx_layout_convert_host(0, rows, length, qt, st, q2, s2)
    assert (q2 == q).all() and (s2 == s).all()


def test_device_layout_convert_validation(L):
    A16 = 1 << 20
    C = mx.mx_layout_convert
    assert _status(C, 1, -1, 8, A16, A16, A16, A16, 0) == mx.MX_ERR_INVALID_ARGUMENT
    assert _status(C, 1, 4, 8, 0, A16, A16, A16, 0) == mx.MX_ERR_INVALID_ARGUMENT
    assert _status(C, 0, 4, 8, A16, A16, A16, 0, 0) == mx.MX_ERR_INVALID_ARGUMENT
    assert _status(C, 1, 4, 8, A16 + 4, A16, A16, A16, 0) == mx.MX_ERR_MISALIGNED
    assert _status(C, 1, 4, 8, A16, A16, A16 + 8, A16, 0) == mx.MX_ERR_MISALIGNED
    assert _status(C, 1, 4, 8, A16, A16 + 4, A16, A16, 0) == mx.MX_ERR_MISALIGNED
    assert _status(C, 0, 4, 8, A16, A16, A16, A16 + 1, 0) == mx.MX_ERR_MISALIGNED
    assert _status(C, 1, 0, 8, A16, A16, A16, A16, 0) == mx.MX_SUCCESS


def test_device_supported_without_gpu(L):
    # no GPU in a CPU-only container: the query reports unsupported instead of crashing
    if _gpu_present():
        pytest.skip("GPU present")
    assert mx.mx_device_supported(0) is False


def _every_launching_call(A16):
    """One valid-argument call of every entry point that launches work."""
    T = mx.MX_LAYOUT_TILED
    o = mx.quant_opts()
    return {
        "mx_quantize_rowwise": lambda: mx.mx_quantize_rowwise(A16, 4, 8, 8, o, T, A16, A16, 0),
        "mx_quantize_dual": lambda: mx.mx_quantize_dual(A16, 4, 8, 8, o, o, T, A16, A16, A16, A16, 0),
        "mx_quantize_dual_mul": lambda: mx.mx_quantize_dual_mul(A16, A16, 4, 8, 8, 8, o, o, T, A16, A16, A16,
                                                                A16, 0),
        "mx_gemm_a4w4": lambda: mx.mx_gemm_a4w4(0, 1, 4, 8, 128, A16, A16, A16, A16, T, mx.MX_BF16, A16, 8, 0),
        "mx_gemm_a4w4_bias": lambda: mx.mx_gemm_a4w4_bias(0, 1, 4, 8, 128, A16, A16, A16, A16, T, mx.MX_F32, A16,
                                                          A16, 8, 0),
        "mx_quantize_fp6": lambda: mx.mx_quantize_fp6(A16, 4, 8, 8, mx.MX_FP6_E2M3, o, mx.MX_FP6_E3M2, o, T, A16,
                                                      A16, A16, A16, 0),
        "mx_gemm_fp6": lambda: mx.mx_gemm_fp6(0, 1, 4, 8, 128, mx.MX_FP6_E2M3, A16, A16, mx.MX_FP6_E3M2, A16, A16,
                                              T, mx.MX_BF16, A16, 8, 0),
        "mx_quantize_fp8_tw": lambda: mx.mx_quantize_fp8_tw(A16, 4, 8, 8, T, A16, A16, A16, 0),
        "mx_gemm_f8_tw": lambda: mx.mx_gemm_f8_tw(0, 1, 4, 8, 128, A16, A16, A16, A16, T, mx.MX_BF16, A16, 8, 0),
        "mx_layout_convert": lambda: mx.mx_layout_convert(1, 4, 8, A16, A16, A16, A16, 0),
        "mx_dequantize": lambda: mx.mx_dequantize(A16, A16, 4, 8, T, A16, 8, 0),
        "mx_measure_mfma": lambda: mx.mx_measure_mfma(4, 4, A16, 1, 1, A16, 0),
    }


def test_forced_unsupported_device(L):
    """The device check of every launching entry point, forced to see another
    architecture through the query hook: MX_ERR_DEVICE_UNSUPPORTED naming it,
    after validation and before any launch (fail loudly, as the page
    "primus_turbo_mxfp4_local.py" has check_mxfp4_support() refuse to build
    an FP4 layer on an unsupported device)."""
    try:
        mx.mx_set_device_arch_override("gfx942")
        assert mx.mx_device_supported(0) is False and mx.mx_device_supported(5) is False
        for name, call in _every_launching_call(1 << 20).items():
            with pytest.raises(mx.MXError) as e:
                call()
            assert e.value.status == mx.MX_ERR_DEVICE_UNSUPPORTED, name
            assert "gfx942" in mx.mx_last_error(), name
        # validation still answers first
        assert _status(mx.mx_quantize_rowwise, 0, 4, 8, 8, None, 1, 1 << 20, 1 << 20, 0) == \
            mx.MX_ERR_INVALID_ARGUMENT
        mx.mx_set_device_arch_override("gfx950:sramecc+:xnack-")
        assert mx.mx_device_supported(0) is True
        mx.mx_set_device_arch_override("gfx9500")
        assert mx.mx_device_supported(0) is False
        with pytest.raises(mx.MXError) as e:
            mx.mx_set_device_arch_override("g" * 64)
        assert e.value.status == mx.MX_ERR_INVALID_ARGUMENT
    finally:
        mx.mx_set_device_arch_override("gfx000" if _gpu_present() else None)


def test_forced_launch_failure_reports_hip_error(L):
    """With the device check forced to pass on a machine whose runtime has no
    device, every launching entry point gets as far as the launch, which
    fails: MX_ERR_HIP with HIP's own error text, no crash, no fallback."""
    if _gpu_present():
        pytest.skip("needs a machine without a GPU (the fake addresses would reach a real launch)")
    try:
        mx.mx_set_device_arch_override("gfx950")
        assert mx.mx_device_supported(0) is True
        for name, call in _every_launching_call(1 << 20).items():
            with pytest.raises(mx.MXError) as e:
                call()
            assert e.value.status == mx.MX_ERR_HIP, name
            msg = mx.mx_last_error()
            assert "launch failed" in msg and name in msg, (name, msg)
    finally:
        mx.mx_set_device_arch_override(None)


def test_fp8_validation_and_sizes(L):
    A16 = 1 << 20
    assert mx.mx_fp8_blob_bytes(37, 200, mx.MX_LAYOUT_CANONICAL) == 37 * 256
    assert mx.mx_fp8_blob_bytes(37, 200, mx.MX_LAYOUT_TILED) == 48 * 256
    Q = mx.mx_quantize_fp8_tw
    assert _status(Q, A16, 4, 8, 8, 1, 0, 0, A16, 0) == mx.MX_ERR_INVALID_ARGUMENT      # no output
    assert _status(Q, A16, 4, 8, 8, 1, A16, 0, 0, 0) == mx.MX_ERR_INVALID_ARGUMENT      # info NULL
    assert _status(Q, A16, 4, 8, 8, 1, A16 + 4, 0, A16, 0) == mx.MX_ERR_MISALIGNED
    assert _status(Q, A16, 4, 8, 8, 7, A16, 0, A16, 0) == mx.MX_ERR_UNSUPPORTED
    assert _status(Q, A16, 0, 8, 8, 1, A16, 0, A16, 0) == mx.MX_SUCCESS
    G = mx.mx_gemm_f8_tw
    assert _status(G, 0, 0, 4, 4, 4, A16, A16, A16, A16, 1, 0, A16, 8, 0) == mx.MX_ERR_UNSUPPORTED
    assert _status(G, 0, 1, 4, 4, 4, A16, 0, A16, A16, 1, 0, A16, 8, 0) == mx.MX_ERR_INVALID_ARGUMENT
    assert _status(G, 0, 1, 4, 4, 4, A16, A16, A16, A16, 0, 0, A16, 8, 0) == mx.MX_ERR_UNSUPPORTED
    assert _status(G, 0, 1, 4, 4, 4, A16, A16, A16, A16, 1, 0, A16, 12, 0) == mx.MX_ERR_MISALIGNED
    assert _status(G, 0, 1, 0, 4, 4, A16, A16, A16, A16, 1, 0, A16, 8, 0) == mx.MX_SUCCESS


def test_fp6_validation_and_sizes(L):
    A16 = 1 << 20
    C, T = mx.MX_LAYOUT_CANONICAL, mx.MX_LAYOUT_TILED
    assert mx.mx_fp6_blob_bytes(37, 200, C) == (37 * 192, 37 * 8)
    assert mx.mx_fp6_blob_bytes(37, 200, T) == (48 * 192, 48 * 16)
    Q = mx.mx_quantize_fp6
    o = mx.quant_opts()
    no_device = (mx.MX_ERR_DEVICE_UNSUPPORTED, mx.MX_ERR_HIP)     # valid arguments reach the device check
    assert _status(Q, A16, 4, 8, 8, 2, o, 3, o, T, A16, A16, A16, A16, 0) in no_device
    assert _status(Q, A16, 4, 8, 8, 4, o, 3, o, T, A16, A16, A16, A16, 0) == mx.MX_ERR_UNSUPPORTED
    assert _status(Q, A16, 4, 8, 8, 2, o, 1, o, T, A16, A16, A16, A16, 0) == mx.MX_ERR_UNSUPPORTED
    assert _status(Q, A16, 4, 8, 8, 2, o, 1, o, T, A16, A16, None, None, 0) in no_device   # col fmt unused
    assert _status(Q, A16, 4, 8, 8, 2, mx.quant_opts(rht=5), 3, o, T, A16, A16, None, None, 0) == \
        mx.MX_ERR_UNSUPPORTED
    assert _status(Q, A16, 4, 8, 8, 2, o, 3, o, T, A16 + 8, A16, None, None, 0) == mx.MX_ERR_MISALIGNED
    assert _status(Q, A16, 4, 8, 8, 2, o, 3, o, T, A16, A16, A16, None, 0) == mx.MX_ERR_INVALID_ARGUMENT
    assert _status(Q, A16, 4, 8, 8, 2, o, 3, o, 5, A16, A16, None, None, 0) == mx.MX_ERR_UNSUPPORTED
    assert _status(Q, A16, 0, 8, 8, 2, o, 3, o, T, A16, A16, None, None, 0) == mx.MX_SUCCESS


def test_multiply_prologue_validation(L):
    A16 = 1 << 20
    T = mx.MX_LAYOUT_TILED
    Q = mx.mx_quantize_dual_mul
    o = mx.quant_opts()
    no_device = (mx.MX_ERR_DEVICE_UNSUPPORTED, mx.MX_ERR_HIP)
    assert _status(Q, A16, A16, 4, 8, 8, 8, o, o, T, A16, A16, A16, A16, 0) in no_device
    assert _status(Q, A16, 0, 4, 8, 8, 8, o, o, T, A16, A16, A16, A16, 0) == mx.MX_ERR_INVALID_ARGUMENT
    assert _status(Q, A16, A16 + 2, 4, 8, 8, 8, o, o, T, A16, A16, A16, A16, 0) == mx.MX_ERR_MISALIGNED
    assert _status(Q, A16, A16, 4, 8, 8, 12, o, o, T, A16, A16, A16, A16, 0) == mx.MX_ERR_MISALIGNED
    assert _status(Q, A16, A16, 4, 8, 8, 4, o, o, T, A16, A16, A16, A16, 0) == mx.MX_ERR_INVALID_ARGUMENT
    assert _status(Q, A16, A16, 4, 8, 8, 8, mx.quant_opts(rht=3), o, T, A16, A16, A16, A16, 0) == \
        mx.MX_ERR_UNSUPPORTED
    assert _status(Q, A16, A16, 4, 8, 8, 8, o, o, T, A16, A16, None, None, 0) in no_device
    assert _status(Q, A16, A16, 0, 8, 8, 8, o, o, T, A16, A16, None, None, 0) == mx.MX_SUCCESS
