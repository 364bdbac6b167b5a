"""GPU parity of the MXFP6 path (OCP FP6 E2M3 / E3M2 elements, E8M0 block
scales): quantizer bytes bit-exact against the oracle in both layouts."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mxfp4_precision_amd as mx
from mxfp4_precision_amd import synth

from gpu_util import host, log, to_dev_bf16

pytestmark = pytest.mark.gpu

CANON, TILED = mx.MX_LAYOUT_CANONICAL, mx.MX_LAYOUT_TILED
E2M3, E3M2 = mx.MX_FP6_E2M3, mx.MX_FP6_E3M2


def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def fp6_blob(rows, length, layout):
    """Output buffers poisoned with 0xAB / 0xCD: every byte must be written."""
    d, s = mx.mx_fp6_blob_bytes(rows, length, layout)
    return (torch.full((max(d, 16),), 0xAB, dtype=torch.uint8, device="cuda"),
            torch.full((max(s, 16),), 0xCD, dtype=torch.uint8, device="cuda"))


def oracle_blob(oracle_mod, x, direction, fmt, layout, kw):
    q, s = oracle_mod.quantize_fp6(x, direction, fmt, **kw)
    rows, length = x.shape if direction == 0 else x.shape[::-1]
    if layout == TILED:
        return oracle_mod.fp6_to_tiled(q, s, rows, length)
    return q.reshape(-1), s.reshape(-1)


def assert_equal_bytes(got, want, what):
    got = np.asarray(got).ravel()[: np.asarray(want).size]
    want = np.asarray(want).ravel()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "%s: %d bytes differ, first at %s: got %s want %s" % (
        what, bad.size, bad[:5].tolist(), got[bad[:5]].tolist(), want[bad[:5]].tolist())


def check_fp6(oracle_mod, x, layout, row_fmt, col_fmt=None, rkw=None, ckw=None):
    """col_fmt None: row-wise only."""
    M, N = x.shape
    xd, ldx = to_dev_bf16(x)
    qr, sr = fp6_blob(M, N, layout)
    qc = sc = None
    if col_fmt is not None:
        qc, sc = fp6_blob(N, M, layout)
    mx.mx_quantize_fp6(xd, M, N, ldx, row_fmt, mx.quant_opts(**(rkw or {})), col_fmt or 0,
                       mx.quant_opts(**(ckw or {})), layout, qr, sr, qc, sc)
    okw = lambda kw: {k: v for k, v in (kw or {}).items() if k != "use_2d_block"} | (
        {"use_2d": True} if (kw or {}).get("use_2d_block") else {})
    qw, sw = oracle_blob(oracle_mod, x, 0, row_fmt, layout, okw(rkw))
    assert_equal_bytes(host(qr), qw, "row data %s fmt %d" % (x.shape, row_fmt))
    assert_equal_bytes(host(sr), sw, "row scale %s" % (x.shape,))
    d, s = mx.mx_fp6_blob_bytes(M, N, layout)
    assert (host(qr)[d:] == 0xAB).all() and (host(sr)[s:] == 0xCD).all()
    if col_fmt is not None:
        qw, sw = oracle_blob(oracle_mod, x, 1, col_fmt, layout, okw(ckw))
        assert_equal_bytes(host(qc), qw, "col data %s fmt %d" % (x.shape, col_fmt))
        assert_equal_bytes(host(sc), sw, "col scale %s" % (x.shape,))


SHAPES = [(1, 1), (33, 70), (127, 129), (128, 128), (200, 1000), (300, 136)]


@pytest.mark.parametrize("layout", [CANON, TILED])
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("fmt", [E2M3, E3M2])
def test_fp6_rowwise(oracle_mod, layout, shape, fmt):
    _require_gpu()
    log("fp6 rowwise %s fmt %d layout %d" % (shape, fmt, layout))
    x = synth.random_bf16(300 + shape[0] + shape[1], shape, std=2.0)
    check_fp6(oracle_mod, x, layout, fmt)


@pytest.mark.parametrize("layout", [CANON, TILED])
@pytest.mark.parametrize("shape", SHAPES)
def test_fp6_dual_mixed_formats(oracle_mod, layout, shape):
    _require_gpu()
    log("fp6 dual %s layout %d" % (shape, layout))
    x = synth.random_bf16(400 + shape[0] * 3 + shape[1], shape, std=0.05)
    check_fp6(oracle_mod, x, layout, E2M3, E3M2)
    check_fp6(oracle_mod, x, layout, E3M2, E2M3)


@pytest.mark.parametrize("layout", [CANON, TILED])
def test_fp6_stochastic_rounding(oracle_mod, layout):
    """Both directions stochastic (the paired-lane path: N and bases multiples of 16),
    then an odd width and a base off 16 (each lane draws its own bytes), plus 2D."""
    _require_gpu()
    x = synth.random_bf16(71, (160, 256), std=0.3)
    rk = dict(use_sr=True, seed=11, tensor_id=4, index_base=32)
    ck = dict(use_sr=True, seed=(9 << 35) + 3, tensor_id=5, index_base=4096)
    log("fp6 sr pairs layout %d" % layout)
    check_fp6(oracle_mod, x, layout, E3M2, E3M2, rk, ck)
    y = synth.random_bf16(72, (97, 200), std=0.3)
    log("fp6 sr ragged layout %d" % layout)
    check_fp6(oracle_mod, y, layout, E2M3, E3M2, dict(rk, index_base=5), ck)
    log("fp6 sr 2d layout %d" % layout)
    check_fp6(oracle_mod, x, layout, E2M3, E2M3, dict(rk, use_2d_block=True), dict(ck, use_2d_block=True))


@pytest.mark.parametrize("fmt", [E2M3, E3M2])
def test_fp6_specials_and_every_bf16(oracle_mod, fmt):
    """Every finite bf16 pattern once (blocks of mixed magnitudes), then Inf/NaN
    blocks, zeros, signed zeros and subnormal-range values."""
    _require_gpu()
    allbits = np.arange(0, 0x10000, dtype=np.uint16)
    allbits = allbits[((allbits >> 7) & 0xFF) != 0xFF]
    rng = np.random.default_rng(12)
    x = rng.permutation(allbits)[: (allbits.size // 512) * 512].reshape(-1, 512)
    log("fp6 all bf16 fmt %d" % fmt)
    check_fp6(oracle_mod, x, TILED, fmt, fmt)
    sp = synth.random_bf16(13, (64, 256), std=1.0)
    sp[0, 5] = 0x7F80; sp[1, 40] = 0xFF80; sp[2, 77] = 0x7FC1; sp[3, :] = 0x8000; sp[4, :32] = 0
    sp[5, :] = 0x0001; sp[6, 3] = 0x0080
    log("fp6 specials fmt %d" % fmt)
    check_fp6(oracle_mod, sp, CANON, fmt, fmt)
    check_fp6(oracle_mod, sp, TILED, fmt, fmt, dict(use_sr=True, seed=3), dict(use_sr=True, seed=4, tensor_id=1))
