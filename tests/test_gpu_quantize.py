"""GPU parity of the quantizers: bytes and scales bit-exact against the oracle.

Canonical-layout outputs are compared with the oracle's canonical blobs;
tiled-layout outputs with the oracle's own tiled permutation of them.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mxfp4_precision_amd as mx
from mxfp4_precision_amd import synth

import input_digests
from gpu_util import canon_shape, host, log, quantize_dual, quantize_rowwise, to_dev_bf16

pytestmark = pytest.mark.gpu

CANON, TILED = mx.MX_LAYOUT_CANONICAL, mx.MX_LAYOUT_TILED


def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def assert_equal_bytes(got, want, what):
    got = np.asarray(got).ravel()
    want = np.asarray(want).ravel()
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "%s: %d bytes differ, first at %s: got %s want %s" % (
        what, bad.size, bad[:5].tolist(), got[bad[:5]].tolist(), want[bad[:5]].tolist())


def check_rowwise(oracle_mod, x, layout, opts=None, okw=None, ldx=None):
    M, N = x.shape
    xd, ldx = to_dev_bf16(x, ldx)
    q, s = quantize_rowwise(xd, M, N, ldx, layout, opts)
    qw, sw = oracle_mod.quantize(x, 0, **(okw or {}))
    q, s = host(q), host(s)
    if layout == CANON:
        qg, sg = canon_shape(oracle_mod, M, N, q, s)
    else:
        qg, sg = q, s
        qw, sw = oracle_mod.to_tiled(qw, sw, M, N)
    assert_equal_bytes(qg, qw, "row data %s" % (x.shape,))
    assert_equal_bytes(sg, sw, "row scale %s" % (x.shape,))


def check_dual(oracle_mod, x, layout, row_opts=None, col_opts=None, rkw=None, ckw=None, ldx=None):
    M, N = x.shape
    xd, ldx = to_dev_bf16(x, ldx)
    qr, sr, qc, sc = quantize_dual(xd, M, N, ldx, layout, row_opts, col_opts)
    qrw, srw = oracle_mod.quantize(x, 0, **(rkw or {}))
    qcw, scw = oracle_mod.quantize(x, 1, **(ckw or {}))
    qr, sr, qc, sc = host(qr), host(sr), host(qc), host(sc)
    if layout == CANON:
        qr, sr = canon_shape(oracle_mod, M, N, qr, sr)
        qc, sc = canon_shape(oracle_mod, N, M, qc, sc)
    else:
        qrw, srw = oracle_mod.to_tiled(qrw, srw, M, N)
        qcw, scw = oracle_mod.to_tiled(qcw, scw, N, M)
    assert_equal_bytes(qr, qrw, "dual row data %s" % (x.shape,))
    assert_equal_bytes(sr, srw, "dual row scale %s" % (x.shape,))
    assert_equal_bytes(qc, qcw, "dual col data %s" % (x.shape,))
    assert_equal_bytes(sc, scw, "dual col scale %s" % (x.shape,))


SHAPES = [(1, 1), (1, 8), (33, 70), (127, 129), (128, 128), (200, 1000), (256, 512), (300, 136)]


@pytest.mark.parametrize("layout", [CANON, TILED])
@pytest.mark.parametrize("shape", SHAPES)
def test_rowwise_ragged(oracle_mod, layout, shape):
    _require_gpu()
    log("rowwise %s layout %d" % (shape, layout))
    x = synth.random_bf16(100 + shape[0] + shape[1], shape, std=1.5)
    check_rowwise(oracle_mod, x, layout)


@pytest.mark.parametrize("layout", [CANON, TILED])
@pytest.mark.parametrize("shape", SHAPES)
def test_dual_ragged(oracle_mod, layout, shape):
    _require_gpu()
    log("dual %s layout %d" % (shape, layout))
    x = synth.random_bf16(200 + shape[0] + shape[1], shape, std=0.7)
    check_dual(oracle_mod, x, layout)


@pytest.mark.parametrize("layout", [CANON, TILED])
def test_strided_input(oracle_mod, layout):
    _require_gpu()
    x = synth.random_bf16(5, (70, 100))
    check_rowwise(oracle_mod, x, layout, ldx=136)
    check_dual(oracle_mod, x, layout, ldx=104)


@pytest.mark.parametrize("layout", [CANON, TILED])
def test_tiny_workload(oracle_mod, layout):
    """256x512 and 384x512 N(0,1), seed 0, row-wise RNE."""
    _require_gpu()
    d = synth.tiny()
    check_rowwise(oracle_mod, d["A"], layout)
    check_rowwise(oracle_mod, d["W"], layout)


@pytest.mark.parametrize("layout", [CANON, TILED])
def test_dual_4600x3072_outliers_zero_tiles(oracle_mod, layout):
    """The 4600x3072 dual-quantize workload (seed 1): 128-padding of M, outliers, zero tiles."""
    _require_gpu()
    log("dual 4600x3072 layout %d" % layout)
    x = synth.dual()["X"]
    check_dual(oracle_mod, x, layout)


def test_special_values(oracle_mod):
    _require_gpu()
    x = synth.random_bf16(9, (96, 256), std=1.0)
    x[0, 5] = 0x7F80        # +Inf
    x[1, 40] = 0xFFC0       # NaN
    x[40, 100] = 0xFF80     # -Inf (column block too)
    x[2, :32] = 0x8000      # -0 block
    x[3, 32:64] = 0x0001    # subnormal block (amax subnormal -> scale 0)
    x[4, 64:96] = np.array([0x0080 + k for k in range(32)], dtype=np.uint16)  # min-normal region
    x[5, :] = 0x7F7F        # bf16 max
    x[6, 0] = 0x0001
    x[6, 1:32] = 0
    x[64:96, 200:232] = 0   # zero 32x32 tile
    for layout in (CANON, TILED):
        check_dual(oracle_mod, x, layout)


def test_exhaustive_element_sweep(oracle_mod):
    """Every finite bf16 magnitude at every scale that can hold it (the oracle's brute-force
    sweep, here through the GPU row-wise kernel), both signs."""
    _require_gpu()
    mags = np.arange(0x7F80, dtype=np.uint16)
    mval = (mags.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    blocks = []
    for e in range(-127, 126):
        sel = mval < 8.0 * 2.0 ** e
        if e > -120:
            sel &= mval >= 2.0 ** (e - 10)
        xs = mags[sel]
        xs = np.concatenate([xs, xs | np.uint16(0x8000)])
        per = 31
        nrow = -(-xs.size // per)
        blk = np.zeros((nrow, 32), dtype=np.uint16)
        blk[:, 0] = synth.bf16_bits(np.float32(4.0 * 2.0 ** e))
        flat = np.zeros(nrow * per, dtype=np.uint16)
        flat[: xs.size] = xs
        blk[:, 1:] = flat.reshape(nrow, per)
        blocks.append(blk)
    X = np.concatenate(blocks)
    log("exhaustive sweep rows %d" % X.shape[0])
    check_rowwise(oracle_mod, X, CANON)
    check_dual(oracle_mod, X[:4096], CANON)


def _special_tensor(seed, shape):
    x = synth.random_bf16(seed, shape, std=1.0)
    x[0, 5] = 0x7F80        # +Inf
    x[1, 40] = 0xFFC0       # NaN
    x[40, 100] = 0xFF80     # -Inf (column block too)
    x[2, :32] = 0x8000      # -0 block
    x[3, 32:64] = 0x0001    # subnormal block (amax subnormal -> scale 0)
    x[4, 64:96] = np.array([0x0080 + k for k in range(32)], dtype=np.uint16)  # min-normal region
    x[5, :] = 0x7F7F        # bf16 max
    x[6, 0] = 0x0001
    x[6, 1:32] = 0
    x[64:96, 200:232] = 0   # zero 32x32 tile
    return x


@pytest.mark.parametrize("layout", [CANON, TILED])
def test_special_values_stochastic(oracle_mod, layout):
    """The special blocks of test_special_values with stochastic rounding in both
    directions: Inf/NaN blocks (scale 0xFF, zero codes), -0, subnormal amax
    (scale 0), bf16 max; N = 256 takes the paired Philox path, N = 250 the
    unpaired one."""
    _require_gpu()
    sr = mx.quant_opts(use_sr=True, seed=11, tensor_id=4)
    kw = dict(use_sr=True, seed=11, tensor_id=4)
    x = _special_tensor(9, (96, 256))
    check_dual(oracle_mod, x, layout, sr, sr, kw, kw)
    check_dual(oracle_mod, np.ascontiguousarray(x[:, :250]), layout, sr, sr, kw, kw)


def test_exhaustive_element_sweep_stochastic(oracle_mod):
    """Every finite bf16 magnitude at every scale that can hold it, both signs,
    with stochastic rounding: row-wise over the whole sweep, dual on a slice
    (paired Philox path), and row-wise on a slice 31 columns wide (unpaired)."""
    _require_gpu()
    mags = np.arange(0x7F80, dtype=np.uint16)
    mval = (mags.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    blocks = []
    for e in range(-127, 126):
        sel = mval < 8.0 * 2.0 ** e
        if e > -120:
            sel &= mval >= 2.0 ** (e - 10)
        xs = mags[sel]
        xs = np.concatenate([xs, xs | np.uint16(0x8000)])
        per = 31
        nrow = -(-xs.size // per)
        blk = np.zeros((nrow, 32), dtype=np.uint16)
        blk[:, 0] = synth.bf16_bits(np.float32(4.0 * 2.0 ** e))
        flat = np.zeros(nrow * per, dtype=np.uint16)
        flat[: xs.size] = xs
        blk[:, 1:] = flat.reshape(nrow, per)
        blocks.append(blk)
    X = np.tile(np.concatenate(blocks), (1, 2))     # 64 columns: two blocks per row
    sr = mx.quant_opts(use_sr=True, seed=5, tensor_id=3)
    kw = dict(use_sr=True, seed=5, tensor_id=3)
    log("exhaustive SR sweep rows %d" % X.shape[0])
    check_rowwise(oracle_mod, X, CANON, sr, kw)
    check_dual(oracle_mod, X[:4096], CANON, sr, sr, kw, kw)
    check_rowwise(oracle_mod, np.ascontiguousarray(X[:, :31]), CANON, sr, kw)


@pytest.mark.parametrize("layout", [CANON, TILED])
def test_stochastic_rounding(oracle_mod, layout):
    """SR with Philox bytes keyed by (seed, tensor_id, direction, element index), both directions."""
    _require_gpu()
    x = synth.random_bf16(17, (192, 384), std=1e-3)
    ro = mx.quant_opts(use_sr=True, seed=7, tensor_id=2)
    kw = dict(use_sr=True, seed=7, tensor_id=2)
    check_dual(oracle_mod, x, layout, ro, ro, kw, kw)
    # a 64-bit seed, a large index_base and an unaligned width (N % 16 != 0)
    x2 = synth.random_bf16(18, (70, 200), std=2.0)
    o2 = mx.quant_opts(use_sr=True, seed=(5 << 40) | 123, tensor_id=9, index_base=(1 << 33) + 5)
    kw2 = dict(use_sr=True, seed=(5 << 40) | 123, tensor_id=9, index_base=(1 << 33) + 5)
    check_rowwise(oracle_mod, x2, layout, o2, kw2)
    check_dual(oracle_mod, x2, layout, o2, o2, kw2, kw2)


@pytest.mark.parametrize("layout", [CANON, TILED])
def test_2d_blocks(oracle_mod, layout):
    """32x32 2D blocks in both directions (the weight recipe), including ragged edge tiles."""
    _require_gpu()
    for shape in [(96, 160), (100, 70), (3072 // 16, 12288 // 16)]:
        x = synth.random_bf16(19 + shape[0], shape, std=0.02)
        o = mx.quant_opts(use_2d_block=True)
        check_dual(oracle_mod, x, layout, o, o, dict(use_2d=True), dict(use_2d=True))
        check_rowwise(oracle_mod, x, layout, o, dict(use_2d=True))


def test_mixed_direction_options(oracle_mod):
    """Row RNE with column SR, and row 2D with column 1D."""
    _require_gpu()
    x = synth.random_bf16(23, (130, 260))
    sr = mx.quant_opts(use_sr=True, seed=3, tensor_id=1)
    check_dual(oracle_mod, x, TILED, None, sr, {}, dict(use_sr=True, seed=3, tensor_id=1))
    d2 = mx.quant_opts(use_2d_block=True)
    check_dual(oracle_mod, x, CANON, d2, None, dict(use_2d=True), {})


def test_fc2_full_size_dual(oracle_mod):
    """Full-size 18432x12288 GELU activation (seed 4), dual, tiled layout, every byte."""
    _require_gpu()
    log("fc2 X 18432x12288 dual")
    d = synth.fc2()
    input_digests.check("fc2", d)
    x = d["X"]
    check_dual(oracle_mod, x, TILED)


def test_fc2_full_size_sr_and_2d(oracle_mod):
    """Full-size fc2 dY (SR, seed 7, id 2) and W (2D) in the tiled layout."""
    _require_gpu()
    d = synth.fc2()
    sr = mx.quant_opts(use_sr=True, seed=7, tensor_id=2)
    log("fc2 dY 18432x3072 SR dual")
    check_dual(oracle_mod, d["dY"], TILED, sr, sr, dict(use_sr=True, seed=7, tensor_id=2),
               dict(use_sr=True, seed=7, tensor_id=2))
    w2 = mx.quant_opts(use_2d_block=True, tensor_id=1)
    log("fc2 W 3072x12288 2D dual")
    check_dual(oracle_mod, d["W"], TILED, w2, w2, dict(use_2d=True, tensor_id=1), dict(use_2d=True, tensor_id=1))


def test_device_dequantize(oracle_mod):
    _require_gpu()
    x = synth.random_bf16(29, (50, 300), std=4.0)
    for layout in (CANON, TILED):
        xd, ldx = to_dev_bf16(x)
        q, s = quantize_rowwise(xd, 50, 300, ldx, layout)
        out = torch.empty((50, 304), dtype=torch.float32, device="cuda")
        mx.mx_dequantize(q, s, 50, 300, layout, out, 304)
        got = host(out)[:, :300].astype(np.float64)
        qw, sw = oracle_mod.quantize(x, 0)
        want = oracle_mod.dequantize(qw, sw, 50, 300)[:, :300]
        assert (got == want).all()


@pytest.mark.parametrize("layout", [CANON, TILED])
def test_stochastic_rounding_distinct_direction_keys(oracle_mod, layout):
    """Both directions stochastic with different seeds, tensor ids and index bases
    (multiples of 16, so lane pairs share Philox blocks), plus a 2D row direction."""
    _require_gpu()
    x = synth.random_bf16(24, (160, 256), std=0.3)
    ro = mx.quant_opts(use_sr=True, seed=11, tensor_id=4, index_base=32)
    co = mx.quant_opts(use_sr=True, seed=(9 << 35) + 3, tensor_id=5, index_base=4096)
    rkw = dict(use_sr=True, seed=11, tensor_id=4, index_base=32)
    ckw = dict(use_sr=True, seed=(9 << 35) + 3, tensor_id=5, index_base=4096)
    check_dual(oracle_mod, x, layout, ro, co, rkw, ckw)
    ro2 = mx.quant_opts(use_sr=True, use_2d_block=True, seed=11, tensor_id=4)
    check_dual(oracle_mod, x, layout, ro2, co, dict(use_sr=True, use_2d=True, seed=11, tensor_id=4), ckw)


@pytest.mark.parametrize("rows,length", [(1, 1), (37, 640), (40, 700), (16, 512), (333, 3000)])
def test_device_layout_convert(oracle_mod, rows, length):
    """Canonical -> tiled on the device equals the oracle's own permutation of
    the oracle's canonical blob (padding rows and scale slots written as 0 over
    a poisoned destination); tiled -> canonical gives the canonical blob back."""
    _require_gpu()
    x = synth.random_bf16(rows * 11 + length, (rows, length))
    q, s = oracle_mod.quantize(x, 0)
    qt_ref, st_ref = oracle_mod.to_tiled(q, s, rows, length)
    log("device layout convert %dx%d" % (rows, length))
    qd = torch.from_numpy(q.reshape(-1).copy()).cuda()
    sd = torch.from_numpy(s.reshape(-1).copy()).cuda()
    dt, sz = mx.mx_blob_bytes(rows, length, TILED)
    qt = torch.full((dt,), 0xAB, dtype=torch.uint8, device="cuda")
    st = torch.full((sz,), 0xCD, dtype=torch.uint8, device="cuda")
    mx.mx_layout_convert(1, rows, length, qd, sd, qt, st)
    assert (host(qt) == qt_ref).all() and (host(st) == st_ref).all()
    q2 = torch.full_like(qd, 0x5A)
    s2 = torch.full_like(sd, 0x5A)
    mx.mx_layout_convert(0, rows, length, qt, st, q2, s2)
    assert (host(q2) == q.reshape(-1)).all() and (host(s2) == s.reshape(-1)).all()


RHT_SHAPES = [(1, 1), (33, 70), (127, 129), (200, 1000), (300, 136)]


@pytest.mark.parametrize("layout", [CANON, TILED])
@pytest.mark.parametrize("shape", RHT_SHAPES)
def test_rht_column_wise(oracle_mod, layout, shape):
    """Random Hadamard transform on the column-wise blob (the recipe's wgrad
    operands), RNE, every byte against the oracle; ragged shapes put real
    elements and pads in one transformed block."""
    _require_gpu()
    x = synth.random_bf16(300 + shape[0] + shape[1], shape, std=1.0)
    col = mx.quant_opts(rht=0x1234)
    check_dual(oracle_mod, x, layout, None, col, None, dict(rht=0x1234))


@pytest.mark.parametrize("layout", [CANON, TILED])
@pytest.mark.parametrize("shape", RHT_SHAPES)
def test_rht_both_directions_stochastic(oracle_mod, layout, shape):
    """RHT on both blobs with stochastic rounding, different seeds per direction;
    an index base that is not a multiple of 16 (Philox windows straddle counters)."""
    _require_gpu()
    x = synth.random_bf16(400 + shape[0] + shape[1], shape, std=0.3)
    row = mx.quant_opts(use_sr=True, seed=5, tensor_id=2, index_base=7, rht=77)
    col = mx.quant_opts(use_sr=True, seed=6, tensor_id=2, index_base=7, rht=78)
    check_dual(oracle_mod, x, layout, row, col, dict(use_sr=True, seed=5, tensor_id=2, index_base=7, rht=77),
               dict(use_sr=True, seed=6, tensor_id=2, index_base=7, rht=78))


@pytest.mark.parametrize("layout", [CANON, TILED])
@pytest.mark.parametrize("shape", [(200, 80), (97, 160)])
def test_rht_stochastic_paired_lanes_with_pads(oracle_mod, layout, shape):
    """RHT and stochastic rounding on both blobs with N and both index bases
    multiples of 16 (neighbouring lanes share Philox blocks, one per
    direction), M and N short of the 128-padding: pad blocks of the row blob
    (columns past N) and pad rows of the column blob draw from their own
    counter space."""
    _require_gpu()
    x = synth.random_bf16(450 + shape[0] + shape[1], shape, std=0.3)
    row = mx.quant_opts(use_sr=True, seed=15, tensor_id=2, index_base=32, rht=91)
    col = mx.quant_opts(use_sr=True, seed=16, tensor_id=2, index_base=4096, rht=92)
    check_dual(oracle_mod, x, layout, row, col, dict(use_sr=True, seed=15, tensor_id=2, index_base=32, rht=91),
               dict(use_sr=True, seed=16, tensor_id=2, index_base=4096, rht=92))


def test_rht_rowwise_and_specials(oracle_mod):
    """Row-wise RHT through mx_quantize_rowwise, with Inf/NaN blocks (scale 0xFF,
    zero codes), signed zeros and large/small magnitudes in other blocks."""
    _require_gpu()
    x = synth.random_bf16(41, (96, 256), std=1.0)
    x[3, 5] = 0x7F80                   # +Inf
    x[40, 200] = 0xFFC0                # NaN
    x[70, 32:64] = 0x8000              # a block of -0
    x[80, 64:96] = synth.bf16_bits(np.full(32, 3e38, np.float32))
    x[90, 96:128] = synth.bf16_bits(np.full(32, 1e-38, np.float32))
    check_rowwise(oracle_mod, x, TILED, mx.quant_opts(rht=3), dict(rht=3))
    check_rowwise(oracle_mod, x, CANON, mx.quant_opts(use_sr=True, seed=9, rht=3), dict(use_sr=True, seed=9, rht=3))


def test_fc2_full_size_rht_recipe(oracle_mod):
    """The recipe's backward operands at full size: dY 18432x3072 dual with SR on
    both blobs and RHT on the column-wise one, every byte; then the wgrad GEMM of
    the RHT'd dY and X column-wise blobs (same sign seed) on sampled entries."""
    _require_gpu()
    d = synth.fc2()
    row = mx.quant_opts(use_sr=True, seed=7, tensor_id=2)
    col = mx.quant_opts(use_sr=True, seed=7, tensor_id=2, rht=0xABCD)
    log("fc2 dY 18432x3072 SR + column RHT")
    check_dual(oracle_mod, d["dY"], TILED, row, col, dict(use_sr=True, seed=7, tensor_id=2),
               dict(use_sr=True, seed=7, tensor_id=2, rht=0xABCD))
    # wgrad on a 2048-token slice: dW = dY^T X with both column blobs transformed
    T, din, dout = 2048, 12288, 3072
    g = np.ascontiguousarray(d["dY"][:T])
    xx = np.ascontiguousarray(d["X"][:T])
    gd, ldg = to_dev_bf16(g)
    xd, ldxx = to_dev_bf16(xx)
    _, _, gq, gs = quantize_dual(gd, T, dout, ldg, TILED, None, col)
    _, _, xq, xs = quantize_dual(xd, T, din, ldxx, TILED, None, mx.quant_opts(rht=0xABCD))
    C = torch.empty((dout, din), dtype=torch.float32, device="cuda")
    mx.mx_gemm_a4w4(0, 1, dout, din, T, gq, gs, xq, xs, TILED, mx.MX_F32, C, din)
    got = host(C)
    oqg, osg = oracle_mod.quantize(g, 1, use_sr=True, seed=7, tensor_id=2, rht=0xABCD)
    oqx, osx = oracle_mod.quantize(xx, 1, rht=0xABCD)
    rng = np.random.default_rng(3)
    ii, jj = rng.integers(0, dout, 2048), rng.integers(0, din, 2048)
    ref = oracle_mod.gemm_entries(oqg, osg, oqx, osx, dout, din, T, ii, jj)
    rel = np.linalg.norm(got[ii, jj] - ref) / np.linalg.norm(ref)
    assert rel <= 1e-5, rel


def check_mul(oracle_mod, x, g, layout, row_opts=None, col_opts=None, rkw=None, ckw=None, dual=True, ldx=None):
    """mx_quantize_dual_mul(x, g) against the oracle's quantization of bf16(fp32(x * g))."""
    M, N = x.shape
    xd, ldx = to_dev_bf16(x, ldx)
    gd, ldg = to_dev_bf16(g, (ldx or 8) + 8)
    qr, sr = mx.empty_blob(M, N, layout)
    qc = sc = None
    if dual:
        qc, sc = mx.empty_blob(N, M, layout)
    mx.mx_quantize_dual_mul(xd, gd, M, N, ldx, ldg, row_opts or mx.quant_opts(), col_opts or mx.quant_opts(), layout,
                            qr, sr, qc, sc)
    y = oracle_mod.bf16_mul(x, g)
    dirs = [(0, qr, sr, rkw, M, N)] + ([(1, qc, sc, ckw, N, M)] if dual else [])
    for d, q, s, kw, rows, length in dirs:
        qw, sw = oracle_mod.quantize(y, d, **(kw or {}))
        q, s = host(q), host(s)
        if layout == CANON:
            q, s = canon_shape(oracle_mod, rows, length, q, s)
        else:
            qw, sw = oracle_mod.to_tiled(qw, sw, rows, length)
        assert_equal_bytes(q, qw, "mul dir %d data %s" % (d, (M, N)))
        assert_equal_bytes(s, sw, "mul dir %d scale %s" % (d, (M, N)))


@pytest.mark.parametrize("layout", [CANON, TILED])
@pytest.mark.parametrize("shape", [(1, 1), (33, 70), (127, 129), (200, 1000), (300, 136)])
def test_multiply_prologue(oracle_mod, layout, shape):
    """Quantizer prologue: bf16(x * g) formed in the staging read, both blobs
    bit-exact against the oracle's quantization of the product; row-only too;
    g has its own row stride."""
    _require_gpu()
    log("mul prologue %s layout %d" % (shape, layout))
    x = synth.random_bf16(500 + shape[0], shape, std=1.0)
    g = synth.random_bf16(600 + shape[1], shape, std=0.7)
    check_mul(oracle_mod, x, g, layout)
    check_mul(oracle_mod, x, g, layout, dual=False)


@pytest.mark.parametrize("layout", [CANON, TILED])
def test_multiply_prologue_sr_2d_specials(oracle_mod, layout):
    """SR on both directions (paired Philox path), 2D blocks, and factors that
    make Inf, NaN (0 * Inf), subnormal and overflowing products."""
    _require_gpu()
    x = synth.random_bf16(77, (160, 256), std=0.3)
    g = synth.random_bf16(78, (160, 256), std=4.0)
    x[0, 3] = 0x7F80; g[0, 3] = 0x0000          # Inf * 0 = NaN
    x[1, 9] = 0x7F7F; g[1, 9] = 0x4000          # overflow to Inf
    x[2, :] = 0x0080; g[2, :] = 0x0100          # far below the fp32 normal range
    x[3, 40] = 0xFF80; g[3, 40] = 0x3F80        # -Inf
    ro = mx.quant_opts(use_sr=True, seed=11, tensor_id=4)
    co = mx.quant_opts(use_sr=True, seed=12, tensor_id=5)
    check_mul(oracle_mod, x, g, layout, ro, co, dict(use_sr=True, seed=11, tensor_id=4),
              dict(use_sr=True, seed=12, tensor_id=5))
    w2 = mx.quant_opts(use_2d_block=True)
    check_mul(oracle_mod, x, g, layout, w2, w2, dict(use_2d=True), dict(use_2d=True))


def test_tall_input_spans_launches(oracle_mod):
    """8,388,928 rows (65,539 tiles of 128 rows; grid dimension y holds at
    most 65,536 workgroups, so the launcher covers them with two launches,
    the second starting at tile 65,535) x 48 columns, dual, both directions
    with stochastic rounding (the paired Philox path), canonical layout.  The
    input is zero except three windows of seeded values: the first 256 rows,
    the 256 rows around the second launch's first row (8,388,480), and the
    last 192 rows (ragged, padded to 128).  Every window's row-blob rows and
    column-blob bytes and scales equal the oracle's dual quantize of the
    window alone with index_base moved to the window's first element; zero
    rows elsewhere encode to zero bytes."""
    _require_gpu()
    M, N, ldx = 65538 * 128 + 64, 48, 48
    base = 1 << 20
    wins = [(0, 256), (65535 * 128 - 128, 65535 * 128 + 128), (65538 * 128 - 128, M)]
    xd = torch.zeros((M, ldx), dtype=torch.int16, device="cuda")
    wx = []
    for k, (r0, r1) in enumerate(wins):
        w = synth.random_bf16(900 + k, (r1 - r0, N), std=1.0)
        xd[r0:r1] = torch.from_numpy(w.view(np.int16)).cuda()
        wx.append(w)
    o = mx.quant_opts(use_sr=True, seed=(3 << 33) + 17, tensor_id=6, index_base=base)
    log("tall input %dx%d: %d row tiles" % (M, N, -(-M // 128)))
    qr, sr, qc, sc = quantize_dual(xd, M, N, ldx, CANON, o, o)
    torch.cuda.synchronize()
    del xd
    M_pad = -(-M // 128) * 128
    qr, sr = qr.view(M, -1), sr.view(M, -1)
    qc, sc = qc.view(N, M_pad // 2), sc.view(N, M_pad // 32)
    for (r0, r1), w in zip(wins, wx):
        kw = dict(use_sr=True, seed=(3 << 33) + 17, tensor_id=6, index_base=base + r0 * N)
        qrw, srw = oracle_mod.quantize(w, 0, **kw)
        qcw, scw = oracle_mod.quantize(w, 1, **kw)
        what = "rows [%d, %d)" % (r0, r1)
        assert_equal_bytes(host(qr[r0:r1]), qrw, "tall row data " + what)
        assert_equal_bytes(host(sr[r0:r1]), srw, "tall row scale " + what)
        assert_equal_bytes(host(qc[:, r0 // 2: r0 // 2 + qcw.shape[1]]), qcw, "tall col data " + what)
        assert_equal_bytes(host(sc[:, r0 // 32: r0 // 32 + scw.shape[1]]), scw, "tall col scale " + what)
    # zero rows between the windows: zero codes and scale bytes everywhere
    for r in (256, 4_000_000, 65535 * 128 + 128, 65538 * 128 - 129):
        assert not host(qr[r]).any() and not host(sr[r]).any(), r
    assert not host(qc[:, 128:1_000_000]).any() and not host(sc[:, 8:60_000]).any()


# Per-direction option sets: every kernel instance of the MXFP4 quantizer
# (round-to-nearest or stochastic rounding per direction, with or without the
# Hadamard transform) and the 32x32 block option, which is a run-time choice.
_MODES = {
    "rne": dict(),
    "rne2d": dict(use_2d=True),
    "sr": dict(use_sr=True),
    "sr2d": dict(use_sr=True, use_2d=True),
    "rht": dict(rht=True),
    "rhtsr": dict(rht=True, use_sr=True),
}


def _mode_kwargs(mode, rng):
    """(device options, oracle keywords) for one direction's mode, with seeded
    random seeds, tensor ids, index bases and transform seeds."""
    m = _MODES[mode]
    kw = {}
    if m.get("use_2d"):
        kw["use_2d"] = True
    if m.get("use_sr"):
        kw.update(use_sr=True, seed=int(rng.integers(0, 2 ** 63)), tensor_id=int(rng.integers(0, 2 ** 32)),
                  index_base=int(rng.integers(0, 2 ** 40)))
    if m.get("rht"):
        kw["rht"] = int(rng.integers(1, 2 ** 32))
    dev = mx.quant_opts(use_2d_block=kw.get("use_2d", False), use_sr=kw.get("use_sr", False),
                        seed=kw.get("seed", 0), tensor_id=kw.get("tensor_id", 0),
                        index_base=kw.get("index_base", 0), rht=kw.get("rht", 0))
    return dev, kw


def _matrix_input(rng, case):
    M, N = int(rng.integers(1, 300)), int(rng.integers(1, 420))
    x = synth.random_bf16(1000 + case, (M, N), std=float(rng.choice([1e-3, 1.0, 50.0])))
    if case % 2:
        # non-finite values in some blocks: the waves holding them take the
        # general encode, the others the all-finite one
        for bits in (0x7F80, 0xFFC0, 0xFF80):
            x[int(rng.integers(0, M)), int(rng.integers(0, N))] = bits
    if case % 3 == 0 and M >= 32 and N >= 32:
        x[:32, :32] = 0                 # an all-zero block in both directions
    ldx = (N + 7) // 8 * 8 + 8 * int(rng.integers(0, 3))
    return x, ldx


@pytest.mark.parametrize("layout", [CANON, TILED])
def test_option_matrix_rowwise(oracle_mod, layout):
    """Row-wise quantize under every per-direction mode, on seeded ragged shapes
    with strided input and non-finite values in half the cases, bit-exact."""
    _require_gpu()
    rng = np.random.Generator(np.random.PCG64(71 + layout))
    for case, mode in enumerate(_MODES):
        x, ldx = _matrix_input(rng, case)
        dev, kw = _mode_kwargs(mode, rng)
        log("row matrix %s layout %d shape %s ldx %d" % (mode, layout, x.shape, ldx))
        check_rowwise(oracle_mod, x, layout, dev, kw, ldx=ldx)


@pytest.mark.parametrize("layout", [CANON, TILED])
def test_option_matrix_dual(oracle_mod, layout):
    """Dual quantize under every pair of per-direction modes (36 pairs: every
    dual kernel instance, each 32x32-block and transform combination across
    the two directions), seeded ragged shapes, strided input, non-finite values
    in half the cases; both blobs bit-exact."""
    _require_gpu()
    rng = np.random.Generator(np.random.PCG64(83 + layout))
    case = 0
    for rmode in _MODES:
        for cmode in _MODES:
            x, ldx = _matrix_input(rng, case)
            rdev, rkw = _mode_kwargs(rmode, rng)
            cdev, ckw = _mode_kwargs(cmode, rng)
            log("dual matrix %s/%s layout %d shape %s ldx %d" % (rmode, cmode, layout, x.shape, ldx))
            check_dual(oracle_mod, x, layout, rdev, cdev, rkw, ckw, ldx=ldx)
            case += 1


@pytest.mark.parametrize("layout", [CANON, TILED])
def test_option_matrix_multiply_prologue(oracle_mod, layout):
    """Quantizer prologue under every pair of per-direction modes without the
    transform (16 pairs, every dual prologue instance, stochastic rounding in
    one direction only included) and each mode row-wise only, seeded ragged
    shapes, strided inputs, non-finite factors in half the cases; bit-exact."""
    _require_gpu()
    rng = np.random.Generator(np.random.PCG64(89 + layout))
    modes = [m for m in _MODES if not _MODES[m].get("rht")]
    pairs = [(r, c) for r in modes for c in modes] + [(r, None) for r in modes]
    for case, (rmode, cmode) in enumerate(pairs):
        x, ldx = _matrix_input(rng, case)
        g = synth.random_bf16(3000 + case, x.shape, std=float(rng.choice([0.5, 4.0])))
        rdev, rkw = _mode_kwargs(rmode, rng)
        cdev, ckw = _mode_kwargs(cmode or "rne", rng)
        log("mul matrix %s/%s layout %d shape %s ldx %d" % (rmode, cmode, layout, x.shape, ldx))
        check_mul(oracle_mod, x, g, layout, rdev, cdev if cmode else None, rkw, ckw if cmode else None,
                  dual=cmode is not None, ldx=ldx)
