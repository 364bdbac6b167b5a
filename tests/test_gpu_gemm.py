"""GPU parity of the block-scaled a4w4 GEMM against the oracle's fp64 NT product.

Bar (elementwise, bf16 output): |C - bf16(C_ref)| <= 2 ulp_bf16(max(|bf16(C_ref)|, tau)),
tau = (K_pad/32) 2^-24 sum_k |a_ik b_jk| (worst-case fp32 summation error of
exact per-block partial sums).  Bar (fp32 output): relative Frobenius error
<= 1e-5 against the fp64 reference.  Full-size shapes are checked on sampled
entries the oracle computes one by one, in the launch configuration the
benchmark times.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mxfp4_precision_amd as mx
from mxfp4_precision_amd import synth

from gpu_util import (check_gemm_bf16, gemm, host, log, quantize_dual, quantize_rowwise,
                      tau_bound, to_dev_bf16)

pytestmark = pytest.mark.gpu
TILED = mx.MX_LAYOUT_TILED


def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_case(oracle_mod, a_bits, b_bits, full=True, nsample=2048, seed=0, what=""):
    M, K = a_bits.shape
    N, K2 = b_bits.shape
    assert K == K2
    ad, lda = to_dev_bf16(a_bits)
    bd, ldb = to_dev_bf16(b_bits)
    qa, sa = quantize_rowwise(ad, M, K, lda, TILED)
    qb, sb = quantize_rowwise(bd, N, K, ldb, TILED)
    Cb = gemm(qa, sa, qb, sb, M, N, K, mx.MX_BF16)
    Cf = gemm(qa, sa, qb, sb, M, N, K, mx.MX_F32)
    cb = host(Cb)[:M, :N].view(np.uint16)
    cf = host(Cf)[:M, :N].astype(np.float64)
    oqa, osa = oracle_mod.quantize(a_bits, 0)
    oqb, osb = oracle_mod.quantize(b_bits, 0)
    if full:
        ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        ii, jj = ii.ravel(), jj.ravel()
    else:
        rng = np.random.default_rng(seed)
        ii = np.concatenate([rng.integers(0, M, nsample), [0, M - 1, M - 1, 0]])
        jj = np.concatenate([rng.integers(0, N, nsample), [0, N - 1, 0, N - 1]])
    ref = oracle_mod.gemm_entries(oqa, osa, oqb, osb, M, N, K, ii, jj)
    tau = tau_bound(oracle_mod, oqa, osa, oqb, osb, M, N, K, ii, jj)
    exact, tau_only = check_gemm_bf16(cb[ii, jj], ref, tau, oracle_mod, what)
    gotf = cf[ii, jj]
    rel = np.linalg.norm(gotf - ref) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= 1e-5, (what, rel)
    log("%s: %d/%d bf16 exact, %d tau-floor only, fp32 rel %.3g" % (what, exact, ii.size, tau_only, rel))
    return cb, cf


def test_tiny_workload(oracle_mod):
    """256x512 . (384x512)^T, seed 0, every entry."""
    _require_gpu()
    d = synth.tiny()
    run_case(oracle_mod, d["A"], d["W"], full=True, what="tiny")


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (17, 33, 129), (100, 70, 300), (128, 128, 128),
                                   (129, 257, 640), (64, 16, 2048), (250, 130, 900)])
def test_ragged(oracle_mod, M, N, K):
    _require_gpu()
    a = synth.random_bf16(M * 3 + K, (M, K), std=1.0)
    b = synth.random_bf16(N * 5 + K, (N, K), std=0.05)
    run_case(oracle_mod, a, b, full=True, what="ragged %dx%dx%d" % (M, N, K))


def test_k_zero_writes_zeros(oracle_mod):
    _require_gpu()
    C = torch.full((5, 8), 7, dtype=torch.int16, device="cuda")
    dummy = torch.zeros(16, dtype=torch.uint8, device="cuda")
    mx.mx_gemm_a4w4(0, 1, 5, 6, 0, dummy, dummy, dummy, dummy, TILED, mx.MX_BF16, C, 8)
    c = host(C)
    assert (c[:, :6] == 0).all() and (c[:, 6:] == 7).all()


def test_ldc_and_untouched_padding(oracle_mod):
    """C rows are written at stride ldc; columns N..ldc-1 stay untouched."""
    _require_gpu()
    a = synth.random_bf16(41, (40, 256))
    b = synth.random_bf16(42, (24, 256))
    ad, lda = to_dev_bf16(a)
    bd, ldb = to_dev_bf16(b)
    qa, sa = quantize_rowwise(ad, 40, 256, lda, TILED)
    qb, sb = quantize_rowwise(bd, 24, 256, ldb, TILED)
    C = gemm(qa, sa, qb, sb, 40, 24, 256, mx.MX_BF16, ldc=40)
    c = host(C)
    assert (c[:, 24:] == -1).all()
    C2 = gemm(qa, sa, qb, sb, 40, 24, 256, mx.MX_BF16)
    assert (host(C2)[:, :24] == c[:, :24]).all()


def test_special_scales(oracle_mod):
    """Outliers, zero blocks, scale-0 (tiny) blocks and saturated blocks in both operands."""
    _require_gpu()
    a = synth.random_bf16(43, (64, 512), std=1.0)
    b = synth.random_bf16(44, (48, 512), std=1.0)
    a[3, :32] = 0
    a[5, 100] = synth.bf16_bits(np.array([3e4], np.float32))[0]
    b[7, 200:232] = 0x0001
    b[9, :] = 0x7F7F >> 1
    run_case(oracle_mod, a, b, full=True, what="special scales")


def test_nan_scale_propagates(oracle_mod):
    """A NaN in an input block gives scale 0xFF; the affected outputs are NaN."""
    _require_gpu()
    a = synth.random_bf16(45, (32, 256))
    b = synth.random_bf16(46, (32, 256))
    a[4, 10] = 0x7FC0
    ad, lda = to_dev_bf16(a)
    bd, ldb = to_dev_bf16(b)
    qa, sa = quantize_rowwise(ad, 32, 256, lda, TILED)
    qb, sb = quantize_rowwise(bd, 32, 256, ldb, TILED)
    C = host(gemm(qa, sa, qb, sb, 32, 32, 256, mx.MX_F32))
    assert np.isnan(C[4, :32]).all()
    assert np.isfinite(np.delete(C[:, :32], 4, axis=0)).all()


def test_qkv_full_size_sampled(oracle_mod):
    """QKV forward 4608x3072 . (9216x3072)^T (seed 2), sampled entries."""
    _require_gpu()
    d = synth.qkv()
    log("qkv full size")
    run_case(oracle_mod, d["A"], d["W"], full=False, nsample=4096, what="qkv")


def test_many_tiles_ragged_and_repeatable(oracle_mod):
    """4500x4100 output = 306 tiles of 256x256 (more than one round on 256
    CUs, ragged last row and column of tiles) with K 700 -> 768 (a k-group
    whose second half is padding).  Sampled entries against the oracle, then
    two more calls must give bit-identical output."""
    _require_gpu()
    M, N, K = 4500, 4100, 700
    a = synth.random_bf16(71, (M, K), std=1.0)
    b = synth.random_bf16(72, (N, K), std=0.05)
    log("many tiles %dx%dx%d" % (M, N, K))
    cb, _ = run_case(oracle_mod, a, b, full=False, nsample=16384, what="many-tiles")
    ad, lda = to_dev_bf16(a)
    bd, ldb = to_dev_bf16(b)
    qa, sa = quantize_rowwise(ad, M, K, lda, TILED)
    qb, sb = quantize_rowwise(bd, N, K, ldb, TILED)
    for _ in range(2):
        again = host(gemm(qa, sa, qb, sb, M, N, K, mx.MX_BF16))[:M, :N].view(np.uint16)
        assert np.array_equal(again, cb)


_FC2 = {}


def _fc2_operands(which):
    if not _FC2:
        _FC2.update(synth.fc2())
    X, W, dY = _FC2["X"], _FC2["W"], _FC2["dY"]
    if which == "fwd":      # Y = X W^T: 18432 x 3072, K 12288
        return X, W
    if which == "dgrad":    # dX = dY W: 18432 x 12288, K 3072
        return dY, np.ascontiguousarray(W.T)
    return np.ascontiguousarray(dY.T), np.ascontiguousarray(X.T)   # dW = dY^T X: 3072 x 12288, K 18432


@pytest.mark.parametrize("which", ["fwd", "dgrad", "wgrad"])
def test_fc2_full_size_sampled(oracle_mod, which):
    """The three GEMMs of the fc2 training step at full size (18432 tokens,
    12288 -> 3072), sampled entries, in the launch configuration the benchmark
    times (864, 3456 and 576 output tiles).  Every entry of the bf16 output
    (persistent kernel plus tail kernel, 96, 24 and 144 k-steps per tile, the
    last being the longest K the persistent kernel takes) equals the
    round-to-nearest-even of the fp32 output (one tile per workgroup, the
    same accumulation order)."""
    _require_gpu()
    a, b = _fc2_operands(which)
    log("fc2 %s %dx%dx%d" % (which, a.shape[0], b.shape[0], a.shape[1]))
    cb, cf = run_case(oracle_mod, a, b, full=False, nsample=4096, seed=5, what="fc2-" + which)
    bad = np.count_nonzero(cb != _rne_bf16_bits(cf))
    assert bad == 0, ("fc2-" + which, bad)
    log("fc2-%s: all %d bf16 entries equal RNE of the fp32 output" % (which, cb.size))


def gemm_bias(A, As, B, Bs, M, N, K, bias, out_dtype=mx.MX_BF16):
    ldc = (N + 7) // 8 * 8
    dt = torch.int16 if out_dtype == mx.MX_BF16 else torch.float32
    C = torch.full((max(M, 1), ldc), -1, dtype=dt, device="cuda")
    mx.mx_gemm_a4w4_bias(0, 1, M, N, K, A, As, B, Bs, TILED, out_dtype, bias, C, ldc)
    return C


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (100, 70, 300), (300, 257, 1000), (512, 513, 640)])
def test_bias_epilogue(oracle_mod, M, N, K):
    """C = A.B^T + bias (bias added to the fp32 accumulator, one rounding):
    every entry against the oracle's exact sum, bf16 within 2 ulp of the
    correctly rounded value (tau floor as above), fp32 rel. Frobenius <= 1e-5.
    N not a multiple of 8 exercises the bias reads past the last column."""
    _require_gpu()
    a = synth.random_bf16(M * 13 + K, (M, K), std=1.0)
    b = synth.random_bf16(N * 17 + K, (N, K), std=0.05)
    bias = synth.random_bf16(N + 5, (N,), std=2.0)
    log("bias epilogue %dx%dx%d" % (M, N, K))
    ad, lda = to_dev_bf16(a)
    bd, ldb = to_dev_bf16(b)
    qa, sa = quantize_rowwise(ad, M, K, lda, TILED)
    qb, sb = quantize_rowwise(bd, N, K, ldb, TILED)
    bias_d = torch.zeros(((N + 7) // 8 * 8,), dtype=torch.int16)
    bias_d[:N] = torch.from_numpy(bias.view(np.int16))
    bias_d = bias_d.cuda()
    cb = host(gemm_bias(qa, sa, qb, sb, M, N, K, bias_d, mx.MX_BF16))[:M, :N].view(np.uint16)
    cf = host(gemm_bias(qa, sa, qb, sb, M, N, K, bias_d, mx.MX_F32))[:M, :N].astype(np.float64)
    oqa, osa = oracle_mod.quantize(a, 0)
    oqb, osb = oracle_mod.quantize(b, 0)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ii, jj = ii.ravel(), jj.ravel()
    ref = oracle_mod.gemm_bias_entries(oqa, osa, oqb, osb, M, N, K, bias, ii, jj)
    tau = tau_bound(oracle_mod, oqa, osa, oqb, osb, M, N, K, ii, jj)
    check_gemm_bf16(cb[ii, jj], ref, tau, oracle_mod, "bias")
    rel = np.linalg.norm(cf[ii, jj] - ref) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= 1e-5, rel


def test_bias_k_zero_writes_bias(oracle_mod):
    """K == 0: every row of C is the bias, exactly, in both output types."""
    _require_gpu()
    M, N = 33, 20
    bias = synth.random_bf16(64, (N,), std=2.0)
    bias_d = torch.zeros((24,), dtype=torch.int16)
    bias_d[:N] = torch.from_numpy(bias.view(np.int16))
    bias_d = bias_d.cuda()
    dummy = torch.zeros(16, dtype=torch.uint8, device="cuda")
    cb = host(gemm_bias(dummy, dummy, dummy, dummy, M, N, 0, bias_d, mx.MX_BF16))[:M, :N].view(np.uint16)
    cf = host(gemm_bias(dummy, dummy, dummy, dummy, M, N, 0, bias_d, mx.MX_F32))[:M, :N]
    assert (cb == bias[None, :]).all()
    assert (cf.astype(np.float64) == oracle_mod.bf16_to_double(bias)[None, :]).all()


@pytest.mark.parametrize("K", [384, 1100, 2048])
def test_tail_tiles_bias_every_entry_of_tail_rows(oracle_mod, K):
    """Tile count past one round on 256 CUs with a small last round: the last
    round runs as 128x128 tiles (4597x4349 -> 18x17 = 306 tiles of 256x256; the
    last 50 of the tile order, which hold the ragged last row and column of
    tiles, become 200 tiles of 128x128).  K 384: one workgroup of 4 waves per
    small tile; K 1100 (3 k-groups: 2 + 1, the second group's last steps past
    K) and 2048 (4 k-groups: 2 + 2): at most one small tile per CU, so each
    runs as two K groups of 4 waves summed through LDS.  With a bias, in bf16
    and fp32: every entry of rows in the main and the tail region, against
    the oracle, and the bf16 output equal to the rounding of the fp32 one."""
    _require_gpu()
    M, N = 4597, 4349
    a = synth.random_bf16(91 + K, (M, K), std=1.0)
    b = synth.random_bf16(92 + K, (N, K), std=0.05)
    bias = synth.random_bf16(93, (N,), std=2.0)
    log("tail tiles with bias %dx%dx%d" % (M, N, K))
    ad, lda = to_dev_bf16(a)
    bd, ldb = to_dev_bf16(b)
    qa, sa = quantize_rowwise(ad, M, K, lda, TILED)
    qb, sb = quantize_rowwise(bd, N, K, ldb, TILED)
    bias_d = torch.zeros(((N + 7) // 8 * 8,), dtype=torch.int16)
    bias_d[:N] = torch.from_numpy(bias.view(np.int16))
    bias_d = bias_d.cuda()
    cb = host(gemm_bias(qa, sa, qb, sb, M, N, K, bias_d, mx.MX_BF16))[:M, :N].view(np.uint16)
    cf = host(gemm_bias(qa, sa, qb, sb, M, N, K, bias_d, mx.MX_F32))[:M, :N].astype(np.float64)
    oqa, osa = oracle_mod.quantize(a, 0)
    oqb, osb = oracle_mod.quantize(b, 0)
    rows = np.array([0, 127, 128, 2047, 2048 + 77, 4095, 4096, 4096 + 128, M - 2, M - 1])
    ii = np.repeat(rows, N)
    jj = np.tile(np.arange(N), rows.size)
    ref = oracle_mod.gemm_bias_entries(oqa, osa, oqb, osb, M, N, K, bias, ii, jj)
    tau = tau_bound(oracle_mod, oqa, osa, oqb, osb, M, N, K, ii, jj)
    exact, _ = check_gemm_bf16(cb[ii, jj], ref, tau, oracle_mod, "tail-bias")
    rel = np.linalg.norm(cf[ii, jj] - ref) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= 1e-5, rel
    assert np.array_equal(cb, _rne_bf16_bits(cf))
    log("tail-bias K %d: %d/%d bf16 exact, fp32 rel %.3g" % (K, exact, ii.size, rel))


def _rne_bf16_bits(f32):
    """bf16 bits of finite fp32 values, round to nearest even."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("K", [200, 700, 1536, 18560])
def test_several_tiles_per_workgroup(oracle_mod, K):
    """5020x7640 output = 20x30 = 600 tiles of 256x256: two whole rounds on
    256 CUs, where each persistent workgroup runs two tiles back to back (the
    DMAs of the first tile's last k-steps fetch the second tile's first ones,
    its stores overlap the second tile's first k-steps, the second tile's
    bias loads follow them), plus an 88-tile tail; ragged last row and column
    of tiles.  K 200 (fewer k-steps than the pipeline depth), 700 (padded
    k-group), 1536, and 18560 (145 k-steps, one past the longest K the
    persistent kernel takes, so the bf16 output comes from one tile per
    workgroup too).  Without and with a bias: sampled entries against the
    oracle, and the bf16 output (persistent kernel) equal to the round-to-
    nearest-even of the fp32 output (one tile per workgroup), which
    accumulates in the same order; nothing written past column N of the
    ldc-strided output."""
    _require_gpu()
    M, N = 5020, 7640
    a = synth.random_bf16(101 + K, (M, K), std=1.0)
    b = synth.random_bf16(102 + K, (N, K), std=0.05)
    bias = synth.random_bf16(103 + K, (N,), std=2.0)
    log("several tiles per workgroup %dx%dx%d" % (M, N, K))
    cb, cf = run_case(oracle_mod, a, b, full=False, nsample=8192, seed=K, what="stream-%d" % K)
    assert np.array_equal(cb, _rne_bf16_bits(cf))
    ad, lda = to_dev_bf16(a)
    bd, ldb = to_dev_bf16(b)
    qa, sa = quantize_rowwise(ad, M, K, lda, TILED)
    qb, sb = quantize_rowwise(bd, N, K, ldb, TILED)
    bias_d = torch.zeros(((N + 7) // 8 * 8,), dtype=torch.int16)
    bias_d[:N] = torch.from_numpy(bias.view(np.int16))
    bias_d = bias_d.cuda()
    cbb = host(gemm_bias(qa, sa, qb, sb, M, N, K, bias_d, mx.MX_BF16))[:M, :N].view(np.uint16)
    cfb = host(gemm_bias(qa, sa, qb, sb, M, N, K, bias_d, mx.MX_F32))[:M, :N]
    assert np.array_equal(cbb, _rne_bf16_bits(cfb))
    oqa, osa = oracle_mod.quantize(a, 0)
    oqb, osb = oracle_mod.quantize(b, 0)
    rng = np.random.default_rng(K + 1)
    ii, jj = rng.integers(0, M, 4096), rng.integers(0, N, 4096)
    ref = oracle_mod.gemm_bias_entries(oqa, osa, oqb, osb, M, N, K, bias, ii, jj)
    tau = tau_bound(oracle_mod, oqa, osa, oqb, osb, M, N, K, ii, jj)
    exact, _ = check_gemm_bf16(cbb[ii, jj], ref, tau, oracle_mod, "stream-bias-%d" % K)
    log("stream-bias-%d: %d/%d bf16 exact" % (K, exact, ii.size))
    ldc = N + 24
    Cp = host(gemm(qa, sa, qb, sb, M, N, K, mx.MX_BF16, ldc=ldc)).view(np.uint16)
    assert np.array_equal(Cp[:M, :N], cb)
    assert (Cp[:, N:] == 0xFFFF).all()


def test_output_over_2gib_sampled(oracle_mod):
    """A bf16 output of 33000 x 32776 with ldc 32784 (2.16 GB, past the 2^31
    bytes that 32-bit buffer offsets reach) and K 130 (padded to 256): the
    launcher keeps such an output off the persistent kernel, and the one-tile
    kernel's 64-bit addressed stores reach every row.  Sampled entries (the
    last 256 rows weighted in, the four corners included) against the oracle;
    the padding columns of the last rows stay untouched."""
    _require_gpu()
    M, N, K = 33000, 32776, 130
    ldc = N + 8
    assert M * ldc * 2 >= 2 ** 31
    a = synth.random_bf16(301, (M, K), std=1.0)
    b = synth.random_bf16(302, (N, K), std=0.5)
    ad, lda = to_dev_bf16(a)
    bd, ldb = to_dev_bf16(b)
    qa, sa = quantize_rowwise(ad, M, K, lda, TILED)
    qb, sb = quantize_rowwise(bd, N, K, ldb, TILED)
    log("output over 2 GiB %dx%dx%d ldc %d" % (M, N, K, ldc))
    C = gemm(qa, sa, qb, sb, M, N, K, mx.MX_BF16, ldc=ldc)
    rng = np.random.default_rng(7)
    ii = np.concatenate([rng.integers(0, M, 4096), rng.integers(M - 256, M, 1024), [0, M - 1, M - 1, 0]])
    jj = np.concatenate([rng.integers(0, N, 4096), rng.integers(0, N, 1024), [0, N - 1, 0, N - 1]])
    got = C[torch.from_numpy(ii).cuda(), torch.from_numpy(jj).cuda()].cpu().numpy().view(np.uint16)
    assert (C[M - 64:, N:].cpu().numpy() == -1).all()
    del C
    oqa, osa = oracle_mod.quantize(a, 0)
    oqb, osb = oracle_mod.quantize(b, 0)
    ref = oracle_mod.gemm_entries(oqa, osa, oqb, osb, M, N, K, ii, jj)
    tau = tau_bound(oracle_mod, oqa, osa, oqb, osb, M, N, K, ii, jj)
    exact, _ = check_gemm_bf16(got, ref, tau, oracle_mod, "over-2GiB")
    log("over-2GiB: %d/%d bf16 exact" % (exact, ii.size))
