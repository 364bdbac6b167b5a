"""GPU parity of whole training steps of an MXFP4 linear layer, wired the way a
step uses the blobs: each of X, W and dY is dual-quantized once, the forward
takes the row-wise blobs (X_row . W_row^T), dgrad takes dY_row . W_col^T and
wgrad dY_col . X_col^T, all NT products over the column-wise blobs rather
than over re-quantized transposes ("primus_turbo_mxfp4_local.py", the
autograd Function's forward and backward).

Every quantized byte and scale is compared with the oracle; GEMM outputs are
checked on sampled entries (the oracle computes them one by one from its own
blobs) against the bf16 and fp32 bars of the GEMM tests.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mxfp4_precision_amd as mx
from mxfp4_precision_amd import synth

import input_digests
from gpu_util import check_gemm_bf16, gemm, host, log, quantize_dual, tau_bound, to_dev_bf16

pytestmark = pytest.mark.gpu
TILED = mx.MX_LAYOUT_TILED


def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _assert_same(got, want, what):
    got = np.asarray(got).ravel()
    want = np.asarray(want).ravel()
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "%s: %d bytes differ, first at %s" % (what, bad.size, bad[:5].tolist())


def _dual_checked(oracle_mod, name, x, opts=None, okw=None):
    """Dual-quantize x on the GPU (tiled layout); check all four outputs
    against the oracle; return the device blobs and the oracle's canonical ones."""
    M, N = x.shape
    xd, ldx = to_dev_bf16(x)
    qr, sr, qc, sc = quantize_dual(xd, M, N, ldx, TILED, opts, opts)
    del xd
    orow = oracle_mod.quantize(x, 0, **(okw or {}))
    ocol = oracle_mod.quantize(x, 1, **(okw or {}))
    trow = oracle_mod.to_tiled(orow[0], orow[1], M, N)
    tcol = oracle_mod.to_tiled(ocol[0], ocol[1], N, M)
    for got, want, what in ((qr, trow[0], "row data"), (sr, trow[1], "row scale"),
                            (qc, tcol[0], "col data"), (sc, tcol[1], "col scale")):
        _assert_same(host(got), want, "%s %s" % (name, what))
    log("%s %dx%d dual: all bytes equal" % (name, M, N))
    return (qr, sr, qc, sc), (orow, ocol)


def _gemm_checked(oracle_mod, what, A, B, oA, oB, M, N, K, nsample, seed):
    (qa, sa), (qb, sb) = A, B
    (oqa, osa), (oqb, osb) = oA, oB
    cb = host(gemm(qa, sa, qb, sb, M, N, K, mx.MX_BF16))[:M, :N].view(np.uint16)
    cf = host(gemm(qa, sa, qb, sb, M, N, K, mx.MX_F32))[:M, :N].astype(np.float64)
    rng = np.random.default_rng(seed)
    ii = np.concatenate([rng.integers(0, M, nsample), [0, M - 1, M - 1, 0]])
    jj = np.concatenate([rng.integers(0, N, nsample), [0, N - 1, 0, N - 1]])
    ref = oracle_mod.gemm_entries(oqa, osa, oqb, osb, M, N, K, ii, jj)
    tau = tau_bound(oracle_mod, oqa, osa, oqb, osb, M, N, K, ii, jj)
    exact, tau_only = check_gemm_bf16(cb[ii, jj], ref, tau, oracle_mod, what)
    rel = np.linalg.norm(cf[ii, jj] - ref) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= 1e-5, (what, rel)
    log("%s %dx%dx%d: %d/%d bf16 exact, %d tau-floor only, fp32 rel %.3g"
        % (what, M, N, K, exact, ii.size, tau_only, rel))


def _gemm_full_checked(oracle_mod, what, A, B, oA, oB, M, N, K):
    """Every entry: the bf16 output (the launch the step uses) within the bf16
    bar of the oracle's product, the fp32 output within tau + 2^-24 |C| of it
    elementwise and within 1e-5 relative Frobenius.  The oracle's whole product
    is its dequantization times a float64 matmul (gemm_dense)."""
    (qa, sa), (qb, sb) = A, B
    (oqa, osa), (oqb, osb) = oA, oB
    cb = host(gemm(qa, sa, qb, sb, M, N, K, mx.MX_BF16))[:M, :N].view(np.uint16)
    cf = host(gemm(qa, sa, qb, sb, M, N, K, mx.MX_F32))[:M, :N].astype(np.float64)
    ref, sabs = oracle_mod.gemm_dense(oqa, osa, oqb, osb, M, N, K)
    tau = (oracle_mod.padded(K) / 32) * 2.0 ** -24 * sabs
    del sabs
    exact, tau_only = check_gemm_bf16(cb, ref, tau, oracle_mod, what)
    del cb
    err = np.abs(cf - ref)
    bad = ~(err <= tau + 2.0 ** -24 * np.abs(ref))
    assert not bad.any(), "%s: %d fp32 entries beyond tau, first at %s" % (what, int(bad.sum()),
                                                                          np.argwhere(bad)[:3].tolist())
    rel = np.linalg.norm(cf - ref) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= 1e-5, (what, rel)
    log("%s %dx%dx%d: every entry checked; %d/%d bf16 exact, %d tau-floor only, fp32 rel %.3g, "
        "fp32 max err/tau %.3g" % (what, M, N, K, exact, ref.size, tau_only, rel,
                                    float((err / np.maximum(tau, 1e-300)).max())))


def _step(oracle_mod, X, W, dY, wopts=None, wkw=None, gopts=None, gkw=None, nsample=4096, tag="", full=False):
    T, din = X.shape
    dout = W.shape[0]
    assert W.shape == (dout, din) and dY.shape == (T, dout)
    (xr, xrs, xc, xcs), (oxr, oxc) = _dual_checked(oracle_mod, tag + "X", X)
    (wr, wrs, wc, wcs), (owr, owc) = _dual_checked(oracle_mod, tag + "W", W, wopts, wkw)
    (gr, grs, gc, gcs), (ogr, ogc) = _dual_checked(oracle_mod, tag + "dY", dY, gopts, gkw)
    if full:
        _gemm_full_checked(oracle_mod, tag + "fwd", (xr, xrs), (wr, wrs), oxr, owr, T, dout, din)
        _gemm_full_checked(oracle_mod, tag + "dgrad", (gr, grs), (wc, wcs), ogr, owc, T, din, dout)
        _gemm_full_checked(oracle_mod, tag + "wgrad", (gc, gcs), (xc, xcs), ogc, oxc, dout, din, T)
        return
    # forward Y = X W^T: (T x dout), K = din
    _gemm_checked(oracle_mod, tag + "fwd", (xr, xrs), (wr, wrs), oxr, owr, T, dout, din, nsample, 11)
    # dgrad dX = dY W: A = dY_row (T rows, K = dout), B = W_col (din rows, K = dout)
    _gemm_checked(oracle_mod, tag + "dgrad", (gr, grs), (wc, wcs), ogr, owc, T, din, dout, nsample, 12)
    # wgrad dW = dY^T X: A = dY_col (dout rows, K = T), B = X_col (din rows, K = T)
    _gemm_checked(oracle_mod, tag + "wgrad", (gc, gcs), (xc, xcs), ogc, oxc, dout, din, T, nsample, 13)


def test_fc1_step_full_size(oracle_mod):
    """MLP fc1 training step at full size (9216 tokens, 3072 -> 12288; seed 3):
    X N(0,1), W N(0,0.02), dY N(0,1e-3), round to nearest, 1D blocks."""
    _require_gpu()
    d = synth.fc1()
    input_digests.check("fc1", d)
    log("fc1 step X %s W %s dY %s" % (d["X"].shape, d["W"].shape, d["dY"].shape))
    _step(oracle_mod, d["X"], d["W"], d["dY"], tag="fc1-")


def test_fc2_recipe_step_ragged(oracle_mod):
    """The fc2 recipe (2D weight blocks, stochastic rounding on dY with seed 7)
    on a ragged slice: 1000 tokens, 1100 -> 300, so every padded edge of
    every blob and GEMM tile is crossed."""
    _require_gpu()
    rng = np.random.Generator(np.random.PCG64(41))
    X = synth.gelu_normal(rng, (1000, 1100))
    W = synth.normal(rng, (300, 1100), 0.02)
    dY = synth.normal(rng, (1000, 300), 1e-3)
    w2 = mx.quant_opts(use_2d_block=True, tensor_id=1)
    sr = mx.quant_opts(use_sr=True, seed=7, tensor_id=2)
    _step(oracle_mod, X, W, dY, w2, dict(use_2d=True, tensor_id=1), sr, dict(use_sr=True, seed=7, tensor_id=2),
          nsample=8192, tag="fc2-ragged-")


def test_fc2_step_full_size_every_entry(oracle_mod):
    """The MLP fc2 training step exactly as the benchmark runs it, at full size
    (18432 tokens, 12288 -> 3072; seed 4): X GELU(N(0,1)) plain, W N(0,0.02)
    with 32x32 blocks in both directions, dY N(0,1e-3) with stochastic
    rounding in both directions (seed 7, tensor id 2).  Every byte of the six
    blobs against the oracle; fwd X_row . W_row^T, dgrad dY_row . W_col^T and
    wgrad dY_col . X_col^T from those blobs, every entry of each product
    (bf16 output from the persistent and tail kernels the step launches, and
    fp32 output) against the oracle's product of its own blobs."""
    _require_gpu()
    d = synth.fc2()
    input_digests.check("fc2", d)
    log("fc2 step X %s W %s dY %s" % (d["X"].shape, d["W"].shape, d["dY"].shape))
    w2 = mx.quant_opts(use_2d_block=True, tensor_id=1)
    sr = mx.quant_opts(use_sr=True, seed=7, tensor_id=2)
    _step(oracle_mod, d["X"], d["W"], d["dY"], w2, dict(use_2d=True, tensor_id=1), sr,
          dict(use_sr=True, seed=7, tensor_id=2), tag="fc2-", full=True)
