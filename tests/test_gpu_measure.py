"""The MFMA-rate measurement aid computes what it claims (so the rate it
reports is of real work): zero operands give zeros; a single E2M1 code of 1.0
in one operand lane and 0.5 everywhere in the other gives exactly
iters x (number of products) x 0.5 summed over the lanes; repeated calls are
bit-identical."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mxfp4_precision_amd as mx

pytestmark = pytest.mark.gpu


def _run(ops_words, workgroups, iters):
    ops = torch.from_numpy(ops_words.view(np.uint8)).cuda()
    out = torch.full((workgroups * 512,), float("nan"), dtype=torch.float32, device="cuda")
    mx.mx_measure_mfma_fp4(ops, workgroups, iters, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_measure_mfma_zero_and_counted_products():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wg, iters = 3, 7
    zeros = np.zeros(64 * 64, dtype=np.uint32)
    assert np.all(_run(zeros, wg, iters) == 0.0)
    # every B code 0x1 (E2M1 0.5); A: lane 0 of chain 0 holds one code 0x2 (1.0)
    # in its first nibble, all else 0.  Whatever row/k that nibble maps to, it
    # meets 32 B values of 0.5 (one per output column), so per chain-0 MFMA the
    # outputs sum to 32 * 0.5 = 16, over iters instructions 16 * iters, spread
    # over some lanes of each wave; the lane sums of every wave add up to that.
    ops = np.zeros((64, 64), dtype=np.uint32)
    for k in range(8):
        ops[:, 8 * k + 4: 8 * k + 8] = 0x11111111
    ops[0, 0] = 0x2
    out = _run(ops.ravel(), wg, iters).reshape(wg, 8, 64)
    per_wave = out.sum(axis=2, dtype=np.float64)
    assert np.all(per_wave == 16.0 * iters), per_wave
    again = _run(ops.ravel(), wg, iters).reshape(wg, 8, 64)
    assert np.array_equal(out, again)
    rng = np.random.default_rng(3)
    r = rng.integers(0, 2 ** 32, 64 * 64, dtype=np.uint64).astype(np.uint32)
    o1 = _run(r, wg, iters)
    assert np.all(np.isfinite(o1)) and np.array_equal(o1, _run(r, wg, iters))
