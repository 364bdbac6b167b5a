"""The MFMA-rate measurement aid computes what it claims (so the rate it
reports is of real work): zero operands give zeros; a single element of 1.0
in one chain's A operand against B elements of 0.5 gives exactly
iters x 32 x 0.5 summed over a wave's lanes, for E2M1, FP6 and FP8 codes;
repeated calls are bit-identical."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mxfp4_precision_amd as mx

pytestmark = pytest.mark.gpu


def _run(ops_words, workgroups, iters, fa=4, fb=4):
    ops = torch.from_numpy(ops_words.view(np.uint8)).cuda()
    out = torch.full((workgroups * 512,), float("nan"), dtype=torch.float32, device="cuda")
    mx.mx_measure_mfma(fa, fb, ops, workgroups, iters, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_measure_mfma_zero_and_counted_products():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wg, iters = 3, 7
    zeros = np.zeros(64 * 64, dtype=np.uint32)
    assert np.all(_run(zeros, wg, iters) == 0.0)
    # B elements all 0.5, A: chain 0 of lane 0 holds one element 1.0 (its first
    # code), all else 0.  Whatever row/k that element maps to, it meets 32 B
    # values of 0.5 (one per output column), so each chain-0 instruction adds
    # 32 * 0.5 = 16 to a wave's outputs: 16 * iters over its 64 lane sums.
    # Codes: E2M1 0.5 = 0x1, 1.0 = 0x2 (4-bit); E2M3 0.5 = 0x04, 1.0 = 0x08 and
    # E3M2 0.5 = 0x08, 1.0 = 0x0C (6-bit, packed little-endian); E5M2 0.5 =
    # 0x38, 1.0 = 0x3C (8-bit).
    cases = [(4, 4, 4, 0x1, 0x2), (2, 2, 6, 0x04, 0x08), (3, 3, 6, 0x08, 0x0C), (1, 1, 8, 0x38, 0x3C)]
    for fa, fb, bits, half, one in cases:
        words = {4: 4, 6: 6, 8: 8}[bits]          # dwords one lane's operand uses
        val = 0
        for e in range(words * 32 // bits):       # every element of B = 0.5, packed LSB first
            val |= half << (bits * e)
        ops = np.zeros((64, 64), dtype=np.uint32)
        for k in range(4):
            for w in range(words):
                ops[:, 16 * k + 8 + w] = (val >> (32 * w)) & 0xFFFFFFFF
        ops[0, 0] = one
        out = _run(ops.ravel(), wg, iters, fa, fb).reshape(wg, 8, 64)
        per_wave = out.sum(axis=2, dtype=np.float64)
        assert np.all(per_wave == 16.0 * iters), (fa, fb, per_wave)
        again = _run(ops.ravel(), wg, iters, fa, fb).reshape(wg, 8, 64)
        assert np.array_equal(out, again)
    rng = np.random.default_rng(3)
    r = rng.integers(0, 2 ** 32, 64 * 64, dtype=np.uint64).astype(np.uint32)
    o1 = _run(r, wg, iters)
    assert np.all(np.isfinite(o1)) and np.array_equal(o1, _run(r, wg, iters))
