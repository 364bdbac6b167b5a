"""Pins of the oracle's multiply prologue element (NEXT row: quantizer
prologue).  Reading of the page "Primus PR 1107" (its QKV packer forms the
gradient in the staging read instead of reading back what the producer
stored): the quantized tensor is what a producer multiplying in fp32 and
storing bf16 would have written, y = bf16(fp32(x * g)).  Pinned against
numpy's IEEE float32 multiply and an integer bf16 rounding written here."""
import numpy as np

from mxfp4_precision_amd import synth


def ref_bf16_mul(x, g):
    """numpy fp32 product, then round-to-nearest-even to the upper 16 bits (NaN kept NaN)."""
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    gf = (g.astype(np.uint32) << 16).view(np.float32)
    with np.errstate(over="ignore", invalid="ignore", under="ignore"):
        p = (xf * gf).astype(np.float32)
    u = p.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(p)
    return r, nan


def test_bf16_mul_matches_numpy_fp32(oracle_mod):
    rng = np.random.default_rng(0)
    x = rng.integers(0, 1 << 16, 200000, dtype=np.uint64).astype(np.uint16)
    g = rng.integers(0, 1 << 16, 200000, dtype=np.uint64).astype(np.uint16)
    got = oracle_mod.bf16_mul(x, g)
    want, nan = ref_bf16_mul(x, g)
    gotnan = ((got >> 7) & 0xFF) == 0xFF
    gotnan &= (got & 0x7F) != 0
    assert np.array_equal(gotnan, nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_bf16_mul_edge_values(oracle_mod):
    # subnormal products (fp32 rounding then bf16 rounding), overflow, zeros and signs
    vals = np.array([0x0001, 0x0080, 0x00FF, 0x0100, 0x1F80, 0x2000, 0x3F80, 0x3FC0, 0x7F7F, 0x7F80, 0x8000,
                     0x8001, 0xBF80, 0xFF7F, 0x0000, 0x3F81, 0x40A0, 0x1000, 0x2F80], dtype=np.uint16)
    x = np.repeat(vals, vals.size)
    g = np.tile(vals, vals.size)
    got = oracle_mod.bf16_mul(x, g)
    want, nan = ref_bf16_mul(x, g)
    keep = ~nan
    assert np.array_equal(got[keep], want[keep])
    # exact cases: 1.0 is the identity, 2^k scales exactly
    xs = synth.random_bf16(5, (4096,), std=3.0)
    assert np.array_equal(oracle_mod.bf16_mul(xs, np.full_like(xs, 0x3F80)), xs)
    two = oracle_mod.bf16_mul(xs, np.full_like(xs, 0x4000))
    assert np.array_equal(synth.bf16_to_f32(two), 2 * synth.bf16_to_f32(xs))
