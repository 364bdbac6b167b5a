"""Pins of the oracle's block-scaled NT GEMM, its dequantizer and its bf16 cast.

GEMM: exact rational brute force (Python fractions) on small shapes, numpy's
float64 matmul (a library routine) of the dequantized operands on larger
ones, a hand-worked integer dot product, and the exact doubling when every A
scale byte is raised by one.  Cast: an exhaustive search over the bf16 grid
(bracket + nearest + even mantissa), a different algorithm from the oracle's
rescale-and-round.
"""
from fractions import Fraction

import numpy as np
import pytest

from mxfp4_precision_amd import synth

E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def exact_element(q, s, r, k):
    byte = int(q[r, k // 2])
    nib = byte & 0xF if k % 2 == 0 else byte >> 4
    v = E2M1[nib & 7] * Fraction(2) ** (int(s[r, k // 32]) - 127)
    return -v if nib & 8 else v


def test_gemm_exact_rational_small(oracle_mod):
    M, N, K = 5, 4, 200
    a = synth.random_bf16(31, (M, K), std=2.0)
    b = synth.random_bf16(32, (N, K), std=0.05)
    qa, sa = oracle_mod.quantize(a, 0)
    qb, sb = oracle_mod.quantize(b, 0)
    Kp = 256
    C = oracle_mod.gemm_rows(qa, sa, qb, sb, M, N, K, 0, M)
    for i in range(M):
        for j in range(N):
            exact = sum(exact_element(qa, sa, i, k) * exact_element(qb, sb, j, k) for k in range(Kp))
            assert C[i, j] == float(exact), (i, j)


def test_gemm_entries_match_rows(oracle_mod):
    M, N, K = 40, 24, 300
    a = synth.random_bf16(33, (M, K))
    b = synth.random_bf16(34, (N, K))
    qa, sa = oracle_mod.quantize(a, 0)
    qb, sb = oracle_mod.quantize(b, 0)
    C = oracle_mod.gemm_rows(qa, sa, qb, sb, M, N, K, 0, M)
    ii = np.array([0, 39, 17, 5]); jj = np.array([0, 23, 11, 20])
    e = oracle_mod.gemm_entries(qa, sa, qb, sb, M, N, K, ii, jj)
    assert (e == C[ii, jj]).all()
    part = oracle_mod.gemm_rows(qa, sa, qb, sb, M, N, K, 10, 20)
    assert (part == C[10:20]).all()


def test_gemm_against_numpy_matmul(oracle_mod):
    """P11: equals numpy float64 matmul of the dequantized operands to 1e-12."""
    M, N, K = 64, 48, 1000
    a = synth.random_bf16(35, (M, K))
    b = synth.random_bf16(36, (N, K), std=0.02)
    qa, sa = oracle_mod.quantize(a, 0)
    qb, sb = oracle_mod.quantize(b, 0)
    da = oracle_mod.dequantize(qa, sa, M, K)
    db = oracle_mod.dequantize(qb, sb, N, K)
    ref = da @ db.T
    C = oracle_mod.gemm_rows(qa, sa, qb, sb, M, N, K, 0, M)
    assert np.linalg.norm(C - ref) <= 1e-12 * np.linalg.norm(ref)


def test_gemm_dense_matches_entry_sums(oracle_mod):
    """gemm_dense (dequantize + float64 matmul) against the oracle's own
    entry-by-entry sum on every entry of a ragged shape with outliers and zero
    blocks, and its |product| sums against a direct sum; then a transposed
    operand (a plausible wiring mistake) must fail the same comparison."""
    M, N, K = 70, 45, 777
    a = synth.random_bf16(37, (M, K), std=1.0)
    b = synth.random_bf16(38, (N, K), std=0.02)
    a[3, :64] = 0
    a[5, 10] = synth.bf16_bits(np.array([3e3], np.float32))[0]
    qa, sa = oracle_mod.quantize(a, 0)
    qb, sb = oracle_mod.quantize(b, 0)
    C, S = oracle_mod.gemm_dense(qa, sa, qb, sb, M, N, K)
    ref = oracle_mod.gemm_rows(qa, sa, qb, sb, M, N, K, 0, M)
    assert C.shape == (M, N) and S.shape == (M, N)
    assert np.abs(C - ref).max() <= 1e-13 * S.max()
    da = oracle_mod.dequantize(qa, sa, M, K)
    db = oracle_mod.dequantize(qb, sb, N, K)
    i, j = 5, 7
    assert abs(S[i, j] - sum(abs(da[i, k] * db[j, k]) for k in range(da.shape[1]))) <= 1e-12 * S[i, j]
    assert (S >= np.abs(C) - 1e-12 * S).all()
    Ct, _ = oracle_mod.gemm_dense(qb, sb, qa, sa, N, M, K)
    assert np.abs(Ct.T - C).max() <= 1e-13 * S.max()                   # the product's own symmetry
    Cw, _ = oracle_mod.gemm_dense(qa, sa, qa[:N], sa[:N], M, N, K)   # wrong B operand: must differ
    assert np.abs(Cw - ref).max() > 1e-3 * np.abs(ref).max()


def test_gemm_hand_dot_product(oracle_mod):
    """K = 32 of 1.0 against 0.5 (unit-scale blocks): 32 * 0.5 = 16 in every entry."""
    a = synth.bf16_bits(np.ones((2, 32), np.float32) * 4.0)   # amax 4 -> scale 2^0, code 6
    b = synth.bf16_bits(np.ones((3, 32), np.float32) * 4.0)
    qa, sa = oracle_mod.quantize(a, 0)
    qb, sb = oracle_mod.quantize(b, 0)
    # Replace the codes by hand: A all 1.0 (code 2), B all 0.5 (code 1)
    qa[:, :16] = 0x22
    qb[:, :16] = 0x11
    C = oracle_mod.gemm_rows(qa, sa, qb, sb, 2, 3, 32, 0, 2)
    assert (C == 16.0).all()


def test_gemm_scale_bump_doubles(oracle_mod):
    M, N, K = 16, 16, 256
    a = synth.random_bf16(37, (M, K))
    b = synth.random_bf16(38, (N, K))
    qa, sa = oracle_mod.quantize(a, 0)
    qb, sb = oracle_mod.quantize(b, 0)
    C = oracle_mod.gemm_rows(qa, sa, qb, sb, M, N, K, 0, M)
    C2 = oracle_mod.gemm_rows(qa, (sa + 1).astype(np.uint8), qb, sb, M, N, K, 0, M)
    assert (C2 == 2 * C).all()


def test_gemm_nan_scale_propagates(oracle_mod):
    a = np.full((1, 64), 0x3F80, np.uint16)
    a[0, 3] = 0x7FC0
    b = np.full((2, 64), 0x3F80, np.uint16)
    qa, sa = oracle_mod.quantize(a, 0)
    qb, sb = oracle_mod.quantize(b, 0)
    C = oracle_mod.gemm_rows(qa, sa, qb, sb, 1, 2, 64, 0, 1)
    assert np.isnan(C).all()


def test_dequantize_is_nearest_grid_value(oracle_mod):
    """dequantize(quantize(x)) is the E2M1 grid point nearest to x/2^e, times 2^e."""
    x = synth.random_bf16(39, (20, 64))
    q, s = oracle_mod.quantize(x, 0)
    d = oracle_mod.dequantize(q, s, 20, 64)[:, :64]
    xv = synth.bf16_to_f32(x).astype(np.float64)
    scale = 2.0 ** (np.repeat(s[:, :2].astype(float), 32, axis=1) - 127)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    v = np.abs(xv) / scale
    err = np.abs(np.abs(d) / scale - v)
    best = np.abs(v[..., None] - grid).min(axis=-1)
    assert (err == best).all()


# ---------------------------------------------------------------- bf16 cast

def _bf16_grid():
    bits = np.arange(0, 0x7F81, dtype=np.uint32)     # 0 .. +Inf
    vals = (bits << 16).view(np.float32).astype(np.float64)
    return bits.astype(np.uint16), vals


def _search_round(d):
    """Round |d| to bf16 by bracketing on the full grid; ties to even mantissa."""
    bits, vals = _bf16_grid()
    a = abs(d)
    hi = int(np.searchsorted(vals, a, side="left"))
    if hi < vals.size and vals[hi] == a:
        r = bits[hi]
    else:
        lo = hi - 1
        if hi >= vals.size - 1:  # above bf16 max: compare with the max and the next step
            mx = vals[-2]
            step = vals[-2] - vals[-3]
            r = bits[-1] if a >= mx + step / 2 else bits[-2]
        else:
            dl, dh = a - vals[lo], vals[hi] - a
            if dl < dh:
                r = bits[lo]
            elif dh < dl:
                r = bits[hi]
            else:
                r = bits[lo] if bits[lo] % 2 == 0 else bits[hi]
    return int(r) | (0x8000 if np.signbit(d) else 0)


def test_bf16_cast_against_grid_search(oracle_mod):
    rng = np.random.default_rng(3)
    vals = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 39, 3000))
    # exact ties, subnormals, overflow boundary, zeros
    vals += [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 2.0 ** -133, 2.0 ** -134,
             1.5 * 2.0 ** -133, 3.0 * 2.0 ** -134, 3.3895313892515355e38, 3.3961775292304005e38,
             3.3961775292304e38 * 1.0000001, 0.0, -0.0, 1e-300, 2.0 ** -126 * (1 - 2.0 ** -9)]
    got = oracle_mod.bf16_from_double(np.array(vals))
    for d, g in zip(vals, got):
        assert int(g) == _search_round(d), (d, hex(int(g)))


def test_bf16_cast_specials(oracle_mod):
    got = oracle_mod.bf16_from_double(np.array([np.inf, -np.inf, np.nan, 1e39, -1e39]))
    assert got[0] == 0x7F80 and got[1] == 0xFF80
    assert (got[2] & 0x7F80) == 0x7F80 and (got[2] & 0x7F)
    assert got[3] == 0x7F80 and got[4] == 0xFF80


def test_gemm_bias_hand_value(oracle_mod):
    """The hand dot product above (16 in every entry) plus a bias of -3.5, 0.25
    and 2^-9 per column: 12.5, 16.25 and 16 + 2^-9 exactly."""
    a = synth.bf16_bits(np.ones((2, 32), np.float32) * 4.0)
    b = synth.bf16_bits(np.ones((3, 32), np.float32) * 4.0)
    qa, sa = oracle_mod.quantize(a, 0)
    qb, sb = oracle_mod.quantize(b, 0)
    qa[:, :16] = 0x22
    qb[:, :16] = 0x11
    bias = synth.bf16_bits(np.array([-3.5, 0.25, 2.0 ** -9], np.float32))
    ii, jj = np.meshgrid(np.arange(2), np.arange(3), indexing="ij")
    C = oracle_mod.gemm_bias_entries(qa, sa, qb, sb, 2, 3, 32, bias, ii.ravel(), jj.ravel()).reshape(2, 3)
    assert (C == np.array([[12.5, 16.25, 16 + 2.0 ** -9]] * 2)).all()
    # rounded to bf16 (spacing 1/8 at 16), 16 + 2^-9 becomes 16
    assert (oracle_mod.bf16_from_double(C[0]) == synth.bf16_bits(np.array([12.5, 16.25, 16.0], np.float32))).all()


def test_gemm_bias_special_cases(oracle_mod):
    """K = 0: the output is the bias itself; a zero bias: the plain product."""
    M, N, K = 5, 7, 96
    a = synth.random_bf16(61, (M, K))
    b = synth.random_bf16(62, (N, K))
    bias = synth.random_bf16(63, (N,), std=3.0)
    qa, sa = oracle_mod.quantize(a, 0)
    qb, sb = oracle_mod.quantize(b, 0)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ii, jj = ii.ravel(), jj.ravel()
    z = oracle_mod.gemm_bias_entries(qa, sa, qb, sb, M, N, 0, bias, ii, jj)
    assert (oracle_mod.bf16_from_double(z) == bias[jj]).all()
    plain = oracle_mod.gemm_entries(qa, sa, qb, sb, M, N, K, ii, jj)
    zero = np.zeros(N, np.uint16)
    assert (oracle_mod.gemm_bias_entries(qa, sa, qb, sb, M, N, K, zero, ii, jj) == plain).all()
