"""Pins of the oracle's MXFP6 path (NEXT row: MXFP6 elements).

The pages only name an MXFP6 campaign (Primus PR 1107); the element formats
come from the OCP Microscaling Formats v1.0 spec, sec. 5.3.2 (FP6 E2M3: bias
1, 3 mantissa bits, largest 7.5; FP6 E3M2: bias 3, 2 mantissa bits, largest
28; both with subnormals and no Inf/NaN), the scale rule from its sec. 6.3
(shared exponent floor(log2 amax) - emax_elem, emax_elem 2 and 4).  The
rounding rules and the canonical 6-bit packing are this library's readings,
checked here against brute force and hand-worked bytes.
"""
from fractions import Fraction

import numpy as np
import pytest

from mxfp4_precision_amd import synth

E2M3, E3M2 = 2, 3
EMAX = {E2M3: 2, E3M2: 4}


def spec_table(fmt):
    """The 32 non-negative magnitudes from the spec's field definitions, exact."""
    mb, bias = (3, 1) if fmt == E2M3 else (2, 3)
    out = []
    for c in range(32):
        e, m = c >> mb, c & ((1 << mb) - 1)
        if e == 0:
            out.append(Fraction(m, 1 << mb) * Fraction(2) ** (1 - bias))
        else:
            out.append((1 + Fraction(m, 1 << mb)) * Fraction(2) ** (e - bias))
    return out


@pytest.mark.parametrize("fmt", [E2M3, E3M2])
def test_fp6_decode_spec_anchors(oracle_mod, fmt):
    # OCP MX v1.0 sec. 5.3.2 table: max normal, min normal, max/min subnormal
    anchors = {E2M3: (7.5, 1.0, 0.875, 0.125), E3M2: (28.0, 0.25, 0.1875, 0.0625)}[fmt]
    vals = [oracle_mod.fp6_value(c, fmt) for c in range(64)]
    mags = vals[:32]
    assert mags[31] == anchors[0]
    assert min(v for v in mags if v >= anchors[1]) == anchors[1]
    sub = [v for v in mags if 0 < v < anchors[1]]
    assert max(sub) == anchors[2] and min(sub) == anchors[3]
    assert all(a < b for a, b in zip(mags, mags[1:]))          # strictly increasing in code order
    assert all(vals[32 + c] == -mags[c] for c in range(32))    # bit 5 is the sign
    assert [Fraction(v) for v in mags] == spec_table(fmt)


def _blocks_at_scale(fmt, e, vals):
    """bf16 rows whose block amax pins the shared exponent to e: element 0 of every
    32-block is 2^(e + emax), the rest are the values under test (each exactly bf16)."""
    vals = np.asarray(vals, dtype=np.float64)
    nblk = -(-len(vals) // 31)
    x = np.zeros((nblk, 32), dtype=np.float64)
    x[:, 0] = 2.0 ** (e + EMAX[fmt])
    flat = np.zeros(nblk * 31)
    flat[:len(vals)] = vals
    x[:, 1:] = flat.reshape(nblk, 31)
    bits = synth.bf16_bits(x.astype(np.float32))
    assert np.array_equal(synth.bf16_to_f32(bits).astype(np.float64), x), "inputs must be bf16-exact"
    return bits, x


def _brute_rne(v, table):
    if v >= table[-1]:
        return table[-1]
    best = min(range(32), key=lambda c: (abs(table[c] - v), c & 1))
    return table[best]


@pytest.mark.parametrize("fmt", [E2M3, E3M2])
def test_fp6_rne_against_brute_force(oracle_mod, fmt):
    table = spec_table(fmt)
    e = -3
    sc = Fraction(2) ** e
    cand = []
    for a, b in zip(table, table[1:]):
        mid = (a + b) / 2
        cand += [a, mid, mid + (b - a) / 64, mid - (b - a) / 64]
    top = Fraction(2) ** (EMAX[fmt] + 1)                # the block amax stays below 2^(e+emax+1)
    cand += [(table[-1] + top) / 2, top - top / 128]    # beyond the largest: saturate
    # keep the candidates that are exact bf16 values (all midpoints are: few significant bits)
    exact = [c for c in cand if float(synth.bf16_to_f32(synth.bf16_bits(np.float32([float(c * sc)])))[0]) == c * sc]
    assert len(exact) > 2 * 31
    vals = [float(c * sc) for c in exact] + [-float(c * sc) for c in exact]
    bits, x = _blocks_at_scale(fmt, e, vals)
    q, s = oracle_mod.quantize_fp6(bits, 0, fmt)
    assert (s[:, 0] == e + 127).all()
    deq = oracle_mod.dequantize_fp6(q, s, bits.shape[0], 32, fmt)[:, 1:32].reshape(-1)[:len(vals)]
    for v, d in zip(vals, deq):
        want = _brute_rne(abs(Fraction(v)) / sc, table) * sc
        assert Fraction(abs(d)) == want, (v, d, want)
        assert (d < 0) == (v < 0) or d == 0


@pytest.mark.parametrize("fmt", [E2M3, E3M2])
def test_fp6_every_bf16_magnitude(oracle_mod, fmt):
    """All positive finite bf16 values below 2^(e + emax + 1), one scale: nearest grid value."""
    table = spec_table(fmt)
    e = 0
    top = 2.0 ** (e + EMAX[fmt] + 1)
    allbits = np.arange(1, 0x7F80, dtype=np.uint16)
    vals = synth.bf16_to_f32(allbits).astype(np.float64)
    vals = vals[vals < top]
    bits, _ = _blocks_at_scale(fmt, e, vals)
    q, s = oracle_mod.quantize_fp6(bits, 0, fmt)
    deq = oracle_mod.dequantize_fp6(q, s, bits.shape[0], 32, fmt)[:, 1:32].reshape(-1)[:len(vals)]
    tf = np.array([float(t) for t in table])
    # nearest by distance, ties to even code (vectorised brute force over the table)
    dist = np.abs(vals[:, None] - tf[None, :])
    best = dist.min(axis=1, keepdims=True)
    ties = dist == best
    code = np.where(ties[:, ::2].any(axis=1) & (ties.sum(axis=1) > 1),
                    np.argmax(ties * (np.arange(32) % 2 == 0), axis=1), np.argmin(dist, axis=1))
    want = np.where(vals >= tf[-1], tf[-1], tf[code])
    assert np.array_equal(deq, want)


@pytest.mark.parametrize("fmt", [E2M3, E3M2])
def test_fp6_scale_rule_and_specials(oracle_mod, fmt):
    # amax in [2^k, 2^(k+1)) -> byte k - emax + 127; zero block -> 0; Inf/NaN block -> 0xFF, codes 0
    x = np.zeros((4, 128), dtype=np.float32)
    x[0, :32] = 1.5 * 2.0 ** 5
    x[0, 32:64] = 0.75
    x[1, :32] = np.inf
    x[1, 64] = np.nan
    x[2, 40] = -2.0 ** -100
    bits = synth.bf16_bits(x)
    q, s = oracle_mod.quantize_fp6(bits, 0, fmt)
    em = EMAX[fmt]
    assert s[0, 0] == 5 - em + 127 and s[0, 1] == -1 - em + 127 and s[0, 2] == 0 and s[0, 3] == 0
    assert s[1, 0] == 0xFF and s[1, 2] == 0xFF and s[1, 1] == 0
    assert s[2, 1] == -100 - em + 127
    assert (q[1, :24] == 0).all() and (q[1, 48:72] == 0).all()
    # scale clamps at 2^-127 for tiny blocks: amax 2^-130 -> e = -127 (byte 0)
    y = synth.bf16_bits(np.full((1, 32), 2.0 ** -130, dtype=np.float32))
    _, s2 = oracle_mod.quantize_fp6(y, 0, fmt)
    assert s2[0, 0] == 0


def test_fp6_packing_worked_bytes(oracle_mod):
    """Six bits per element, little-endian bit string: code k occupies bits [6k, 6k+6),
    so c0 | c1<<6 | c2<<12 | ... and element 5 straddles bytes 3 and 4 (worked by hand)."""
    # scale e = 0 (amax 4 = 2^(0+2)); E2M3 codes: 0.125 -> 1, 0.25 -> 2, 0.375 -> 3,
    # -0.5 -> 32|4 = 36, 4.0 -> exponent 3, mantissa 0 = 24, 0.875 -> 7
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :6] = [0.125, 0.25, 0.375, -0.5, 4.0, 0.875]
    q, s = oracle_mod.quantize_fp6(synth.bf16_bits(x), 0, E2M3)
    assert s[0, 0] == 127
    assert list(q[0, :5]) == [0x81, 0x30, 0x90, 0xD8, 0x01]
    assert (q[0, 5:] == 0).all() and q.shape == (1, 96)


def test_fp6_e2m3_contains_mxfp4(oracle_mod):
    """E2M1 magnitudes are E2M3 grid points and both formats take emax_elem = 2: on
    inputs whose scaled values sit on the E2M1 grid the two oracles agree exactly
    (independent encoders)."""
    rng = np.random.default_rng(3)
    e2m1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    x = rng.choice(e2m1, size=(40, 256)) * rng.choice([-1.0, 1.0], size=(40, 256))
    # one exponent per aligned 32x32 tile, so row blocks and column blocks both see a
    # single power of two; the tile diagonal carries 6 * 2^e
    ex = rng.integers(-5, 5, size=(2, 8)).repeat(32, axis=0)[:40].repeat(32, axis=1)
    x *= 2.0 ** ex
    r = np.arange(40)
    for b in range(8):
        x[r, 32 * b + r % 32] = 6.0 * 2.0 ** ex[r, 32 * b]
    bits = synth.bf16_bits(x.astype(np.float32))
    for d in (0, 1):
        q4, s4 = oracle_mod.quantize(bits, d)
        q6, s6 = oracle_mod.quantize_fp6(bits, d, E2M3)
        rows, length = (40, 256) if d == 0 else (256, 40)
        assert np.array_equal(s4, s6)
        assert np.array_equal(oracle_mod.dequantize(q4, s4, rows, length),
                              oracle_mod.dequantize_fp6(q6, s6, rows, length, E2M3))


@pytest.mark.parametrize("fmt", [E2M3, E3M2])
def test_fp6_sr_unbiased_and_bracketing(oracle_mod, fmt):
    """Stochastic rounding lands on one of the two neighbours, and the fraction
    rounded up matches floor(256 frac)/256 over many draws."""
    table = spec_table(fmt)
    lo, hi = table[20], table[21]
    frac = Fraction(3, 8)
    v = lo + frac * (hi - lo)
    e = 1
    n = 31 * 400
    bits, _ = _blocks_at_scale(fmt, e, [float(v * 2 ** e)] * n)
    q, s = oracle_mod.quantize_fp6(bits, 0, fmt, use_sr=True, seed=77, tensor_id=3)
    deq = oracle_mod.dequantize_fp6(q, s, bits.shape[0], 32, fmt)[:, 1:32].reshape(-1)[:n] / 2.0 ** e
    assert set(np.unique(deq)) <= {float(lo), float(hi)}
    up = float(np.mean(deq == float(hi)))
    p = float(Fraction(int(256 * frac), 256))
    assert abs(up - p) < 4 * np.sqrt(p * (1 - p) / n)
    # grid points never move, and values past the largest saturate
    bits2, _ = _blocks_at_scale(fmt, e, [float(table[7] * 2 ** e), float(table[31] * 2 ** e)])
    q2, s2 = oracle_mod.quantize_fp6(bits2, 0, fmt, use_sr=True, seed=5)
    d2 = oracle_mod.dequantize_fp6(q2, s2, 1, 32, fmt)[0, 1:3] / 2.0 ** e
    assert list(d2) == [float(table[7]), float(table[31])]


def test_fp6_sr_byte_rule(oracle_mod):
    """Each element's decision follows its own Philox byte: up iff byte < floor(256 frac)."""
    fmt = E3M2
    table = spec_table(fmt)
    e = 0
    vals, fr = [], []
    rng = np.random.default_rng(1)
    for _ in range(31 * 8):
        c = int(rng.integers(0, 31))
        f = Fraction(int(rng.integers(0, 4)), 4)
        vals.append(float(table[c] + f * (table[c + 1] - table[c])))
        fr.append((c, f))
    bits, _ = _blocks_at_scale(fmt, e, vals)
    q, s = oracle_mod.quantize_fp6(bits, 0, fmt, use_sr=True, seed=123, tensor_id=9)
    deq = oracle_mod.dequantize_fp6(q, s, bits.shape[0], 32, fmt)
    for t, (c, f) in enumerate(fr):
        r, col = divmod(t, 31)
        byte = oracle_mod.sr_byte(123, 9, 0, r * 32 + col + 1)
        want = table[c + 1] if byte < int(256 * f) else table[c]
        assert Fraction(deq[r, col + 1]) == want


def test_fp6_gemm_entries_match_dense_product(oracle_mod):
    rng = np.random.default_rng(4)
    M, N, K = 20, 12, 200
    a = synth.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    b = synth.bf16_bits((0.1 * rng.standard_normal((N, K))).astype(np.float32))
    for fa, fb in [(E2M3, E2M3), (E3M2, E2M3), (E3M2, E3M2)]:
        qa, sa = oracle_mod.quantize_fp6(a, 0, fa)
        qb, sb = oracle_mod.quantize_fp6(b, 0, fb)
        da = oracle_mod.dequantize_fp6(qa, sa, M, K, fa)
        db = oracle_mod.dequantize_fp6(qb, sb, N, K, fb)
        ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        got, gabs = oracle_mod.gemm_fp6_entries(qa, sa, fa, qb, sb, fb, M, N, K, ii.reshape(-1), jj.reshape(-1))
        ref = da @ db.T
        assert np.allclose(got.reshape(M, N), ref, rtol=1e-12, atol=1e-12)
        assert np.allclose(gabs.reshape(M, N), np.abs(da) @ np.abs(db).T, rtol=1e-12)
        # quantization error is within the grid spacing: |deq - x| <= 2^-mbits * 2^e relative
        xa = synth.bf16_to_f32(a).astype(np.float64)
        rel = np.abs(da[:, :K] - xa).max() / np.abs(xa).max()
        assert rel < (2.0 ** -3 if fa == E2M3 else 2.0 ** -2)


def test_fp6_to_tiled_places_every_byte(oracle_mod):
    """The tiled blob is a permutation of the canonical bytes plus zero padding:
    each 24-byte lane slice reappears as 16 bytes at 16*lane and 8 at 1024 + 8*lane."""
    rng = np.random.default_rng(6)
    rows, length = 37, 700
    x = synth.bf16_bits(rng.standard_normal((rows, length)).astype(np.float32))
    q, s = oracle_mod.quantize_fp6(x, 0, E3M2)
    qt, st = oracle_mod.fp6_to_tiled(q, s, rows, length)
    lp = 768
    ksteps = lp // 128
    for r in (0, 15, 16, 36):
        for kb in (0, 3, 4, 23):
            lane = (r % 16) + 16 * (kb % 4)
            atom = ((r // 16) * ksteps + kb // 4) * 1536
            got = np.concatenate([qt[atom + 16 * lane: atom + 16 * lane + 16],
                                  qt[atom + 1024 + 8 * lane: atom + 1024 + 8 * lane + 8]])
            assert np.array_equal(got, q[r, 24 * kb: 24 * kb + 24])
    assert qt.size == 48 * lp * 3 // 4 and int(qt.sum()) == int(q.astype(np.int64).sum())
    q4t, s4t = oracle_mod.to_tiled(np.zeros((rows, lp // 2), np.uint8), s, rows, length)
    assert np.array_equal(st, s4t)
