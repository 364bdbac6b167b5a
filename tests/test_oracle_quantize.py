"""Pins of the oracle's quantizer against things other than itself.

Hand tables and a hand-worked block (OCP MX v1.0 definitions, typed in
tests/golden/), an exhaustive nearest-grid brute force (a different algorithm
from the oracle's midpoint table), round-trip and scaling invariants, the
dual/2D consistency identities, and the blob-size contract of the fake
dual-quantize op on the page "primus_turbo_mxfp4_local.py".
"""
import json
import math
import os

import numpy as np
import pytest

from mxfp4_precision_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def bf16(values):
    return synth.bf16_bits(np.asarray(values, dtype=np.float32))


def bf16_val(bits):
    return synth.bf16_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def parse_amount(s):
    if s == "bf16max":
        return (2.0 - 2.0 ** -7) * 2.0 ** 127
    if s.startswith("2^"):
        return 2.0 ** int(s[2:])
    return float(s)


def nibbles_of(q, length):
    """Split canonical data bytes into nibbles along the row (element 2j low)."""
    lo = q & 0xF
    hi = q >> 4
    out = np.empty((q.shape[0], q.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


# ----------------------------------------------------------------- tables

def test_e2m1_nibble_table(oracle_mod):
    """P1: dequantizing each nibble at scale 2^0 gives the OCP E2M1 table."""
    tab = json.load(open(os.path.join(GOLDEN, "e2m1_e8m0.json")))["e2m1_nibble_values"]
    q = np.zeros((1, 64), dtype=np.uint8)
    for n in range(16):
        q[0, n // 2] |= (n << 4) if n % 2 else n
    s = np.full((1, 4), 127, dtype=np.uint8)
    d = oracle_mod.dequantize(q, s, 1, 128)[0]
    for n in range(16):
        want = tab[str(n)]
        assert d[n] == want and math.copysign(1.0, d[n]) == math.copysign(1.0, want), n


def test_e8m0_values(oracle_mod):
    """E8M0 byte b scales by 2^(b-127); 0xFF is NaN."""
    tab = json.load(open(os.path.join(GOLDEN, "e2m1_e8m0.json")))["e8m0_byte_values"]
    for b, v in tab.items():
        q = np.full((1, 64), 0x22, dtype=np.uint8)  # every element 1.0
        s = np.full((1, 4), int(b), dtype=np.uint8)
        d = oracle_mod.dequantize(q, s, 1, 128)[0, 0]
        if v == "NaN":
            assert math.isnan(d)
        else:
            assert d == 2.0 ** int(v[2:])


def test_scale_hand_cases(oracle_mod):
    """P2: hand-worked amax -> E8M0 byte (and the amax element's nibble)."""
    cases = json.load(open(os.path.join(GOLDEN, "e2m1_e8m0.json")))["scale_cases"]
    for c in cases:
        a = parse_amount(c["amax"])
        x = np.zeros((1, 32), dtype=np.float64)
        x[0, 5] = a
        bits = synth.bf16_bits(x.astype(np.float32))
        assert bf16_val(bits)[0, 5] == a, c  # every hand value is exact in bf16
        q, s = oracle_mod.quantize(bits, 0)
        assert s[0, 0] == c["scale_byte"], c
        assert s.shape == (1, 4) and list(s[0, 1:]) == [0, 0, 0]  # pad-only blocks
        if "amax_nibble" in c:
            assert nibbles_of(q, 128)[0, 5] == c["amax_nibble"], c


def test_worked_block(oracle_mod):
    """P4: the hand-worked 8-element block."""
    wb = json.load(open(os.path.join(GOLDEN, "e2m1_e8m0.json")))["worked_block"]
    vals = [float(v) for v in wb["values"]] + [0.0] * (32 - len(wb["values"]))
    bits = bf16(np.array(vals).reshape(1, 32))
    assert bits[0, 7] == 0x8000  # -0.0 kept
    q, s = oracle_mod.quantize(bits, 0)
    assert s[0, 0] == wb["scale_byte"]
    assert list(nibbles_of(q, 128)[0, :8]) == wb["nibbles"]
    assert list(q[0, :4]) == wb["bytes_first4"]
    assert not q[0, 4:].any()


# --------------------------------------------------- exhaustive brute force

def nearest_even_code(v):
    """Nearest E2M1 magnitude by exhaustive search; ties -> even code (vectorised)."""
    d = np.abs(v[:, None] - GRID[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates prefer the even code
    codes = np.arange(8)[None, :]
    even = cand & (codes % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return pick


def all_finite_bf16_magnitudes():
    m = np.arange(0x7F80, dtype=np.uint16)  # every finite non-negative pattern
    return m


def test_exhaustive_rne_against_nearest_search(oracle_mod):
    """P3: every finite bf16 magnitude, at every scale exponent that can hold it,
    rounds to the nearest E2M1 value (ties to even, saturating at 6)."""
    mags = all_finite_bf16_magnitudes()
    mval = bf16_val(mags)
    rows_bits = []
    expect = []
    for e in range(-127, 126):
        anchor = 4.0 * 2.0 ** e          # fixes the block scale at e while |x| < 8*2^e
        lim = 8.0 * 2.0 ** e
        sel = mval < lim
        if e > -120:
            sel &= mval >= 2.0 ** (e - 10)   # below this every value rounds to 0; covered at e <= -120
        xs = mags[sel]
        if xs.size == 0:
            continue
        v = mval[sel] / 2.0 ** e
        code = nearest_even_code(v)
        # random signs, deterministic
        sign = (np.arange(xs.size) * 2654435761 % 7 < 3).astype(np.uint16)
        xs = xs | (sign << 15)
        nib = (sign.astype(np.int64) << 3) | code
        n = xs.size
        per = 31
        nrow = -(-n // per)
        blk = np.zeros((nrow, 32), dtype=np.uint16)
        want = np.zeros((nrow, 32), dtype=np.int64)
        anchor_bits = bf16(np.float32(anchor))
        blk[:, 0] = anchor_bits
        want[:, 0] = 6
        flat = np.zeros(nrow * per, dtype=np.uint16)
        flat[:n] = xs
        wflat = np.zeros(nrow * per, dtype=np.int64)
        wflat[:n] = nib
        blk[:, 1:] = flat.reshape(nrow, per)
        want[:, 1:] = wflat.reshape(nrow, per)
        rows_bits.append(blk)
        expect.append((e, want))
    X = np.concatenate(rows_bits)
    q, s = oracle_mod.quantize(X, 0)
    nib = nibbles_of(q, 128)[:, :32]
    r0 = 0
    for e, want in expect:
        r1 = r0 + want.shape[0]
        assert (s[r0:r1, 0] == e + 127).all(), e
        bad = np.nonzero(nib[r0:r1] != want)
        assert bad[0].size == 0, (e, bad[0][:5], bad[1][:5])
        r0 = r1


def test_subnormal_and_clamped_scale(oracle_mod):
    """Blocks whose amax is tiny clamp the exponent at -127; elements then scale by 2^127."""
    x = np.zeros((1, 32), dtype=np.float64)
    x[0, 0] = 2.0 ** -127   # bf16 subnormal
    x[0, 1] = 2.0 ** -128
    x[0, 2] = 3 * 2.0 ** -129
    bits = bf16(x)
    assert bf16_val(bits)[0, 0] == 2.0 ** -127
    q, s = oracle_mod.quantize(bits, 0)
    assert s[0, 0] == 0
    nib = nibbles_of(q, 128)[0]
    # v = x * 2^127: 1.0 -> code 2; 0.5 -> code 1; 0.75 -> tie -> code 2
    assert list(nib[:3]) == [2, 1, 2]


def test_nonfinite_block(oracle_mod):
    """A block holding Inf or NaN gets scale 0xFF and all-zero nibbles; others unaffected."""
    x = np.ones((2, 64), dtype=np.float32)
    x[0, 3] = np.inf
    x[1, 40] = np.nan
    bits = bf16(x)
    q, s = oracle_mod.quantize(bits, 0)
    assert s[0, 0] == 0xFF and s[0, 1] == 125
    assert s[1, 0] == 125 and s[1, 1] == 0xFF
    nib = nibbles_of(q, 128)
    assert not nib[0, :32].any() and (nib[0, 32:64] == 6).all()  # 1.0 at scale 2^-2 is 4.0
    assert (nib[1, :32] == 6).all() and not nib[1, 32:64].any()


def test_padding_and_zero_blocks(oracle_mod):
    """Axis padded to 128 with +0 nibbles; pad-only and all-zero blocks get scale 0."""
    x = synth.random_bf16(11, (3, 200))
    x[1, 32:64] = 0
    q, s = oracle_mod.quantize(x, 0)
    assert q.shape == (3, 128) and s.shape == (3, 8)
    nib = nibbles_of(q, 256)
    assert not nib[:, 200:].any()
    assert (s[:, 7] == 0).all()          # blocks 224..255: pad only
    assert s[1, 1] == 0 and not nib[1, 32:64].any()
    assert (s[:, 6] != 0).all()           # block 192..223 holds 8 real elements


# ------------------------------------------------------------- invariants

def test_roundtrip_rne_1d(oracle_mod):
    """P5: quantize(dequantize(q)) == q (dequantized values are exact in bf16)."""
    x = synth.random_bf16(5, (64, 300))
    x[3, :] = 0
    x[7, 10] = 0x8000
    for d in (0, 1):
        q, s = oracle_mod.quantize(x, d)
        rows, length = (64, 300) if d == 0 else (300, 64)
        deq = oracle_mod.dequantize(q, s, rows, length)[:, :length]
        xb = oracle_mod.bf16_from_double(deq)
        assert (bf16_val(xb) == deq).all()
        q2, s2 = oracle_mod.quantize(xb, 0)
        assert (q2 == q).all() and (s2 == s).all()


@pytest.mark.parametrize("mode", ["sr", "2d"])
def test_roundtrip_modes(oracle_mod, mode):
    x = synth.random_bf16(6, (96, 160), std=3.0)
    kw = dict(use_sr=True, seed=9, tensor_id=3) if mode == "sr" else dict(use_2d=True)
    q, s = oracle_mod.quantize(x, 0, **kw)
    deq = oracle_mod.dequantize(q, s, 96, 160)[:, :160]
    xb = oracle_mod.bf16_from_double(deq)
    q2, s2 = oracle_mod.quantize(xb, 0, **kw)
    assert (q2 == q).all() and (s2 == s).all()


def test_power_of_two_scaling(oracle_mod):
    """P6: x * 2^k keeps every nibble and shifts every scale byte by k."""
    x = synth.random_bf16(7, (16, 256))
    q, s = oracle_mod.quantize(x, 0)
    for k in (-20, -1, 1, 9):
        xk = bf16(bf16_val(x) * 2.0 ** k)
        qk, sk = oracle_mod.quantize(xk, 0)
        assert (qk == q).all()
        assert (sk.astype(int) == s.astype(int) + k).all()


def test_sign_flip_and_permutation(oracle_mod):
    x = synth.random_bf16(8, (8, 128))
    q, s = oracle_mod.quantize(x, 0)
    qn, sn = oracle_mod.quantize(x ^ np.uint16(0x8000), 0)
    assert (sn == s).all()
    assert (nibbles_of(qn, 128) == (nibbles_of(q, 128) ^ 8)).all()
    perm = np.random.default_rng(0).permutation(32)
    xp = x.copy()
    xp[:, :32] = x[:, :32][:, perm]
    qp, sp = oracle_mod.quantize(xp, 0)
    assert (sp == s).all()
    assert (nibbles_of(qp, 128)[:, :32] == nibbles_of(q, 128)[:, :32][:, perm]).all()


def test_saturation_bound(oracle_mod):
    """Every dequantized element lies within +-6 * 2^e of its block and keeps x's sign."""
    x = synth.random_bf16(12, (32, 512), std=10.0)
    q, s = oracle_mod.quantize(x, 0)
    deq = oracle_mod.dequantize(q, s, 32, 512)
    scale = 2.0 ** (np.repeat(s.astype(np.float64), 32, axis=1) - 127)
    assert (np.abs(deq) <= 6 * scale).all()
    xv = bf16_val(x)
    nz = deq != 0
    assert (np.sign(deq[nz]) == np.sign(xv[nz])).all()


def test_dual_consistency(oracle_mod):
    """P7: colwise(X) == rowwise(X^T), byte-exact including padding (RNE, 1D and 2D)."""
    x = synth.random_bf16(13, (200, 72))
    for two_d in (False, True):
        qc, sc = oracle_mod.quantize(x, 1, use_2d=two_d)
        qr, sr = oracle_mod.quantize(np.ascontiguousarray(x.T), 0, use_2d=two_d)
        assert (qc == qr).all() and (sc == sr).all()


def test_2d_consistency(oracle_mod):
    """P8: with 2D blocks and RNE, colwise codes transposed equal rowwise codes and
    every scale is constant over its 32x32 tile."""
    M, N = 96, 160
    x = synth.random_bf16(14, (M, N), std=2.0)
    qr, sr = oracle_mod.quantize(x, 0, use_2d=True)
    qc, sc = oracle_mod.quantize(x, 1, use_2d=True)
    nr = nibbles_of(qr, 256)[:, :N]
    nc = nibbles_of(qc, 128)[:, :M]
    assert (nr == nc.T).all()
    for ti in range(M // 32):
        for tj in range(N // 32):
            tile = sr[32 * ti:32 * ti + 32, tj]
            assert (tile == tile[0]).all()
            assert (sc[32 * tj:32 * tj + 32, ti] == tile[0]).all()
    # 2D scale is the scale of the tile's amax
    xv = np.abs(bf16_val(x))
    amax = xv[0:32, 32:64].max()
    assert sr[0, 1] == math.floor(math.log2(amax)) - 2 + 127


def test_size_contract(oracle_mod):
    """P9: blob shapes equal the fake dual-quantize op's formulas (page
    "primus_turbo_mxfp4_local.py"): row data (M, N_pad/2), row scale
    (M, cdiv(N_pad,32)), col data (N, M_pad/2), col scale (N, cdiv(M_pad,32))."""
    for M, N in [(1, 1), (4600, 3072), (127, 129), (256, 512), (33, 4600)]:
        Mp = -(-M // 128) * 128
        Np = -(-N // 128) * 128
        x = np.zeros((M, N), dtype=np.uint16)
        qr, sr = oracle_mod.quantize(x, 0)
        qc, sc = oracle_mod.quantize(x, 1)
        assert qr.shape == (M, Np // 2) and sr.shape == (M, -(-Np // 32))
        assert qc.shape == (N, Mp // 2) and sc.shape == (N, -(-Mp // 32))


def test_strided_input_equals_contiguous(oracle_mod):
    """ldx > N reads only the first N elements of each row."""
    x = synth.random_bf16(15, (10, 100))
    big = np.full((10, 136), 0x7FC0, dtype=np.uint16)  # NaN in the gap
    big[:, :100] = x
    import ctypes
    L = oracle_mod.lib()
    q = np.zeros((10, 64), dtype=np.uint8)
    s = np.zeros((10, 4), dtype=np.uint8)
    L.oracle_quantize(big.ctypes.data, 10, 100, 136, 0, 0, 0, 0, 0, 0, 0, q.ctypes.data, s.ctypes.data)
    q0, s0 = oracle_mod.quantize(x, 0)
    assert (q == q0).all() and (s == s0).all()


# -------------------------------------------------------------- tiled layout

def test_tiled_layout_hand_offsets(oracle_mod):
    """The oracle's tiled permutation puts hand-picked elements where the layout's
    definition (worked by hand) says."""
    g = json.load(open(os.path.join(GOLDEN, "tiled_layout.json")))
    R, L = g["shape"]["rows"], g["shape"]["length"]
    Lp = g["shape"]["L_pad"]
    for e in g["data"]:
        q = np.zeros((R, Lp // 2), dtype=np.uint8)
        s = np.zeros((R, Lp // 32), dtype=np.uint8)
        r, k = e["r"], e["k"]
        q[r, k // 2] = (0x5 << 4) if k % 2 else 0x5
        qt, st = oracle_mod.to_tiled(q, s, R, L)
        nz = np.nonzero(qt)[0]
        assert list(nz) == [e["byte"]], e
        assert qt[e["byte"]] == (0x50 if e["high"] else 0x05), e
    for e in g["scale"]:
        q = np.zeros((R, Lp // 2), dtype=np.uint8)
        s = np.zeros((R, Lp // 32), dtype=np.uint8)
        s[e["r"], e["kb"]] = 0x9A
        qt, st = oracle_mod.to_tiled(q, s, R, L)
        assert list(np.nonzero(st)[0]) == [e["byte"]], e


def test_tiled_layout_is_a_permutation(oracle_mod):
    R, L = 37, 640
    rng = np.random.default_rng(1)
    q = rng.integers(0, 256, size=(R, L // 2), dtype=np.uint8)
    s = rng.integers(1, 256, size=(R, L // 32), dtype=np.uint8)
    qt, st = oracle_mod.to_tiled(q, s, R, L)
    assert qt.size == 48 * 320 and st.size == 48 * 2 * 16
    # same multiset of nibbles (padding rows add zeros only)
    def hist(a):
        return np.bincount(np.concatenate([a & 0xF, a >> 4]).ravel(), minlength=16)
    h = hist(q.ravel())
    ht = hist(qt)
    ht[0] -= (qt.size - q.size) * 2
    assert (h == ht).all()
    assert sorted(st[st != 0].tolist()) == sorted(s.ravel().tolist())
