"""Pins of the oracle's stochastic rounding and of its Philox-4x32-10.

The Philox pin is rocRAND's own engine (an independent implementation of
Salmon et al., SC'11), compiled from its header here and fed counters and keys
directly.  The SR rule (round up iff r < floor(256 p)) is pinned statistically:
over 2^20 copies the round-up fraction must sit within 6 sigma of t/256, which
separates r < t from r <= t (a 1/256 shift, ~8 sigma).
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from mxfp4_precision_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _rocrand_available():
    return shutil.which("g++") and os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h")


@pytest.fixture(scope="module")
def rocrand_philox():
    if not _rocrand_available():
        pytest.skip("rocRAND headers or g++ missing")
    d = tempfile.mkdtemp()
    exe = os.path.join(d, "philox_ref")
    subprocess.check_call(["g++", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                           os.path.join(HERE, "philox_rocrand_ref.cpp"), "-o", exe])

    def run(rows):
        inp = "".join("%x %x %x %x %x %x\n" % tuple(int(v) for v in r) for r in rows)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return np.array([[int(w, 16) for w in line.split()] for line in out.strip().split("\n")],
                        dtype=np.uint32)
    yield run
    shutil.rmtree(d, ignore_errors=True)


def test_philox_against_rocrand(oracle_mod, rocrand_philox):
    rng = np.random.default_rng(42)
    rows = [(0, 0, 0, 0, 0, 0), (0xFFFFFFFF,) * 6, (1, 0, 0, 0, 0, 0), (0, 0, 0, 1, 0, 0),
            (0, 0, 0, 0, 7, 0), (5, 0, 2, 1, 7, 0)]
    rows += [tuple(int(v) for v in rng.integers(0, 2 ** 32, size=6)) for _ in range(200)]
    ref = rocrand_philox(rows)
    for r, want in zip(rows, ref):
        got = oracle_mod.philox4x32_10(np.array(r[:4]), np.array(r[4:]))
        assert (got == want).all(), r


def test_sr_byte_layout(oracle_mod, rocrand_philox):
    """Byte n%16 of the Philox block for counter (n>>4, tensor_id, dir), little-endian words."""
    seed = (3 << 32) | 7
    ns = [0, 1, 15, 16, 17, 1000003, (5 << 36) + 9]
    rows = []
    for n in ns:
        g = n >> 4
        rows.append((g & 0xFFFFFFFF, g >> 32, 2, 1, seed & 0xFFFFFFFF, seed >> 32))
    ref = rocrand_philox(rows)
    for n, words in zip(ns, ref):
        raw = words.astype("<u4").tobytes()
        assert oracle_mod.sr_byte(seed, 2, 1, n) == raw[n % 16]


def _sr_rows(value_bits, copies, seed, tensor_id=0):
    """Blocks of 32: element 0 anchors the scale at 2^0 (amax 4.0), the rest are copies."""
    per = 31
    nrow = -(-copies // per)
    x = np.zeros((nrow, 32), dtype=np.uint16)
    x[:, 0] = synth.bf16_bits(np.float32(4.0))
    x[:, 1:] = value_bits
    return x


@pytest.mark.parametrize("value,lo,hi", [
    (0.2578125, 0.0, 0.5),
    (1.0 + 1 / 64, 1.0, 1.5),
    (2.5, 2.0, 3.0),
    (3.984375, 3.0, 4.0),
    (5.0, 4.0, 6.0),
    (0.001953125, 0.0, 0.5),
])
def test_sr_rounding_rate(oracle_mod, value, lo, hi):
    """The round-up fraction over 2^20 copies is t/256 with t = floor(256 (v-lo)/(hi-lo))."""
    t = int(np.floor(256 * (value - lo) / (hi - lo)))
    bits = synth.bf16_bits(np.float32(value))
    assert synth.bf16_to_f32(bits) == np.float32(value)
    copies = 1 << 20
    x = _sr_rows(bits, copies, 0)
    q, s = oracle_mod.quantize(x, 0, use_sr=True, seed=1234, tensor_id=5)
    assert (s[:, 0] == 127).all()
    lo_code = int(np.searchsorted([0, 0.5, 1, 1.5, 2, 3, 4, 6], lo))
    nib = np.empty((q.shape[0], 2 * q.shape[1]), dtype=np.uint8)
    nib[:, 0::2] = q & 0xF
    nib[:, 1::2] = q >> 4
    got = nib[:, 1:32].ravel()
    assert set(np.unique(got).tolist()) <= {lo_code, lo_code + 1}
    frac = float((got == lo_code + 1).mean())
    p = t / 256
    sigma = max(np.sqrt(p * (1 - p) / got.size), 1 / got.size)
    assert abs(frac - p) <= 6 * sigma, (frac, p, sigma)


def test_sr_properties(oracle_mod):
    x = synth.random_bf16(21, (64, 256), std=0.7)
    q1, s1 = oracle_mod.quantize(x, 0, use_sr=True, seed=7, tensor_id=2)
    q2, s2 = oracle_mod.quantize(x, 0, use_sr=True, seed=7, tensor_id=2)
    q3, s3 = oracle_mod.quantize(x, 0, use_sr=True, seed=8, tensor_id=2)
    q4, _ = oracle_mod.quantize(x, 0, use_sr=True, seed=7, tensor_id=3)
    qr, sr = oracle_mod.quantize(x, 0)
    assert (q1 == q2).all() and (s1 == s2).all()          # deterministic
    assert (q1 != q3).any() and (q1 != q4).any()          # keyed
    assert (s1 == sr).all() and (s3 == sr).all()          # scale never depends on SR
    # SR result is one of the two neighbours: |deq_sr - x| < grid spacing
    deq = oracle_mod.dequantize(q1, s1, 64, 256)
    deqr = oracle_mod.dequantize(qr, sr, 64, 256)
    spacing = 2.0 ** (np.repeat(s1.astype(float), 32, axis=1) - 127) * 2
    assert (np.abs(deq - deqr) <= spacing).all()


def test_sr_grid_points_fixed(oracle_mod):
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -6, -3, 1], dtype=np.float32)
    x = np.tile(np.concatenate([grid, np.zeros(20, np.float32)]), (50, 1))
    x[:, 7] = 6.0
    bits = synth.bf16_bits(x)
    qs, ss = oracle_mod.quantize(bits, 0, use_sr=True, seed=99)
    qr, sr = oracle_mod.quantize(bits, 0)
    assert (qs == qr).all() and (ss == sr).all()


def test_sr_index_base_shift(oracle_mod):
    """index_base shifts the element index: a tensor quantized as the lower half of a
    larger one (index_base = rows*N) matches that half of the larger result."""
    x = synth.random_bf16(22, (64, 128))
    qa, sa = oracle_mod.quantize(x, 0, use_sr=True, seed=5, tensor_id=1)
    qb, sb = oracle_mod.quantize(x[32:], 0, use_sr=True, seed=5, tensor_id=1, index_base=32 * 128)
    assert (qa[32:] == qb).all() and (sa[32:] == sb).all()


def test_sr_uniform_bytes(oracle_mod):
    """Chi-square of 65536 SR bytes over 256 bins (loose bound; catches stuck bits)."""
    b = np.array([oracle_mod.sr_byte(11, 0, 0, n) for n in range(65536)])
    h = np.bincount(b, minlength=256)
    chi2 = float(((h - 256.0) ** 2 / 256.0).sum())
    assert 150 < chi2 < 380, chi2
