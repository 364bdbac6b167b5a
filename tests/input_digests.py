"""Check seeded inputs against the SHA-256 digests recorded in
tests/golden/input_sha256.json (written by tests/golden/make_input_hashes.py)."""
import hashlib
import json
import os

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "input_sha256.json")
_REC = None


def check(config, tensors):
    """Assert that every tensor of `config` (name -> bf16 bits) matches its digest."""
    global _REC
    if _REC is None:
        _REC = json.load(open(_PATH))["inputs"]
    for name, bits in tensors.items():
        want = _REC["%s.%s" % (config, name)]
        assert list(bits.shape) == want["shape"], (config, name, bits.shape)
        got = hashlib.sha256(bits.tobytes()).hexdigest()
        assert got == want["sha256"], "%s.%s: seeded input drifted (%s)" % (config, name, got)
