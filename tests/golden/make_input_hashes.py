"""Write tests/golden/input_sha256.json: SHA-256 of the bf16 bytes of every
seeded synthetic input (mxfp4_precision_amd.synth), so that a change in the
generator or in numpy's streams shows up as a failing CPU test instead of as
silently different parity and benchmark inputs.  The digests describe the
inputs only; no expected output of the method is stored here.

Usage: python tests/golden/make_input_hashes.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from mxfp4_precision_amd import synth  # noqa: E402


def digests():
    out = {}
    for name, fn in (("tiny", synth.tiny), ("dual", synth.dual), ("qkv", synth.qkv), ("fc1", synth.fc1),
                     ("fc2", synth.fc2)):
        for tensor, bits in fn().items():
            out["%s.%s" % (name, tensor)] = {"shape": list(bits.shape),
                                             "sha256": hashlib.sha256(bits.tobytes()).hexdigest()}
    return out


if __name__ == "__main__":
    rec = {"_source": "SHA-256 of the uint16 (bf16) bytes, row-major, of each seeded input of "
                      "mxfp4_precision_amd/synth.py, written by tests/golden/make_input_hashes.py",
           "inputs": digests()}
    with open(os.path.join(HERE, "input_sha256.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print("wrote", len(rec["inputs"]), "digests")
