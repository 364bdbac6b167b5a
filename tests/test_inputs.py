"""The seeded synthetic inputs are the recorded ones (SHA-256 of their bf16
bytes).  The small configurations are checked here; the fc1 and fc2 inputs,
slow to draw on a small host, are checked by the GPU tests that use them."""
from mxfp4_precision_amd import synth

import input_digests


def test_small_inputs_match_recorded_digests():
    for name, fn in (("tiny", synth.tiny), ("dual", synth.dual), ("qkv", synth.qkv)):
        input_digests.check(name, fn())
