"""Regression snapshot of the oracle on the 64-token fp32 reference workload (CPU only).

The pages print no worked example for this step, so this fixture is not a pin of correctness
(the pins in oracle_pins.py are); it catches drift of the oracle or the input generator.
"""
import json
import os

from golden.make_golden import OUT, snapshot


def test_tiny_ref_snapshot():
    with open(OUT) as f:
        stored = json.load(f)
    now = snapshot()
    assert now["input_sha256"] == stored["input_sha256"], "input generator drifted"
    assert now == stored, "oracle output drifted from the stored snapshot"
