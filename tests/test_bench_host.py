"""bench.py's host-side helpers (no GPU): the byte counts it divides by and
the traffic table lookup."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from int4_quantized_decode_amd import synth  # noqa: E402


def test_algorithmic_bytes_8b_ctx4096():
    # 8B layer at one row and context 4096: 112,459,776 weight + scale bytes
    # and 4096 tokens x 8 kv heads x 2 x (64 + 2) bytes of cache
    total, w, kv = bench.algorithmic_bytes(synth.SHAPE_8B, np.array([4096]))
    assert w == 112_459_776
    assert kv == 4096 * 8 * 2 * 66
    assert total == 116_785_152


def test_gate_up_bytes_8b():
    assert bench.gate_up_bytes(synth.SHAPE_8B) == 60_555_264


def test_traffic_lookup_requires_matching_kernel():
    assert bench.traffic_of("8b_m1_ctx4096", "some other kernel") is None
    assert bench.traffic_of("no such workload", "step_m1_kernel (one-launch decode step)") is None
