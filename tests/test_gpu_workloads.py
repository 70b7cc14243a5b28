"""Full-size parity: the decode block at the workload shapes, in the launch
configuration bench.py times (automatic split count), against the oracle's
complete fp64 block on the same seeded inputs.

Bounds (block output relative RMS <= 1e-2, attention max-abs/RMS <= 2e-2)
as in the stage tests; the appended token's codes are reported (they can
differ from the oracle's only where the bf16 rounding of the new k or v
differs between an fp32 and an fp64 projection).
"""
import numpy as np
import pytest

import oracle as O
from int4_quantized_decode_amd import synth
from tests.gpu_helpers import say
from tests.test_gpu_stages import check_block, gpu, run_block  # noqa: F401

pytestmark = pytest.mark.gpu


def _workload(name):
    wl = synth.WORKLOADS[name]
    return wl, synth.make_lengths(wl)


def test_1b_layer_m1_ctx256(gpu):
    wl, lengths = _workload("1b_m1_ctx256")
    check_block(run_block(gpu, wl.shape, wl.seed, lengths), wl.name)


def test_8b_layer_m1_ctx4096(gpu):
    wl, lengths = _workload("8b_m1_ctx4096")
    check_block(run_block(gpu, wl.shape, wl.seed, lengths), wl.name)


def test_8b_layer_m32_ragged(gpu):
    wl, lengths = _workload("8b_m32_ragged")
    assert lengths.min() >= 1024 and lengths.max() <= 4096 and len(set(lengths.tolist())) > 16
    check_block(run_block(gpu, wl.shape, wl.seed, lengths), wl.name)


@pytest.fixture(scope="module")
def layer70(gpu):
    wl = synth.WORKLOADS["70b_ctx4096"]
    say("generating the 70B-shape layer")
    lw = synth.make_layer(wl.shape, wl.seed)
    return wl, lw, {}, {}


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 16, 32])
def test_70b_layer_ctx4096(gpu, layer70, M):
    wl, lw, dense, memo = layer70
    lengths = synth.make_lengths(wl, M)
    check_block(run_block(gpu, wl.shape, wl.seed, lengths, dense_cache=dense, lw=lw, memo=memo),
                f"{wl.name} M={M}")


def test_8b_layer_m1_ctx32768_16_splits(gpu):
    """One layer of the full-model workload (8B shape, context 32768, 16 KV
    splits: the split count bench.py's full-model run passes), through the
    one-launch step."""
    wl = synth.WORKLOADS["8b_32layer_ctx32768"]
    lengths = synth.make_lengths(wl)
    assert int(lengths[0]) == 32768 and wl.num_splits == 16
    check_block(run_block(gpu, wl.shape, wl.seed, lengths, num_splits=wl.num_splits), "8b_ctx32768 S=16")
