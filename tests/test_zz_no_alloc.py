"""The no-allocation decode step (i4d_decode_block_step_noalloc) against
the workspace entry point (i4d_decode_block_step) on the same inputs,
through the C ABI: outputs and attention bit-identical (the same kernels on
the same inputs; both match the oracle, which the other block tests check),
over consecutive calls on the library's one scratch array, each later call
smaller than the one before (fewer rows, another layout of the
intermediates, the one-launch step), and again after a larger call."""
import numpy as np
import pytest

import oracle as O
from int4_quantized_decode_amd import synth
from tests.gpu_helpers import norm_maxabs, rel_rms, say
from tests.test_gpu_stages import SPLIT_SHAPE, gpu  # noqa: F401

pytestmark = pytest.mark.gpu


def _inputs(torch, D, shape, seed, lengths):
    lengths = np.asarray(lengths, np.int32)
    M = len(lengths)
    lw = synth.make_layer(shape, seed)
    pre = synth.make_cache_prefill(shape, lengths, seed)
    layer = D.DeviceLayer(shape, lw)
    caches = []
    for _ in range(2):
        c = D.DeviceCache(shape, lengths)
        c.prefill(pre)
        caches.append(c)
    x = D.to_device_u16(synth.make_x(shape, M, seed))
    ctx = torch.from_numpy(lengths).cuda()
    return lw, pre, layer, caches, x, ctx, lengths


def _compare(gpu, shape, seed, lengths, check_oracle=False):
    torch, B, D = gpu
    lw, pre, layer, caches, x, ctx, lengths = _inputs(torch, D, shape, seed, lengths)
    M, maxL = len(lengths), int(lengths.max())
    nq = shape.n_q_heads * shape.head_dim
    ws = D.Workspace(shape, M, maxL, 0)
    out_ref = torch.empty_like(x)
    out_na = torch.full_like(x, 0x7fff)
    att_ref = torch.empty((M, nq), dtype=torch.float32, device="cuda")
    att_na = torch.full((M, nq), float("nan"), dtype=torch.float32, device="cuda")
    say(f"no-alloc step d={shape.d_model} M={M} maxL={maxL}")
    B.i4d_decode_block_step(layer.struct, caches[0].struct, x, out_ref, ctx, M, maxL, 0, ws.buf, ws.nbytes, att_ref)
    B.i4d_decode_block_step_noalloc(layer.struct, caches[1].struct, x, out_na, ctx, M, maxL, 0, att_na)
    torch.cuda.synchronize()
    assert caches[0].errors() == 0 and caches[1].errors() == 0
    assert torch.equal(out_ref, out_na)
    assert torch.equal(att_ref, att_na)
    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
        assert torch.equal(getattr(caches[0], name), getattr(caches[1], name)), name
    if check_oracle:
        ref = O.decode_block(shape, O.quantize_layer(lw), O.build_cache(shape, lengths, pre),
                             synth.make_x(shape, M, seed), lengths)
        assert rel_rms(D.bf16_tensor_to_f32(out_na), ref.out) <= 1e-2
        assert norm_maxabs(att_na.cpu().numpy(), ref.attn) <= 2e-2


def test_noalloc_matches_workspace_step_on_consecutive_calls(gpu):
    rng = np.random.default_rng(3)
    # 32 rows with the K split of the down projection (split counters and
    # partials), then 5 rows, then one row (the one-launch step: its sync
    # counters), then 32 rows again
    _compare(gpu, SPLIT_SHAPE, 41, list(rng.integers(1, 600, 32)), check_oracle=True)
    _compare(gpu, synth.SHAPE_SMALL128, 42, [300, 33, 1, 64, 129])
    _compare(gpu, synth.LayerShape(1024, 8, 2, 128, 2048), 43, [700])
    _compare(gpu, SPLIT_SHAPE, 44, list(rng.integers(1, 600, 32)))


def test_noalloc_rejects_oversized_step(gpu):
    torch, B, D = gpu
    shape = synth.SHAPE_SMALL128   # 32 rows x 8 heads x 256 splits: 34 MB of split partials
    lengths = np.full(32, 4096, np.int32)
    cache = D.DeviceCache(shape, lengths)
    x = torch.zeros((32, shape.d_model), dtype=torch.int16, device="cuda")
    ctx = torch.from_numpy(lengths).cuda()
    layer = D.DeviceLayer(shape, synth.make_layer(shape, 1))
    with pytest.raises(B.I4DError) as ei:
        B.i4d_decode_block_step_noalloc(layer.struct, cache.struct, x, torch.empty_like(x), ctx, 32, 4096, 256)
    assert ei.value.status == -5
