"""GPU parity of the E4M3 decode-weight variant (reading R12 of the oracle:
the summary page's "premises and limits" section reports E4M3 decode
weights beside the INT4 path) against the CPU oracle, through the C ABI.

* the decode of every E4M3 code by the projection kernel is exact: with a
  one-hot input row and a zero residual the O stage returns a weight column,
  which must equal the oracle's dequantized weight bit for bit (an E4M3
  value times an fp16 scale is exact in fp32), at M = 1 and 17 (one and two
  x tiles);
* the whole block with E4M3 weights: block output rel-RMS <= 1e-2 and
  attention max-abs/RMS <= 2e-2 against the oracle's fp64 block on the
  same E4M3 grid, with the appended token bit-exact, at small shapes and at
  the 8B (M = 1, context 4096) and 70B (M = 1, 32; context 4096) shapes.
"""
import numpy as np
import pytest

import oracle as O
from int4_quantized_decode_amd import synth
from tests.gpu_helpers import assert_appended_exact, norm_maxabs, rel_rms, say

pytestmark = pytest.mark.gpu

REL_TOL = 1e-2
ATT_TOL = 2e-2


@pytest.fixture(scope="module")
def gpu():
    import torch
    from int4_quantized_decode_amd import binding as B
    from int4_quantized_decode_amd import device as D
    assert torch.cuda.is_available()
    B.lib()
    return torch, B, D


def _all_code_weights(rng, N, K):
    """W whose E4M3 codes run over all 254 finite codes and whose every
    128-group holds +-448 * 2^-6, so the scale is exactly 2^-6 and the
    codes are the chosen ones."""
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    codes = finite[np.arange(N * K) % finite.size].reshape(N, K)
    codes = codes[rng.permutation(N)][:, rng.permutation(K)].copy()
    g = codes.reshape(N, K // 128, 128)
    g[:, :, 0] = np.where(rng.random((N, K // 128)) < 0.5, 0x7E, 0xFE)
    W = (O.e4m3_decode(codes) * 2.0 ** -6).astype(np.float32)
    q, s, _ = O.quantize_weight_e4m3(W)
    assert np.all(s.astype(np.float64) == 2.0 ** -6) and np.array_equal(q, codes)
    return W, q, s


@pytest.mark.parametrize("M", [1, 17])
def test_e4m3_decode_exact_through_the_o_stage(gpu, M):
    torch, B, D = gpu
    shape = synth.LayerShape(256, 4, 2, 64, 512)
    rng = np.random.default_rng(M)
    d, K = shape.d_model, shape.n_q_heads * shape.head_dim
    lw = synth.make_layer(shape, 3)
    W, q, s = _all_code_weights(rng, d, K)
    lw.w_o = W
    layer = D.DeviceLayer(shape, lw, fmt="e4m3")
    W_hat = O.dense((q, s, "e4m3"))
    x = torch.zeros((M, d), dtype=torch.int16, device="cuda")
    h32 = torch.empty((M, d), dtype=torch.float32, device="cuda")
    h16 = torch.empty((M, d), dtype=torch.int16, device="cuda")
    covered = 0
    for k0 in range(0, K, M):
        ks = [min(k0 + m, K - 1) for m in range(M)]
        onehot = np.zeros((M, K), np.float32)
        onehot[np.arange(M), ks] = 1.0
        attn = D.to_device_u16(synth.f32_to_bf16_bits(onehot))
        B.i4d_attn_out_proj_e4m3(layer.struct, attn, x, M, h32, h16)
        torch.cuda.synchronize()
        got = h32.cpu().numpy().astype(np.float64)
        np.testing.assert_array_equal(got, W_hat[:, ks].T)
        covered += M
    say(f"e4m3 decode exact over {K} columns x {d} rows (all 254 finite codes), M={M}")


def _run_block_e4m3(gpu, shape, seed, lengths, lw=None, memo=None):
    torch, B, D = gpu
    lengths = np.asarray(lengths, np.int32)
    M = len(lengths)
    memo = {} if memo is None else memo
    lw = lw or synth.make_layer(shape, seed)
    if "layer" not in memo:
        memo["layer"] = D.DeviceLayer(shape, lw, fmt="e4m3")
        memo["ql"] = O.quantize_layer_e4m3(lw)
        memo["dense"] = {}
    pre = synth.make_cache_prefill(shape, lengths, seed)
    xb = synth.make_x(shape, M, seed)
    cache = D.DeviceCache(shape, lengths)
    cache.prefill(pre)
    maxL = int(lengths.max())
    ws = D.Workspace(shape, M, maxL, 0)
    x_in = D.to_device_u16(xb)
    x_out = torch.empty_like(x_in)
    ctx = torch.from_numpy(lengths).cuda()
    attn = torch.empty((M, shape.n_q_heads * shape.head_dim), dtype=torch.float32, device="cuda")
    say(f"e4m3 block d={shape.d_model} M={M} maxL={maxL}")
    B.i4d_decode_block_step_e4m3(memo["layer"].struct, cache.struct, x_in, x_out, ctx, M, maxL, 0, ws.buf,
                                 ws.nbytes, attn)
    torch.cuda.synchronize()
    assert cache.errors() == 0
    ref = O.decode_block(shape, memo["ql"], O.build_cache(shape, lengths, pre), xb, lengths, memo["dense"])
    e_out = rel_rms(D.bf16_tensor_to_f32(x_out), ref.out)
    e_att = norm_maxabs(attn.cpu().numpy(), ref.attn)
    say(f"  out rel-RMS {e_out:.3e}  attn max-abs/rms {e_att:.3e}")
    assert_appended_exact(cache, ws, shape, lengths)
    assert e_out <= REL_TOL
    assert e_att <= ATT_TOL


@pytest.mark.parametrize("shape,lengths", [
    (synth.SHAPE_TINY, [1, 2, 5, 67]),
    (synth.SHAPE_TINY, [70]),
    (synth.SHAPE_SMALL128, [1, 33, 300]),
    (synth.SHAPE_SMALL128, [4096] * 2 + [1000] * 15),   # M = 17: two x tiles
    (synth.SHAPE_SMALL128, list(range(100, 3300, 100))),  # M = 32
])
def test_e4m3_block_small(gpu, shape, lengths):
    _run_block_e4m3(gpu, shape, 23, lengths)


def test_e4m3_block_8b_m1_ctx4096(gpu):
    wl = synth.WORKLOADS["8b_m1_ctx4096"]
    _run_block_e4m3(gpu, wl.shape, wl.seed, synth.make_lengths(wl))


@pytest.fixture(scope="module")
def layer70_e4m3(gpu):
    wl = synth.WORKLOADS["70b_ctx4096"]
    say("generating the 70B-shape layer")
    return wl, synth.make_layer(wl.shape, wl.seed), {}


@pytest.mark.parametrize("M", [1, 32])
def test_e4m3_block_70b_ctx4096(gpu, layer70_e4m3, M):
    wl, lw, memo = layer70_e4m3
    _run_block_e4m3(gpu, wl.shape, wl.seed, synth.make_lengths(wl, M), lw=lw, memo=memo)
