"""GPU parity of the FP8 prefill of the QKV projection (reading R13 of the
oracle: the summary page's "how it works" section) against the CPU oracle,
through the C ABI.

Per call:
* the FP8 activations x8 (read from the head of the workspace) equal the
  oracle's E4M3(fp32(x / s_x)) bit for bit, and max |x| is exact;
* q: every E4M3 code is a correct rounding (half a step) of a value within
  2e-3 rms(q) of the oracle's q (the oracle rounds its fp64 q, the kernel
  its fp32 q), at most 1% of the codes differ, and max |q| agrees to 1e-3;
* the bf16 keys and values the call places next to the cache: rel-RMS
  <= 1e-2 against the oracle's fp64 projection rounded to bf16;
* the INT4 cache: at every written slot the codes and fp16 scales equal the
  oracle's encoding (rotation, scale, rounding) of the call's own bf16 key
  and value, bit for bit; slots the call does not own keep what they held
  (earlier tokens of a value block sharing dwords with new ones included);
* the delayed scale update is the oracle's max / 448 exactly.
Cases: one token, ragged packed requests over several 128-token tiles and
request ends inside value blocks, capacity edges, an out-of-range position
(its writes are skipped and the error bit is set), the 8B-shape S = 2048
and variable-length batches at full size, the 70B shape on sampled tokens,
and a decode step reading a cache the prefill filled.
"""
import numpy as np
import pytest

import oracle as O
from int4_quantized_decode_amd import synth
from tests.gpu_helpers import rel_rms, say, norm_maxabs

pytestmark = pytest.mark.gpu

KV_TOL = 1e-2
Q_DELTA = 2e-3


@pytest.fixture(scope="module")
def gpu():
    import torch
    from int4_quantized_decode_amd import binding as B
    from int4_quantized_decode_amd import device as D
    assert torch.cuda.is_available()
    B.lib()
    return torch, B, D


_LAYERS = {}


def _layer(gpu, shape, seed):
    torch, B, D = gpu
    key = (shape, seed)
    if key not in _LAYERS:
        say(f"packing the prefill weights d={shape.d_model} seed={seed}")
        lw = synth.make_layer(shape, seed)
        qkv = O.quantize_weight_e4m3_mx(lw.w_qkv, lw.gamma_attn)
        _LAYERS.clear()
        _LAYERS[key] = (lw, D.PrefillWeights(shape, lw), qkv, O.dense(qkv))
    return _LAYERS[key]


def x8_from_workspace(ws, T, d):
    """Token-major E4M3 codes [T, d] from the operand-order head of the workspace."""
    T128 = -(-T // 128) * 128
    a = ws[: T128 * d].cpu().numpy().reshape(T128 // 16, d // 128, 2, 4, 16, 2, 8)
    # (tile, group, half, j, r, kb-in-half, e) -> token (tile, r), channel (group, half, kb, j, e)
    a = a.transpose(0, 4, 1, 2, 5, 3, 6).reshape(T128, d)
    return a[:T]


class Run:
    pass


def run_prefill(gpu, shape, seed, seqlens, starts, caps=None, sx=None, sq=None, prior=None, lw_seed=None):
    """One prefill call; returns the device results and the cache."""
    torch, B, D = gpu
    lw, layer, qkv, W = _layer(gpu, shape, seed if lw_seed is None else lw_seed)
    seqlens = [int(n) for n in seqlens]
    starts = [int(s) for s in starts]
    R = len(seqlens)
    T = sum(seqlens)
    cu = synth.prefill_offsets(seqlens)
    if caps is None:
        caps = [s + n + 5 for s, n in zip(starts, seqlens)]
    cache = D.DeviceCache(shape, caps)
    if prior is not None:
        cache.prefill(prior)
    before = [cache.read_codes(r, 0, cache.capacities[r]) for r in range(R)]
    xb = synth.make_prefill_x(shape, T, seed)
    x = synth.bf16_bits_to_f32(xb)
    sx = np.float32(np.max(np.abs(x)) / 448.0) if sx is None else np.float32(sx)
    sq = np.float32(0.05) if sq is None else np.float32(sq)
    scales = torch.tensor([sx, sq, 0.0, 0.0], dtype=torch.float32, device="cuda")
    cshape = B.make_shape(shape)
    nbytes = B.i4d_prefill_workspace_bytes(cshape, T)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    q8 = torch.zeros((max(T, 1), shape.n_q_heads * shape.head_dim), dtype=torch.uint8, device="cuda")
    total = int(cache.row_base_host[-1])
    kd = torch.zeros(total * shape.n_kv_heads * shape.head_dim, dtype=torch.int16, device="cuda")
    vd = torch.zeros_like(kd)
    say(f"prefill d={shape.d_model} R={R} T={T} seqlens={seqlens[:8]} starts={starts[:8]}")
    B.i4d_prefill_qkv_e4m3(layer.struct, cache.struct, D.to_device_u16(xb) if T else None, T,
                           torch.from_numpy(cu).cuda(), torch.tensor(starts, dtype=torch.int32, device="cuda"), R,
                           scales, q8, kd, vd, ws, nbytes)
    torch.cuda.synchronize()
    out = Run()
    out.__dict__.update(dict(shape=shape, lw=lw, qkv=qkv, W=W, xb=xb, x=x, cu=cu, starts=starts, seqlens=seqlens,
                             T=T, R=R, sx=sx, sq=sq, scales=scales, ws=ws, q8=q8, kd=kd, vd=vd, cache=cache,
                             before=before, caps=caps, layer=layer))
    return out


def slot_of(run, r, pos, j):
    cap = run.cache.capacities[r]
    return int(run.cache.row_base_host[r]) * run.shape.n_kv_heads + j * cap + pos


def check_run(run, sample=None):
    """All checks of one call against the oracle (sample: token subset)."""
    shape, T = run.shape, run.T
    hd, nkv, nq = shape.head_dim, shape.n_kv_heads, shape.n_q_heads
    rows, pos = O.prefill_token_map(run.cu, run.starts)
    toks = np.arange(T) if sample is None else np.asarray(sample)
    if sample is None:
        ref = O.prefill_qkv(shape, run.qkv, run.xb, run.cu, run.starts, run.sx, run.sq, W_dense=run.W)
    else:
        ref = O.prefill_qkv(shape, run.qkv, run.xb[toks], synth.prefill_offsets([1] * len(toks)), pos[toks],
                            run.sx, run.sq, W_dense=run.W)
    # FP8 activations and max |x|: exact
    x8 = x8_from_workspace(run.ws, T, shape.d_model)
    np.testing.assert_array_equal(x8[toks], ref.x8)
    assert float(run.scales[2].item()) == np.float32(np.max(np.abs(run.x)))
    # q: each code is a correct rounding of a value within Q_DELTA * rms(q)
    # of the oracle's q (the oracle rounds its fp64 q, the kernel its fp32
    # q), and at most 1% of the codes differ from the oracle's
    q8 = run.q8[:T].cpu().numpy().reshape(T, nq, hd)[toks]
    frac = float(np.mean(q8 != ref.q8))
    qc = np.clip(ref.q / float(run.sq), -448.0, 448.0)
    aq = np.abs(qc)
    half = np.where(aq >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(aq, 2.0 ** -6))) - 4), 2.0 ** -10)
    delta = Q_DELTA * np.sqrt(np.mean(ref.q ** 2)) / float(run.sq)
    excess = np.abs(O.e4m3_decode(q8) - qc) - half
    say(f"  q codes differing: {frac:.2e} (largest excess over half a step {excess.max() / delta:.2f} delta)")
    assert excess.max() <= delta and frac <= 0.01
    if sample is None:
        amq = float(run.scales[3].item())
        assert abs(amq - ref.amax_q) <= 1e-3 * ref.amax_q
    # bf16 k, v at their slots; cache codes exact against their encoding
    kd = run.kd.cpu().numpy().view(np.uint16).reshape(-1, hd)
    vd = run.vd.cpu().numpy().view(np.uint16).reshape(-1, hd)
    k_gpu = np.zeros((len(toks), nkv, hd), np.uint16)
    v_gpu = np.zeros_like(k_gpu)
    for i, t in enumerate(toks):
        for j in range(nkv):
            s = slot_of(run, rows[t], pos[t], j)
            k_gpu[i, j], v_gpu[i, j] = kd[s], vd[s]
    kf, vf = synth.bf16_bits_to_f32(k_gpu), synth.bf16_bits_to_f32(v_gpu)
    ek, ev = rel_rms(kf, ref.k_new), rel_rms(vf, ref.v_new)
    say(f"  k rel-RMS {ek:.2e}  v rel-RMS {ev:.2e}")
    assert ek <= KV_TOL and ev <= KV_TOL
    kq, ks = O.quantize_kv(kf)
    vq, vs = O.quantize_kv(vf)
    after = {}
    for i, t in enumerate(toks):
        r = int(rows[t])
        if r not in after:
            after[r] = run.cache.read_codes(r, 0, run.cache.capacities[r])
        kc, vc, kss, vss = after[r]
        p = int(pos[t])
        np.testing.assert_array_equal(kc[p], kq[i])
        np.testing.assert_array_equal(vc[p], vq[i])
        np.testing.assert_array_equal(kss[p], ks[i].view(np.uint16))
        np.testing.assert_array_equal(vss[p], vs[i].view(np.uint16))
    mism = float(np.mean(kq != ref.k_codes))
    say(f"  k codes differing from the oracle's own projection: {mism:.2e} (reported only)")
    return ref, rows, pos


def check_untouched(run, rows, pos):
    """Slots the call does not own keep their earlier contents."""
    for r in range(run.R):
        after = run.cache.read_codes(r, 0, run.cache.capacities[r])
        own = np.zeros(run.cache.capacities[r], bool)
        own[pos[rows == r]] = True
        for a, b in zip(run.before[r], after):
            np.testing.assert_array_equal(a[~own], b[~own])


SMALL = synth.SHAPE_SMALL128


@pytest.mark.parametrize("seqlens,starts", [
    ([1], [0]),
    ([37], [5]),
    ([3, 0, 5, 130, 1, 19], [7, 2, 30, 0, 200, 13]),
    ([128, 128], [0, 64]),
    ([300], [29]),
])
def test_prefill_small(gpu, seqlens, starts):
    run = run_prefill(gpu, SMALL, 31, seqlens, starts)
    assert run.cache.errors() == 0
    ref, rows, pos = check_run(run)
    check_untouched(run, rows, pos)


def test_prefill_keeps_earlier_tokens_of_shared_value_blocks(gpu):
    """Requests continue sequences whose earlier positions are already in the
    cache: the new tokens share value dwords with them (atomic nibble
    writes), which must keep the earlier codes."""
    torch, B, D = gpu
    seqlens, starts = [20, 45, 3], [13, 70, 31]
    rng = np.random.default_rng(9)
    prior_k = [synth.f32_to_bf16_bits(rng.standard_normal((s, SMALL.n_kv_heads, 128)).astype(np.float32))
               for s in starts]
    prior_v = [synth.f32_to_bf16_bits(rng.standard_normal((s, SMALL.n_kv_heads, 128)).astype(np.float32))
               for s in starts]
    prior = synth.CachePrefill(prior_k, prior_v)
    run = run_prefill(gpu, SMALL, 32, seqlens, starts, caps=[s + n + 40 for s, n in zip(starts, seqlens)],
                      prior=prior)
    assert run.cache.errors() == 0
    ref, rows, pos = check_run(run)
    check_untouched(run, rows, pos)
    # the earlier tokens are still the oracle's encoding of their own values
    for r in range(len(starts)):
        kc, vc, _, _ = run.cache.read_codes(r, 0, starts[r])
        kq, _ = O.quantize_kv(synth.bf16_bits_to_f32(prior_k[r]))
        vq, _ = O.quantize_kv(synth.bf16_bits_to_f32(prior_v[r]))
        np.testing.assert_array_equal(kc, kq)
        np.testing.assert_array_equal(vc, vq)


def test_prefill_capacity_edges_and_out_of_range_positions(gpu):
    # request 0 ends exactly at its capacity; request 1 runs past it (its last
    # 7 tokens have no slot: skipped, error bit set); request 2 is fine
    seqlens, starts = [32, 20, 9], [0, 19, 3]
    caps = [32, 32, 64]
    run = run_prefill(gpu, SMALL, 33, seqlens, starts, caps=caps)
    from int4_quantized_decode_amd import binding as B
    assert run.cache.errors() & B.I4D_DEVERR_APPEND_POS
    rows, pos = O.prefill_token_map(run.cu, run.starts)
    ok = np.array([p < caps[r] for r, p in zip(rows, pos)])
    assert (~ok).sum() == 7
    check_run(run, sample=np.nonzero(ok)[0])
    check_untouched(run, rows[ok], pos[ok])


def test_delayed_scaling_update_and_second_call(gpu):
    torch, B, D = gpu
    run = run_prefill(gpu, SMALL, 34, [50, 77], [0, 0], sx=1.0, sq=1.0)
    ref = O.prefill_qkv(SMALL, run.qkv, run.xb, run.cu, run.starts, run.sx, run.sq, W_dense=run.W)
    B.i4d_fp8_scales_update(run.scales)
    torch.cuda.synchronize()
    s = run.scales.cpu().numpy()
    assert s[0] == O.delayed_scale(np.float32(np.max(np.abs(run.x))), 1.0)
    assert abs(float(s[1]) - float(O.delayed_scale(ref.amax_q, 1.0))) <= 1e-3 * float(s[1])
    assert s[2] == 0 and s[3] == 0
    # the next call with the updated scales: the largest |x| maps to +-448
    run2 = run_prefill(gpu, SMALL, 34, [50, 77], [0, 0], sx=s[0], sq=s[1])
    x8 = x8_from_workspace(run2.ws, run2.T, SMALL.d_model)
    i = np.unravel_index(np.argmax(np.abs(run2.x)), run2.x.shape)
    assert x8[i] & 0x7F == 0x7E
    check_run(run2)


def test_prefill_8b_s2048(gpu):
    wl = synth.PREFILL_WORKLOADS["8b_prefill_s2048"]
    run = run_prefill(gpu, wl.shape, wl.seed, wl.seqlens, wl.starts, caps=[2048])
    assert run.cache.errors() == 0
    check_run(run)


def test_prefill_8b_varlen(gpu):
    wl = synth.PREFILL_WORKLOADS["8b_prefill_varlen"]
    run = run_prefill(gpu, wl.shape, wl.seed, wl.seqlens, wl.starts, caps=[2048] + [128] * 7)
    assert run.cache.errors() == 0
    check_run(run)


def test_prefill_70b_s2048_sampled(gpu):
    wl = synth.PREFILL_WORKLOADS["70b_prefill_s2048"]
    run = run_prefill(gpu, wl.shape, wl.seed, wl.seqlens, wl.starts, caps=[2048])
    assert run.cache.errors() == 0
    rng = np.random.default_rng(5)
    sample = np.sort(np.concatenate([[0, 1, 127, 128, 2047], rng.choice(2048, 59, replace=False)]))
    check_run(run, sample=np.unique(sample))


def test_decode_step_reads_the_prefilled_cache(gpu):
    """The INT4 decode step of the same layer at position L_r - 1 after a
    prefill of positions 0 .. L_r - 2: GPU block output against the oracle's
    decode over the cache the prefill wrote (read back; its codes are checked
    exact above)."""
    torch, B, D = gpu
    shape = SMALL
    lengths = np.array([5, 130, 300, 64], np.int32)
    run = run_prefill(gpu, shape, 35, list(lengths - 1), [0] * len(lengths), caps=list(lengths))
    assert run.cache.errors() == 0
    check_run(run)
    layer4 = D.DeviceLayer(shape, run.lw)
    ql4 = O.quantize_layer(run.lw)
    M = len(lengths)
    xb = synth.make_x(shape, M, 36)
    ws = D.Workspace(shape, M, int(lengths.max()), 0)
    x_in = D.to_device_u16(xb)
    x_out = torch.empty_like(x_in)
    ctx = torch.from_numpy(lengths).cuda()
    attn = torch.empty((M, shape.n_q_heads * shape.head_dim), dtype=torch.float32, device="cuda")
    cache_rows = []
    for r, L in enumerate(lengths):
        kc, vc, ks, vs = run.cache.read_codes(r, 0, int(L))
        cache_rows.append(O.RowCache(kc.copy(), ks.view(np.float16).copy(), vc.copy(), vs.view(np.float16).copy()))
    B.i4d_decode_block_step(layer4.struct, run.cache.struct, x_in, x_out, ctx, M, int(lengths.max()), 0, ws.buf,
                            ws.nbytes, attn)
    torch.cuda.synchronize()
    assert run.cache.errors() == 0
    ref = O.decode_block(shape, ql4, cache_rows, xb, lengths, {})
    e_out = rel_rms(D.bf16_tensor_to_f32(x_out), ref.out)
    e_att = norm_maxabs(attn.cpu().numpy(), ref.attn)
    say(f"  decode after prefill: out rel-RMS {e_out:.2e}  attn {e_att:.2e}")
    assert e_out <= 1e-2 and e_att <= 2e-2


def test_prepare_then_project_equals_the_fused_call(gpu):
    """The two-call form gives the fused call's results bit for bit, and a
    repeated projection over the same workspace changes nothing."""
    torch, B, D = gpu
    seqlens, starts = [70, 129, 1], [3, 40, 0]
    run = run_prefill(gpu, SMALL, 37, seqlens, starts)
    cache2 = D.DeviceCache(SMALL, run.caps)
    scales2 = torch.tensor([run.sx, run.sq, 0.0, 0.0], dtype=torch.float32, device="cuda")
    ws2 = torch.zeros_like(run.ws)
    q2 = torch.zeros_like(run.q8)
    kd2, vd2 = torch.zeros_like(run.kd), torch.zeros_like(run.vd)
    cu = torch.from_numpy(run.cu).cuda()
    st = torch.tensor(starts, dtype=torch.int32, device="cuda")
    B.i4d_prefill_prepare(run.layer.struct, cache2.struct, D.to_device_u16(run.xb), run.T, cu, st, run.R, scales2,
                          ws2, ws2.numel())
    for _ in range(2):
        B.i4d_prefill_project(run.layer.struct, cache2.struct, run.T, cu, st, run.R, scales2, q2, kd2, vd2, ws2,
                              ws2.numel())
    torch.cuda.synchronize()
    for a, b in ((run.q8, q2), (run.kd, kd2), (run.vd, vd2), (run.scales, scales2), (run.ws, ws2),
                 (run.cache.k_codes, cache2.k_codes), (run.cache.v_codes, cache2.v_codes),
                 (run.cache.k_scales, cache2.k_scales), (run.cache.v_scales, cache2.v_scales)):
        assert torch.equal(a, b)
