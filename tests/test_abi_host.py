"""Host-side checks of the C ABI (no GPU work is enqueued by any test here).

* the library loads and exports every function include/i4d.h declares;
* argument validation rejects bad calls before anything reaches the GPU;
* the host packer is bit-exact against the oracle's quantizer, and the
  packed bytes sit where the documented device layout says;
* the KV-cache decoder reads the documented cache layout.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from int4_quantized_decode_amd import binding as B
from int4_quantized_decode_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "i4d.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(i4d_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = B.lib()
    names = declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/i4d.h but not exported"
    assert sorted(B.exported_names()) == names
    assert "gfx950" in B.i4d_version()


# ---------------------------------------------------------------------------
# validation (every call below fails in host checks, before any HIP call)
# ---------------------------------------------------------------------------

def _shape(**kw):
    s = B.make_shape(synth.SHAPE_TINY)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


FAKE = 1 << 20  # never dereferenced: each call fails validation first


def _layer(shape=None, **ptrs):
    f = dict(qkv_codes=FAKE, qkv_scales=FAKE, o_codes=FAKE, o_scales=FAKE, gu_codes=FAKE,
             gu_scales=FAKE, down_codes=FAKE, down_scales=FAKE)
    f.update(ptrs)
    return B.i4d_layer(shape or _shape(), **f)


def _cache(**kw):
    c = B.i4d_kv_cache(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 64, 256, None)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _status(fn):
    with pytest.raises(B.I4DError) as e:
        fn()
    return e.value.status


def test_shape_validation():
    assert _status(lambda: B.i4d_workspace_bytes(_shape(head_dim=96, hadamard_block=96), 1, 16)) == -3
    assert _status(lambda: B.i4d_workspace_bytes(_shape(hadamard_block=32), 1, 16)) == -3
    assert _status(lambda: B.i4d_workspace_bytes(_shape(group=64), 1, 16)) == -3
    assert _status(lambda: B.i4d_workspace_bytes(_shape(n_kv_heads=3), 1, 16)) == -2
    assert _status(lambda: B.i4d_workspace_bytes(_shape(d_model=200), 1, 16)) == -2
    assert _status(lambda: B.i4d_workspace_bytes(_shape(n_q_heads=24, n_kv_heads=2), 1, 16)) == -3
    assert _status(lambda: B.i4d_workspace_bytes(_shape(), 0, 16)) == -6
    assert _status(lambda: B.i4d_workspace_bytes(_shape(), 33, 16)) == -6
    assert _status(lambda: B.i4d_workspace_bytes(_shape(), 1, 0)) == -6
    assert _status(lambda: B.i4d_workspace_bytes(_shape(), 1, 16, 257)) == -6
    assert B.i4d_workspace_bytes(_shape(), 32, 4096) > 0


def test_device_entry_points_reject_bad_arguments_before_launch():
    lay, ws = _layer(), FAKE
    big = 1 << 40
    # NULL layer / pointers
    assert B.lib().i4d_decode_block_step(None, ctypes.byref(_cache()), FAKE, FAKE + 16, FAKE, 1, 16, 0,
                                         ws, big, None, None) == -1
    assert _status(lambda: B.i4d_decode_block_step(_layer(o_codes=0), _cache(), FAKE, FAKE + 16, FAKE, 1,
                                                   16, 0, ws, big)) == -1
    # misaligned pointers
    assert _status(lambda: B.i4d_decode_block_step(_layer(gu_scales=FAKE + 2), _cache(), FAKE, FAKE + 16,
                                                   FAKE, 1, 16, 0, ws, big)) == -4
    assert _status(lambda: B.i4d_decode_block_step(lay, _cache(), FAKE + 8, FAKE + 16, FAKE, 1, 16, 0,
                                                   ws, big)) == -4
    # rows out of range / more rows than the cache
    assert _status(lambda: B.i4d_decode_block_step(lay, _cache(), FAKE, FAKE + 16, FAKE, 0, 16, 0, ws, big)) == -6
    assert _status(lambda: B.i4d_decode_block_step(lay, _cache(), FAKE, FAKE + 16, FAKE, 5, 16, 0, ws, big)) == -2
    # cache/layer mismatch, bad capacity
    assert _status(lambda: B.i4d_decode_block_step(lay, _cache(head_dim=128), FAKE, FAKE + 16, FAKE, 1, 16,
                                                   0, ws, big)) == -2
    assert _status(lambda: B.i4d_decode_block_step(lay, _cache(total_capacity=100), FAKE, FAKE + 16, FAKE,
                                                   1, 16, 0, ws, big)) == -2
    # max_ctx_len beyond capacity, aliasing, workspace too small
    assert _status(lambda: B.i4d_decode_block_step(lay, _cache(), FAKE, FAKE + 16, FAKE, 1, 257, 0, ws,
                                                   big)) == -6
    assert _status(lambda: B.i4d_decode_block_step(lay, _cache(), FAKE, FAKE, FAKE, 1, 16, 0, ws, big)) == -6
    assert _status(lambda: B.i4d_decode_block_step(lay, _cache(), FAKE, FAKE + 16, FAKE, 1, 16, 0, ws, 64)) == -5
    # stage entry points
    assert _status(lambda: B.i4d_attn_qkv(lay, None, FAKE, 1, FAKE, FAKE, FAKE, 0)) == -1
    assert _status(lambda: B.i4d_ffn_gate_up(lay, FAKE, 40, FAKE, 0)) == -6
    assert _status(lambda: B.i4d_ffn_down(_layer(shape=_shape(head_dim=80)), FAKE, FAKE, 1, FAKE, 0)) == -3
    assert _status(lambda: B.i4d_attention(_cache(), _shape(), FAKE, FAKE, 1, 16, 0, ws, 16, None, FAKE, 0)) == -5
    assert _status(lambda: B.i4d_kv_append(_cache(), FAKE, FAKE, None, FAKE, 9, 0)) == -2
    assert _status(lambda: B.i4d_kv_append(_cache(), FAKE, FAKE, None, FAKE, -1, 0)) == -6
    assert _status(lambda: B.i4d_lm_head_argmax(FAKE, 100, 128, FAKE, 1, 1e-5, None, FAKE, ws, big, 0)) == -2
    assert _status(lambda: B.i4d_lm_head_argmax(FAKE, 128, 128, FAKE, 1, 0.0, None, FAKE, ws, big, 0)) == -6
    assert "epsilon" in B.i4d_last_error() or "rms_eps" in B.i4d_last_error()


def test_pack_argument_errors():
    W = np.zeros((16, 100), np.float32)
    assert _status(lambda: B.i4d_pack_weights(B.I4D_PROJ_PLAIN, W)) == -2
    W = np.zeros((20, 128), np.float32)
    assert _status(lambda: B.i4d_pack_weights(B.I4D_PROJ_PLAIN, W)) == -2
    W = np.zeros((64, 128), np.float32)
    assert _status(lambda: B.i4d_pack_weights(B.I4D_PROJ_GATE_UP, W)) == -1
    assert _status(lambda: B.i4d_pack_weights(B.I4D_PROJ_QKV, W, head_dim=96)) == -3
    assert _status(lambda: B.i4d_pack_weights(B.I4D_PROJ_PLAIN, W, gamma=np.ones(128, np.float32))) == -6


# ---------------------------------------------------------------------------
# packer: bit-exact codes and scales
# ---------------------------------------------------------------------------

def _check_pack(kind, W0, W1, gamma, hd=0):
    codes, scales = B.i4d_pack_weights(kind, W0, W1, gamma, hd)
    q, s = B.i4d_unpack_weights(kind, codes, scales, W0.shape[0], W0.shape[1], hd)
    rq, rs = O.quantize_weight(W0, gamma)
    if kind == B.I4D_PROJ_GATE_UP:
        rq2, rs2 = O.quantize_weight(W1, gamma)
        rq, rs = np.concatenate([rq, rq2]), np.concatenate([rs, rs2])
    np.testing.assert_array_equal(q, rq)
    np.testing.assert_array_equal(s, rs.view(np.uint16))
    return codes, scales


@pytest.mark.parametrize("shape", [synth.SHAPE_TINY, synth.SHAPE_1B], ids=["tiny", "1b"])
def test_packer_bit_exact_full_layer(shape):
    lw = synth.make_layer(shape, 5 if shape is synth.SHAPE_TINY else 0)
    _check_pack(B.I4D_PROJ_QKV, lw.w_qkv, None, lw.gamma_attn, shape.head_dim)
    _check_pack(B.I4D_PROJ_PLAIN, lw.w_o, None, None)
    _check_pack(B.I4D_PROJ_GATE_UP, lw.w_gate, lw.w_up, lw.gamma_ffn)
    _check_pack(B.I4D_PROJ_PLAIN, lw.w_down, None, None)


def test_packer_bit_exact_sampled_8b_rows():
    # 8B-shape distributions on a row sample (every K of the 8B layer)
    rng = np.random.default_rng(1)
    for K in (4096, 14336):
        W = (rng.standard_normal((256, K)) * 0.02).astype(np.float32)
        g = rng.uniform(0.5, 1.5, K).astype(np.float32)
        _check_pack(B.I4D_PROJ_PLAIN, W, None, None)
        _check_pack(B.I4D_PROJ_GATE_UP, W[:128], W[128:], g)
    W = (rng.standard_normal((6 * 128, 4096)) * 0.02).astype(np.float32)
    _check_pack(B.I4D_PROJ_QKV, W, None, rng.uniform(0.5, 1.5, 4096).astype(np.float32), 128)


def test_packer_edge_values():
    # ties, zero groups, scale overflow (saturates), scale underflow (s = 0), tiny and huge values
    W = np.zeros((32, 1024), np.float32)
    W[0, :7] = [2.5, 3.5, -2.5, 0.5, 7.0, -1.5, -0.5]       # s = 1 exactly, ties to even
    W[1, 128:131] = [0.7, -0.35, 0.05]                       # fp16-rounded scale example
    W[2, 256] = 1e6                                          # absmax/7 > 65504 -> scale saturates
    W[3, 384] = 1e-9                                         # scale rounds to 0 -> codes 0
    W[4, 512:640] = np.linspace(-3e-5, 3e-5, 128)            # subnormal fp16 scale
    W[5, 640:768] = -np.float32(3.0)                         # all equal negative
    rng = np.random.default_rng(3)
    W[8:] = (rng.standard_normal((24, 1024)) * np.exp(rng.uniform(-8, 8, (24, 1))).astype(np.float32))
    _check_pack(B.I4D_PROJ_PLAIN, W, None, None)
    q, s = O.quantize_weight(W)
    assert s[2, 2] == np.float16(65504) and s[3, 3] == 0 and np.all(q[3] == 0)


def test_packed_bytes_follow_documented_layout():
    """Place one code per group and find its nibble where the layout says."""
    N, K = 32, 256
    W = np.zeros((N, K), np.float32)
    rng = np.random.default_rng(4)
    pos = {}
    for n in range(N):
        for g in range(K // 128):
            k = 128 * g + int(rng.integers(0, 128))
            W[n, k] = 7.0 * (n + 1)                           # code +7 -> nibble 15, others nibble 8
            pos[(n, g)] = k
    codes, scales = B.i4d_pack_weights(B.I4D_PROJ_PLAIN, W)
    G = K // 128
    for (n, g), k in pos.items():
        t, r, kk = n // 16, n % 16, k % 128
        kb, j, e = kk // 32, (kk % 32) // 8, kk % 8
        slot = 4 * (e & 1) + (e >> 1)                         # nibble slots hold e = 0,2,4,6,1,3,5,7
        byte = ((t * G + g) * 64 + 16 * j + r) * 16 + kb * 4 + slot // 2
        nib = (codes[byte] >> 4) if slot & 1 else (codes[byte] & 15)
        assert nib == 15
        # scale layout [strip][group][row]
        assert scales[(t * G + g) * 16 + r] == np.float16(n + 1).view(np.uint16)
    # every other nibble encodes code 0
    assert np.count_nonzero(codes == 0x88) == codes.size - len(pos)


def test_qkv_and_gate_up_strip_interleave():
    hd, N, K = 64, 3 * 64, 128
    W = np.zeros((N, K), np.float32)
    for n in range(N):
        W[n, 0] = 7.0 * (n + 1)
    codes, scales = B.i4d_pack_weights(B.I4D_PROJ_QKV, W, None, None, hd)
    sc = scales.view(np.float16).reshape(N // 16, 1, 16)[:, 0, :]
    for t in range(N // 16):
        head, sp = t // (hd // 16), t % (hd // 16)
        want = [head * hd + 8 * sp + i for i in range(8)] + [head * hd + hd // 2 + 8 * sp + i for i in range(8)]
        np.testing.assert_array_equal(sc[t], np.array(want, np.float32) + 1)
    F = 32
    Wg = np.zeros((F, K), np.float32)
    Wu = np.zeros((F, K), np.float32)
    Wg[:, 0] = 7.0 * (np.arange(F) + 1)
    Wu[:, 0] = -7.0 * (np.arange(F) + 101)
    codes, scales = B.i4d_pack_weights(B.I4D_PROJ_GATE_UP, Wg, Wu)
    sc = scales.view(np.float16).reshape(2 * F // 16, 1, 16)[:, 0, :]
    for t in range(2 * F // 16):
        np.testing.assert_array_equal(sc[t, :8], np.arange(8 * t, 8 * t + 8) + 1)
        np.testing.assert_array_equal(sc[t, 8:], np.arange(8 * t, 8 * t + 8) + 101)


# ---------------------------------------------------------------------------
# pre-quantized import: the layout permutation alone
# ---------------------------------------------------------------------------

def _random_codes(rng, rows, K):
    q = rng.integers(-8, 8, (rows, K)).astype(np.int8)
    s = (rng.uniform(1e-4, 0.05, (rows, K // 128)) * rng.choice([1, -1], (rows, K // 128))).astype(np.float16)
    return q, s.view(np.uint16)


@pytest.mark.parametrize("kind,N,K,hd", [(0, 48, 384, 0), (1, 3 * 128, 256, 128), (1, 6 * 64, 128, 64),
                                         (2, 32, 512, 0)], ids=["plain", "qkv128", "qkv64", "gate_up"])
def test_pack_codes_round_trip(kind, N, K, hd):
    """Arbitrary codes and scales (any sign, not from round-to-nearest) come
    back unchanged through the device layout."""
    rng = np.random.default_rng(8 + kind)
    rows = 2 * N if kind == B.I4D_PROJ_GATE_UP else N
    q, s = _random_codes(rng, rows, K)
    codes, scales = B.i4d_pack_codes(kind, q, s, N, K, hd)
    q2, s2 = B.i4d_unpack_weights(kind, codes, scales, N, K, hd)
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(s2, s)


def test_pack_codes_places_bytes_as_the_quantizing_packer():
    """Importing the codes and scales the quantizing packer produced gives
    the same bytes (every projection kind of a layer)."""
    shape = synth.SHAPE_TINY
    lw = synth.make_layer(shape, 9)
    hd = shape.head_dim
    for kind, W0, W1, g in [(B.I4D_PROJ_QKV, lw.w_qkv, None, lw.gamma_attn), (B.I4D_PROJ_PLAIN, lw.w_o, None, None),
                            (B.I4D_PROJ_GATE_UP, lw.w_gate, lw.w_up, lw.gamma_ffn),
                            (B.I4D_PROJ_PLAIN, lw.w_down, None, None)]:
        N, K = W0.shape
        h = hd if kind == B.I4D_PROJ_QKV else 0
        codes, scales = B.i4d_pack_weights(kind, W0, W1, g, h)
        q, s = B.i4d_unpack_weights(kind, codes, scales, N, K, h)
        c2, s2 = B.i4d_pack_codes(kind, q, s, N, K, h)
        np.testing.assert_array_equal(c2, codes)
        np.testing.assert_array_equal(s2, scales)


def test_pack_codes_rejects_bad_input():
    rng = np.random.default_rng(12)
    q, s = _random_codes(rng, 32, 256)
    for bad in (-9, 8):
        qb = q.copy()
        qb[17, 200] = bad
        assert _status(lambda: B.i4d_pack_codes(B.I4D_PROJ_PLAIN, qb, s, 32, 256)) == -6
        assert "outside [-8, 7]" in B.i4d_last_error()
    for bits in (0x7c00, 0xfc00, 0x7e00):          # +inf, -inf, nan
        sb = s.copy()
        sb[5, 1] = bits
        assert _status(lambda: B.i4d_pack_codes(B.I4D_PROJ_PLAIN, q, sb, 32, 256)) == -6
        assert "not finite" in B.i4d_last_error()
    assert _status(lambda: B.i4d_pack_codes(B.I4D_PROJ_PLAIN, q[:, :200], s[:, :1], 32, 200)) == -2
    L = B.lib()
    assert L.i4d_pack_codes(B.I4D_PROJ_PLAIN, None, None, 32, 256, 0, None, None, 0) == -1


def test_lm_head_pack_matches_oracle_bf16():
    rng = np.random.default_rng(6)
    W = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    g = rng.uniform(0.5, 1.5, 256).astype(np.float32)
    out = B.i4d_pack_lm_head(W, g)
    assert out.shape == (64 // 16, 256 // 32, 16, 32)
    ref = O.lm_head_weight_bf16(W, g)
    # tiles [V/16][d/32][16 rows][32 channels] back to [V][d]
    natural = out.transpose(0, 2, 1, 3).reshape(64, 256)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(natural).astype(np.float64), ref)
    # documented offset of element (v, k)
    flat = out.reshape(-1)
    for v, k in [(0, 0), (17, 33), (63, 255), (5, 130)]:
        o = ((v // 16 * (256 // 32) + k // 32) * 16 + v % 16) * 32 + k % 32
        assert synth.bf16_bits_to_f32(flat[o:o + 1])[0] == ref[v, k]


# ---------------------------------------------------------------------------
# KV cache layout decoder
# ---------------------------------------------------------------------------

def test_kv_unpack_reads_documented_layout():
    """Build a cache by hand from the documented layout; the library decodes it."""
    nkv, hd = 2, 128
    caps = [64, 32]
    rb = np.array([0, 64, 96], np.int64)
    total = 96
    rng = np.random.default_rng(8)
    codes_k = rng.integers(-8, 8, (total * nkv, hd)).astype(np.int8)   # per slot, logical channels
    codes_v = rng.integers(-8, 8, (total * nkv, hd)).astype(np.int8)
    sk = rng.integers(0, 1 << 15, total * nkv).astype(np.uint16)
    sv = rng.integers(0, 1 << 15, total * nkv).astype(np.uint16)
    kbuf = np.zeros(total * nkv * hd // 2, np.uint8)
    vbuf = np.zeros(total * nkv * hd // 8, np.uint32)
    for slot in range(total * nkv):
        for c in range(hd):
            kb, jj, e = c // 32, (c % 32) // 8, c % 8
            ns = 4 * (e & 1) + (e >> 1)
            byte = slot * hd // 2 + jj * 16 + kb * 4 + ns // 2
            kbuf[byte] |= (int(codes_k[slot, c]) + 8) << (4 * (ns & 1))
            w = slot % 32
            jv, ev = (w // 4, w % 4) if w < 16 else ((w - 16) // 4, 4 + (w - 16) % 4)
            nsv = 4 * (ev & 1) + (ev >> 1)
            dw = (slot // 32) * 4 * hd + jv * hd + (c % 16) * (hd // 16) + c // 16
            vbuf[dw] |= np.uint32((int(codes_v[slot, c]) + 8) << (4 * nsv))
    hc = B.i4d_kv_cache(kbuf.ctypes.data, vbuf.ctypes.data, sk.ctypes.data, sv.ctypes.data, rb.ctypes.data,
                        2, nkv, hd, total, None)
    for row, cap in enumerate(caps):
        k, v, ks, vs = B.i4d_kv_unpack_host(hc, rb, row, 0, cap)
        for j in range(nkv):
            slots = rb[row] * nkv + j * cap + np.arange(cap)
            np.testing.assert_array_equal(k[:, j], codes_k[slots])
            np.testing.assert_array_equal(v[:, j], codes_v[slots])
            np.testing.assert_array_equal(ks[:, j], sk[slots])
            np.testing.assert_array_equal(vs[:, j], sv[slots])


# ---------------------------------------------------------------------------
# projection launch plans
# ---------------------------------------------------------------------------

PLAN_SHAPES = [synth.SHAPE_1B, synth.SHAPE_8B, synth.SHAPE_70B, synth.SHAPE_TINY, synth.SHAPE_SMALL128,
               synth.LayerShape(640, 5, 5, 128, 1152), synth.LayerShape(4096, 8, 2, 128, 8192),
               synth.LayerShape(1024, 8, 2, 128, 16384), synth.LayerShape(1024, 16, 4, 64, 2048)]


@pytest.mark.parametrize("shape", PLAN_SHAPES, ids=lambda s: f"d{s.d_model}_f{s.d_ffn}_hd{s.head_dim}")
def test_every_projection_plan_has_a_kernel(shape):
    """For every stage and every batch size the decode step takes, the plan
    it would launch names a kernel the library holds (a plan without one
    fails the call with I4D_ERR_UNSUPPORTED rather than launching nothing),
    and it fits the 160 KiB of LDS of a CU."""
    cs = B.make_shape(shape)
    for M in range(1, B.I4D_MAX_ROWS + 1):
        for stage in range(4):
            p = B.i4d_projection_plan_of(cs, stage, M)
            assert p.instantiated == 1, (M, stage, p.strips_per_workgroup, p.k_slices, p.depth, p.persistent)
            assert p.kernel == 0 if M == 1 else (p.kernel in (1, 2) and (p.kernel == 1 or M <= 8))
            assert 0 < p.lds_bytes <= 160 * 1024 and p.grid >= 1
            if p.kernel == 1:
                assert p.waves == 8 and p.strips_per_workgroup in (1, 2, 3, 4, 5, 7)


def test_one_launch_coverage():
    """The M = 1 step of the 8B shape runs as one launch, more rows do not;
    the 70B shape (FFN 28672, beyond the one-launch x staging of 16384) and
    more than 16 kv heads keep one launch per stage."""
    cs8 = B.make_shape(synth.SHAPE_8B)
    assert B.i4d_decode_step_is_one_launch(cs8, 1) == 1
    assert B.i4d_decode_step_is_one_launch(cs8, 2) == 0
    for shape in (synth.SHAPE_70B, synth.LayerShape(4096, 32, 32, 128, 2048)):
        assert B.i4d_decode_step_is_one_launch(B.make_shape(shape), 1) == 0


def test_multi_row_gemv_plans():
    """The multi-row GEMV runs at M = 2 and 3 wherever its x staging fits:
    every 8B stage and the 70B ones with K = 8192 to M = 3, the 70B down
    projection (K = 28672) at M = 2 only (M x K fp16 beyond the staging)."""
    cs8, cs70 = B.make_shape(synth.SHAPE_8B), B.make_shape(synth.SHAPE_70B)
    for M in range(2, 9):
        for stage in range(3):
            assert B.i4d_projection_plan_of(cs8, stage, M).kernel == (2 if M <= 3 else 1)
            assert B.i4d_projection_plan_of(cs70, stage, M).kernel == (2 if M <= 3 else 1)
        assert B.i4d_projection_plan_of(cs8, 3, M).kernel == (2 if M <= 3 else 1)
        assert B.i4d_projection_plan_of(cs70, 3, M).kernel == (2 if M == 2 else 1)
    for M in (9, 16, 32):
        assert all(B.i4d_projection_plan_of(cs8, st, M).kernel == 1 for st in range(4))


def test_projection_plan_splits_large_k_only_with_many_rows():
    cs = B.make_shape(synth.SHAPE_8B)
    # down projection (K = 14336): unsplit at 16 rows, split at 32
    assert B.i4d_projection_plan_of(cs, 3, 16).k_slices == 1
    assert B.i4d_projection_plan_of(cs, 3, 32).k_slices > 1
    with pytest.raises(B.I4DError):
        B.i4d_projection_plan_of(cs, 4, 1)


def test_noalloc_step_rejects_a_step_larger_than_its_scratch():
    """A step whose intermediates exceed the library-owned scratch is
    refused on the host, before any device call (70B shape, 32 rows, 256
    forced KV splits: 272 MB of split partials)."""
    shape = B.make_shape(synth.SHAPE_70B)
    layer = _layer(shape)
    cache = _cache(n_kv_heads=8, head_dim=128, total_capacity=32 * 4096, n_rows=32)
    with pytest.raises(B.I4DError) as ei:
        B.i4d_decode_block_step_noalloc(layer, cache, FAKE, FAKE + 4096, FAKE, 32, 4096, 256)
    assert ei.value.status == -5 and "scratch" in str(ei.value)
    # the same step fits a caller's workspace of the reported size
    assert B.i4d_workspace_bytes(shape, 32, 4096, 256) > B.I4D_NOALLOC_SCRATCH_BYTES


# ---------------------------------------------------------------------------
# E4M3 decode-weight packer
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [synth.SHAPE_TINY, synth.SHAPE_SMALL128], ids=["tiny", "small128"])
def test_e4m3_packer_bit_exact_full_layer(shape):
    """Codes and fp16 scales of every projection kind equal the oracle's
    E4M3 encoding (gain folded) after undoing the layout permutation."""
    lw = synth.make_layer(shape, 9)
    ql = O.quantize_layer_e4m3(lw)
    hd, d, F = shape.head_dim, shape.d_model, shape.d_ffn
    nq = shape.n_q_heads * hd
    cases = [
        (B.I4D_PROJ_QKV, lw.w_qkv, None, lw.gamma_attn, hd, [ql.qkv]),
        (B.I4D_PROJ_PLAIN, lw.w_o, None, None, 0, [ql.o]),
        (B.I4D_PROJ_GATE_UP, lw.w_gate, lw.w_up, lw.gamma_ffn, 0, [ql.gate, ql.up]),
        (B.I4D_PROJ_PLAIN, lw.w_down, None, None, 0, [ql.down]),
    ]
    for kind, W0, W1, g, h, refs in cases:
        codes, scales = B.i4d_pack_weights_e4m3(kind, W0, W1, g, h)
        N, K = W0.shape
        assert codes.size == (2 if W1 is not None else 1) * N * K
        q, s = B.i4d_unpack_weights_e4m3(kind, codes, scales, N, K, h)
        np.testing.assert_array_equal(q, np.concatenate([r[0] for r in refs]))
        np.testing.assert_array_equal(s, np.concatenate([r[1] for r in refs]).view(np.uint16))


@pytest.mark.parametrize("shape", [synth.SHAPE_TINY, synth.SHAPE_SMALL128])
def test_mx_packer_bit_exact(shape):
    """Codes and E8M0 scale bytes of the prefill weight format equal the
    oracle's encoding on every projection kind, and the edge cases: a zero
    group, tiny and huge magnitudes, exact powers of two at 448 * 2^e."""
    lw = synth.make_layer(shape, 11)
    hd = shape.head_dim
    W = lw.w_qkv.copy()
    W[0, :128] = 0.0
    W[1, :128] *= np.float32(1e-30)
    W[2, :128] *= np.float32(1e30)
    W[3, :128] = np.float32(448.0 * 2.0 ** -5)
    W[4, 128:256] = -np.float32(2.0 ** -20)
    cases = [
        (B.I4D_PROJ_QKV, W, None, lw.gamma_attn, hd),
        (B.I4D_PROJ_QKV, W, None, None, hd),
        (B.I4D_PROJ_PLAIN, lw.w_o, None, None, 0),
        (B.I4D_PROJ_GATE_UP, lw.w_gate, lw.w_up, lw.gamma_ffn, 0),
    ]
    for kind, W0, W1, g, h in cases:
        codes, scales = B.i4d_pack_weights_mx(kind, W0, W1, g, h)
        N, K = W0.shape
        q, s = B.i4d_unpack_weights_mx(kind, codes, scales, N, K, h)
        refs = [O.quantize_weight_e4m3_mx(W0, g)] + ([O.quantize_weight_e4m3_mx(W1, g)] if W1 is not None else [])
        np.testing.assert_array_equal(q, np.concatenate([r[0] for r in refs]))
        np.testing.assert_array_equal(s, np.concatenate([r[1] for r in refs]))
    # the layout is the E4M3 atom layout: same code bytes as the E4M3 packer would place
    codes, _ = B.i4d_pack_weights_mx(B.I4D_PROJ_PLAIN, lw.w_o, None, None, 0)
    q_ref = O.quantize_weight_e4m3_mx(lw.w_o)[0]
    N, K = lw.w_o.shape
    for (n, k) in [(0, 0), (5, 131), (17, 255), (N - 1, K - 1)]:
        t, r, gi, kk = n // 16, n % 16, k // 128, k % 128
        kb, j, e = kk // 32, (kk % 32) // 8, kk % 8
        off = ((t * (K // 128) + gi) * 64 + 16 * j + r) * 32 + kb * 8 + e
        assert codes[off] == q_ref[n, k]


def test_e4m3_packer_edge_values_and_layout():
    """Saturation, subnormals, ties, signed zeros and a zero group, against
    the oracle; and the documented byte position of (row, k) in an atom."""
    N, K = 16, 256
    W = np.zeros((N, K), np.float32)
    W[0, :128] = np.linspace(-1, 1, 128, dtype=np.float32)
    W[1, :128] = np.float32(2.0 ** -12) * np.arange(128, dtype=np.float32)  # subnormal codes
    W[2, :128] = -0.0
    W[3, :128] = np.float32(448.0)
    W[3, 5] = np.float32(-448.0)
    W[4, :128] = np.array([1 + 1 / 16, 1 + 3 / 16] * 64, np.float32) * np.float32(448.0 / 1.25)
    W[5:, 128:] = np.random.default_rng(4).standard_normal((11, 128)).astype(np.float32)
    codes, scales = B.i4d_pack_weights_e4m3(B.I4D_PROJ_PLAIN, W)
    rq, rs, _ = O.quantize_weight_e4m3(W)
    q, s = B.i4d_unpack_weights_e4m3(B.I4D_PROJ_PLAIN, codes, scales, N, K)
    np.testing.assert_array_equal(q, rq)
    np.testing.assert_array_equal(s, rs.view(np.uint16))
    # byte of (row r, k = 128 g + 32 kb + 8 j + e) at ((g * 64 + 16 j + r) * 32 + 8 kb + e)
    for r, k in [(0, 0), (3, 5), (7, 127), (15, 200), (9, 128 + 32 * 3 + 8 * 2 + 6)]:
        g, kk = divmod(k, 128)
        kb, rem = divmod(kk, 32)
        j, e = divmod(rem, 8)
        assert codes[(g * 64 + 16 * j + r) * 32 + 8 * kb + e] == rq[r, k]
