"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Every check here is a closed form, an invariant, a special case with a known
answer, an independent library routine, or a value the pages state.  They are
chosen so that a plausible slip in the oracle (a dropped term, a wrong sign or
index, a transposed operand, the wrong rounding) fails at least one of them;
tests/test_oracle_mutations.py plants such slips and checks that they do.
"""
import os
import struct

import numpy as np
import pytest

import oracle as O
from int4_quantized_decode_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits << 16))[0]


# ---------------------------------------------------------------------------
# rounding helpers
# ---------------------------------------------------------------------------

def test_fp16_round_ties_and_saturation():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -10)
    # exact halfway between 1 and 1+ulp -> even (1.0)
    assert O.fp16_round(one + ulp / 2) == np.float16(1.0)
    # halfway between 1+ulp (odd significand) and 1+2ulp (even) -> 1+2ulp
    assert O.fp16_round(one + np.float32(1.5) * ulp) == np.float16(1.0 + 2 * 2.0 ** -10)
    # just above halfway rounds up
    assert O.fp16_round(np.nextafter(one + ulp / 2, np.float32(2))) == np.float16(1.0 + 2.0 ** -10)
    # overflow saturates at the largest finite fp16
    assert O.fp16_round(np.float32(1e6)) == np.float16(65504)
    assert O.fp16_round(np.float32(-1e6)) == np.float16(-65504)
    # smallest subnormal survives; half of it is a tie -> 0
    assert O.fp16_round(np.float32(2.0 ** -24)) == np.float16(2.0 ** -24)
    assert O.fp16_round(np.float32(2.0 ** -25)) == np.float16(0.0)


def test_round_to_bf16_ties_and_idempotence():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> even (1)
    assert O.round_to_bf16(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 halfway between 1+2^-7 (odd) and 1+2^-6 (even)
    assert O.round_to_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert O.round_to_bf16(-(1.0 + 3 * 2.0 ** -8)) == -(1.0 + 2.0 ** -6)
    # carry into the exponent
    assert O.round_to_bf16(2.0 - 2.0 ** -9) == 2.0
    # bf16 values are fixed points
    for bits in (0x3F80, 0x4049, 0xC2F7, 0x0080, 0x7F7F):
        v = bf16_bits_value(bits)
        assert O.round_to_bf16(v) == v


def test_round_to_bf16_matches_bit_level_rounding():
    # independent implementation: integer rounding of the fp32 bit pattern
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    bits = synth.f32_to_bf16_bits(x)
    ref = synth.bf16_bits_to_f32(bits).astype(np.float64)
    np.testing.assert_array_equal(O.round_to_bf16(x.astype(np.float64)), ref)


# ---------------------------------------------------------------------------
# weight quantizer (R1) and nibble code (R2)
# ---------------------------------------------------------------------------

def test_nibble_rule_golden_table():
    """The pages' decode rule: bf16 128.0 with the nibble in its mantissa, minus 136."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "nibble_bf16_128.txt")) if not l.startswith("#")]
    assert len(rows) == 16
    for u_s, bits_s, val_s, code_s in rows:
        u, bits, val, code = int(u_s), int(bits_s, 16), int(val_s), int(code_s)
        assert bf16_bits_value(bits) == val          # format fact, checked with struct
        assert O.code_of_nibble_via_bf16_128(u) == code
        assert O.nibble_of_code(code) == u
    assert [int(r[3]) for r in rows] == list(range(-8, 8))


def test_quantizer_absmax_maps_to_seven():
    rng = np.random.default_rng(1)
    W = rng.standard_normal((64, 512)).astype(np.float32) * np.float32(0.02)
    q, s = O.quantize_weight(W)
    g = W.reshape(64, 4, 128)
    idx = np.argmax(np.abs(g), axis=2)
    top = np.take_along_axis(q.reshape(64, 4, 128), idx[..., None], axis=2)[..., 0]
    sign = np.sign(np.take_along_axis(g, idx[..., None], axis=2)[..., 0])
    np.testing.assert_array_equal(top, (7 * sign).astype(np.int8))
    assert q.min() >= -7 and q.max() <= 7     # absmax/7 never produces -8


def test_quantizer_ties_half_to_even():
    # group absmax exactly 7 -> s = fp16(7/7) = 1 exactly -> codes = rint(w)
    g = np.zeros(128, np.float32)
    g[:7] = [2.5, 3.5, -2.5, 0.5, 7.0, -1.5, -0.5]
    q, s = O.quantize_rtn_lastaxis(g)
    assert s == np.float16(1.0)
    np.testing.assert_array_equal(q[:7], [2, 4, -2, 0, 7, -2, 0])


def test_quantizer_worked_example_fp16_scale():
    # absmax 0.7: fp32 0.7/7 rounds to fp16 0.0999755859375; -0.35/s = -3.50085 (not a tie) -> -4
    g = np.zeros(128, np.float32)
    g[:3] = [0.7, -0.35, 0.05]
    q, s = O.quantize_rtn_lastaxis(g)
    assert float(s) == 0.0999755859375
    np.testing.assert_array_equal(q[:3], [7, -4, 1])


def test_quantizer_round_trip_idempotence_symmetry():
    rng = np.random.default_rng(2)
    W = rng.standard_normal((32, 1024)).astype(np.float32) * np.float32(0.05)
    q, s = O.quantize_weight(W)
    Wh = O.dequantize_weight(q, s)
    sf = np.repeat(s.astype(np.float64), 128, axis=1)
    assert np.all(np.abs(Wh - W) <= sf / 2 * (1 + 2.0 ** -9))
    # quantizing the dequantized grid reproduces it exactly
    q2, s2 = O.quantize_weight(Wh.astype(np.float32))
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(s2, s)
    # odd symmetry
    qn, sn = O.quantize_weight(-W)
    np.testing.assert_array_equal(qn, -q)
    np.testing.assert_array_equal(sn, s)


def test_quantizer_zero_group_and_group_axis():
    # W[n, k] = (n + 1) * (k // 128 + 1) * sign pattern: group scales follow a closed form
    N, K = 5, 384
    n = np.arange(N)[:, None] + 1
    gk = np.arange(K)[None, :] // 128 + 1
    sign = np.where(np.arange(K) % 3 == 0, -1.0, 1.0)[None, :]
    W = (n * gk * sign * 0.125).astype(np.float32)
    W[2, 128:256] = 0.0
    q, s = O.quantize_weight(W)
    expect = (n * np.arange(1, 4)[None, :] * 0.125 / 7).astype(np.float32).astype(np.float16)
    expect[2, 1] = 0
    np.testing.assert_array_equal(s, expect)
    assert np.all(q[2, 128:256] == 0)
    np.testing.assert_array_equal(q[s.repeat(128, axis=1) != 0], (7 * sign * np.ones((N, K)))[s.repeat(128, axis=1) != 0])


def test_gain_fold_identity():
    """rho * (x . (gamma (.) W)^T) == (rho x (.) gamma) . W^T: the gain scales input channels."""
    rng = np.random.default_rng(3)
    W = rng.standard_normal((48, 256)).astype(np.float32)
    gam = rng.uniform(0.5, 1.5, 256).astype(np.float32)
    x = rng.standard_normal((3, 256))
    rho = O.rms_factor(x, 1e-5)
    lhs = rho[:, None] * (x @ O.fold_gain(W, gam).astype(np.float64).T)
    rhs = ((rho[:, None] * x) * gam.astype(np.float64)) @ W.astype(np.float64).T
    # the only difference is the fp32 rounding of each product gamma*W (relative 2^-24)
    bound = 2.0 ** -24 * (rho[:, None] * (np.abs(x) * gam) @ np.abs(W.astype(np.float64)).T) + 1e-12
    assert np.all(np.abs(lhs - rhs) <= bound)


# ---------------------------------------------------------------------------
# Hadamard (R5) and KV encoding (R6)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("b", [1, 2, 4, 8, 16, 32, 64, 128])
def test_fwht_is_sylvester_and_orthogonal(b):
    H = O.fwht(np.eye(b))          # transform of the unit vectors = columns of H
    Hd = O.sylvester(b)
    np.testing.assert_array_equal(H.T, Hd)
    np.testing.assert_array_equal(Hd, Hd.T)
    np.testing.assert_array_equal(Hd @ Hd.T, b * np.eye(b))
    if b == 2:
        np.testing.assert_array_equal(Hd, [[1, 1], [1, -1]])


def test_fwht_fp32_exact_on_integers_and_close_on_floats():
    rng = np.random.default_rng(4)
    xi = rng.integers(-1000, 1000, (50, 128)).astype(np.float32)
    np.testing.assert_array_equal(O.fwht(xi, np.float32), (O.sylvester(128) @ xi.T.astype(np.float64)).T)
    xf = rng.standard_normal((50, 128)).astype(np.float32)
    ref = (O.sylvester(128) @ xf.T.astype(np.float64)).T
    err = np.abs(O.fwht(xf, np.float32) - ref)
    assert err.max() <= 128 * 2.0 ** -24 * np.abs(xf).sum(axis=1).max()


def test_fwht_stage_order_fp32():
    # b = 4, stages h=1 then h=2, each add rounded to fp32 (order matters for rounding)
    e = 2.0 ** -24
    x = np.array([1.0, e, 0.0, e], np.float32)
    y = O.fwht(x, np.float32)
    f = np.float32
    a0, a1 = f(x[0] + x[1]), f(x[0] - x[1])
    a2, a3 = f(x[2] + x[3]), f(x[2] - x[3])
    np.testing.assert_array_equal(y, [f(a0 + a2), f(a1 + a3), f(a0 - a2), f(a1 - a3)])
    assert y[0] == 1.0                     # (1 + e) ties to 1, then + e ties to 1 again
    # the opposite stage order (h=2 first) rounds differently here, so the order is pinned
    b0, b1 = f(x[0] + x[2]), f(x[1] + x[3])
    assert f(b0 + b1) == 1.0 + 2.0 ** -23 != y[0]


def test_rotation_preserves_dot_products():
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal((2, 20, 128))
    lhs = np.sum(O.fwht(q) * O.fwht(k), axis=-1)
    np.testing.assert_allclose(lhs, 128 * np.sum(q * k, axis=-1), rtol=1e-12, atol=1e-9)


def test_kv_encoding_one_hot_and_round_trip():
    x = np.zeros(64, np.float32)
    x[5] = 3.0
    q, s = O.quantize_kv(x)          # H e5 * 3 = +-3 everywhere
    assert s == O.fp16_round(np.float32(3.0) / np.float32(7.0))
    np.testing.assert_array_equal(np.abs(q), 7)
    np.testing.assert_array_equal(np.sign(q), O.sylvester(64)[:, 5])
    rng = np.random.default_rng(6)
    xs = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(rng.standard_normal((100, 128)).astype(np.float32)))
    qq, ss = O.quantize_kv(xs)
    rec = O.dequantize_kv(qq, ss)
    Hx = O.fwht(xs)
    assert np.all(np.abs(rec - Hx) <= ss.astype(np.float64)[:, None] / 2 * (1 + 2.0 ** -9) + 1e-4)


def test_rotation_reduces_outlier_cache_error():
    """The pages' claim: the rotation cuts cache quantization error from outlier channels."""
    wl = synth.WORKLOADS["1b_m1_ctx256"]
    pre = synth.make_cache_prefill(wl.shape, np.array([257]), 11)
    k = synth.bf16_bits_to_f32(pre.k[0]).astype(np.float64)           # [256, 8, 64]
    q_rot, s_rot = O.quantize_kv(k)
    rec_rot = O.fwht(O.dequantize_kv(q_rot, s_rot)) / 64               # back to the un-rotated basis
    q_pl, s_pl = O.quantize_rtn_lastaxis(k.astype(np.float32))
    rec_pl = O.dequantize_kv(q_pl, s_pl)
    e_rot = np.linalg.norm(rec_rot - k) / np.linalg.norm(k)
    e_pl = np.linalg.norm(rec_pl - k) / np.linalg.norm(k)
    assert e_rot < 0.7 * e_pl


# ---------------------------------------------------------------------------
# norm, RoPE, SwiGLU
# ---------------------------------------------------------------------------

def test_rms_factor_closed_form():
    x = np.full((2, 512), 0.75)
    np.testing.assert_allclose(O.rms_factor(x, 1e-5), 1.0 / np.sqrt(0.75 ** 2 + 1e-5), rtol=1e-15)


def test_rope_pairs_frequencies_and_relative_position():
    hd, theta = 64, 500000.0
    # position 0 is the identity
    v = np.random.default_rng(8).standard_normal((3, hd))
    np.testing.assert_array_equal(O.rope(v, np.zeros(3), theta), v)
    # unit vector e_i rotates inside the pair (i, i + hd/2) by p * theta^(-2i/hd)
    for i in (0, 5, 31):
        e = np.zeros(hd)
        e[i] = 1.0
        p = 1234
        r = O.rope(e, np.array(p), theta)
        ang = p * theta ** (-2.0 * i / hd)
        expect = np.zeros(hd)
        expect[i], expect[i + hd // 2] = np.cos(ang), np.sin(ang)
        np.testing.assert_allclose(r, expect, atol=1e-12)
    # norms kept, dot products depend only on the position difference
    q, k = np.random.default_rng(9).standard_normal((2, hd))
    d1 = O.rope(q, np.array(100), theta) @ O.rope(k, np.array(90), theta)
    d2 = O.rope(q, np.array(1010), theta) @ O.rope(k, np.array(1000), theta)
    np.testing.assert_allclose(d1, d2, rtol=1e-9)
    np.testing.assert_allclose(np.linalg.norm(O.rope(q, np.array(77), theta)), np.linalg.norm(q), rtol=1e-13)


def test_silu_closed_forms():
    assert O.silu(0.0) == 0.0
    np.testing.assert_allclose(O.silu(1.0), 1.0 / (1.0 + np.exp(-1.0)), rtol=1e-15)
    np.testing.assert_allclose(O.silu(40.0), 40.0, rtol=1e-15)
    assert abs(O.silu(-40.0)) < 1e-15


# ---------------------------------------------------------------------------
# attention (R5, R7, R8)
# ---------------------------------------------------------------------------

def _random_cache(L, nkv, hd, seed):
    rng = np.random.default_rng(seed)
    kc = rng.integers(-8, 8, (L, nkv, hd)).astype(np.int8)
    vc = rng.integers(-8, 8, (L, nkv, hd)).astype(np.int8)
    ks = rng.uniform(0.05, 0.5, (L, nkv)).astype(np.float16)
    vs = rng.uniform(0.05, 0.5, (L, nkv)).astype(np.float16)
    return kc, ks, vc, vs


def test_attention_single_token_returns_its_value():
    kc, ks, vc, vs = _random_cache(1, 2, 64, 10)
    q = np.random.default_rng(0).standard_normal((4, 64))
    o = O.attention_one_row(q, kc, ks, vc, vs, 1, 64)
    v0 = O.dequantize_kv(vc[0], vs[0])                 # [2, 64], rotated basis
    for h in range(4):
        np.testing.assert_allclose(o[h], O.sylvester(64) @ v0[h // 2] / 64, rtol=1e-13, atol=1e-13)


def test_attention_equal_scores_average_values():
    kc, ks, vc, vs = _random_cache(7, 2, 64, 11)
    kc[:] = kc[0]
    ks[:] = ks[0]
    q = np.random.default_rng(1).standard_normal((4, 64))
    o = O.attention_one_row(q, kc, ks, vc, vs, 7, 64)
    vbar = O.dequantize_kv(vc, vs).mean(axis=0)
    for h in range(4):
        np.testing.assert_allclose(o[h], O.sylvester(64) @ vbar[h // 2] / 64, rtol=1e-12, atol=1e-13)


def test_attention_matches_expanded_heads_bruteforce():
    """GQA without expansion == repeat_kv expansion + plain softmax in the un-rotated basis."""
    from scipy.special import softmax
    L, nkv, nq, hd = 37, 2, 8, 64
    kc, ks, vc, vs = _random_cache(L, nkv, hd, 12)
    q = np.random.default_rng(2).standard_normal((nq, hd))
    o = O.attention_one_row(O.fwht(q), kc, ks, vc, vs, L, hd)
    H = O.sylvester(hd)
    k_un = np.einsum("ij,tnj->tni", H, O.dequantize_kv(kc, ks)) / hd     # H^-1 = H / b
    v_un = np.einsum("ij,tnj->tni", H, O.dequantize_kv(vc, vs)) / hd
    k_exp = np.repeat(k_un, nq // nkv, axis=1)                             # [L, nq, hd]
    v_exp = np.repeat(v_un, nq // nkv, axis=1)
    for h in range(nq):
        p = softmax(k_exp[:, h, :] @ q[h] / np.sqrt(hd))
        np.testing.assert_allclose(o[h], p @ v_exp[:, h, :], rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("S", [1, 2, 3, 16, 37, 50])
def test_split_kv_reduction_equals_unsplit(S):
    L, nkv, nq, hd = 37, 2, 4, 64
    kc, ks, vc, vs = _random_cache(L, nkv, hd, 13)
    qr = O.fwht(np.random.default_rng(3).standard_normal((nq, hd)))
    ref = O.attention_one_row(qr, kc, ks, vc, vs, L, hd)
    chunk = -(-L // S)
    for h in range(nq):
        j = h // (nq // nkv)
        parts = []
        for s in range(S):
            lo, hi = s * chunk, min(L, (s + 1) * chunk)
            if lo >= hi:
                parts.append((-np.inf, 0.0, np.zeros(hd)))
                continue
            sc = O.dequantize_kv(kc[lo:hi, j], ks[lo:hi, j]) @ qr[h] / (hd * np.sqrt(hd))
            m = sc.max()
            e = np.exp(sc - m)
            parts.append((m, e.sum(), e @ O.dequantize_kv(vc[lo:hi, j], vs[lo:hi, j])))
        mstar = max(p[0] for p in parts)
        w = [np.exp(p[0] - mstar) if p[1] > 0 else 0.0 for p in parts]
        lsum = sum(wi * p[1] for wi, p in zip(w, parts))
        ot = sum(wi * p[2] for wi, p in zip(w, parts)) / lsum
        np.testing.assert_allclose(O.fwht(ot) / hd, ref[h], rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------------------
# LM head (R11)
# ---------------------------------------------------------------------------

def test_lm_head_argmax_ties_lowest_index_and_fold():
    d, V = 128, 10
    h = np.ones((1, d))
    W = np.zeros((V, d), np.float32)
    W[3, 0] = W[7, 0] = 2.0        # tie between 3 and 7
    W[5, 1] = 1.0
    logits, tok = O.lm_head_argmax(h, O.lm_head_weight_bf16(W, np.ones(d, np.float32)), 1e-5)
    assert tok[0] == 3
    np.testing.assert_allclose(logits[0, 3], 2.0 / np.sqrt(1 + 1e-5), rtol=1e-15)
    # gain fold picks the scaled column: gamma[1] = 3 makes row 5 win (3 > 2)
    g = np.ones(d, np.float32)
    g[1] = 3.0
    _, tok2 = O.lm_head_argmax(h, O.lm_head_weight_bf16(W, g), 1e-5)
    assert tok2[0] == 5
