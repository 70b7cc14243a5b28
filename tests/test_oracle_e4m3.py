"""Pins of the oracle's E4M3 decode-weight encoding (reading R12 of the
oracle: the summary page's "premises and limits" section reports E4M3
decode weights beside the INT4 ones; the format is OCP FP8 E4M3, the scale
one fp16 per (row, 128-group) = fp16(absmax / 448)).

Each pin fixes the encoding by something other than the oracle itself:
closed forms of the format's definition, constructed ties, exhaustive round
trips over the 256 codes, and PyTorch's own float8_e4m3fn conversion (a
library routine; it rounds to nearest even and agrees with saturation on
every value below 448).  A planted mistake in the encoder fails one of
them (test_planted_mistakes_fail_a_pin).
"""
import numpy as np
import pytest
import torch

import oracle as O
import oracle.reference as R

TABLE = [
    # value, code: the format's definition written out
    (0.0, 0x00), (-0.0, 0x80), (1.0, 0x38), (-1.0, 0xB8), (2.0 ** -6, 0x08), (2.0 ** -9, 0x01),
    (7 * 2.0 ** -9, 0x07), (448.0, 0x7E), (-448.0, 0xFE), (1.875, 0x3F), (256.0, 0x78), (0.5, 0x30),
    (3.0, 0x44), (0.1015625, 0x1D),  # 0.1015625 = 2^-4 * 1.625 -> e = 3, m = 5
]


def test_e4m3_closed_forms():
    vals = np.array([v for v, _ in TABLE], np.float32)
    codes = np.array([c for _, c in TABLE], np.uint8)
    np.testing.assert_array_equal(O.e4m3_encode(vals), codes)
    dec = O.e4m3_decode(codes)
    np.testing.assert_array_equal(np.abs(dec), np.abs(vals.astype(np.float64)))
    assert np.isnan(O.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_ties_to_even_and_saturation():
    cases = [
        (1 + 1 / 16, 0x38),      # halfway between 1 and 1.125 -> even mantissa 0
        (1 + 3 / 16, 0x3A),      # halfway between 1.125 and 1.25 -> even mantissa 2
        (2.0 ** -10, 0x00),      # halfway between 0 and 2^-9 -> 0
        (3 * 2.0 ** -10, 0x02),  # halfway between 2^-9 and 2^-8 -> 2^-8
        (15 * 2.0 ** -10, 0x08),  # halfway between 7 * 2^-9 and 2^-6 -> 2^-6 (even)
        (464.0, 0x7E), (448.5, 0x7E), (1e6, 0x7E), (-1e30, 0xFE),
        (0.96875, 0x38),         # halfway between 0.9375 and 1.0 -> 1.0 (next exponent)
        (-2.0 ** -11, 0x80),     # rounds to zero, keeps its sign
    ]
    for v, c in cases:
        assert int(O.e4m3_encode(np.array([v], np.float32))[0]) == c, (v, hex(c))


def test_e4m3_exhaustive_round_trip():
    codes = np.arange(256, dtype=np.uint8)
    vals = O.e4m3_decode(codes)
    fin = ~np.isnan(vals)
    assert fin.sum() == 254
    np.testing.assert_array_equal(O.e4m3_encode(vals[fin].astype(np.float32)), codes[fin])
    # monotone over the positive codes, spacing 2^-9 below 2^-6
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)
    np.testing.assert_array_equal(pos[:9], np.arange(9) * 2.0 ** -9)


def test_e4m3_matches_torch_float8():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000) * 30, rng.standard_normal(20000) * 1e-2,
                        rng.uniform(-448, 448, 20000)]).astype(np.float32)
    # every finite fp16 value below 448 in magnitude, exhaustively
    h = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float32)
    h = h[np.isfinite(h) & (np.abs(h) < 448)]
    for v in (x, h):
        ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(O.e4m3_encode(v), ref)


def test_e4m3_quantizer_absmax_zero_group_and_round_trip():
    rng = np.random.default_rng(2)
    W = (rng.standard_normal((32, 384)) * 0.02).astype(np.float32)
    W[3, 128:256] = 0.0                               # zero group
    W[5, 0:128] = rng.uniform(-1, 1, 128).astype(np.float32)
    W[5, 7] = -448.0 * 2.0 ** -7                       # absmax whose fp16 scale is exact
    q, s, fmt = O.quantize_weight_e4m3(W)
    assert fmt == "e4m3" and q.dtype == np.uint8 and s.dtype == np.float16 and s.shape == (32, 3)
    assert s[3, 1] == 0 and np.all(q[3, 128:256] == 0)
    assert float(s[5, 0]) == 2.0 ** -7 and q[5, 7] == 0xFE
    W_hat = O.dense((q, s, fmt))
    sf = np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(W_hat - W.astype(np.float64))
    # half a step: 2^-4 relative for normals, 2^-10 s for subnormals, plus
    # the absmax element's saturation (s rounded down by up to 2^-11)
    assert np.all(err <= 2.0 ** -4 * np.abs(W) + 2.0 ** -10 * sf + 2.0 ** -11 * 448 * sf + 1e-12)
    # idempotence: the dequantized weight encodes to the same codes and scales
    q2, s2, _ = O.quantize_weight_e4m3(W_hat.astype(np.float32))
    np.testing.assert_array_equal(s2, s)
    np.testing.assert_array_equal(q2, q)
    # sign symmetry (a zero-scale group stores code 0 whatever the sign)
    qn, sn, _ = O.quantize_weight_e4m3(-W)
    np.testing.assert_array_equal(sn, s)
    live = np.repeat(s != 0, 128, axis=1)
    np.testing.assert_array_equal(qn[live], (q ^ 0x80)[live])
    assert np.all(qn[~live] == 0)


def test_e4m3_layer_gain_fold():
    """The gains fold into QKV, gate and up as for INT4 (R3): quantizing
    gamma * W directly gives the same codes."""
    from int4_quantized_decode_amd import synth
    lw = synth.make_layer(synth.SHAPE_TINY, 5)
    ql = O.quantize_layer_e4m3(lw)
    q, s, _ = O.quantize_weight_e4m3(lw.w_qkv * lw.gamma_attn[None, :])
    np.testing.assert_array_equal(ql.qkv[0], q)
    np.testing.assert_array_equal(ql.qkv[1], s)
    q, s, _ = O.quantize_weight_e4m3(lw.w_down)
    np.testing.assert_array_equal(ql.down[0], q)


def _round_half_away(x):
    return np.sign(x) * np.floor(np.abs(x) + 0.5)


@pytest.mark.parametrize("mistake", ["half_away", "no_saturation", "bias8", "sub_step"])
def test_planted_mistakes_fail_a_pin(monkeypatch, mistake):
    pins = [test_e4m3_closed_forms, test_e4m3_ties_to_even_and_saturation, test_e4m3_exhaustive_round_trip,
            test_e4m3_matches_torch_float8]
    if mistake == "half_away":
        monkeypatch.setattr(R.np, "rint", _round_half_away, raising=True)
    elif mistake == "no_saturation":
        orig_enc = R.e4m3_encode

        def enc(x):  # a conversion without saturation: NaN code above the largest finite value
            x = np.asarray(x, np.float32)
            c = orig_enc(x)
            return np.where(np.abs(x) > 448.0, (c & 0x80) | 0x7F, c).astype(np.uint8)
        monkeypatch.setattr(R, "e4m3_encode", enc)
        monkeypatch.setattr(O, "e4m3_encode", enc)
    elif mistake == "bias8":
        orig = R.e4m3_decode
        monkeypatch.setattr(R, "e4m3_decode", lambda c: orig(c) * 0.5)
        monkeypatch.setattr(O, "e4m3_decode", R.e4m3_decode)
    elif mistake == "sub_step":
        orig_enc = R.e4m3_encode

        def enc(x):
            x = np.asarray(x, np.float32)
            c = orig_enc(x).astype(np.int64)
            a = np.abs(x.astype(np.float64))
            wrong = np.where(a < 2.0 ** -6, np.floor(a * 512.0), c & 0x7F)  # truncating subnormals
            return ((c & 0x80) | wrong.astype(np.int64)).astype(np.uint8)
        monkeypatch.setattr(R, "e4m3_encode", enc)
        monkeypatch.setattr(O, "e4m3_encode", enc)
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, mistake
