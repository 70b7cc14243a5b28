"""Planted mistakes in the oracle must be caught by its pins.

Each case swaps one oracle function for a plausible wrong variant (on the CPU,
inside this process only) and checks that at least one pin or the brute-force
block comparison now fails.  This is evidence that the pins constrain the
oracle, not a test of the HIP path.
"""
import numpy as np
import pytest

import oracle
import oracle.reference as R
from tests import test_oracle_bruteforce as BF
from tests import test_oracle_pins as P


def _fails(fn, *a):
    try:
        fn(*a)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def _block_check(shape):
    return BF.test_block_matches_bruteforce(shape)


def mut_gqa_modulo(q_rot, k_codes, k_scales, v_codes, v_scales, L, b):
    n_q, hd = q_rot.shape
    n_kv = k_codes.shape[1]
    out = np.empty((n_q, hd))
    for h in range(n_q):
        j = h % n_kv                                  # wrong head map
        k_hat = R.dequantize_kv(k_codes[:L, j, :], k_scales[:L, j])
        v_hat = R.dequantize_kv(v_codes[:L, j, :], v_scales[:L, j])
        sc = (k_hat @ q_rot[h]) / (b * np.sqrt(hd))
        p = np.exp(sc - sc.max())
        p /= p.sum()
        out[h] = R.fwht(p @ v_hat) / b
    return out


def _attn_generic(q_rot, k_codes, k_scales, v_codes, v_scales, L, b, out_div, score_div):
    n_q, hd = q_rot.shape
    G = n_q // k_codes.shape[1]
    out = np.empty((n_q, hd))
    for h in range(n_q):
        j = h // G
        k_hat = R.dequantize_kv(k_codes[:L, j, :], k_scales[:L, j])
        v_hat = R.dequantize_kv(v_codes[:L, j, :], v_scales[:L, j])
        sc = (k_hat @ q_rot[h]) / score_div(b, hd)
        p = np.exp(sc - sc.max())
        p /= p.sum()
        out[h] = R.fwht(p @ v_hat) / out_div(b)
    return out


def mut_rope_adjacent_pairs(v, pos, theta):
    v = np.asarray(v, dtype=np.float64)
    hd = v.shape[-1]
    inv_freq = theta ** (-2.0 * np.arange(hd // 2) / hd)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    a, bb = v[..., 0::2], v[..., 1::2]                # interleaved pairs instead of halves
    out = np.empty_like(v)
    out[..., 0::2] = a * c - bb * s
    out[..., 1::2] = bb * c + a * s
    return out


def mut_quant_absmax_over_8(v):
    v = np.asarray(v, dtype=np.float32)
    a = np.max(np.abs(v), axis=-1)
    s = R.fp16_round(a / np.float32(8.0))
    sf = s.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.clip(np.rint(v / sf), -8, 7)
    q = np.where(sf == 0, 0.0, q)
    return q.astype(np.int8), s


def mut_quant_round_half_away(v):
    v = np.asarray(v, dtype=np.float32)
    a = np.max(np.abs(v), axis=-1)
    s = R.fp16_round(a / np.float32(7.0))
    sf = s.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = v / sf
    q = np.clip(np.sign(r) * np.floor(np.abs(r) + 0.5), -8, 7)
    q = np.where(sf == 0, 0.0, q)
    return q.astype(np.int8), s


def mut_fwht_swapped_signs(x, dtype=np.float64):
    y = np.array(x, dtype=dtype, copy=True)
    b = y.shape[-1]
    lead = y.shape[:-1]
    h = 1
    while h < b:
        y = y.reshape(lead + (b // (2 * h), 2, h))
        lo, hi = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :] = lo - hi
        y[..., 1, :] = lo + hi
        y = y.reshape(lead + (b,))
        h *= 2
    return y


def mut_fold_gain_rows(W, gamma):
    W = np.asarray(W, dtype=np.float32)
    if gamma is None:
        return W
    g = np.asarray(gamma, dtype=np.float32)
    return W * np.resize(g, W.shape[0])[:, None]      # gain applied per output row


def mut_rms_no_eps(x, eps):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / np.sqrt(np.mean(x * x, axis=-1))


def mut_silu_sigmoid_only(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


def mut_round_bf16_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.trunc(m * 256.0) / 256.0, e)


TINY = BF.synth.SHAPE_TINY

CASES = [
    ("attention_one_row", mut_gqa_modulo, [(_block_check, TINY)]),
    ("attention_one_row",
     lambda *a: _attn_generic(*a, out_div=lambda b: 1.0, score_div=lambda b, hd: b * np.sqrt(hd)),
     [(P.test_attention_single_token_returns_its_value,)]),
    ("attention_one_row",
     lambda *a: _attn_generic(*a, out_div=lambda b: b, score_div=lambda b, hd: np.sqrt(hd)),
     [(P.test_attention_matches_expanded_heads_bruteforce,)]),
    ("rope", mut_rope_adjacent_pairs, [(P.test_rope_pairs_frequencies_and_relative_position,)]),
    ("quantize_rtn_lastaxis", mut_quant_absmax_over_8, [(P.test_quantizer_absmax_maps_to_seven,)]),
    ("quantize_rtn_lastaxis", mut_quant_round_half_away, [(P.test_quantizer_ties_half_to_even,)]),
    ("fwht", mut_fwht_swapped_signs, [(P.test_fwht_is_sylvester_and_orthogonal, 4)]),
    ("fold_gain", mut_fold_gain_rows, [(_block_check, TINY), (P.test_gain_fold_identity,)]),
    ("rms_factor", mut_rms_no_eps, [(P.test_rms_factor_closed_form,)]),
    ("silu", mut_silu_sigmoid_only, [(P.test_silu_closed_forms,)]),
    ("round_to_bf16", mut_round_bf16_truncate, [(P.test_round_to_bf16_ties_and_idempotence,)]),
]


@pytest.mark.parametrize("name,mutant,checks", CASES, ids=[f"{c[0]}-{i}" for i, c in enumerate(CASES)])
def test_planted_mistake_is_caught(monkeypatch, name, mutant, checks):
    # the unmutated oracle passes the same checks
    for fn, *args in checks:
        fn(*args)
    # the package re-exports the module's names: patch both bindings
    monkeypatch.setattr(R, name, mutant)
    monkeypatch.setattr(oracle, name, mutant)
    assert any(_fails(fn, *args) for fn, *args in checks)


def test_wrong_residual_or_transpose_caught(monkeypatch):
    """Dropping the attention residual, or using W_o untransposed, breaks the block check."""
    orig = R.decode_block

    def no_residual(shape, ql, cache, x_bits, lengths, dense_cache=None):
        res = orig(shape, ql, cache, x_bits, lengths, dense_cache)
        return R.BlockResult(res.out - R._bf16_bits_to_values(np.asarray(x_bits).reshape(len(lengths), -1)),
                             *[getattr(res, f) for f in ("attn", "h", "q", "k_new", "v_new", "k_codes_new",
                                                         "k_scales_new", "v_codes_new", "v_scales_new")])

    monkeypatch.setattr(R, "decode_block", no_residual)
    monkeypatch.setattr(BF.O, "decode_block", no_residual)
    assert _fails(_block_check, TINY)

    monkeypatch.setattr(R, "decode_block", orig)
    monkeypatch.setattr(BF.O, "decode_block", orig)
    dq = R.dense

    def transposed(part):
        W = dq(part)
        return W.T if W.shape[0] == W.shape[1] else W

    monkeypatch.setattr(R, "dense", transposed)
    assert _fails(_block_check, TINY)
