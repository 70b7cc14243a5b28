"""Brute force on tiny shapes: the whole decode block written a second way.

The second formulation shares only the encodings with the oracle (quantizer,
KV encoding, bf16 rounding: each pinned on its own in test_oracle_pins.py)
and computes everything else by a different route: explicit per-head slicing,
RoPE as complex multiplication, keys and values rotated back with the dense
Sylvester matrix (H^-1 = H / b) instead of rotating the queries, repeat_kv
head expansion instead of the h // G map, scipy's softmax and expit, and
explicit per-group scale multiplication for the dense weights.
"""
import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle as O
from int4_quantized_decode_amd import synth


def dense_by_groups(q, s):
    N, K = q.shape
    W = np.zeros((N, K))
    for g in range(K // 128):
        W[:, g * 128:(g + 1) * 128] = q[:, g * 128:(g + 1) * 128] * s[:, g].astype(np.float64)[:, None]
    return W


def bruteforce_block(shape, lw, prefill, x_bits, lengths):
    d, hd, nq, nkv, F = shape.d_model, shape.head_dim, shape.n_q_heads, shape.n_kv_heads, shape.d_ffn
    eps, theta = shape.rms_eps, shape.rope_theta
    M = len(lengths)
    x = synth.bf16_bits_to_f32(x_bits).astype(np.float64).reshape(M, d)

    # gains folded here (fp32 product per weight), then the pinned quantizer
    Wqkv = dense_by_groups(*O.quantize_weight(lw.w_qkv * lw.gamma_attn[None, :]))
    Wo = dense_by_groups(*O.quantize_weight(lw.w_o))
    Wg = dense_by_groups(*O.quantize_weight(lw.w_gate * lw.gamma_ffn[None, :]))
    Wu = dense_by_groups(*O.quantize_weight(lw.w_up * lw.gamma_ffn[None, :]))
    Wd = dense_by_groups(*O.quantize_weight(lw.w_down))
    H = O.sylvester(hd)

    out = np.zeros((M, d))
    attn_all = np.zeros((M, nq * hd))
    for r in range(M):
        L = int(lengths[r])
        xr = x[r]
        rho = (np.sum(xr ** 2) / d + eps) ** -0.5
        y = np.array([np.dot(Wqkv[n], xr) for n in range(Wqkv.shape[0])]) * rho

        def head(idx):
            return y[idx * hd:(idx + 1) * hd]

        def rot(v):
            half = hd // 2
            z = v[:half] + 1j * v[half:]
            w = z * np.exp(1j * (L - 1) * theta ** (-np.arange(half) * 2.0 / hd))
            return np.concatenate([w.real, w.imag])

        qs = [rot(head(h)) for h in range(nq)]
        ks = [O.round_to_bf16(rot(head(nq + j))) for j in range(nkv)]
        vs = [O.round_to_bf16(head(nq + nkv + j)) for j in range(nkv)]

        # cache: prefill tokens then the new one, all through the KV encoding
        Kt = np.zeros((L, nkv, hd))
        Vt = np.zeros((L, nkv, hd))
        if L > 1:
            kq, kss = O.quantize_kv(synth.bf16_bits_to_f32(prefill.k[r]))
            vq, vss = O.quantize_kv(synth.bf16_bits_to_f32(prefill.v[r]))
            Kt[:L - 1] = kq * kss.astype(np.float64)[..., None]
            Vt[:L - 1] = vq * vss.astype(np.float64)[..., None]
        for j in range(nkv):
            kq, kss = O.quantize_kv(ks[j])
            vq, vss = O.quantize_kv(vs[j])
            Kt[L - 1, j] = kq * np.float64(kss)
            Vt[L - 1, j] = vq * np.float64(vss)
        K_un = Kt @ H.T / hd          # rows: H^-1 (H k) = k
        V_un = Vt @ H.T / hd
        K_exp = np.repeat(K_un, nq // nkv, axis=1)
        V_exp = np.repeat(V_un, nq // nkv, axis=1)
        attn = np.concatenate([softmax(K_exp[:, h, :] @ qs[h] / np.sqrt(hd)) @ V_exp[:, h, :]
                               for h in range(nq)])
        attn_all[r] = attn
        hres = xr + Wo @ attn
        rho2 = (np.sum(hres ** 2) / d + eps) ** -0.5
        g = rho2 * (Wg @ hres)
        u = rho2 * (Wu @ hres)
        a = g * expit(g) * u
        out[r] = hres + Wd @ a
    return out, attn_all


@pytest.mark.parametrize("shape", [synth.SHAPE_TINY, synth.SHAPE_SMALL128], ids=["hd64", "hd128"])
def test_block_matches_bruteforce(shape):
    lengths = np.array([1, 2, 5, 67], np.int32)
    lw = synth.make_layer(shape, 42)
    pre = synth.make_cache_prefill(shape, lengths, 42)
    xb = synth.make_x(shape, len(lengths), 42)
    ql = O.quantize_layer(lw)
    cache = O.build_cache(shape, lengths, pre)
    res = O.decode_block(shape, ql, cache, xb, lengths)
    out_bf, attn_bf = bruteforce_block(shape, lw, pre, xb, lengths)
    np.testing.assert_allclose(res.attn, attn_bf, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(res.out, out_bf, rtol=1e-9, atol=1e-11)
