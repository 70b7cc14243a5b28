"""Shared helpers of the GPU parity tests: run the HIP path and the oracle on
the same seeded inputs and measure the differences."""
import sys

import numpy as np

import oracle as O
from int4_quantized_decode_amd import synth


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_rms(a, ref) -> float:
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(a - ref) / max(np.linalg.norm(ref), 1e-300))


def norm_maxabs(a, ref) -> float:
    """max |a - ref| / rms(ref): the attention-output error measure."""
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(a - ref).max() / max(np.sqrt(np.mean(ref ** 2)), 1e-300))


def random_bf16(rng, shape, scale=1.0, outlier_channels=0):
    x = rng.standard_normal(shape).astype(np.float32) * np.float32(scale)
    if outlier_channels:
        hd = shape[-1]
        ch = rng.permutation(hd)[:outlier_channels]
        x[..., ch] *= np.float32(20.0)
    return synth.f32_to_bf16_bits(x)


def bf16_values(bits) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def oracle_cache_from_tokens(shape, k_rows, v_rows):
    """Oracle cache rows from per-row bf16 token arrays [L_r, n_kv, hd]."""
    rows = []
    for k, v in zip(k_rows, v_rows):
        kq, ks = O.quantize_kv(synth.bf16_bits_to_f32(k))
        vq, vs = O.quantize_kv(synth.bf16_bits_to_f32(v))
        rows.append(O.RowCache(kq, ks, vq, vs))
    return rows


def assert_appended_exact(cache, ws, shape, lengths):
    """The codes and fp16 scales the decode step appended at position L-1
    of every row equal the oracle's encoding (rotation, scale, rounding) of
    the step's own bf16 key and value, read back from the workspace.  The
    encoding is exact, so this is a bit-for-bit check of the in-step append
    (the oracle's own fp64 projection may round a k or v differently to bf16;
    that comparison is only reported)."""
    import torch
    from int4_quantized_decode_amd import device as D
    M = len(lengths)
    n = M * shape.n_kv_heads * shape.head_dim
    kb = D.to_host_u16(ws.view("k", torch.int16, n)).reshape(M, shape.n_kv_heads, shape.head_dim)
    vb = D.to_host_u16(ws.view("v", torch.int16, n)).reshape(M, shape.n_kv_heads, shape.head_dim)
    rk, rks = O.quantize_kv(synth.bf16_bits_to_f32(kb))
    rv, rvs = O.quantize_kv(synth.bf16_bits_to_f32(vb))
    for r, L in enumerate(lengths):
        k, v, ks, vs = cache.read_codes(r, int(L) - 1, int(L))
        np.testing.assert_array_equal(k[0], rk[r], err_msg=f"key codes of row {r}")
        np.testing.assert_array_equal(ks[0], rks[r].view(np.uint16), err_msg=f"key scales of row {r}")
        np.testing.assert_array_equal(v[0], rv[r], err_msg=f"value codes of row {r}")
        np.testing.assert_array_equal(vs[0], rvs[r].view(np.uint16), err_msg=f"value scales of row {r}")
