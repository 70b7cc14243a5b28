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
