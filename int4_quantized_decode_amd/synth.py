"""Seeded synthetic inputs for the INT4 decode block.

This module only draws random numbers and rounds them to the bf16 storage
format the block takes as input.  It holds none of the method's arithmetic
(no quantizer, no rotation, no projection): both the CPU oracle and the HIP
path consume exactly the arrays produced here.

Workload shapes follow the Llama-style layer shapes the FuTransformer pages
evaluate (1B / 8B / 70B layer shapes, decode batches 1-32; FuTransformer
paper, "premises and limits" section of the onedev.kr summary and the English
abstract).  Value distributions:

* projection weights N(0, 0.02^2) in fp32;
* RMSNorm gains U(0.5, 1.5);
* cached keys / values N(0, 1) with hd/16 outlier channels per KV head
  (chosen without replacement, independently for K and V, fixed across
  tokens) multiplied by 20, then rounded to bf16;
* block input x ~ N(0, 1) rounded to bf16;
* prefill activations N(0, 1) with d/128 outlier channels multiplied by
  20, rounded to bf16.

Random streams are keyed by (seed, purpose) through numpy's SeedSequence so
that the weights of a layer do not depend on the batch size or the context
lengths drawn for a step.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

# purposes of the independent random streams of one (config, layer) seed
_P_WEIGHTS, _P_CACHE, _P_X, _P_LENGTHS, _P_LMHEAD, _P_PREFILL = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class LayerShape:
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    group: int = 128
    rms_eps: float = 1e-5
    rope_theta: float = 500000.0

    @property
    def hadamard_block(self) -> int:
        return self.head_dim

    @property
    def n_qkv(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def gqa_group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


SHAPE_1B = LayerShape(2048, 32, 8, 64, 8192)
SHAPE_8B = LayerShape(4096, 32, 8, 128, 14336)
SHAPE_70B = LayerShape(8192, 64, 8, 128, 28672)
# tiny shape for brute-force checks and fast parity cases (every K a multiple
# of the 128-wide weight group, several 16-row strips, GQA group 2)
SHAPE_TINY = LayerShape(256, 4, 2, 64, 512)
SHAPE_SMALL128 = LayerShape(512, 8, 2, 128, 1024)

LM_VOCAB = 128256
# seed of the LM head of the 32-layer 8B-shape model (its layers take seeds 4000..4031)
LM_HEAD_SEED = 4999


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    M: int
    ctx: int                      # context per row (incl. the new token); 0 = ragged
    seed: int
    ctx_lo: int = 0               # ragged rows: lengths ~ U{ctx_lo..ctx_hi}
    ctx_hi: int = 0
    n_layers: int = 1
    num_splits: int = 0           # 0 = library's automatic choice


WORKLOADS = {
    # 1B-shape layer, one row, context 256, seed 0
    "1b_m1_ctx256": Workload("1b_m1_ctx256", SHAPE_1B, 1, 256, 0),
    # 8B-shape layer, one row, context 4096
    "8b_m1_ctx4096": Workload("8b_m1_ctx4096", SHAPE_8B, 1, 4096, 1000),
    # 8B-shape layer, 32 independent rows with ragged contexts 1024..4096
    "8b_m32_ragged": Workload("8b_m32_ragged", SHAPE_8B, 32, 0, 2000, 1024, 4096),
    # 70B-shape layer, context 4096 (batch swept 1..32 by the caller)
    "70b_ctx4096": Workload("70b_ctx4096", SHAPE_70B, 1, 4096, 3000),
    # 32 stacked 8B-shape layers + bf16 LM head, context 32768, 16 KV splits
    "8b_32layer_ctx32768": Workload("8b_32layer_ctx32768", SHAPE_8B, 1, 32768, 4000,
                                    n_layers=32, num_splits=16),
}


@dataclasses.dataclass(frozen=True)
class PrefillWorkload:
    """A packed prefill batch: request r has seqlens[r] new tokens at positions
    starts[r], starts[r] + 1, ... of its cache row."""
    name: str
    shape: LayerShape
    seqlens: tuple
    starts: tuple
    seed: int

    @property
    def T(self) -> int:
        return int(sum(self.seqlens))


PREFILL_WORKLOADS = {
    # 8B-shape layer, one 2048-token prompt from position 0 (the pages' 8B
    # prefill shape at S = 2048)
    "8b_prefill_s2048": PrefillWorkload("8b_prefill_s2048", SHAPE_8B, (2048,), (0,), 5000),
    # 8B shape, a packed batch of 8: one 2048-token prompt and seven of 128
    # (the pages' variable-length case, B = 8, S_max = 2048)
    "8b_prefill_varlen": PrefillWorkload("8b_prefill_varlen", SHAPE_8B, (2048,) + (128,) * 7, (0,) * 8, 5001),
    # 70B-shape layer, one 2048-token prompt
    "70b_prefill_s2048": PrefillWorkload("70b_prefill_s2048", SHAPE_70B, (2048,), (0,), 5002),
}


def prefill_offsets(seqlens) -> np.ndarray:
    """Prefix sums of the request lengths: int32 [R + 1], starting at 0."""
    return np.concatenate([[0], np.cumsum(np.asarray(seqlens, dtype=np.int64))]).astype(np.int32)


def make_prefill_x(shape: LayerShape, T: int, seed: int) -> np.ndarray:
    """Packed prefill activations, bf16 bits [T, d]: N(0, 1) with d/128
    outlier channels (fixed across tokens) multiplied by 20."""
    r = _rng(seed, _P_PREFILL)
    d = shape.d_model
    m = np.ones(d, dtype=np.float32)
    m[r.permutation(d)[: max(1, d // 128)]] = np.float32(20.0)
    return f32_to_bf16_bits(r.standard_normal((T, d), dtype=np.float32) * m[None])


def _rng(seed: int, purpose: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(purpose)]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Input preparation only: the generated activations and cache entries are
    bf16 tensors, and this is how they are stored.  Inputs are finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class LayerWeights:
    """fp32 weights of one layer in PyTorch [out, in] convention."""
    w_qkv: np.ndarray     # [(n_q + 2 n_kv) hd, d]: q rows, then k rows, then v rows
    w_o: np.ndarray       # [d, n_q hd]
    w_gate: np.ndarray    # [F, d]
    w_up: np.ndarray      # [F, d]
    w_down: np.ndarray    # [d, F]
    gamma_attn: np.ndarray  # [d]
    gamma_ffn: np.ndarray   # [d]


def make_layer(shape: LayerShape, seed: int) -> LayerWeights:
    r = _rng(seed, _P_WEIGHTS)
    d, F = shape.d_model, shape.d_ffn
    nqh = shape.n_q_heads * shape.head_dim

    def w(n, k):
        a = r.standard_normal((n, k), dtype=np.float32)
        a *= np.float32(0.02)
        return a

    w_qkv = w(shape.n_qkv, d)
    w_o = w(d, nqh)
    w_gate = w(F, d)
    w_up = w(F, d)
    w_down = w(d, F)
    g_attn = r.uniform(0.5, 1.5, d).astype(np.float32)
    g_ffn = r.uniform(0.5, 1.5, d).astype(np.float32)
    return LayerWeights(w_qkv, w_o, w_gate, w_up, w_down, g_attn, g_ffn)


def make_lengths(wl: Workload, M: Optional[int] = None) -> np.ndarray:
    """Context length per row, counting the token appended this step."""
    M = wl.M if M is None else M
    if wl.ctx > 0:
        return np.full(M, wl.ctx, dtype=np.int32)
    r = _rng(wl.seed, _P_LENGTHS)
    return r.integers(wl.ctx_lo, wl.ctx_hi, size=M, endpoint=True).astype(np.int32)


@dataclasses.dataclass
class CachePrefill:
    """bf16 keys/values already in the cache before the step (rows are ragged).

    k[r], v[r]: uint16 bf16 bits of shape [L_r - 1, n_kv, hd] (positions 0..L_r-2).
    """
    k: List[np.ndarray]
    v: List[np.ndarray]


def make_cache_prefill(shape: LayerShape, lengths: np.ndarray, seed: int) -> CachePrefill:
    r = _rng(seed, _P_CACHE)
    hd, nkv = shape.head_dim, shape.n_kv_heads
    n_out = max(1, hd // 16)
    mult = {}
    for which in ("k", "v"):
        m = np.ones((nkv, hd), dtype=np.float32)
        for j in range(nkv):
            ch = r.permutation(hd)[:n_out]
            m[j, ch] = np.float32(20.0)
        mult[which] = m
    ks, vs = [], []
    for L in lengths:
        n = int(L) - 1
        kk = r.standard_normal((n, nkv, hd), dtype=np.float32) * mult["k"][None]
        vv = r.standard_normal((n, nkv, hd), dtype=np.float32) * mult["v"][None]
        ks.append(f32_to_bf16_bits(kk))
        vs.append(f32_to_bf16_bits(vv))
    return CachePrefill(ks, vs)


def make_x(shape: LayerShape, M: int, seed: int) -> np.ndarray:
    """Block input rows, bf16 bits [M, d]."""
    r = _rng(seed, _P_X)
    return f32_to_bf16_bits(r.standard_normal((M, shape.d_model), dtype=np.float32))


def make_lm_head(d: int, vocab: int, seed: int):
    """fp32 LM head weight [vocab, d] ~ N(0, 0.02^2) and final-norm gain U(0.5, 1.5)."""
    r = _rng(seed, _P_LMHEAD)
    w = r.standard_normal((vocab, d), dtype=np.float32)
    w *= np.float32(0.02)
    g = r.uniform(0.5, 1.5, d).astype(np.float32)
    return w, g
