"""Plain fp64 CPU definition of the INT4 decode step of a Llama-style block.

TEST INFRASTRUCTURE ONLY (see the package docstring): slow, obviously
correct, and independent of the HIP library.

Sources.  The method is described by three web pages about one preprint,
"FuTransformer: FP8 prefill and INT4 decode for Llama-style inference on
Hopper" (Wei Wang, 16 Oct 2026):

* [P1]  onedev.kr structured summary, title "FuTransformer는 Hopper에서 프리필과
        디코드를 분리해 최적화한다", sections "what it is", "how it works",
        "how it differs", "how to use", "premises and limits";
* [P2]  atlas360.news article "FuTransformer cuts Llama decode step to 2.8 ms
        on H100";
* [P3]  BAAI hub page with the preprint's abstract (Chinese and English).

Citations below name the page and the section, e.g. [P1 how-it-differs].

What the method computes.  It is an *encoding* (INT4 group-quantized weights;
an INT4 copy of the KV cache written through a block-diagonal Hadamard
rotation) followed by ordinary arithmetic on the encoded values [P1
how-it-differs; P3 abstract].  The oracle therefore has two parts:

1. the encodings, step by step, in the precision they are defined in
   (fp32 arithmetic, fp16 scales), so that codes and scales can be compared
   bit for bit;
2. the plain fp64 definition of the block on the dequantized values, the
   "simulated reference on the same quantization grid" the pages validate
   their kernels against [P1 premises-and-limits; P3 abstract].

Readings of points the pages leave open (each is restated where it is used):

R1  weight quantizer: symmetric round-to-nearest [P1 premises-and-limits]
    over groups of 128 consecutive input channels (the group axis is the
    reduction axis because group scales are applied after accumulation
    [P1 how-it-differs]); scale s = fp16(absmax / 7) so codes lie in
    [-7, 7]; ties round half to even; an all-zero group (or a scale that
    rounds to zero in fp16) gives s = 0 and zero codes; an fp16 overflow of
    the scale saturates at 65504.
R2  the nibble stores u = q + 8 (offset binary): the pages decode a nibble by
    placing it in the mantissa of bf16 128.0 and subtracting 136
    [P1 how-it-differs], i.e. value = 128 + u - 136 = u - 8.
R3  RMSNorm gain folded before quantization, W' = gamma * W as one fp32
    product [P1 how-it-works]; rho = 1/sqrt(mean(x^2) + eps), eps = 1e-5,
    applied to the projection output [P1 how-it-works].
R4  RoPE (the pages only say "Llama-style"): rotate-half pairs (i, i+hd/2),
    theta = 500000, position = L - 1 for the appended token; cached entries
    count as already positioned.
R5  Hadamard: unnormalised Sylvester matrix H_b with b = head_dim (one block
    per head), applied by the fast transform in the stage order
    h = 1, 2, 4, ...; the cache stores H k and H v, the queries are rotated
    the same way, the factor 1/b goes into the score scale and into the
    inverse rotation of the attention output, so that (Hq).(Hk)/b = q.k
    [P1 how-it-differs; P3 abstract].
R6  KV quantizer: per (token, kv head) scale over the head_dim rotated
    channels, same rule as R1, applied to the bf16-rounded key/value after
    RoPE; the rotation runs in fp32.
R7  GQA: query head h reads kv head floor(h / G), G = n_q / n_kv, directly
    from the 8-head cache [P1 premises-and-limits].
R8  softmax scale 1/sqrt(head_dim), no mask beyond the context length; the
    context L counts the appended token.
R9  SwiGLU: a = silu(gate) * up with silu(z) = z / (1 + exp(-z)).
R10 the block's new k and v are rounded to bf16 before they are encoded
    into the cache (the cache is written from bf16 keys/values).
R11 final norm and LM head: gamma_f folded into the bf16 LM head weight
    (fp32 product, then bf16 rounding), rho_f applied to the logits, argmax
    with ties to the lowest index.
R12 E4M3 decode-weight variant: the pages report E4M3 decode weights beside
    the INT4 ones [P1 premises-and-limits: +0.02 perplexity; the INT4 decode
    path is 31-51% faster than the FP8 path; P3 abstract] and say nothing of
    their scale.  Reading: only the weight format changes (the activations,
    the gain fold, rho and the rotated INT4 KV cache stay as in the INT4
    block); one fp16 scale per (output row, 128 consecutive input channels),
    s = fp16(absmax / 448) with the R1 arithmetic, codes = E4M3 of
    fp32(w / s) rounded to nearest, ties to even, saturating at +-448 (the
    OCP FP8 E4M3 format: 1 sign, 4 exponent bits with bias 7, 3 mantissa
    bits, subnormals m 2^-9, no infinities, largest finite 448); s == 0
    gives zero codes.  The sign of a value that rounds to zero is kept
    (code 0x80 for negative inputs).
R13 FP8 prefill of the QKV projection, the step that fills the cache the
    decode step reads [P1 how-it-works: FP8 GEMM whose QKV epilogue writes K
    and V straight to offset(request, head, position, channel); gain folded,
    rho in the epilogue; packed prefill by prefix sums, no padding rows;
    delayed per-tensor scaling: the FP8 output is written in the producing
    epilogue and the current maximum gives the next call's scale; P3
    abstract].  Reading: R requests, request r owns tokens [cu[r], cu[r+1])
    at positions start[r], start[r] + 1, ...; the activations are E4M3 of
    fp32(x / s_x) with one per-tensor scale s_x (R12 encoding); the weights
    are E4M3 codes of the gain-folded QKV weight with one power-of-two scale
    per (row, 128-group) (the pages give no scale form for the prefill
    weights; a power of two is the E8M0 scale gfx950's FP8 MFMA applies in
    the instruction, OCP MX style): e = the smallest integer with absmax <=
    448 2^e, codes = E4M3(fp32(w 2^-e)); y = rho_t (sum_k W_hat[n, k] x_hat[t, k])
    in fp64 with x_hat = s_x E4M3(x8); RoPE (R4) at the token's position;
    q is written as E4M3 of fp32(q / s_q) with its own per-tensor scale; k
    and v are rounded to bf16 (R10) and encoded (R6) at their slot.  The
    call reports max |x| and max |q|; the next call's scale is max / 448
    (fp32), a zero maximum keeping the previous scale.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

GROUP = 128
FP16_MAX = np.float16(65504.0)

# ---------------------------------------------------------------------------
# rounding helpers
# ---------------------------------------------------------------------------


def fp16_round(x) -> np.ndarray:
    """fp32 -> fp16, round to nearest even, saturating at +-65504 (R1)."""
    with np.errstate(over="ignore"):
        s = np.asarray(x, dtype=np.float32).astype(np.float16)
    return np.where(np.isinf(s), np.copysign(FP16_MAX, s), s).astype(np.float16)


def round_to_bf16(x) -> np.ndarray:
    """Round to the nearest bf16 value (8 significant bits), ties to even.

    Exact for inputs in the normal bf16 range: frexp gives x = m 2^e with
    0.5 <= |m| < 1, so m*256 is an integer-valued 8-bit significand after
    rint (which rounds half to even).  Returned as float64.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


# ---------------------------------------------------------------------------
# INT4 group quantizer (R1, R2)
# ---------------------------------------------------------------------------


def quantize_rtn_lastaxis(v) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric INT4 round-to-nearest over the last axis (one scale per vector).

    s = fp16(absmax / 7), the division in fp32 (correctly rounded);
    q = clamp(rint(v / fp32(s)), -8, 7), the division in fp32; s == 0 -> q = 0.
    [P1 premises-and-limits: round-to-nearest; R1]
    """
    v = np.asarray(v, dtype=np.float32)
    a = np.max(np.abs(v), axis=-1)
    s = fp16_round(a / np.float32(7.0))
    sf = s.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = v / sf
    q = np.clip(np.rint(r), -8, 7)
    q = np.where(sf == 0, 0.0, q)
    return q.astype(np.int8), s


def fold_gain(W, gamma) -> np.ndarray:
    """W' = gamma (.) W, one fp32 product per weight [P1 how-it-works; R3]."""
    W = np.asarray(W, dtype=np.float32)
    if gamma is None:
        return W
    return W * np.asarray(gamma, dtype=np.float32)[None, :]


def quantize_weight(W, gamma=None) -> tuple[np.ndarray, np.ndarray]:
    """Group-128 INT4 RTN of a [N, K] weight (groups along K), gain folded first.

    Returns codes q [N, K] int8 in [-8, 7] and scales s [N, K/128] fp16.
    [P1 how-it-differs: group scales applied after accumulation -> groups run
    along the reduction axis; P1 how-it-works: W' = gamma W before quantization]
    """
    Wp = fold_gain(W, gamma)
    N, K = Wp.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    q, s = quantize_rtn_lastaxis(Wp.reshape(N, K // GROUP, GROUP))
    return q.reshape(N, K), s


def dequantize_weight(q, s) -> np.ndarray:
    """W_hat[n, k] = fp64(s[n, k // 128]) * q[n, k]."""
    q = np.asarray(q)
    N, K = q.shape
    sf = np.asarray(s, dtype=np.float16).astype(np.float64)
    return (q.reshape(N, K // GROUP, GROUP).astype(np.float64) * sf[:, :, None]).reshape(N, K)


def nibble_of_code(q) -> np.ndarray:
    """Stored nibble u = q + 8 (offset binary) [P1 how-it-differs; R2]."""
    return (np.asarray(q, dtype=np.int16) + 8).astype(np.uint8)


def code_of_nibble_via_bf16_128(u) -> np.ndarray:
    """Decode a nibble the way the pages describe: bf16 bits 0x4300|u is
    128 + u; subtracting 136 leaves u - 8 [P1 how-it-differs]."""
    u = np.asarray(u, dtype=np.uint32)
    bits = (np.uint32(0x4300) | u) << np.uint32(16)
    return bits.view(np.float32).astype(np.float64) - 136.0


# ---------------------------------------------------------------------------
# E4M3 weight encoding (R12)
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of E4M3 codes (uint8) as fp64: (-1)^s 2^(e-7) (1 + m/8) for
    exponent field e > 0, (-1)^s m 2^-9 for e == 0; the two NaN codes
    (0x7F, 0xFF) decode to NaN.  [OCP FP8 E4M3]"""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """fp32 values -> E4M3 codes: nearest representable value, ties to the
    even mantissa, magnitudes of 448 and above saturate to 448 (code 0x7E).
    Below 2^-6 the spacing is 2^-9 (subnormals); in [2^E, 2^(E+1)) it is
    2^(E-3).  The input sign is kept, also on zero.  [R12]"""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    sign = np.where(np.signbit(x), 0x80, 0x00).astype(np.int64)
    a = np.abs(x)
    # the exponent E of a normal magnitude, and its spacing
    E = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    E = np.clip(E, -6, 8)
    step = np.exp2((E - 3).astype(np.float64))
    q = np.rint(a / step)                                   # mantissa steps, ties to even
    # rounding up to the next power of two moves to the next exponent
    bump = q >= 16
    E = np.where(bump, E + 1, E)
    q = np.where(bump, 8.0, q)
    normal = np.where(E + 7 > 15, 0x7E, ((E + 7) << 3) | (q.astype(np.int64) - 8))
    # subnormal range: multiples of 2^-9 (rounding up to 2^-6 gives code 0x08)
    sub = np.rint(np.minimum(a, 1.0) * 512.0).astype(np.int64)
    mag = np.where(a < 2.0 ** -6, sub, normal)
    mag = np.where(a >= E4M3_MAX, 0x7E, np.minimum(mag, 0x7E))
    return (sign | mag).astype(np.uint8)


def quantize_weight_e4m3(W, gamma=None) -> tuple[np.ndarray, np.ndarray, str]:
    """Group-128 E4M3 codes of a [N, K] weight (gain folded first, R3):
    per (row, group) s = fp16(absmax / 448) (fp32 division), codes =
    E4M3(fp32(w / fp32(s))); s == 0 -> codes 0.  Returns (codes uint8
    [N, K], scales fp16 [N, K/128], "e4m3").  [R12]"""
    Wp = fold_gain(W, gamma)
    N, K = Wp.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    g = Wp.reshape(N, K // GROUP, GROUP)
    a = np.max(np.abs(g), axis=-1)
    s = fp16_round(a / np.float32(E4M3_MAX))
    sf = s.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = g / sf
    codes = e4m3_encode(np.where(sf == 0, np.float32(0.0), r))
    return codes.reshape(N, K), s, "e4m3"


def mx_exponent(absmax) -> np.ndarray:
    """The smallest integer e with absmax <= 448 * 2^e (exact: with
    absmax = m 2^x, 0.5 <= m < 1, and 448 = 0.875 2^9, e = x - 9 when
    m <= 0.875, else x - 8), clamped to the E8M0 range [-127, 127]; an
    all-zero group takes -127.  [R13]"""
    a = np.asarray(absmax, dtype=np.float64)
    m, x = np.frexp(a)
    e = np.where(m <= 0.875, x - 9, x - 8)
    e = np.where(a == 0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize_weight_e4m3_mx(W, gamma=None) -> tuple[np.ndarray, np.ndarray, str]:
    """Group-128 E4M3 codes with one power-of-two scale per (row, group), the
    scale form gfx950's FP8 MFMA applies by itself (an E8M0 byte, exponent
    + 127, as in the OCP MX formats): gain folded first (R3); e =
    mx_exponent(absmax); codes = E4M3(fp32(w * 2^-e)) (the scaling is exact,
    and no code saturates since |w| 2^-e <= 448).  Returns (codes uint8
    [N, K], E8M0 bytes uint8 [N, K/128], "e4m3mx").  [R13]"""
    Wp = fold_gain(W, gamma)
    N, K = Wp.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    g = Wp.reshape(N, K // GROUP, GROUP)
    e = mx_exponent(np.max(np.abs(g), axis=-1))
    r = np.ldexp(g.astype(np.float64), -e[..., None]).astype(np.float32)
    codes = e4m3_encode(r)
    return codes.reshape(N, K), (e + 127).astype(np.uint8), "e4m3mx"


def dequantize_weight_e4m3_mx(codes, e8m0) -> np.ndarray:
    """W_hat[n, k] = 2^(e8m0[n, k // 128] - 127) * E4M3 value of code[n, k]."""
    c = np.asarray(codes)
    N, K = c.shape
    e = np.asarray(e8m0, dtype=np.int64) - 127
    return np.ldexp(e4m3_decode(c).reshape(N, K // GROUP, GROUP), e[:, :, None]).reshape(N, K)


def dequantize_weight_e4m3(codes, s) -> np.ndarray:
    """W_hat[n, k] = fp64(s[n, k // 128]) * E4M3 value of code[n, k]."""
    c = np.asarray(codes)
    N, K = c.shape
    sf = np.asarray(s, dtype=np.float16).astype(np.float64)
    return (e4m3_decode(c).reshape(N, K // GROUP, GROUP) * sf[:, :, None]).reshape(N, K)


# ---------------------------------------------------------------------------
# Hadamard rotation (R5) and the KV-cache encoding (R6)
# ---------------------------------------------------------------------------


def fwht(x, dtype=np.float64) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform over the last axis.

    Stages h = 1, 2, 4, ..., b/2; in stage h every index j with (j & h) == 0
    is paired with j + h and (x_j, x_{j+h}) <- (x_j + x_{j+h}, x_j - x_{j+h}).
    The result equals H_b x for the Sylvester matrix H_b (H_1 = [1],
    H_2n = [[H_n, H_n], [H_n, -H_n]]).  Every add is done in ``dtype``.
    """
    y = np.array(x, dtype=dtype, copy=True)
    b = y.shape[-1]
    if b & (b - 1):
        raise ValueError("block size must be a power of two")
    lead = y.shape[:-1]
    h = 1
    while h < b:
        y = y.reshape(lead + (b // (2 * h), 2, h))
        lo = y[..., 0, :].copy()
        hi = y[..., 1, :].copy()
        y[..., 0, :] = lo + hi
        y[..., 1, :] = lo - hi
        y = y.reshape(lead + (b,))
        h *= 2
    return y


def sylvester(b: int) -> np.ndarray:
    """Dense unnormalised Sylvester-Hadamard matrix H_b (fp64)."""
    H = np.ones((1, 1))
    while H.shape[0] < b:
        H = np.block([[H, H], [H, -H]])
    return H


def quantize_kv(x_bf16_values) -> tuple[np.ndarray, np.ndarray]:
    """Encode keys or values for the INT4 cache copy.

    x: bf16 values (given as float32/float64 holding bf16-representable
    numbers), shape [..., hd].  Steps: fp32 copy -> FWHT in fp32 -> one
    per-vector INT4 RTN scale (R1 rule).  Returns codes [..., hd] int8 and
    scales [...] fp16.  The cache holds H x (unnormalised).
    [P1 how-it-differs: rotation applied before cache quantization; R6]
    """
    y = fwht(np.asarray(x_bf16_values, dtype=np.float32), dtype=np.float32)
    return quantize_rtn_lastaxis(y)


def dequantize_kv(q, s) -> np.ndarray:
    return np.asarray(q, dtype=np.float64) * np.asarray(s, dtype=np.float16).astype(np.float64)[..., None]


# ---------------------------------------------------------------------------
# block pieces
# ---------------------------------------------------------------------------


def rms_factor(x, eps: float) -> np.ndarray:
    """rho = 1 / sqrt(mean(x^2) + eps) per row [P1 how-it-works; R3]."""
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)


def rope(v, pos, theta: float) -> np.ndarray:
    """Rotate-half RoPE on the last axis (hd) at integer positions ``pos``.

    v: [..., hd] with pos broadcastable to v.shape[:-1]; pair (i, i + hd/2)
    rotates by angle pos * theta^(-2i/hd).  (R4)
    """
    v = np.asarray(v, dtype=np.float64)
    hd = v.shape[-1]
    half = hd // 2
    inv_freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / hd)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    a, b = v[..., :half], v[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(z) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def attention_one_row(q_rot, k_codes, k_scales, v_codes, v_scales, L: int, b: int) -> np.ndarray:
    """Decode attention for one row over its first L cached tokens.

    q_rot: H q per query head, [n_q, hd] fp64.  Cache: codes [L_cap, n_kv, hd],
    scales [L_cap, n_kv].  Query head h reads kv head h // G (R7).
    score_t = q_rot . k_hat_t / (b sqrt(hd)); p = softmax over t < L (R8);
    o_h = H (sum_t p_t v_hat_t) / b (R5).  Unsplit: the plain definition.
    """
    n_q, hd = q_rot.shape
    n_kv = k_codes.shape[1]
    G = n_q // n_kv
    out = np.empty((n_q, hd))
    for j in range(n_kv):
        # the G query heads of kv head j read the same dequantized entries
        k_hat = dequantize_kv(k_codes[:L, j, :], k_scales[:L, j])     # [L, hd]
        v_hat = dequantize_kv(v_codes[:L, j, :], v_scales[:L, j])
        for h in range(j * G, (j + 1) * G):
            sc = (k_hat @ q_rot[h]) / (b * np.sqrt(hd))
            p = np.exp(sc - sc.max())
            p /= p.sum()
            out[h] = fwht(p @ v_hat) / b
    return out


# ---------------------------------------------------------------------------
# layer containers
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class QuantLayer:
    """Encoded projections of one layer (codes int8 in [-8, 7], fp16 scales)."""
    qkv: tuple
    o: tuple
    gate: tuple
    up: tuple
    down: tuple


def quantize_layer(lw) -> QuantLayer:
    """gamma_attn folds into QKV, gamma_ffn into gate and up; O and down take
    un-normalised inputs and carry no gain [P1 how-it-works; R3]."""
    return QuantLayer(
        qkv=quantize_weight(lw.w_qkv, lw.gamma_attn),
        o=quantize_weight(lw.w_o, None),
        gate=quantize_weight(lw.w_gate, lw.gamma_ffn),
        up=quantize_weight(lw.w_up, lw.gamma_ffn),
        down=quantize_weight(lw.w_down, None),
    )


def quantize_layer_e4m3(lw) -> QuantLayer:
    """The same layer with E4M3 decode weights (R12); gains fold as for INT4."""
    return QuantLayer(
        qkv=quantize_weight_e4m3(lw.w_qkv, lw.gamma_attn),
        o=quantize_weight_e4m3(lw.w_o, None),
        gate=quantize_weight_e4m3(lw.w_gate, lw.gamma_ffn),
        up=quantize_weight_e4m3(lw.w_up, lw.gamma_ffn),
        down=quantize_weight_e4m3(lw.w_down, None),
    )


@dataclasses.dataclass
class RowCache:
    """Oracle-side INT4 cache of one row: logical codes per token."""
    k_codes: np.ndarray   # [cap, n_kv, hd] int8
    k_scales: np.ndarray  # [cap, n_kv] fp16
    v_codes: np.ndarray
    v_scales: np.ndarray


def build_cache(shape, lengths: Sequence[int], prefill) -> List[RowCache]:
    """Encode the bf16 prefill of every row (positions 0..L_r-2) with R6 and
    leave room for the token appended at L_r - 1."""
    rows = []
    hd, nkv = shape.head_dim, shape.n_kv_heads
    for r, L in enumerate(lengths):
        L = int(L)
        kc = np.zeros((L, nkv, hd), np.int8)
        vc = np.zeros((L, nkv, hd), np.int8)
        ks = np.zeros((L, nkv), np.float16)
        vs = np.zeros((L, nkv), np.float16)
        if L > 1:
            kq, kss = quantize_kv(_bf16_bits_to_values(prefill.k[r]))
            vq, vss = quantize_kv(_bf16_bits_to_values(prefill.v[r]))
            kc[: L - 1], ks[: L - 1] = kq, kss
            vc[: L - 1], vs[: L - 1] = vq, vss
        rows.append(RowCache(kc, ks, vc, vs))
    return rows


def _bf16_bits_to_values(bits) -> np.ndarray:
    """Interpret uint16 bf16 bit patterns as float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def dense(ql_part) -> np.ndarray:
    """fp64 weights of an encoded projection: INT4 (codes, scales) or E4M3
    (codes, scales, "e4m3")."""
    if len(ql_part) == 3 and ql_part[2] == "e4m3":
        return dequantize_weight_e4m3(ql_part[0], ql_part[1])
    if len(ql_part) == 3 and ql_part[2] == "e4m3mx":
        return dequantize_weight_e4m3_mx(ql_part[0], ql_part[1])
    return dequantize_weight(*ql_part)


# ---------------------------------------------------------------------------
# the block step
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class BlockResult:
    out: np.ndarray          # [M, d] block output (fp64)
    attn: np.ndarray         # [M, n_q * hd] attention output (un-rotated, fp64)
    h: np.ndarray            # [M, d] residual stream after attention
    q: np.ndarray            # [M, n_q, hd] queries after rho and RoPE, before rotation
    k_new: np.ndarray        # [M, n_kv, hd] bf16-rounded new keys (after RoPE)
    v_new: np.ndarray        # [M, n_kv, hd] bf16-rounded new values
    k_codes_new: np.ndarray  # [M, n_kv, hd] codes appended for the new token
    k_scales_new: np.ndarray
    v_codes_new: np.ndarray
    v_scales_new: np.ndarray


def qkv_stage(shape, W_qkv_hat, x, lengths):
    """rho1 -> x . W'qkv^T (gain folded) -> RoPE on q and k at position L-1.

    x fp64 [M, d]; returns q [M, n_q, hd], k and v [M, n_kv, hd] (fp64, k/v not
    yet rounded to bf16).  [P1 how-it-works; R3, R4]
    """
    d, hd = shape.d_model, shape.head_dim
    nq, nkv = shape.n_q_heads, shape.n_kv_heads
    M = x.shape[0]
    rho1 = rms_factor(x, shape.rms_eps)
    qkv = rho1[:, None] * (x @ W_qkv_hat.T)
    q = qkv[:, : nq * hd].reshape(M, nq, hd)
    k = qkv[:, nq * hd: (nq + nkv) * hd].reshape(M, nkv, hd)
    v = qkv[:, (nq + nkv) * hd:].reshape(M, nkv, hd)
    pos = np.asarray(lengths, dtype=np.float64) - 1.0
    return rope(q, pos[:, None], shape.rope_theta), rope(k, pos[:, None], shape.rope_theta), v


def attention_stage(shape, cache: List[RowCache], q, lengths):
    """Rotated query against each row's INT4 cache, unsplit softmax, inverse
    rotation; returns the attention output [M, n_q * hd].  [P1 how-it-differs; R5, R7, R8]"""
    M = q.shape[0]
    q_rot = fwht(q)
    out = np.empty((M,) + q.shape[1:])
    for r in range(M):
        c = cache[r]
        out[r] = attention_one_row(q_rot[r], c.k_codes, c.k_scales, c.v_codes, c.v_scales,
                                   int(lengths[r]), shape.head_dim)
    return out.reshape(M, -1)


def o_stage(W_o_hat, x, attn):
    """h = x + attn . Wo^T (no gain: the input is not normalised)."""
    return x + attn @ W_o_hat.T


def gate_up_stage(shape, W_gate_hat, W_up_hat, h):
    """rho2 -> gate, up (gain folded) -> a = silu(gate) * up.  [P1 how-it-works; R3, R9]"""
    rho2 = rms_factor(h, shape.rms_eps)
    g = rho2[:, None] * (h @ W_gate_hat.T)
    u = rho2[:, None] * (h @ W_up_hat.T)
    return silu(g) * u


def down_stage(W_down_hat, h, a):
    """out = h + a . Wdown^T."""
    return h + a @ W_down_hat.T


def append_stage(cache: List[RowCache], k, v, lengths):
    """Round the new k, v to bf16 (R10), encode them (R6) and store them at
    position L-1 of each row.  Returns the bf16 values and the codes."""
    k_b = round_to_bf16(k)
    v_b = round_to_bf16(v)
    kq, ks = quantize_kv(k_b)
    vq, vs = quantize_kv(v_b)
    for r in range(len(lengths)):
        p = int(lengths[r]) - 1
        cache[r].k_codes[p], cache[r].k_scales[p] = kq[r], ks[r]
        cache[r].v_codes[p], cache[r].v_scales[p] = vq[r], vs[r]
    return k_b, v_b, kq, ks, vq, vs


def decode_block(shape, ql: QuantLayer, cache: List[RowCache], x_bits, lengths,
                 dense_cache: Optional[dict] = None) -> BlockResult:
    """One decode step of the block for M rows (row r attends L_r tokens).

    Data flow [P1 how-it-differs; P1 how-it-works; P1 premises-and-limits]:
      rho1 -> QKV (gain folded, rho1 on the output) -> RoPE(q, k) ->
      bf16(k, v) -> INT4 append at L-1 (through the rotation) ->
      attention with rotated q over the INT4 cache (GQA, unsplit) ->
      inverse rotation -> O + residual -> rho2 -> gate/up -> SwiGLU ->
      down + residual.
    ``cache`` is updated in place with the appended token.
    ``dense_cache`` (optional dict) memoises the dequantized fp64 weights.
    """
    lengths = [int(L) for L in lengths]
    M = len(lengths)

    def W(name):
        if dense_cache is not None:
            if name not in dense_cache:
                dense_cache[name] = dense(getattr(ql, name))
            return dense_cache[name]
        return dense(getattr(ql, name))

    x = _bf16_bits_to_values(np.asarray(x_bits).reshape(M, shape.d_model)).astype(np.float64)
    q, k, v = qkv_stage(shape, W("qkv"), x, lengths)
    k_b, v_b, kq, ks, vq, vs = append_stage(cache, k, v, lengths)
    attn = attention_stage(shape, cache, q, lengths)
    h = o_stage(W("o"), x, attn)
    a = gate_up_stage(shape, W("gate"), W("up"), h)
    out = down_stage(W("down"), h, a)
    return BlockResult(out, attn, h, q, k_b, v_b, kq, ks, vq, vs)


# ---------------------------------------------------------------------------
# LM head (R11)
# ---------------------------------------------------------------------------


def lm_head_weight_bf16(W_lm, gamma_f) -> np.ndarray:
    """bf16(fp32(gamma_f (.) W_lm)) as fp64 values [vocab, d]."""
    return round_to_bf16(fold_gain(W_lm, gamma_f))


def lm_head_argmax(h, W_hat_lm, eps: float) -> tuple[np.ndarray, np.ndarray]:
    """logits = rho_f * (h . W_hat_lm^T); token = argmax, lowest index on ties."""
    h = np.asarray(h, dtype=np.float64)
    rho = rms_factor(h, eps)
    logits = rho[:, None] * (h @ np.asarray(W_hat_lm, dtype=np.float64).T)
    return logits, np.argmax(logits, axis=-1)


# ---------------------------------------------------------------------------
# FP8 prefill of the QKV projection (R13)
# ---------------------------------------------------------------------------


def prefill_token_map(cu_seqlens, start_pos):
    """Request and position of every packed token: request r owns tokens
    cu[r] .. cu[r+1]-1 at positions start[r], start[r] + 1, ... (R13)."""
    rows, pos = [], []
    for r in range(len(cu_seqlens) - 1):
        n = int(cu_seqlens[r + 1]) - int(cu_seqlens[r])
        rows += [r] * n
        pos += list(range(int(start_pos[r]), int(start_pos[r]) + n))
    return np.array(rows, dtype=np.int64), np.array(pos, dtype=np.int64)


def delayed_scale(amax, prev) -> np.float32:
    """The next call's per-tensor E4M3 scale: fp32(max) / 448, or the previous
    scale when the maximum is zero (R13)."""
    a = np.float32(amax)
    return np.float32(a / np.float32(E4M3_MAX)) if a > 0 else np.float32(prev)


@dataclasses.dataclass
class PrefillResult:
    x8: np.ndarray        # [T, d] E4M3 codes of the activations
    rho: np.ndarray       # [T] RMS factor of each token
    q: np.ndarray         # [T, n_q, hd] fp64 queries after RoPE
    q8: np.ndarray        # [T, n_q, hd] E4M3 codes of q / s_q
    k_new: np.ndarray     # [T, n_kv, hd] bf16-rounded keys after RoPE
    v_new: np.ndarray
    k_codes: np.ndarray   # [T, n_kv, hd] cache codes (R6) and scales
    k_scales: np.ndarray
    v_codes: np.ndarray
    v_scales: np.ndarray
    rows: np.ndarray      # [T] request of each token
    pos: np.ndarray       # [T] position of each token
    amax_x: float
    amax_q: float


def fp8_quantize(v, scale) -> np.ndarray:
    """E4M3 codes of fp32(v) / fp32(scale) (fp32 division, R12 encoding):
    the FP8 activation or query of the prefill (R13)."""
    return e4m3_encode(np.asarray(v, np.float32) / np.float32(scale))


def fp8_dequantize(codes, scale) -> np.ndarray:
    """fp64 values scale * E4M3(codes) (R13)."""
    return e4m3_decode(codes) * np.float64(np.float32(scale))


def prefill_qkv(shape, qkv_e4m3, x_bits, cu_seqlens, start_pos, x_scale, q_scale,
                W_dense: Optional[np.ndarray] = None) -> PrefillResult:
    """The FP8 prefill of the QKV projection for packed tokens (R13).

    x_bits: bf16 bits [T, d] of the packed tokens; qkv_e4m3: (codes, E8M0
    bytes, "e4m3mx") of the gain-folded QKV weight from
    quantize_weight_e4m3_mx (any encoded form dense() takes), or its fp64
    dense form in W_dense.  Steps: token map; rho of each token from its bf16 values; x8 =
    E4M3(x / s_x); y = rho (s_x dec(x8)) W_hat^T; RoPE of q and k at the
    token's position; q8 = E4M3(q / s_q); k and v rounded to bf16 and encoded
    for the INT4 cache."""
    T = int(cu_seqlens[-1])
    hd, nq, nkv = shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    x = _bf16_bits_to_values(np.asarray(x_bits).reshape(T, shape.d_model))
    rows, pos = prefill_token_map(cu_seqlens, start_pos)
    rho = rms_factor(x.astype(np.float64), shape.rms_eps)
    x8 = fp8_quantize(x, x_scale)
    x_hat = fp8_dequantize(x8, x_scale)
    W = dense(qkv_e4m3) if W_dense is None else W_dense
    y = rho[:, None] * (x_hat @ W.T)
    q = y[:, : nq * hd].reshape(T, nq, hd)
    k = y[:, nq * hd: (nq + nkv) * hd].reshape(T, nkv, hd)
    v = y[:, (nq + nkv) * hd:].reshape(T, nkv, hd)
    q = rope(q, pos[:, None], shape.rope_theta)
    k = rope(k, pos[:, None], shape.rope_theta)
    q8 = fp8_quantize(q, q_scale)
    k_b, v_b = round_to_bf16(k), round_to_bf16(v)
    kq, ks = quantize_kv(k_b)
    vq, vs = quantize_kv(v_b)
    amax_x = float(np.max(np.abs(x))) if T else 0.0
    amax_q = float(np.max(np.abs(q.astype(np.float32)))) if T else 0.0
    return PrefillResult(x8, rho, q, q8, k_b, v_b, kq, ks, vq, vs, rows, pos, amax_x, amax_q)
