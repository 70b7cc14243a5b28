"""ctypes binding of libi4d.so: one Python function per C entry point, same names.

Argument marshalling only.  Pointers may be given as torch tensors (their
``data_ptr()``), numpy arrays (host memory), plain integers or None (NULL).
Streams default to torch's current stream.  Every non-zero status raises
:class:`I4DError` with the library's message.  All computation happens in
the library; if it is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libi4d.so")

c_size_p = ctypes.POINTER(ctypes.c_size_t)

I4D_PROJ_PLAIN, I4D_PROJ_QKV, I4D_PROJ_GATE_UP = 0, 1, 2
I4D_MAX_ROWS = 32
I4D_MAX_SPLITS = 256
I4D_DEVERR_APPEND_POS = 1
I4D_DEVERR_CTX_LEN = 2
I4D_DEVERR_SYNC = 4
I4D_DEVERR_SCALE = 8
I4D_NOALLOC_SCRATCH_BYTES = 16 << 20
I4D_STEP_STAMPS = 10

STATUS_NAMES = {0: "I4D_OK", -1: "I4D_ERR_NULL", -2: "I4D_ERR_SHAPE", -3: "I4D_ERR_UNSUPPORTED",
                -4: "I4D_ERR_ALIGN", -5: "I4D_ERR_WORKSPACE", -6: "I4D_ERR_RANGE", -7: "I4D_ERR_HIP"}


class I4DError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class i4d_layer_shape(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int), ("n_q_heads", ctypes.c_int), ("n_kv_heads", ctypes.c_int),
                ("head_dim", ctypes.c_int), ("d_ffn", ctypes.c_int), ("group", ctypes.c_int),
                ("hadamard_block", ctypes.c_int), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float)]


class i4d_kv_cache(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
                ("row_base", ctypes.c_void_p), ("n_rows", ctypes.c_int),
                ("n_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int),
                ("total_capacity", ctypes.c_int64), ("err_word", ctypes.c_void_p)]


class i4d_layer(ctypes.Structure):
    _fields_ = [("shape", i4d_layer_shape),
                ("qkv_codes", ctypes.c_void_p), ("qkv_scales", ctypes.c_void_p),
                ("o_codes", ctypes.c_void_p), ("o_scales", ctypes.c_void_p),
                ("gu_codes", ctypes.c_void_p), ("gu_scales", ctypes.c_void_p),
                ("down_codes", ctypes.c_void_p), ("down_scales", ctypes.c_void_p)]


class i4d_projection_plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("kernel", "waves", "strips_per_workgroup", "k_slices", "depth",
                                            "persistent", "grid")] + \
               [("lds_bytes", ctypes.c_size_t), ("instantiated", ctypes.c_int)]


class i4d_prefill_weights(ctypes.Structure):
    _fields_ = [("shape", i4d_layer_shape), ("qkv_codes", ctypes.c_void_p), ("qkv_scales", ctypes.c_void_p)]


class i4d_fp8_scales(ctypes.Structure):
    _fields_ = [(n, ctypes.c_float) for n in ("x_scale", "q_scale", "x_amax", "q_amax")]


class i4d_workspace_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("q", "k", "v", "attn", "h", "h_bf16", "a", "attn_ws", "split_cnt", "split_part", "sync",
                                               "total")]


_VP = ctypes.c_void_p
_I = ctypes.c_int
_SIGS = {
    "i4d_last_error": (ctypes.c_char_p, []),
    "i4d_version": (ctypes.c_char_p, []),
    "i4d_packed_sizes": (_I, [_I, _I, _I, _I, c_size_p, c_size_p]),
    "i4d_pack_weights": (_I, [_I, _VP, _VP, _VP, _I, _I, _I, _VP, _VP, _I]),
    "i4d_unpack_weights": (_I, [_I, _VP, _VP, _I, _I, _I, _VP, _VP]),
    "i4d_pack_codes": (_I, [_I, _VP, _VP, _I, _I, _I, _VP, _VP, _I]),
    "i4d_pack_lm_head": (_I, [_VP, _VP, _I, _I, _VP, _I]),
    "i4d_packed_sizes_e4m3": (_I, [_I, _I, _I, _I, c_size_p, c_size_p]),
    "i4d_pack_weights_e4m3": (_I, [_I, _VP, _VP, _VP, _I, _I, _I, _VP, _VP, _I]),
    "i4d_unpack_weights_e4m3": (_I, [_I, _VP, _VP, _I, _I, _I, _VP, _VP]),
    "i4d_packed_sizes_mx": (_I, [_I, _I, _I, _I, c_size_p, c_size_p]),
    "i4d_pack_weights_mx": (_I, [_I, _VP, _VP, _VP, _I, _I, _I, _VP, _VP, _I]),
    "i4d_unpack_weights_mx": (_I, [_I, _VP, _VP, _I, _I, _I, _VP, _VP]),
    "i4d_kv_cache_bytes": (_I, [_I, _I, ctypes.c_int64, c_size_p, c_size_p, c_size_p, c_size_p]),
    "i4d_kv_append": (_I, [ctypes.POINTER(i4d_kv_cache), _VP, _VP, _VP, _VP, _I, _VP]),
    "i4d_kv_unpack_host": (_I, [ctypes.POINTER(i4d_kv_cache), _VP, _I, _I, _I, _VP, _VP, _VP, _VP]),
    "i4d_attn_qkv": (_I, [ctypes.POINTER(i4d_layer), _VP, _VP, _I, _VP, _VP, _VP, _VP]),
    "i4d_attention_workspace_bytes": (_I, [ctypes.POINTER(i4d_layer_shape), _I, _I, _I, c_size_p]),
    "i4d_attention": (_I, [ctypes.POINTER(i4d_kv_cache), ctypes.POINTER(i4d_layer_shape), _VP, _VP, _I,
                           _I, _I, _VP, ctypes.c_size_t, _VP, _VP, _VP]),
    "i4d_attn_out_proj": (_I, [ctypes.POINTER(i4d_layer), _VP, _VP, _I, _VP, _VP, _VP]),
    "i4d_ffn_gate_up": (_I, [ctypes.POINTER(i4d_layer), _VP, _I, _VP, _VP]),
    "i4d_ffn_down": (_I, [ctypes.POINTER(i4d_layer), _VP, _VP, _I, _VP, _VP]),
    "i4d_workspace_bytes": (_I, [ctypes.POINTER(i4d_layer_shape), _I, _I, _I, c_size_p]),
    "i4d_workspace_layout_of": (_I, [ctypes.POINTER(i4d_layer_shape), _I, _I, _I,
                                     ctypes.POINTER(i4d_workspace_layout)]),
    "i4d_workspace_init": (_I, [_VP, ctypes.c_size_t, _VP]),
    "i4d_projection_plan_of": (_I, [ctypes.POINTER(i4d_layer_shape), _I, _I, ctypes.POINTER(i4d_projection_plan)]),
    "i4d_decode_step_is_one_launch": (_I, [ctypes.POINTER(i4d_layer_shape), _I, ctypes.POINTER(_I)]),
    "i4d_decode_block_step": (_I, [ctypes.POINTER(i4d_layer), ctypes.POINTER(i4d_kv_cache), _VP, _VP, _VP,
                                   _I, _I, _I, _VP, ctypes.c_size_t, _VP, _VP]),
    "i4d_decode_block_step_e4m3": (_I, [ctypes.POINTER(i4d_layer), ctypes.POINTER(i4d_kv_cache), _VP, _VP, _VP,
                                        _I, _I, _I, _VP, ctypes.c_size_t, _VP, _VP]),
    "i4d_decode_block_step_timeline": (_I, [ctypes.POINTER(i4d_layer), ctypes.POINTER(i4d_kv_cache), _VP, _VP,
                                            _VP, _I, _I, _I, _VP, ctypes.c_size_t, _VP, _VP, ctypes.c_size_t,
                                            _VP]),
    "i4d_attn_out_proj_e4m3": (_I, [ctypes.POINTER(i4d_layer), _VP, _VP, _I, _VP, _VP, _VP]),
    "i4d_decode_block_step_noalloc": (_I, [ctypes.POINTER(i4d_layer), ctypes.POINTER(i4d_kv_cache), _VP, _VP,
                                           _VP, _I, _I, _I, _VP, _VP]),
    "i4d_prefill_workspace_bytes": (_I, [ctypes.POINTER(i4d_layer_shape), _I, c_size_p]),
    "i4d_prefill_qkv_e4m3": (_I, [ctypes.POINTER(i4d_prefill_weights), ctypes.POINTER(i4d_kv_cache), _VP, _I, _VP, _VP, _I,
                                  _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
    "i4d_prefill_prepare": (_I, [ctypes.POINTER(i4d_prefill_weights), ctypes.POINTER(i4d_kv_cache), _VP, _I, _VP, _VP, _I,
                                 _VP, _VP, ctypes.c_size_t, _VP]),
    "i4d_prefill_project": (_I, [ctypes.POINTER(i4d_prefill_weights), ctypes.POINTER(i4d_kv_cache), _I, _VP, _VP, _I,
                                 _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
    "i4d_fp8_scales_update": (_I, [_VP, _VP]),
    "i4d_lm_head_workspace_bytes": (_I, [_I, _I, c_size_p]),
    "i4d_lm_head_argmax": (_I, [_VP, _I, _I, _VP, _I, ctypes.c_float, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libi4d.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(or python int4_quantized_decode_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_names():
    return list(_SIGS)


def _check(st: int):
    if st != 0:
        raise I4DError(st, lib().i4d_last_error().decode(errors="replace"))


def ptr(x):
    """Address of a torch tensor, numpy array, int, or None (NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    raise TypeError(f"cannot take the address of {type(x)}")


def stream_handle(stream):
    if stream is None:
        import torch
        if not torch.cuda.is_available():
            return 0  # NULL stream; only reached by calls that fail host validation
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_shape(s) -> i4d_layer_shape:
    return i4d_layer_shape(s.d_model, s.n_q_heads, s.n_kv_heads, s.head_dim, s.d_ffn, 128, s.head_dim,
                           float(s.rms_eps), float(s.rope_theta))


# ---------------------------------------------------------------------------
# host calls
# ---------------------------------------------------------------------------

def i4d_version() -> str:
    return lib().i4d_version().decode()


def i4d_last_error() -> str:
    return lib().i4d_last_error().decode()


def i4d_packed_sizes(kind: int, N: int, K: int, head_dim: int = 0):
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().i4d_packed_sizes(kind, N, K, head_dim, ctypes.byref(cb), ctypes.byref(sb)))
    return cb.value, sb.value


def i4d_pack_weights(kind: int, W0, W1=None, gamma=None, head_dim: int = 0, threads: int = 0):
    """fp32 host weights -> (codes uint8, scales uint16) in the device layout."""
    W0 = np.ascontiguousarray(W0, dtype=np.float32)
    N, K = W0.shape
    W1 = None if W1 is None else np.ascontiguousarray(W1, dtype=np.float32)
    gamma = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.float32)
    cb, sb = i4d_packed_sizes(kind, N, K, head_dim)
    codes = np.empty(cb, np.uint8)
    scales = np.empty(sb // 2, np.uint16)
    _check(lib().i4d_pack_weights(kind, ptr(W0), ptr(W1), ptr(gamma), N, K, head_dim,
                                  ptr(codes), ptr(scales), threads))
    return codes, scales


def i4d_pack_codes(kind: int, q, s, N: int, K: int, head_dim: int = 0, threads: int = 0):
    """Pre-quantized codes q [rows][K] int8 in [-8, 7] and fp16 scale bits
    s [rows][K/128] (rows = N, or 2N for gate/up: gate rows then up rows)
    -> (codes uint8, scales uint16) in the device layout."""
    rows = 2 * N if kind == I4D_PROJ_GATE_UP else N
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.uint16)
    if q.shape != (rows, K) or s.shape != (rows, K // 128):
        raise ValueError(f"q {q.shape} / s {s.shape}: expected ({rows}, {K}) / ({rows}, {K // 128})")
    cb, sb = i4d_packed_sizes(kind, N, K, head_dim)
    codes = np.empty(cb, np.uint8)
    scales = np.empty(sb // 2, np.uint16)
    _check(lib().i4d_pack_codes(kind, ptr(q), ptr(s), N, K, head_dim, ptr(codes), ptr(scales), threads))
    return codes, scales


def i4d_unpack_weights(kind: int, codes, scales, N: int, K: int, head_dim: int = 0):
    rows = 2 * N if kind == I4D_PROJ_GATE_UP else N
    q = np.empty((rows, K), np.int8)
    s = np.empty((rows, K // 128), np.uint16)
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    _check(lib().i4d_unpack_weights(kind, ptr(codes), ptr(scales), N, K, head_dim, ptr(q), ptr(s)))
    return q, s


def i4d_packed_sizes_e4m3(kind: int, N: int, K: int, head_dim: int = 0):
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().i4d_packed_sizes_e4m3(kind, N, K, head_dim, ctypes.byref(cb), ctypes.byref(sb)))
    return cb.value, sb.value


def i4d_pack_weights_e4m3(kind: int, W0, W1=None, gamma=None, head_dim: int = 0, threads: int = 0):
    """fp32 host weights -> (E4M3 codes uint8, fp16 scales uint16) in the device layout."""
    W0 = np.ascontiguousarray(W0, dtype=np.float32)
    N, K = W0.shape
    W1 = None if W1 is None else np.ascontiguousarray(W1, dtype=np.float32)
    gamma = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.float32)
    cb, sb = i4d_packed_sizes_e4m3(kind, N, K, head_dim)
    codes = np.empty(cb, np.uint8)
    scales = np.empty(sb // 2, np.uint16)
    _check(lib().i4d_pack_weights_e4m3(kind, ptr(W0), ptr(W1), ptr(gamma), N, K, head_dim,
                                       ptr(codes), ptr(scales), threads))
    return codes, scales


def i4d_unpack_weights_e4m3(kind: int, codes, scales, N: int, K: int, head_dim: int = 0):
    rows = 2 * N if kind == I4D_PROJ_GATE_UP else N
    q = np.empty((rows, K), np.uint8)
    s = np.empty((rows, K // 128), np.uint16)
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    _check(lib().i4d_unpack_weights_e4m3(kind, ptr(codes), ptr(scales), N, K, head_dim, ptr(q), ptr(s)))
    return q, s


def i4d_packed_sizes_mx(kind: int, N: int, K: int, head_dim: int = 0):
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().i4d_packed_sizes_mx(kind, N, K, head_dim, ctypes.byref(cb), ctypes.byref(sb)))
    return cb.value, sb.value


def i4d_pack_weights_mx(kind: int, W0, W1=None, gamma=None, head_dim: int = 0, threads: int = 0):
    """fp32 host weights -> (E4M3 codes uint8, E8M0 scale bytes uint8) in the device layout."""
    W0 = np.ascontiguousarray(W0, dtype=np.float32)
    N, K = W0.shape
    W1 = None if W1 is None else np.ascontiguousarray(W1, dtype=np.float32)
    gamma = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.float32)
    cb, sb = i4d_packed_sizes_mx(kind, N, K, head_dim)
    codes = np.empty(cb, np.uint8)
    scales = np.empty(sb, np.uint8)
    _check(lib().i4d_pack_weights_mx(kind, ptr(W0), ptr(W1), ptr(gamma), N, K, head_dim, ptr(codes), ptr(scales),
                                     threads))
    return codes, scales


def i4d_unpack_weights_mx(kind: int, codes, scales, N: int, K: int, head_dim: int = 0):
    rows = 2 * N if kind == I4D_PROJ_GATE_UP else N
    q = np.empty((rows, K), np.uint8)
    s = np.empty((rows, K // 128), np.uint8)
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    _check(lib().i4d_unpack_weights_mx(kind, ptr(codes), ptr(scales), N, K, head_dim, ptr(q), ptr(s)))
    return q, s


def i4d_pack_lm_head(W, gamma=None, threads: int = 0):
    """fp32 [V][d] -> bf16 bits in tiles [V/16][d/32][16][32]."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    V, d = W.shape
    gamma = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.float32)
    out = np.empty((V // 16, d // 32, 16, 32) if V % 16 == 0 and d % 32 == 0 else (V, d), np.uint16)
    _check(lib().i4d_pack_lm_head(ptr(W), ptr(gamma), V, d, ptr(out), threads))
    return out


def i4d_kv_cache_bytes(n_kv_heads: int, head_dim: int, total_capacity: int):
    a, b, c, d = (ctypes.c_size_t() for _ in range(4))
    _check(lib().i4d_kv_cache_bytes(n_kv_heads, head_dim, total_capacity, ctypes.byref(a), ctypes.byref(b),
                                    ctypes.byref(c), ctypes.byref(d)))
    return a.value, b.value, c.value, d.value


def i4d_kv_unpack_host(host_cache: i4d_kv_cache, row_base_host, row: int, t0: int, t1: int):
    nkv, hd = host_cache.n_kv_heads, host_cache.head_dim
    n = t1 - t0
    k = np.empty((n, nkv, hd), np.int8)
    v = np.empty((n, nkv, hd), np.int8)
    ks = np.empty((n, nkv), np.uint16)
    vs = np.empty((n, nkv), np.uint16)
    rb = np.ascontiguousarray(row_base_host, dtype=np.int64)
    _check(lib().i4d_kv_unpack_host(ctypes.byref(host_cache), ptr(rb), row, t0, t1, ptr(k), ptr(v),
                                    ptr(ks), ptr(vs)))
    return k, v, ks, vs


def i4d_attention_workspace_bytes(shape: i4d_layer_shape, M: int, max_ctx_len: int, num_splits: int = 0):
    b = ctypes.c_size_t()
    _check(lib().i4d_attention_workspace_bytes(ctypes.byref(shape), M, max_ctx_len, num_splits, ctypes.byref(b)))
    return b.value


def i4d_workspace_bytes(shape: i4d_layer_shape, M: int, max_ctx_len: int, num_splits: int = 0):
    b = ctypes.c_size_t()
    _check(lib().i4d_workspace_bytes(ctypes.byref(shape), M, max_ctx_len, num_splits, ctypes.byref(b)))
    return b.value


def i4d_workspace_layout_of(shape: i4d_layer_shape, M: int, max_ctx_len: int, num_splits: int = 0):
    out = i4d_workspace_layout()
    _check(lib().i4d_workspace_layout_of(ctypes.byref(shape), M, max_ctx_len, num_splits, ctypes.byref(out)))
    return out


def i4d_decode_step_is_one_launch(shape: i4d_layer_shape, M: int) -> bool:
    out = _I()
    _check(lib().i4d_decode_step_is_one_launch(ctypes.byref(shape), M, ctypes.byref(out)))
    return bool(out.value)


def i4d_projection_plan_of(shape: i4d_layer_shape, stage: int, M: int) -> i4d_projection_plan:
    out = i4d_projection_plan()
    _check(lib().i4d_projection_plan_of(ctypes.byref(shape), stage, M, ctypes.byref(out)))
    return out


def i4d_workspace_init(workspace, nbytes: int, stream=None):
    _check(lib().i4d_workspace_init(ptr(workspace), nbytes, stream_handle(stream)))


def i4d_lm_head_workspace_bytes(V: int, M: int):
    b = ctypes.c_size_t()
    _check(lib().i4d_lm_head_workspace_bytes(V, M, ctypes.byref(b)))
    return b.value


# ---------------------------------------------------------------------------
# device calls (asynchronous on `stream`)
# ---------------------------------------------------------------------------

def i4d_kv_append(cache: i4d_kv_cache, k, v, row_idx, pos, T: int, stream=None):
    _check(lib().i4d_kv_append(ctypes.byref(cache), ptr(k), ptr(v), ptr(row_idx), ptr(pos), T,
                               stream_handle(stream)))


def i4d_attn_qkv(layer: i4d_layer, x, ctx_len, M: int, q_out, k_out, v_out, stream=None):
    _check(lib().i4d_attn_qkv(ctypes.byref(layer), ptr(x), ptr(ctx_len), M, ptr(q_out), ptr(k_out),
                              ptr(v_out), stream_handle(stream)))


def i4d_attention(cache: i4d_kv_cache, shape: i4d_layer_shape, q, ctx_len, M: int, max_ctx_len: int,
                  num_splits: int, workspace, workspace_bytes: int, attn_f32, attn_bf16, stream=None):
    _check(lib().i4d_attention(ctypes.byref(cache), ctypes.byref(shape), ptr(q), ptr(ctx_len), M,
                               max_ctx_len, num_splits, ptr(workspace), workspace_bytes, ptr(attn_f32),
                               ptr(attn_bf16), stream_handle(stream)))


def i4d_attn_out_proj(layer: i4d_layer, attn_bf16, x, M: int, h_f32, h_bf16, stream=None):
    _check(lib().i4d_attn_out_proj(ctypes.byref(layer), ptr(attn_bf16), ptr(x), M, ptr(h_f32), ptr(h_bf16),
                                   stream_handle(stream)))


def i4d_ffn_gate_up(layer: i4d_layer, h_bf16, M: int, a_out, stream=None):
    _check(lib().i4d_ffn_gate_up(ctypes.byref(layer), ptr(h_bf16), M, ptr(a_out), stream_handle(stream)))


def i4d_ffn_down(layer: i4d_layer, a, h_f32, M: int, x_out, stream=None):
    _check(lib().i4d_ffn_down(ctypes.byref(layer), ptr(a), ptr(h_f32), M, ptr(x_out), stream_handle(stream)))


def i4d_decode_block_step(layer: i4d_layer, cache: i4d_kv_cache, x_in, x_out, ctx_len, M: int,
                          max_ctx_len: int, num_splits: int, workspace, workspace_bytes: int,
                          attn_f32=None, stream=None):
    _check(lib().i4d_decode_block_step(ctypes.byref(layer), ctypes.byref(cache), ptr(x_in), ptr(x_out),
                                       ptr(ctx_len), M, max_ctx_len, num_splits, ptr(workspace),
                                       workspace_bytes, ptr(attn_f32), stream_handle(stream)))


def i4d_decode_block_step_timeline(layer: i4d_layer, cache: i4d_kv_cache, x_in, x_out, ctx_len, M: int,
                                   max_ctx_len: int, num_splits: int, workspace, workspace_bytes: int, stamps,
                                   stamps_count: int, attn_f32=None, stream=None):
    _check(lib().i4d_decode_block_step_timeline(ctypes.byref(layer), ctypes.byref(cache), ptr(x_in), ptr(x_out),
                                                ptr(ctx_len), M, max_ctx_len, num_splits, ptr(workspace),
                                                workspace_bytes, ptr(attn_f32), ptr(stamps), stamps_count,
                                                stream_handle(stream)))


def i4d_decode_block_step_e4m3(layer: i4d_layer, cache: i4d_kv_cache, x_in, x_out, ctx_len, M: int,
                               max_ctx_len: int, num_splits: int, workspace, workspace_bytes: int,
                               attn_f32=None, stream=None):
    _check(lib().i4d_decode_block_step_e4m3(ctypes.byref(layer), ctypes.byref(cache), ptr(x_in), ptr(x_out),
                                            ptr(ctx_len), M, max_ctx_len, num_splits, ptr(workspace),
                                            workspace_bytes, ptr(attn_f32), stream_handle(stream)))


def i4d_attn_out_proj_e4m3(layer: i4d_layer, attn_bf16, x, M: int, h_f32, h_bf16, stream=None):
    _check(lib().i4d_attn_out_proj_e4m3(ctypes.byref(layer), ptr(attn_bf16), ptr(x), M, ptr(h_f32), ptr(h_bf16),
                                        stream_handle(stream)))


def i4d_decode_block_step_noalloc(layer: i4d_layer, cache: i4d_kv_cache, x_in, x_out, ctx_len, M: int,
                                  max_ctx_len: int, num_splits: int, attn_f32=None, stream=None):
    _check(lib().i4d_decode_block_step_noalloc(ctypes.byref(layer), ctypes.byref(cache), ptr(x_in), ptr(x_out),
                                               ptr(ctx_len), M, max_ctx_len, num_splits, ptr(attn_f32),
                                               stream_handle(stream)))


def i4d_lm_head_argmax(w_lm, V: int, d: int, h, M: int, rms_eps: float, logits_out, token_out,
                       workspace, workspace_bytes: int, stream=None):
    _check(lib().i4d_lm_head_argmax(ptr(w_lm), V, d, ptr(h), M, float(rms_eps), ptr(logits_out),
                                    ptr(token_out), ptr(workspace), workspace_bytes, stream_handle(stream)))


def i4d_prefill_workspace_bytes(shape: i4d_layer_shape, T: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().i4d_prefill_workspace_bytes(ctypes.byref(shape), T, ctypes.byref(b)))
    return b.value


def i4d_prefill_qkv_e4m3(layer: i4d_prefill_weights, cache: i4d_kv_cache, x, T: int, cu_seqlens, start_pos, R: int,
                         scales, q_fp8, k_bf16, v_bf16, workspace, workspace_bytes: int, stream=None):
    """scales: device i4d_fp8_scales (e.g. a float32 tensor of 4 elements)."""
    _check(lib().i4d_prefill_qkv_e4m3(ctypes.byref(layer), ctypes.byref(cache), ptr(x), T, ptr(cu_seqlens),
                                      ptr(start_pos), R, ptr(scales), ptr(q_fp8), ptr(k_bf16), ptr(v_bf16),
                                      ptr(workspace), workspace_bytes, stream_handle(stream)))


def i4d_prefill_prepare(layer: i4d_prefill_weights, cache: i4d_kv_cache, x, T: int, cu_seqlens, start_pos, R: int, scales,
                        workspace, workspace_bytes: int, stream=None):
    _check(lib().i4d_prefill_prepare(ctypes.byref(layer), ctypes.byref(cache), ptr(x), T, ptr(cu_seqlens),
                                     ptr(start_pos), R, ptr(scales), ptr(workspace), workspace_bytes,
                                     stream_handle(stream)))


def i4d_prefill_project(layer: i4d_prefill_weights, cache: i4d_kv_cache, T: int, cu_seqlens, start_pos, R: int, scales,
                        q_fp8, k_bf16, v_bf16, workspace, workspace_bytes: int, stream=None):
    _check(lib().i4d_prefill_project(ctypes.byref(layer), ctypes.byref(cache), T, ptr(cu_seqlens), ptr(start_pos),
                                     R, ptr(scales), ptr(q_fp8), ptr(k_bf16), ptr(v_bf16), ptr(workspace),
                                     workspace_bytes, stream_handle(stream)))


def i4d_fp8_scales_update(scales, stream=None):
    _check(lib().i4d_fp8_scales_update(ptr(scales), stream_handle(stream)))
