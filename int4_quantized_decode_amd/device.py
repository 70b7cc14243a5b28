"""Device-memory plumbing around the C ABI (torch tensors hold GPU buffers).

Nothing here computes anything of the method: weights are packed by the
library's host packer, caches are filled by the library's kv_append, and
these classes only allocate tensors and fill the C structs with pointers.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from . import binding as B
from . import synth


def to_device_u16(a: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bit patterns (bf16/fp16) -> int16 device tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


def to_host_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


def bf16_tensor_to_f32(t: torch.Tensor) -> np.ndarray:
    return synth.bf16_bits_to_f32(to_host_u16(t))


class DeviceLayer:
    """One layer's packed INT4 weights on the GPU and its i4d_layer struct."""

    def __init__(self, shape: synth.LayerShape, lw: synth.LayerWeights, device="cuda", threads: int = 0,
                 fmt: str = "int4"):
        self.fmt = fmt
        self._upload(shape, self.pack_host(shape, lw, threads, fmt), device)

    @staticmethod
    def pack_host(shape: synth.LayerShape, lw: synth.LayerWeights, threads: int = 0, fmt: str = "int4") -> dict:
        """The library's host packer on the four projections of a layer:
        {name: (codes uint8, scales uint16)} in the device layout; fmt
        "int4" (i4d_pack_weights) or "e4m3" (i4d_pack_weights_e4m3)."""
        pack = {"int4": B.i4d_pack_weights, "e4m3": B.i4d_pack_weights_e4m3}[fmt]
        hd = shape.head_dim
        return dict(
            qkv=pack(B.I4D_PROJ_QKV, lw.w_qkv, None, lw.gamma_attn, hd, threads),
            o=pack(B.I4D_PROJ_PLAIN, lw.w_o, None, None, 0, threads),
            gu=pack(B.I4D_PROJ_GATE_UP, lw.w_gate, lw.w_up, lw.gamma_ffn, 0, threads),
            down=pack(B.I4D_PROJ_PLAIN, lw.w_down, None, None, 0, threads))

    @classmethod
    def from_host(cls, shape: synth.LayerShape, host: dict, device="cuda") -> "DeviceLayer":
        obj = cls.__new__(cls)
        obj._upload(shape, host, device)
        return obj

    def _upload(self, shape, host, device):
        self.shape = shape
        self.host = host
        self.tensors = {}
        for name, (codes, scales) in host.items():
            self.tensors[name] = (torch.from_numpy(codes).to(device), to_device_u16(scales, device))
        self.struct = self._make_struct()

    @classmethod
    def from_packed(cls, shape, tensors):
        obj = cls.__new__(cls)
        obj.shape = shape
        obj.host = None
        obj.tensors = tensors
        obj.struct = obj._make_struct()
        return obj

    def clone(self) -> "DeviceLayer":
        """Same bytes at new device addresses (for cache-cold timing)."""
        t = {k: (c.clone(), s.clone()) for k, (c, s) in self.tensors.items()}
        obj = DeviceLayer.from_packed(self.shape, t)
        obj.fmt = getattr(self, "fmt", "int4")
        return obj

    def _make_struct(self) -> B.i4d_layer:
        t = self.tensors
        return B.i4d_layer(B.make_shape(self.shape),
                           t["qkv"][0].data_ptr(), t["qkv"][1].data_ptr(),
                           t["o"][0].data_ptr(), t["o"][1].data_ptr(),
                           t["gu"][0].data_ptr(), t["gu"][1].data_ptr(),
                           t["down"][0].data_ptr(), t["down"][1].data_ptr())

    @property
    def weight_bytes(self) -> int:
        return sum(c.numel() + 2 * s.numel() for c, s in self.tensors.values())


class PrefillWeights:
    """The FP8 prefill's QKV weight on the device: E4M3 atoms with E8M0 group
    scales (i4d_pack_weights_mx, attention gain folded)."""

    def __init__(self, shape: synth.LayerShape, lw: synth.LayerWeights, device="cuda", threads: int = 0):
        codes, scales = B.i4d_pack_weights_mx(B.I4D_PROJ_QKV, lw.w_qkv, None, lw.gamma_attn, shape.head_dim, threads)
        self.shape = shape
        self.codes = torch.from_numpy(codes).to(device)
        self.scales = torch.from_numpy(scales).to(device)
        self.struct = B.i4d_prefill_weights(B.make_shape(shape), self.codes.data_ptr(), self.scales.data_ptr())


class DeviceCache:
    """Paged INT4 KV cache: one row per decode row, capacity rounded up to 32."""

    def __init__(self, shape: synth.LayerShape, capacities, device="cuda"):
        caps = [int(-(-int(c) // 32) * 32) for c in capacities]
        self.shape = shape
        self.capacities = caps
        self.row_base_host = np.concatenate([[0], np.cumsum(caps)]).astype(np.int64)
        total = int(self.row_base_host[-1])
        kcb, vcb, ksb, vsb = B.i4d_kv_cache_bytes(shape.n_kv_heads, shape.head_dim, total)
        self.k_codes = torch.zeros(kcb, dtype=torch.uint8, device=device)
        self.v_codes = torch.zeros(vcb, dtype=torch.uint8, device=device)
        self.k_scales = torch.zeros(ksb // 2, dtype=torch.int16, device=device)
        self.v_scales = torch.zeros(vsb // 2, dtype=torch.int16, device=device)
        self.row_base = torch.from_numpy(self.row_base_host).to(device)
        self.err_word = torch.zeros(4, dtype=torch.int32, device=device)
        self.struct = B.i4d_kv_cache(self.k_codes.data_ptr(), self.v_codes.data_ptr(),
                                     self.k_scales.data_ptr(), self.v_scales.data_ptr(),
                                     self.row_base.data_ptr(), len(caps), shape.n_kv_heads,
                                     shape.head_dim, total, self.err_word.data_ptr())

    def prefill(self, prefill: synth.CachePrefill, stream=None, chunk: int = 1 << 16):
        """Append every prefill token (positions 0..L_r-2 of each row) through kv_append."""
        ks, vs, rows, poss = [], [], [], []
        for r, (k, v) in enumerate(zip(prefill.k, prefill.v)):
            n = k.shape[0]
            if n == 0:
                continue
            ks.append(k.reshape(n, -1))
            vs.append(v.reshape(n, -1))
            rows.append(np.full(n, r, np.int32))
            poss.append(np.arange(n, dtype=np.int32))
        if not ks:
            return
        k = np.concatenate(ks)
        v = np.concatenate(vs)
        row = np.concatenate(rows)
        pos = np.concatenate(poss)
        for s0 in range(0, k.shape[0], chunk):
            s1 = min(k.shape[0], s0 + chunk)
            kd = to_device_u16(k[s0:s1])
            vd = to_device_u16(v[s0:s1])
            rd = torch.from_numpy(row[s0:s1]).to(kd.device)
            pd = torch.from_numpy(pos[s0:s1]).to(kd.device)
            B.i4d_kv_append(self.struct, kd, vd, rd, pd, s1 - s0, stream)
            torch.cuda.current_stream().synchronize()

    def host_view(self):
        """Host copies of the buffers and an i4d_kv_cache struct pointing at them."""
        hk = self.k_codes.cpu().numpy()
        hv = self.v_codes.cpu().numpy()
        hks = self.k_scales.cpu().numpy()
        hvs = self.v_scales.cpu().numpy()
        s = B.i4d_kv_cache(hk.ctypes.data, hv.ctypes.data, hks.ctypes.data, hvs.ctypes.data,
                           self.row_base_host.ctypes.data, len(self.capacities), self.shape.n_kv_heads,
                           self.shape.head_dim, int(self.row_base_host[-1]), None)
        return s, (hk, hv, hks, hvs)

    def read_codes(self, row: int, t0: int, t1: int):
        s, keep = self.host_view()
        out = B.i4d_kv_unpack_host(s, self.row_base_host, row, t0, t1)
        del keep
        return out

    def errors(self) -> int:
        return int(self.err_word[0].item())


class Workspace:
    def __init__(self, shape: synth.LayerShape, M: int, max_ctx_len: int, num_splits: int = 0, device="cuda"):
        self.cshape = B.make_shape(shape)
        self.nbytes = B.i4d_workspace_bytes(self.cshape, M, max_ctx_len, num_splits)
        self.layout = B.i4d_workspace_layout_of(self.cshape, M, max_ctx_len, num_splits)
        self.buf = torch.zeros(self.nbytes, dtype=torch.uint8, device=device)
        self.M, self.shape = M, shape

    def view(self, name: str, dtype, count: int) -> torch.Tensor:
        off = getattr(self.layout, name)
        esize = torch.tensor([], dtype=dtype).element_size()
        return self.buf[off: off + count * esize].view(dtype)


def stacked_layers(shape: synth.LayerShape, seeds, lengths, workers: int = 8, on_host=None):
    """One independently seeded layer per seed, packed and uploaded, each
    with its own KV cache prefilled with that seed's cached tokens (the
    stack of a full-model step).  Weights and cache tokens are drawn and
    packed in `workers` host threads; uploads and the prefill (kv_append)
    run on the calling thread.  ``on_host(seed, lw, prefill)``, if given,
    runs in the worker on the layer's host arrays before they are dropped;
    its results are returned in seed order.  Returns (layers, caches,
    results)."""
    lengths = np.asarray(lengths, np.int32)

    def host(seed):
        lw = synth.make_layer(shape, seed)
        packed = DeviceLayer.pack_host(shape, lw, threads=2)
        pre = synth.make_cache_prefill(shape, lengths, seed)
        extra = on_host(seed, lw, pre) if on_host else None
        del lw
        return packed, pre, extra

    layers, caches, extras = [], [], []
    with ThreadPoolExecutor(max(1, workers)) as ex:
        for packed, pre, extra in ex.map(host, seeds):
            layers.append(DeviceLayer.from_host(shape, packed))
            c = DeviceCache(shape, lengths)
            c.prefill(pre)
            caches.append(c)
            extras.append(extra)
            for name in list(packed):  # the host copies are not needed once uploaded
                packed[name] = None
    return layers, caches, extras
