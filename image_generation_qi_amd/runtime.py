"""Torch-side plumbing around libqi: device buffers, streams and table upload.

PyTorch only allocates device memory and supplies the current HIP stream; every step of
the attention path runs in libqi's kernels (or, for tables, its C++ host helpers).
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import qi as Q

TORCH_DTYPE = {Q.QI_BF16: torch.bfloat16, Q.QI_F32: torch.float32, Q.QI_F16: torch.float16}


def stream_handle(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def dtype_code(name: str) -> int:
    return {"bf16": Q.QI_BF16, "f32": Q.QI_F32, "f16": Q.QI_F16}[name]


class Layout:
    """A segment layout with its host-built rotation tables uploaded to the device."""

    def __init__(self, segments, device="cuda", bands=(16, 56, 56), theta: float = 10000.0, text_pos0: int = -1):
        self.segments = tuple(segments)
        self.c = Q.make_layout(self.segments, 128, bands, theta, text_pos0)
        self.S, self.P, self.T = Q.qi_layout_tokens(self.c)
        cos = np.empty((self.S, 64), np.float32)
        sin = np.empty((self.S, 64), np.float32)
        Q.check(Q.qi_rope3d_tables(self.c, cos, sin), "qi_rope3d_tables")
        self.cos_host, self.sin_host = cos, sin
        self.cos = torch.from_numpy(cos).to(device)
        self.sin = torch.from_numpy(sin).to(device)

    def rows(self, start: int, stop: Optional[int] = None):
        """Device (cos, sin) views of table rows [start, stop)."""
        return self.cos[start:stop], self.sin[start:stop]


class KVCache:
    """Per-layer prefix K/V cache [n_layers][n_head][p_cap][128] (fp16 for bf16 attention)."""

    def __init__(self, n_layers: int, n_head: int, p_cap: int, io_dtype: int = Q.QI_BF16, device="cuda"):
        self.dtype = Q.QI_F16 if io_dtype == Q.QI_BF16 else Q.QI_F32
        td = TORCH_DTYPE[self.dtype]
        self.k = torch.empty((n_layers, n_head, max(p_cap, 1), 128), dtype=td, device=device)
        self.v = torch.empty_like(self.k)
        self.c = Q.make_cache(self.k, self.v, self.dtype, n_layers, n_head, p_cap)


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


class Attention:
    """Owns the workspaces for one (layout, heads, dtype) and issues the ABI calls."""

    def __init__(self, layout: Layout, n_head: int, io_dtype: int = Q.QI_BF16, device="cuda"):
        self.L, self.H, self.dtype, self.device = layout, n_head, io_dtype, device
        self.ws_full_bytes = Q.qi_attn_full_workspace_bytes(layout.c, io_dtype, n_head)
        self.ws_cached_bytes = Q.qi_attn_cached_workspace_bytes(io_dtype, layout.T, n_head)
        self.ws_full = None
        self.ws_cached = None

    def _stride(self, t: torch.Tensor) -> int:
        assert t.dim() == 3 and t.shape[1] == self.H and t.shape[2] == 128 and t.stride(2) == 1 and t.stride(1) == 128
        return t.stride(0)

    def prep(self, rows: slice, q_w=None, k_w=None, eps: float = 1e-6, rotate: bool = True):
        cos, sin = self.L.rows(rows.start, rows.stop) if rotate else (None, None)
        return Q.make_prep(cos, sin, q_w, k_w, eps), (cos, sin)

    def full(self, q, k, v, q_w=None, k_w=None, eps=1e-6, cache: Optional[KVCache] = None, layer: int = 0,
             scale: float = 0.0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        if self.ws_full is None:
            self.ws_full = _ws(self.ws_full_bytes, self.device)
        o = out if out is not None else torch.empty((self.L.S, self.H, 128), dtype=q.dtype, device=self.device)
        io = Q.make_qkv(q, k, v, o, self.dtype, self.L.S, self.H, self._stride(q))
        prep, keep = self.prep(slice(0, self.L.S), q_w, k_w, eps)
        Q.check(Q.qi_attn_blockcausal_full(io, prep, self.L.c, scale, cache.c if cache else None, layer,
                                           self.ws_full, self.ws_full_bytes, stream_handle(self.device)),
                "qi_attn_blockcausal_full")
        return o

    def store(self, k, v, cache: KVCache, layer: int = 0, k_w=None, eps=1e-6):
        prep, keep = self.prep(slice(0, self.L.P), None, k_w, eps)
        Q.check(Q.qi_attn_prefix_store(k, v, self.dtype, self.L.P, self.H, self._stride(k), prep, cache.c, layer,
                                       stream_handle(self.device)), "qi_attn_prefix_store")

    def cached(self, q_t, k_t, v_t, cache: KVCache, layer: int = 0, q_w=None, k_w=None, eps=1e-6,
               scale: float = 0.0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        if self.ws_cached is None:
            self.ws_cached = _ws(self.ws_cached_bytes, self.device)
        T = q_t.shape[0]
        o = out if out is not None else torch.empty((T, self.H, 128), dtype=q_t.dtype, device=self.device)
        io = Q.make_qkv(q_t, k_t, v_t, o, self.dtype, T, self.H, self._stride(q_t))
        prep, keep = self.prep(slice(self.L.P, self.L.P + T), q_w, k_w, eps)
        Q.check(Q.qi_attn_target_cached(io, prep, cache.c, layer, self.L.P, scale, self.ws_cached,
                                        self.ws_cached_bytes, stream_handle(self.device)), "qi_attn_target_cached")
        return o


def euler_step(x: torch.Tensor, v: torch.Tensor, sigma_k: float, sigma_k1: float):
    assert x.dtype == torch.float32 and x.is_contiguous() and v.is_contiguous() and v.numel() == x.numel()
    vd = Q.QI_BF16 if v.dtype == torch.bfloat16 else Q.QI_F32
    Q.check(Q.qi_euler_step(x, v, vd, x.numel(), sigma_k, sigma_k1, stream_handle(x.device)), "qi_euler_step")
    return x


def rope3d_apply(x: torch.Tensor, cos, sin, rms_w=None, eps: float = 1e-6):
    assert x.dim() == 3 and x.shape[2] == 128 and x.stride(2) == 1 and x.stride(1) == 128
    dt = Q.QI_BF16 if x.dtype == torch.bfloat16 else Q.QI_F32
    Q.check(Q.qi_rope3d_apply(x, dt, x.shape[0], x.shape[1], x.stride(0), cos, sin, rms_w, eps,
                              stream_handle(x.device)), "qi_rope3d_apply")
    return x


def from_bits(bits: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Device tensor holding exactly the given stored values (bf16 bit patterns or fp32)."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.float32)).to(device)
