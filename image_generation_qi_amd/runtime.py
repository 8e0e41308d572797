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

# 16-bit activation type of the composed layer paths (DiT, TextProjection, V1Block): fp16 rounds
# each activation to 11 bits instead of bf16's 8 at the same matrix-core rate, which keeps a whole
# layer's residual increment within the bf16 bar; the model's bf16 weights convert to it exactly
# (magnitudes 2^-17 .. 65504).  Values it cannot hold raise the range flags.
ACT = torch.float16


def stream_handle(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def dtype_code(name: str) -> int:
    return {"bf16": Q.QI_BF16, "f32": Q.QI_F32, "f16": Q.QI_F16}[name]


class Layout:
    """A segment layout with its host-built rotation tables uploaded to the device."""

    def __init__(self, segments, device="cuda", bands=(16, 56, 56), theta: float = 10000.0, text_pos0: int = -1,
                 attention: int = Q.QI_ATTN_BLOCK_CAUSAL):
        self.segments = tuple(segments)
        self.attention = attention
        self.c = Q.make_layout(self.segments, 128, bands, theta, text_pos0, attention)
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
    """Per-layer prefix K/V cache (fp16 for bf16 attention, fp32 for fp32 attention).

    k, v: [n_layers][n_head][R][128] storage.  fp32 caches hold row-major K and V rows (R =
    p_cap).  fp16 caches (R = p_cap rounded up to a multiple of 64) hold each head's keys in
    tiles of 64 keys: K as [16 dim chunks][64 keys][8 dims], V as [2 key halves][4 key
    groups][128 dims][8 keys] with element e of group g of half c holding key 32c + 16(e // 4) +
    4g + e % 4; k_rows and v_rows return plain [n_head][R][128] rows."""

    def __init__(self, n_layers: int, n_head: int, p_cap: int, io_dtype: int = Q.QI_BF16, device="cuda"):
        self.dtype = Q.QI_F32 if io_dtype == Q.QI_F32 else Q.QI_F16
        td = TORCH_DTYPE[self.dtype]
        rows = (p_cap + 63) // 64 * 64 if self.dtype == Q.QI_F16 else p_cap
        self.rows = max(rows, 64 if self.dtype == Q.QI_F16 else 1)
        self.k = torch.zeros((n_layers, n_head, self.rows, 128), dtype=td, device=device)
        self.v = torch.zeros_like(self.k)
        self.c = Q.make_cache(self.k, self.v, self.dtype, n_layers, n_head, p_cap)

    def k_rows(self, layer: int) -> torch.Tensor:
        """K of one layer as [n_head][R][128] rows (a copy for fp16 caches)."""
        k = self.k[layer]
        if self.dtype != Q.QI_F16:
            return k
        H = k.shape[0]
        return k.reshape(H, self.rows // 64, 16, 64, 8).permute(0, 1, 3, 2, 4).reshape(H, self.rows, 128)

    def v_rows(self, layer: int) -> torch.Tensor:
        """V of one layer as [n_head][R][128] rows (a copy for fp16 caches)."""
        v = self.v[layer]
        if self.dtype != Q.QI_F16:
            return v
        H = v.shape[0]
        # [tile][half c][group g][dim][e_hi][e_lo] -> key order (c, e_hi, g, e_lo)
        t = v.reshape(H, self.rows // 64, 2, 4, 128, 2, 4).permute(0, 1, 2, 5, 3, 6, 4)
        return t.reshape(H, self.rows, 128)


class KVTiles:
    """fp16 K/V tiles of one key source outside a cache (qi_kvtiles): the target tokens of the fused
    QKV path, written by gemm_qkv_tiles and read by Attention.cached_tiled / full_tiled.  k, v:
    [n_head][R][128] storage in the fp16 cache's tile layout (R = n_keys rounded up to 64)."""

    def __init__(self, n_keys: int, n_head: int, device="cuda"):
        self.rows = max((n_keys + 63) // 64 * 64, 64)
        self.n_head = n_head
        self.k = torch.zeros((n_head, self.rows, 128), dtype=torch.float16, device=device)
        self.v = torch.zeros_like(self.k)
        self.c = Q.make_tiles(self.k, self.v, n_head, self.rows)

    def k_rows(self) -> torch.Tensor:
        """K as [n_head][R][128] rows (a copy)."""
        H = self.n_head
        return self.k.reshape(H, self.rows // 64, 16, 64, 8).permute(0, 1, 3, 2, 4).reshape(H, self.rows, 128)

    def v_rows(self) -> torch.Tensor:
        """V as [n_head][R][128] rows (a copy)."""
        H = self.n_head
        t = self.v.reshape(H, self.rows // 64, 2, 4, 128, 2, 4).permute(0, 1, 2, 5, 3, 6, 4)
        return t.reshape(H, self.rows, 128)


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


class RangeError(RuntimeError):
    """A value did not fit fp16: a q, k or v operand of the attention's matrix cores, or an fp16
    activation of the layer chain."""


class Attention:
    """Owns the workspaces and the range-flag word for one (layout, heads, dtype) and issues the
    ABI calls.  Every call ORs its QI_RANGE_* bits into the flag word; range_flags() reads it."""

    def __init__(self, layout: Layout, n_head: int, io_dtype: int = Q.QI_BF16, device="cuda"):
        self.L, self.H, self.dtype, self.device = layout, n_head, io_dtype, device
        self.ws_full_bytes = Q.qi_attn_full_workspace_bytes(layout.c, io_dtype, n_head)
        self.ws_cached_bytes = Q.qi_attn_cached_workspace_bytes(io_dtype, layout.T, n_head)
        self.ws_tiled_bytes = Q.qi_attn_tiled_workspace_bytes(layout.c, n_head) if io_dtype != Q.QI_F32 else 0
        self.ws_full = None
        self.ws_cached = None
        self.ws_tiled = None
        self.flags = torch.zeros(1, dtype=torch.int32, device=device)

    def range_flags(self, clear: bool = True) -> int:
        """QI_RANGE_* bits raised since the last clear (waits for the device)."""
        v = int(self.flags.item())
        if clear:
            self.flags.zero_()
        return v

    def check_range(self):
        """Raise RangeError if a call since the last check met a value that does not fit fp16."""
        v = self.range_flags()
        if v:
            names = [n for b, n in ((Q.QI_RANGE_Q, "q"), (Q.QI_RANGE_K, "k"), (Q.QI_RANGE_V, "v"),
                                    (Q.QI_RANGE_OUT, "layer outputs")) if v & b]
            raise RangeError(f"values of {', '.join(names)} outside the fp16 range")

    def _stride(self, t: torch.Tensor) -> int:
        assert t.dim() == 3 and t.shape[1] == self.H and t.shape[2] == 128 and t.stride(2) == 1 and t.stride(1) == 128
        return t.stride(0)

    def prep(self, rows: slice, q_w=None, k_w=None, eps: float = 1e-6, rotate: bool = True):
        cos, sin = self.L.rows(rows.start, rows.stop) if rotate else (None, None)
        return Q.make_prep(cos, sin, q_w, k_w, eps), (cos, sin)

    def full(self, q, k, v, q_w=None, k_w=None, eps=1e-6, cache: Optional[KVCache] = None, layer: int = 0,
             scale: float = 0.0, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
             rotate: bool = True) -> torch.Tensor:
        """Step 1 over the layout; lse (optional fp32 [H][S]) receives each row's log-sum-exp;
        rotate=False passes no rotation tables (q and k already rotated)."""
        if self.ws_full is None:
            self.ws_full = _ws(self.ws_full_bytes, self.device)
        o = out if out is not None else torch.empty((self.L.S, self.H, 128), dtype=q.dtype, device=self.device)
        if lse is not None:
            assert lse.dtype == torch.float32 and lse.is_contiguous() and lse.shape == (self.H, self.L.S)
        io = Q.make_qkv(q, k, v, o, self.dtype, self.L.S, self.H, self._stride(q), lse, self.flags)
        prep, keep = self.prep(slice(0, self.L.S), q_w, k_w, eps, rotate)
        Q.check(Q.qi_attn_blockcausal_full(io, prep, self.L.c, scale, cache.c if cache else None, layer,
                                           self.ws_full, self.ws_full_bytes, stream_handle(self.device)),
                "qi_attn_blockcausal_full")
        return o

    def store(self, k, v, cache: KVCache, layer: int = 0, k_w=None, eps=1e-6, rotate: bool = True):
        prep, keep = self.prep(slice(0, self.L.P), None, k_w, eps, rotate)
        Q.check(Q.qi_attn_prefix_store(k, v, self.dtype, self.L.P, self.H, self._stride(k), prep, cache.c, layer,
                                       self.flags, stream_handle(self.device)), "qi_attn_prefix_store")

    def cached(self, q_t, k_t, v_t, cache: KVCache, layer: int = 0, q_w=None, k_w=None, eps=1e-6,
               scale: float = 0.0, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
               rotate: bool = True) -> torch.Tensor:
        """A cached target step; lse (optional fp32 [H][T]) receives each row's log-sum-exp."""
        if self.ws_cached is None:
            self.ws_cached = _ws(self.ws_cached_bytes, self.device)
        T = q_t.shape[0]
        o = out if out is not None else torch.empty((T, self.H, 128), dtype=q_t.dtype, device=self.device)
        if lse is not None:
            assert lse.dtype == torch.float32 and lse.is_contiguous() and lse.shape == (self.H, T)
        io = Q.make_qkv(q_t, k_t, v_t, o, self.dtype, T, self.H, self._stride(q_t), lse, self.flags)
        prep, keep = self.prep(slice(self.L.P, self.L.P + T), q_w, k_w, eps, rotate)
        Q.check(Q.qi_attn_target_cached(io, prep, cache.c, layer, self.L.P, scale, self.ws_cached,
                                        self.ws_cached_bytes, stream_handle(self.device)), "qi_attn_target_cached")
        return o


    def _tiled_ws(self):
        if self.ws_tiled is None:
            self.ws_tiled = _ws(self.ws_tiled_bytes, self.device)
        return self.ws_tiled

    def cached_tiled(self, q_t, cache: KVCache, layer: int, target: KVTiles, q_w=None, eps=1e-6, scale: float = 0.0,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     rotate: bool = True) -> torch.Tensor:
        """A cached target step whose target K/V are already tiles (written by gemm_qkv_tiles)."""
        T = q_t.shape[0]
        o = out if out is not None else torch.empty((T, self.H, 128), dtype=q_t.dtype, device=self.device)
        io = Q.make_qkv(q_t, None, None, o, self.dtype, T, self.H, self._stride(q_t), lse, self.flags)
        prep, keep = self.prep(slice(self.L.P, self.L.P + T), q_w, None, eps, rotate)
        Q.check(Q.qi_attn_target_cached_tiled(io, prep, cache.c, layer, self.L.P, scale, target.c, self._tiled_ws(),
                                              self.ws_tiled_bytes, stream_handle(self.device)),
                "qi_attn_target_cached_tiled")
        return o

    def full_tiled(self, q, cache: KVCache, layer: int, target: KVTiles, q_w=None, eps=1e-6, scale: float = 0.0,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   rotate: bool = True) -> torch.Tensor:
        """Step 1 with the prefix K/V in cache layer `layer` and the target's in `target`, both
        already tiles (written by gemm_qkv_tiles)."""
        o = out if out is not None else torch.empty((self.L.S, self.H, 128), dtype=q.dtype, device=self.device)
        io = Q.make_qkv(q, None, None, o, self.dtype, self.L.S, self.H, self._stride(q), lse, self.flags)
        prep, keep = self.prep(slice(0, self.L.S), q_w, None, eps, rotate)
        Q.check(Q.qi_attn_blockcausal_full_tiled(io, prep, self.L.c, scale, cache.c, layer, target.c, self._tiled_ws(),
                                                 self.ws_tiled_bytes, stream_handle(self.device)),
                "qi_attn_blockcausal_full_tiled")
        return o


def euler_step(x: torch.Tensor, v: torch.Tensor, sigma_k: float, sigma_k1: float):
    assert x.dtype == torch.float32 and x.is_contiguous() and v.is_contiguous() and v.numel() == x.numel()
    vd = Q.QI_BF16 if v.dtype == torch.bfloat16 else Q.QI_F32
    Q.check(Q.qi_euler_step(x, v, vd, x.numel(), sigma_k, sigma_k1, stream_handle(x.device)), "qi_euler_step")
    return x


def code_of(t: torch.Tensor) -> int:
    """qi_dtype of a tensor's element type."""
    return {torch.bfloat16: Q.QI_BF16, torch.float16: Q.QI_F16, torch.float32: Q.QI_F32}[t.dtype]


def rope3d_apply(x: torch.Tensor, cos, sin, rms_w=None, eps: float = 1e-6):
    assert x.dim() == 3 and x.shape[2] == 128 and x.stride(2) == 1 and x.stride(1) == 128
    dt = code_of(x)
    Q.check(Q.qi_rope3d_apply(x, dt, x.shape[0], x.shape[1], x.stride(0), cos, sin, rms_w, eps,
                              stream_handle(x.device)), "qi_rope3d_apply")
    return x


def from_bits(bits: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Device tensor holding exactly the given stored values (bf16 or fp16 bit patterns, or fp32)."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).to(device)
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.float32)).to(device)


# ------------------------------------------------------------------------------------------------
# one single-stream DiT layer and the sampling loop around the attention
# ------------------------------------------------------------------------------------------------

def pack_swiglu(w_gate: torch.Tensor, w_up: torch.Tensor) -> torch.Tensor:
    """Interleave gate and up weights [F][D] into the [2F][D] layout the SwiGLU epilogue reads:
    blocks of 64 rows, 32 gate rows then the 32 up rows of the same features."""
    F, D = w_gate.shape
    assert w_up.shape == (F, D) and F % 32 == 0
    return torch.stack([w_gate.reshape(F // 32, 32, D), w_up.reshape(F // 32, 32, D)], dim=1).reshape(2 * F, D).contiguous()


def pack_qkv_tiles(w_qkv: torch.Tensor, n_head: int) -> torch.Tensor:
    """Rows of W_qkv [3D][D_in] (the Q, K and V rows, D = 128 n_head each) in the tile order that
    gemm_qkv_tiles reads: for each head h, the rows of K_h then of V_h dims 0..63; then the rows of
    V_h dims 64..127 of every head; then the Q rows."""
    D = 128 * n_head
    assert w_qkv.shape[0] == 3 * D
    k = w_qkv[D:2 * D].reshape(n_head, 128, -1)
    v = w_qkv[2 * D:].reshape(n_head, 128, -1)
    first = torch.cat([k, v[:, :64]], dim=1).reshape(n_head * 192, -1)
    return torch.cat([first, v[:, 64:].reshape(n_head * 64, -1), w_qkv[:D]], dim=0).contiguous()


def gemm_qkv_tiles(x: torch.Tensor, w: torch.Tensor, q_out: torch.Tensor, n_head: int, row0: int, P: int, T: int,
                   cache: Optional[KVCache], layer: int, target: Optional[KVTiles], tables=None, k_w=None,
                   eps: float = 1e-6, bias=None, flags=None, fold: Optional["NormFold"] = None):
    """The QKV projection writing Q rows to q_out and K/V as attention tiles (qi_gemm_qkv_tiles):
    x [M][K] rows are tokens row0.. of a sequence of P prefix and T target tokens; w in the tile
    order (pack_qkv_tiles); tables = (cos, sin) rows of those tokens (None: no rotation); k_w the
    K RMSNorm weight (None: no norm)."""
    M, K = x.shape
    assert x.dtype in (torch.bfloat16, torch.float16) and w.dtype == x.dtype and x.stride(1) == 1
    assert w.shape == (384 * n_head, K) and q_out.dtype == x.dtype and q_out.stride(1) == 1 and q_out.shape[0] >= M
    cos, sin = tables if tables is not None else (None, None)
    prep = Q.make_prep(cos, sin, None, k_w, eps)
    fs = None
    if fold is not None:
        fold.check(M, 384 * n_head, K, x.dtype)
        fs = fold.struct()
    Q.check(Q.qi_gemm_qkv_tiles(x, x.stride(0), w, bias, q_out, q_out.stride(0), M, n_head, K, code_of(x), row0, P, T,
                                fs, prep, cache.c if cache is not None else None, layer,
                                target.c if target is not None else None, flags, stream_handle(x.device)),
            "qi_gemm_qkv_tiles")
    return q_out


def unpack_qkv_tiles(w_tiles: torch.Tensor, n_head: int) -> torch.Tensor:
    """The inverse of pack_qkv_tiles: rows back in the Q | K | V order."""
    perm = pack_qkv_tiles(torch.arange(w_tiles.shape[0], device=w_tiles.device, dtype=torch.float32)[:, None],
                          n_head)[:, 0].long()
    w = torch.empty_like(w_tiles)
    w[perm] = w_tiles
    return w


class LayerWeights:
    """Device weights of one layer: fp32 norm weights, bf16 Linear weights [out][in]."""

    def __init__(self, norm1, norm2, q_norm, k_norm, w_qkv, w_out, w_gate, w_up, w_down):
        self.norm1, self.norm2 = norm1.contiguous(), norm2.contiguous()
        self.q_norm, self.k_norm = q_norm.contiguous(), k_norm.contiguous()
        self.w_qkv, self.w_out, self.w_down = w_qkv.contiguous(), w_out.contiguous(), w_down.contiguous()
        self.w_gu = pack_swiglu(w_gate, w_up)
        self.D = self.w_out.shape[0]
        self.F = w_gate.shape[0]

    def as_dtype(self, dtype) -> "LayerWeights":
        """The same layer with its Linear weights converted to `dtype` (fp16 for the fp16 layer
        chain: exact for the bf16 weights of magnitude 2^-17 .. 65504)."""
        W = LayerWeights.__new__(LayerWeights)
        W.norm1, W.norm2, W.q_norm, W.k_norm = self.norm1, self.norm2, self.q_norm, self.k_norm
        W.w_qkv, W.w_out, W.w_down, W.w_gu = (t.to(dtype) for t in (self.w_qkv, self.w_out, self.w_down, self.w_gu))
        W.D, W.F = self.D, self.F
        return W


class SharedWeights:
    """Device weights shared by all layers: timestep MLP, shared modulation, head, img_in."""

    def __init__(self, t_w1, t_w2, w_mod, w_scale, w_head, w_in):
        self.t_w1, self.t_w2, self.w_mod = t_w1.contiguous(), t_w2.contiguous(), w_mod.contiguous()
        self.w_scale, self.w_head, self.w_in = w_scale.contiguous(), w_head.contiguous(), w_in.contiguous()
        self.D = self.w_mod.shape[1]
        self.t_dim = self.t_w1.shape[1]
        self.latent_ch = self.w_head.shape[0]


def gemm(x: torch.Tensor, w: torch.Tensor, out: torch.Tensor, epilogue: int, gate=None, row0: int = 0, P: int = 0,
         tile_n: int = 0, bias=None, flags=None, fold: Optional["NormFold"] = None):
    """y = x W^T with an epilogue; x and w both bf16 (bf16 matrix cores, bf16 16-bit outputs) or
    both fp16 (fp16 matrix cores and outputs).  fold: the norm fold's consuming and/or producing
    side (qi_gemm_norm_fold)."""
    M, K = x.shape
    N = w.shape[0]
    assert x.dtype in (torch.bfloat16, torch.float16) and w.dtype == x.dtype and w.shape[1] == K and x.stride(1) == 1
    assert out.stride(1) == 1 and out.shape[0] == M
    if bias is not None:
        assert bias.dtype == torch.float32 and bias.is_contiguous() and bias.numel() == N
    if fold is None:
        Q.check(Q.qi_gemm(x, x.stride(0), w, bias, out, out.stride(0), M, N, K, code_of(x), epilogue, gate, row0, P,
                          tile_n, flags, stream_handle(x.device)), "qi_gemm")
        return out
    fold.check(M, N, K, x.dtype)
    Q.check(Q.qi_gemm_norm_fold(x, x.stride(0), w, bias, out, out.stride(0), M, N, K, code_of(x), epilogue, gate,
                                row0, P, tile_n, fold.struct(), flags, stream_handle(x.device)), "qi_gemm_norm_fold")
    return out


FOLD_W = 96   # features per partial sum of squares of the norm fold (include/qi.h)


def fold_parts(D: int) -> int:
    """Partial sums of squares per row of D features: ceil(D / 96)."""
    return -(-D // FOLD_W)


class NormFold:
    """Arguments of the norm fold (include/qi.h, qi_norm_fold): the consuming side (sumsq
    [M][ceil(K/96)] of the rows x was formed from, eps, the target rows' bias bias_t) and/or the
    producing side of a gated residual epilogue (xc [M][N] of the activation type, next_w [N],
    next_scale [2][N], sumsq_out [M][ceil(N/96)])."""

    def __init__(self, sumsq=None, eps: float = 1e-6, bias_t=None, xc=None, next_w=None, next_scale=None,
                 sumsq_out=None):
        self.sumsq, self.eps, self.bias_t = sumsq, eps, bias_t
        self.xc, self.next_w, self.next_scale, self.sumsq_out = xc, next_w, next_scale, sumsq_out

    def check(self, M, N, K, dtype):
        if self.sumsq is not None:
            assert self.sumsq.dtype == torch.float32 and self.sumsq.is_contiguous()
            assert self.sumsq.shape[0] >= M and self.sumsq.shape[1] == fold_parts(K)
        if self.bias_t is not None:
            assert self.bias_t.dtype == torch.float32 and self.bias_t.is_contiguous() and self.bias_t.numel() == N
        if self.xc is not None:
            assert self.xc.dtype == dtype and self.xc.stride(1) == 1 and self.xc.shape[0] >= M
            assert self.sumsq_out.dtype == torch.float32 and self.sumsq_out.is_contiguous()
            assert self.sumsq_out.shape[0] >= M and self.sumsq_out.shape[1] == fold_parts(N)

    def struct(self):
        return Q.make_norm_fold(self.sumsq, self.eps, self.bias_t, self.xc,
                                self.xc.stride(0) if self.xc is not None else 0, self.next_w, self.next_scale,
                                self.sumsq_out)


def norm_fold_rows(x: torch.Tensor, xc: torch.Tensor, sumsq: torch.Tensor, w=None, scale=None, row0: int = 0,
                   P: int = 0, flags=None):
    """The norm fold's producing side for fp32 rows: xc = x (1 + w)(1 + scale), sumsq [M][ceil(D/96)]."""
    M, D = x.shape
    assert x.dtype == torch.float32 and x.stride(1) == 1 and xc.stride(1) == 1 and xc.shape[0] >= M
    assert sumsq.dtype == torch.float32 and sumsq.is_contiguous() and sumsq.shape[0] >= M and sumsq.shape[1] == fold_parts(D)
    Q.check(Q.qi_norm_fold_rows(x, x.stride(0), xc, xc.stride(0), sumsq, M, D, w, scale, row0, P, code_of(xc), flags,
                                stream_handle(x.device)), "qi_norm_fold_rows")
    return xc


def linear_multi(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor):
    """y[v] = x[v] W^T for up to 16 fp32 vectors (one pass over W)."""
    nv, I = x.shape
    O_ = w.shape[0]
    assert x.dtype == torch.float32 and x.is_contiguous() and w.is_contiguous() and w.shape[1] == I
    assert y.dtype == torch.float32 and y.is_contiguous() and y.shape == (nv, O_)
    Q.check(Q.qi_linear_multi(x, nv, I, w, code_of(w), O_, y, stream_handle(x.device)), "qi_linear_multi")
    return y


def norm_mod(x: torch.Tensor, out: torch.Tensor, w=None, scale=None, shift=None, row0: int = 0, P: int = 0,
             eps: float = 1e-6, flags=None):
    """ZeroCenterRMSNorm + modulation of fp32 rows into bf16 or fp16 rows (out's type)."""
    M, D = x.shape
    assert x.dtype == torch.float32 and out.dtype in (torch.bfloat16, torch.float16)
    assert x.stride(1) == 1 and out.stride(1) == 1
    Q.check(Q.qi_norm_mod(x, x.stride(0), out, out.stride(0), M, D, w, scale, shift, row0, P, eps, 0, code_of(out),
                          flags, stream_handle(x.device)), "qi_norm_mod")
    return out


def layernorm_mod(x: torch.Tensor, out: torch.Tensor, scale=None, shift=None, row0: int = 0, P: int = 0,
                  eps: float = 1e-6, flags=None):
    """LayerNorm (no affine) + modulation of fp32 rows into bf16 or fp16 rows (out's type)."""
    M, D = x.shape
    assert x.dtype == torch.float32 and out.dtype in (torch.bfloat16, torch.float16)
    assert x.stride(1) == 1 and out.stride(1) == 1
    Q.check(Q.qi_norm_mod(x, x.stride(0), out, out.stride(0), M, D, None, scale, shift, row0, P, eps, 1,
                          code_of(out), flags, stream_handle(x.device)), "qi_norm_mod")
    return out


def cast(x: torch.Tensor, y: torch.Tensor, flags=None):
    """fp32 -> bf16 or fp16 (y's type), nearest even."""
    assert x.dtype == torch.float32 and x.is_contiguous() and y.is_contiguous() and y.numel() >= x.numel()
    Q.check(Q.qi_cast(x, y, x.numel(), code_of(y), flags, stream_handle(x.device)), "qi_cast")
    return y


class TextProjection:
    """The context path of [1B] sections 1-3: ZeroCenterRMSNorm (weights stored as scale - 1),
    Linear, GELU(tanh), Linear; vision-language context rows (fp32 [n][D]) in, the DiT's text
    rows (fp32 [n][D]) out.  Three library calls: the norm, a GEMM with the GELU epilogue, a GEMM
    with the fp32 store.  The normed rows, the GELU output and the weights are fp16 (the weights
    converted once)."""

    def __init__(self, norm_w: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, eps: float = 1e-6):
        self.act = act_dtype = ACT
        self.norm_w, self.eps = norm_w.contiguous(), eps
        self.w1, self.w2 = w1.to(act_dtype).contiguous(), w2.to(act_dtype).contiguous()
        self.D = self.w1.shape[1]
        assert self.w1.shape == (self.D, self.D) and self.w2.shape == (self.D, self.D)
        self.flags = torch.zeros(1, dtype=torch.int32, device=w1.device)

    def __call__(self, x_ctx: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        n, D = x_ctx.shape
        assert D == self.D and x_ctx.dtype == torch.float32
        dev = x_ctx.device
        h = torch.empty((n, D), dtype=self.act, device=dev)
        a = torch.empty((n, D), dtype=self.act, device=dev)
        out = torch.empty((n, D), dtype=torch.float32, device=dev) if out is None else out
        norm_mod(x_ctx, h, self.norm_w, None, None, 0, 0, self.eps, flags=self.flags)
        gemm(h, self.w1, a, Q.QI_EPI_GELU, flags=self.flags)
        gemm(a, self.w2, out, Q.QI_EPI_STORE_F32)
        return out


def linear_small(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor, silu_in: bool, bias=None):
    nv, I = x.shape
    O_ = w.shape[0]
    assert x.is_contiguous() and y.is_contiguous() and w.is_contiguous() and y.shape == (nv, O_)
    if bias is not None:
        assert bias.dtype == torch.float32 and bias.is_contiguous() and bias.numel() == O_
        Q.check(Q.qi_linear_small_bias(x, nv, I, w, bias, O_, silu_in, y, stream_handle(x.device)),
                "qi_linear_small_bias")
        return y
    Q.check(Q.qi_linear_small(x, nv, I, w, O_, silu_in, y, stream_handle(x.device)), "qi_linear_small")
    return y


class DiT:
    """The single-stream denoiser around the attention: per-step conditioning, the layer stack
    (step 1 over the whole sequence filling the prefix caches, then target-only steps), the
    scale-only head and the Euler update.  All arithmetic runs in libqi kernels; this class owns
    buffers and issues the calls in order on the current stream."""

    def __init__(self, layout: Layout, shared: SharedWeights, layers, device="cuda", eps: float = 1e-6,
                 fold: bool = True, kv_tiles: bool = True):
        """The layer chain's 16-bit activations (normed rows, QKV, attention output, SwiGLU output,
        the latents into img_in) and the projection weights are fp16 (the weights converted once
        from the model's bf16).  fold: the layer's two norms folded into its GEMMs (qi_norm_fold)
        instead of launched on their own (two launches more per layer).  kv_tiles: the QKV
        projection writes K (normed, rotated) and V as the attention's fp16 tiles
        (qi_gemm_qkv_tiles, its weights packed once in the tile order), so no K/V preparation
        launch runs and a cached layer is six launches (at the 14,848-token shape the cached
        step takes the same time either way and step 1 is about 0.7 ms shorter: the epilogue's
        norm and rotation, after the MFMA loop of every round of tiles, cost about what the
        preparation launch did)."""
        self.L, self.sw, self.device, self.eps, self.act = layout, shared, device, eps, ACT
        self.fold = fold
        self.kv_tiles = kv_tiles
        act_dtype = ACT
        self.layers = [W.as_dtype(act_dtype) for W in layers]
        if kv_tiles:
            for W in self.layers:
                W.w_qkv = pack_qkv_tiles(W.w_qkv, W.D // 128)
        self.w_in, self.w_head = shared.w_in.to(act_dtype), shared.w_head.to(act_dtype)
        self.D = shared.D
        self.H = self.D // 128
        self.F = self.layers[0].F if self.layers else 0
        self.attn = Attention(layout, self.H, code_of(torch.empty(0, dtype=act_dtype)), device)
        self.cache = KVCache(len(self.layers), self.H, layout.P, self.attn.dtype, device)
        self.kvt = KVTiles(layout.T, self.H, device) if kv_tiles else None
        S, D = layout.S, self.D
        bf, f32 = act_dtype, torch.float32
        self.flags = self.attn.flags                                    # QI_RANGE_* of every call
        self.x = torch.empty((S, D), dtype=f32, device=device)          # residual stream
        self.h = torch.empty((S, D), dtype=bf, device=device)           # normed + modulated
        self.qkv = torch.empty((S, 3 * D), dtype=bf, device=device)
        self.o = torch.empty((S, self.H, 128), dtype=bf, device=device)
        self.a = torch.empty((S, max(self.F, 1)), dtype=bf, device=device)  # SwiGLU output
        self.lat_bf = torch.empty((max(S, 1), shared.latent_ch), dtype=bf, device=device)
        self.vel = torch.empty((layout.T, shared.latent_ch), dtype=f32, device=device)
        self.t = torch.zeros(2, dtype=f32, device=device)
        self.emb = torch.empty((2, shared.t_dim), dtype=f32, device=device)
        self.t_h = torch.empty((2, D), dtype=f32, device=device)
        self.temb = torch.empty((2, D), dtype=f32, device=device)
        self.mods = torch.empty((6, 2, D), dtype=f32, device=device)     # [chunk][prefix | target][D]
        self.hscale = torch.empty((2, D), dtype=f32, device=device)
        # norm fold: partial sums of squares of the rows in h, and the bias tables shift W^T of the
        # QKV and gate|up projections ([prefix (t = 0) | target] of the current conditioning)
        nl = len(self.layers)
        self.sq = torch.empty((S, fold_parts(D)), dtype=f32, device=device)
        self.bq = torch.empty((nl, 2, 3 * D), dtype=f32, device=device)
        self.bgu = torch.empty((nl, 2, 2 * max(self.F, 1)), dtype=f32, device=device)
        self._sched = None     # conditioning of a whole schedule (prepare)
        self._k = None         # the schedule's step whose conditioning is current

    def use_kv_tiles(self, on: bool):
        """Switch the fused QKV path on or off (repacks the QKV weights; the next step prepares
        its schedule's bias tables again, since their columns follow the weight rows)."""
        if on == self.kv_tiles:
            return
        for W in self.layers:
            W.w_qkv = pack_qkv_tiles(W.w_qkv, self.H) if on else unpack_qkv_tiles(W.w_qkv, self.H)
        if on and self.kvt is None:
            self.kvt = KVTiles(self.L.T, self.H, self.device)
        self.kv_tiles = on
        self._sched = None
        self._k = None

    # -- conditioning ------------------------------------------------------------------------
    def condition(self, sigma: float):
        """temb for (t = 0, t = 1000 sigma) and the six shared modulation vectors of each."""
        sw, D = self.sw, self.D
        self.t.copy_(torch.tensor([0.0, 1000.0 * sigma], dtype=torch.float32))
        s = stream_handle(self.device)
        Q.check(Q.qi_timestep_embed(self.t, 2, sw.t_dim, self.emb, s), "qi_timestep_embed")
        linear_small(self.emb, sw.t_w1, self.t_h, False)
        linear_small(self.t_h, sw.t_w2, self.temb, True)
        for c in range(6):
            linear_small(self.temb, sw.w_mod[c * D:(c + 1) * D], self.mods[c], True)
        linear_small(self.temb, sw.w_scale, self.hscale, True)
        self._k = None
        if self.fold:
            for li, W in enumerate(self.layers):
                linear_multi(self.mods[0], W.w_qkv, self.bq[li])
                linear_multi(self.mods[3], W.w_gu, self.bgu[li])

    def prepare(self, sig):
        """The conditioning of every step of the schedule sig (sigmas of n steps + the end point):
        the modulation and head-scale vectors per step, and with the fold the bias tables of every
        layer for all steps in one pass over its weights (entry 0: the prefix rows' t = 0, entry
        1 + k: the target rows at step k).  step() then copies a step's vectors instead of
        recomputing them (and prepares a schedule it has not seen)."""
        n = len(sig) - 1
        assert n >= 1
        D = self.D
        mods = torch.empty((n, 6, 2, D), dtype=torch.float32, device=self.device)
        hsc = torch.empty((n, 2, D), dtype=torch.float32, device=self.device)
        fold = self.fold
        self.fold = False          # the vectors only: the tables below take every step at once
        try:
            for k in range(n):
                self.condition(float(sig[k]))
                mods[k].copy_(self.mods)
                hsc[k].copy_(self.hscale)
        finally:
            self.fold = fold
        tabs = None
        if fold:
            v1 = torch.cat([mods[0, 0, 0:1], mods[:, 0, 1]]).contiguous()   # shift1: t = 0, then each step
            v2 = torch.cat([mods[0, 3, 0:1], mods[:, 3, 1]]).contiguous()   # shift2
            nl = len(self.layers)
            tq = torch.empty((nl, n + 1, 3 * D), dtype=torch.float32, device=self.device)
            tg = torch.empty((nl, n + 1, self.bgu.shape[2]), dtype=torch.float32, device=self.device)
            for li, W in enumerate(self.layers):
                for j in range(0, n + 1, 16):   # (at most 16 vectors per pass over the weights)
                    linear_multi(v1[j:j + 16], W.w_qkv, tq[li, j:j + 16])
                    linear_multi(v2[j:j + 16], W.w_gu, tg[li, j:j + 16])
            tabs = (tq, tg)
        self._sched = (tuple(float(v) for v in sig), mods, hsc, tabs)
        self._k = None

    def _use_step(self, k: int, sig) -> bool:
        """Make step k of a prepared schedule current; False if sig is not the prepared one."""
        if self._sched is None or self._sched[0] != tuple(float(v) for v in sig):
            return False
        _, mods, hsc, _ = self._sched
        self.mods.copy_(mods[k])
        self.hscale.copy_(hsc[k])
        self._k = k
        return True

    def _biases(self, li: int):
        """(prefix, target) bias rows of layer li's QKV and gate|up projections."""
        if self._k is not None:
            tq, tg = self._sched[3]
            return tq[li, 0], tq[li, 1 + self._k], tg[li, 0], tg[li, 1 + self._k]
        return self.bq[li, 0], self.bq[li, 1], self.bgu[li, 0], self.bgu[li, 1]

    # -- one layer ---------------------------------------------------------------------------
    def layer(self, li: int, rows: slice, cached: bool):
        """Layer li over residual rows [rows): the whole sequence at step 1, the target rows after."""
        W, D, F, eps = self.layers[li], self.D, self.F, self.eps
        r0, n, P = rows.start, rows.stop - rows.start, self.L.P
        x, h, qkv, o, a = self.x[rows], self.h[:n], self.qkv[:n], self.o[:n], self.a[:n]
        m, fl = self.mods, self.flags
        if self.fold:
            # h holds x (1 + w)(1 + scale) of the next norm and sq its rows' partial sums of squares:
            # written here for the first layer, else by the previous down-projection's epilogue
            sq = self.sq[:n]
            bq_p, bq_t, bg_p, bg_t = self._biases(li)
            if li == 0:
                norm_fold_rows(x, h, sq, W.norm1, m[1], r0, P, flags=fl)
            qfold, qbias = NormFold(sq, eps, bq_t), bq_p
        else:
            norm_mod(x, h, W.norm1, m[1], m[0], r0, P, eps, flags=fl)
            qfold, qbias = None, None
        if self.kv_tiles:
            # Q rows into qkv[:, :D]; K and V as tiles: prefix tokens into the cache, target tokens
            # into kvt; then the attention on those tiles
            gemm_qkv_tiles(h, W.w_qkv, qkv[:, :D], self.H, r0, P, self.L.T, self.cache, li, self.kvt,
                           self.L.rows(r0, r0 + n), W.k_norm, eps, bias=qbias, flags=fl, fold=qfold)
            qv = qkv[:, :D].view(n, self.H, 128)
            if cached:
                self.attn.cached_tiled(qv, self.cache, li, self.kvt, W.q_norm, eps, out=o)
            else:
                self.attn.full_tiled(qv, self.cache, li, self.kvt, W.q_norm, eps, out=o)
        else:
            gemm(h, W.w_qkv, qkv, Q.QI_EPI_STORE, None, r0, P, bias=qbias, flags=fl, fold=qfold)
            self._attention(li, qkv, o, n, cached)
        self._rest(li, W, x, h, o, a, n, r0, P)

    def _attention(self, li: int, qkv, o, n: int, cached: bool):
        W, D, eps = self.layers[li], self.D, self.eps
        q = qkv[:, :D].view(n, self.H, 128)
        k = qkv[:, D:2 * D].view(n, self.H, 128)
        v = qkv[:, 2 * D:].view(n, self.H, 128)
        if cached:
            self.attn.cached(q, k, v, self.cache, li, W.q_norm, W.k_norm, eps, out=o)
        else:
            self.attn.full(q, k, v, W.q_norm, W.k_norm, eps, cache=self.cache, layer=li, out=o)

    def _rest(self, li: int, W, x, h, o, a, n: int, r0: int, P: int):
        """The out-projection, the FFN and their residual updates."""
        D, eps, m, fl = self.D, self.eps, self.mods, self.flags
        if self.fold:
            sq = self.sq[:n]
            _, _, bg_p, bg_t = self._biases(li)
            gemm(o.view(n, D), W.w_out, x, Q.QI_EPI_GATED_RESIDUAL, m[2], r0, P, flags=fl,
                 fold=NormFold(xc=h, next_w=W.norm2, next_scale=m[4], sumsq_out=sq))
            gemm(h, W.w_gu, a, Q.QI_EPI_SWIGLU, None, r0, P, bias=bg_p, flags=fl, fold=NormFold(sq, eps, bg_t))
            nxt = self.layers[li + 1] if li + 1 < len(self.layers) else None
            gemm(a, W.w_down, x, Q.QI_EPI_GATED_RESIDUAL, m[5], r0, P, flags=fl,
                 fold=NormFold(xc=h, next_w=nxt.norm1, next_scale=m[1], sumsq_out=sq) if nxt else None)
            return
        gemm(o.view(n, D), W.w_out, x, Q.QI_EPI_GATED_RESIDUAL, m[2], r0, P)
        norm_mod(x, h, W.norm2, m[4], m[3], r0, P, eps, flags=fl)
        gemm(h, W.w_gu, a, Q.QI_EPI_SWIGLU, flags=fl)
        gemm(a, W.w_down, x, Q.QI_EPI_GATED_RESIDUAL, m[5], r0, P)

    # -- inputs, head, Euler -----------------------------------------------------------------
    def embed(self, lat: torch.Tensor, out: torch.Tensor):
        """img_in: fp32 latents [n][64] -> the activation type -> fp32 tokens [n][D]."""
        n = lat.shape[0]
        cast(lat, self.lat_bf, self.flags)
        gemm(self.lat_bf[:n], self.w_in, out, Q.QI_EPI_STORE_F32)

    def set_prefix(self, x_text: torch.Tensor, lat_ref: Optional[torch.Tensor]):
        """Fill the prefix rows of the residual stream in segment order: text rows copied from
        x_text (fp32 [n_text][D]), reference-image rows written by img_in from lat_ref."""
        it = ir = row = 0
        for g in self.L.segments[:-1]:
            n = g.n_tokens
            if g.kind == 1:
                self.embed(lat_ref[ir:ir + n], self.x[row:row + n])
                ir += n
            else:
                self.x[row:row + n].copy_(x_text[it:it + n])
                it += n
            row += n

    def head(self, lat: torch.Tensor, sigma_k: float, sigma_k1: float):
        """Scale-only final norm, the velocity projection, and the Euler update of lat (in place)."""
        P, T = self.L.P, self.L.T
        h = self.h[:T]
        norm_mod(self.x[P:], h, None, self.hscale, None, P, P, self.eps, flags=self.flags)
        gemm(h, self.w_head, self.vel, Q.QI_EPI_STORE_F32)
        euler_step(lat, self.vel, sigma_k, sigma_k1)

    def check_range(self):
        """Raise RangeError if any call since the last check met a value that fp16 cannot hold."""
        self.attn.check_range()

    def step(self, k: int, lat: torch.Tensor, sig, x_text=None, lat_ref=None):
        """Euler step k (0-based) of the loop: step 0 runs the whole sequence and fills the caches."""
        S, P = self.L.S, self.L.P
        if not self._use_step(k, sig):   # a schedule not prepared yet: prepare it once
            self.prepare(sig)
            self._use_step(k, sig)
        self.embed(lat, self.x[P:])
        if k == 0:
            self.set_prefix(x_text, lat_ref)
            for li in range(len(self.layers)):
                self.layer(li, slice(0, S), False)
        else:
            for li in range(len(self.layers)):
                self.layer(li, slice(P, S), True)
        self.head(lat, float(sig[k]), float(sig[k + 1]))


# ------------------------------------------------------------------------------------------------
# the v1 / Edit dual-stream block around the unmasked joint attention
# ------------------------------------------------------------------------------------------------

V1_LINEARS = ("img_mod", "txt_mod", "img_qkv", "txt_qkv", "img_out", "txt_out", "img_fc1", "img_fc2", "txt_fc1",
              "txt_fc2")


class V1BlockWeights:
    """Device weights of one v1 dual-stream block: bf16 Linear weights [out][in] with fp32 biases
    (`<name>_w`, `<name>_b` for each name in V1_LINEARS: modulation [6D][D], QKV [3D][D] in
    q | k | v order, out [D][D], MLP [F][D] and [D][F]) and fp32 QK-RMSNorm weights [128]
    (`norm_q`, `norm_k` of the image stream, `norm_added_q`, `norm_added_k` of the text)."""

    def __init__(self, tensors: dict):
        self.t = {k: v.contiguous() for k, v in tensors.items()}
        self.D = self.t["img_out_w"].shape[0]
        self.F = self.t["img_fc1_w"].shape[0]
        for name in V1_LINEARS:
            assert self.t[name + "_w"].dtype == torch.bfloat16 and self.t[name + "_b"].dtype == torch.float32

    def __getitem__(self, key):
        return self.t[key]


class V1Block:
    """One dual-stream block of the v1 / Edit model ("QwenImageTransformer2DModel source reading
    (Qwen-Image-Edit)", section 5.2 for the block, section 6 for the attention processor) as a
    sequence of library calls.  The layout must be the unmasked one (QI_ATTN_FULL) with the text
    first, then the image rows (the noisy target, then the references).  Per stream: six
    conditioning linears (one per modulation chunk, SiLU then Linear with bias), LayerNorm +
    modulation, the QKV GEMM with bias written straight into the joint [text | image] QKV buffer,
    and the stream's QK-RMSNorm in place; then one joint attention over the layout (RoPE applied
    in it); per stream again the out-projection GEMM with bias adding gate1 * y into the residual,
    LayerNorm + modulation, the MLP (GEMM with bias and GELU(tanh), GEMM with bias adding
    gate2 * y)."""

    def __init__(self, W: V1BlockWeights, layout: Layout, n_head: int, device="cuda", eps: float = 1e-6,
                 two_streams: bool = True):
        """The activations and the GEMM weights (converted once) are fp16.  two_streams: the text
        stream's calls on a second stream beside the image stream's (else all on the calling one)."""
        assert layout.attention == Q.QI_ATTN_FULL
        assert W.D == n_head * 128
        act_dtype = ACT
        self.W, self.L, self.H, self.eps, self.device, self.act = W, layout, n_head, eps, device, act_dtype
        self.att = Attention(layout, n_head, code_of(torch.empty(0, dtype=act_dtype)), device)
        self.w = {name: W[name + "_w"].to(act_dtype) for name in V1_LINEARS if not name.endswith("_mod")}
        # the text stream's calls run on a second stream (default priority) beside the image
        # stream's: its 512-row GEMMs fill a fraction of the chip, and the image GEMMs fill the rest
        self.side = torch.cuda.Stream(device=device) if two_streams else None

    def __call__(self, x_txt: torch.Tensor, x_img: torch.Tensor, cond: torch.Tensor, n_noise: Optional[int] = None):
        """x_txt fp32 [Lt][D] and x_img fp32 [Li][D] (updated in place and returned); cond fp32
        [2][D]: row 0 the current t's conditioning, row 1 the t = 0 one, which image rows
        n_noise.. take when n_noise is given (the per-token modulation; the text and, without
        n_noise, every image row take row 0)."""
        W, D, H, eps, dev = self.W, self.W.D, self.H, self.eps, self.device
        Lt, Li = x_txt.shape[0], x_img.shape[0]
        S = Lt + Li
        assert S == self.L.S and x_txt.shape[1] == D and x_img.shape[1] == D
        assert cond.shape == (2, D) and cond.dtype == torch.float32 and cond.is_contiguous()
        streams = (("txt", x_txt, 0, Lt, Lt, "norm_added_q", "norm_added_k"),
                   ("img", x_img, Lt, Li, Li if n_noise is None else n_noise, "norm_q", "norm_k"))
        # every buffer is allocated on the calling stream before the two streams fork
        mods = {name: torch.empty((6, 2, D), dtype=torch.float32, device=dev) for name, *_ in streams}
        h = torch.empty((S, D), dtype=self.act, device=dev)
        qkv = torch.empty((S, 3, H, 128), dtype=self.act, device=dev)
        o = torch.empty((S, H, 128), dtype=self.act, device=dev)
        acts = {name: torch.empty((n, W.F), dtype=self.act, device=dev) for name, _, _, n, *_ in streams}
        fl, w = self.att.flags, self.w
        main = torch.cuda.current_stream(dev)
        side = self.side if self.side is not None else main

        def pre(name, x, r0, n, P, nq, nk):
            # modulation (chunk i of the stream for both conditioning rows, [2][D] each), LayerNorm
            # + modulation, the QKV projection into the joint buffer, the stream's QK-RMSNorm
            m = mods[name]
            for i in range(6):
                linear_small(cond, W[name + "_mod_w"][i * D:(i + 1) * D], m[i], True,
                             W[name + "_mod_b"][i * D:(i + 1) * D])
            layernorm_mod(x, h[r0:r0 + n], m[1], m[0], 0, P, eps, flags=fl)
            gemm(h[r0:r0 + n], w[name + "_qkv"], qkv[r0:r0 + n].view(n, 3 * D), Q.QI_EPI_STORE,
                 bias=W[name + "_qkv_b"], flags=fl)
            rope3d_apply(qkv[r0:r0 + n, 0], None, None, W[nq], eps)
            rope3d_apply(qkv[r0:r0 + n, 1], None, None, W[nk], eps)

        def post(name, x, r0, n, P, nq, nk):
            # out-projection into the residual, LayerNorm + modulation, the GELU MLP into the residual
            m = mods[name]
            gemm(o[r0:r0 + n].view(n, D), w[name + "_out"], x, Q.QI_EPI_GATED_RESIDUAL_LINEAR, m[2], 0, P,
                 bias=W[name + "_out_b"])
            layernorm_mod(x, h[r0:r0 + n], m[4], m[3], 0, P, eps, flags=fl)
            a = acts[name]
            gemm(h[r0:r0 + n], w[name + "_fc1"], a, Q.QI_EPI_GELU, bias=W[name + "_fc1_b"], flags=fl)
            gemm(a, w[name + "_fc2"], x, Q.QI_EPI_GATED_RESIDUAL_LINEAR, m[5], 0, P, bias=W[name + "_fc2_b"])

        # the text stream on the side stream, the image stream on the calling one; they join for the
        # joint attention and at the end (the streams touch disjoint rows of h, qkv and o)
        side.wait_stream(main)
        with torch.cuda.stream(side):
            pre(*streams[0])
        pre(*streams[1])
        main.wait_stream(side)
        self.att.full(qkv[:, 0], qkv[:, 1], qkv[:, 2], out=o)
        side.wait_stream(main)
        with torch.cuda.stream(side):
            post(*streams[0])
        post(*streams[1])
        main.wait_stream(side)
        return x_txt, x_img


class V1Head:
    """The v1 / Edit model's exit ("QwenImageTransformer2DModel source reading (Qwen-Image-Edit)",
    section 5.3) on the image stream: norm_out (SiLU(temb) through one Linear with bias giving
    scale then shift; LayerNorm without affine, times (1 + scale), plus shift) and proj_out
    (Linear D -> 64 with bias).  Two conditioning linears, the norm into fp16 rows and one fp16
    GEMM with the bias and the fp32 store."""

    def __init__(self, norm_out_w: torch.Tensor, norm_out_b: torch.Tensor, proj_out_w: torch.Tensor,
                 proj_out_b: torch.Tensor, eps: float = 1e-6):
        D = proj_out_w.shape[1]
        assert norm_out_w.shape == (2 * D, D) and norm_out_w.dtype == torch.bfloat16
        self.D, self.eps = D, eps
        self.w_scale, self.w_shift = norm_out_w[:D].contiguous(), norm_out_w[D:].contiguous()
        self.b_scale, self.b_shift = norm_out_b[:D].contiguous(), norm_out_b[D:].contiguous()
        self.w_proj = proj_out_w.to(ACT).contiguous()
        self.b_proj = proj_out_b.contiguous()
        self.flags = torch.zeros(1, dtype=torch.int32, device=proj_out_w.device)

    def __call__(self, x_img: torch.Tensor, temb: torch.Tensor) -> torch.Tensor:
        """x_img fp32 [Li][D], temb fp32 [D] -> fp32 [Li][64]."""
        Li, D = x_img.shape
        dev = x_img.device
        cond = temb.reshape(1, D).expand(2, D).contiguous()      # the same vector for both row sets
        scale = torch.empty((2, D), dtype=torch.float32, device=dev)
        shift = torch.empty((2, D), dtype=torch.float32, device=dev)
        linear_small(cond, self.w_scale, scale, True, self.b_scale)
        linear_small(cond, self.w_shift, shift, True, self.b_shift)
        h = torch.empty((Li, D), dtype=ACT, device=dev)
        layernorm_mod(x_img, h, scale, shift, 0, 0, self.eps, flags=self.flags)
        out = torch.empty((Li, self.w_proj.shape[0]), dtype=torch.float32, device=dev)
        gemm(h, self.w_proj, out, Q.QI_EPI_STORE_F32, bias=self.b_proj)
        return out
