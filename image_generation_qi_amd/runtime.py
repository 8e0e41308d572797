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
    tiles of 64 keys: K as [16 dim chunks][64 key slots][8 dims] with the slots of every 16
    keys in the order 0-3, 8-11, 4-7, 12-15, V as [8 key chunks][128 dims][8 keys]; k_rows and
    v_rows return plain [n_head][R][128] rows."""

    # key held by each of the 64 slots of an fp16 K tile (the permutation is its own inverse)
    SLOT_KEY = [(p & ~15) | ((2 if (p >> 2) & 3 == 1 else 1 if (p >> 2) & 3 == 2 else (p >> 2) & 3) << 2) | (p & 3)
                for p in range(64)]

    def __init__(self, n_layers: int, n_head: int, p_cap: int, io_dtype: int = Q.QI_BF16, device="cuda"):
        self.dtype = Q.QI_F16 if io_dtype == Q.QI_BF16 else Q.QI_F32
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
        t = k.reshape(H, self.rows // 64, 16, 64, 8).permute(0, 1, 3, 2, 4).reshape(H, self.rows // 64, 64, 128)
        idx = torch.tensor(self.SLOT_KEY, device=k.device)
        return t[:, :, idx].reshape(H, self.rows, 128)

    def v_rows(self, layer: int) -> torch.Tensor:
        """V of one layer as [n_head][R][128] rows (a copy for fp16 caches)."""
        v = self.v[layer]
        if self.dtype != Q.QI_F16:
            return v
        H = v.shape[0]
        return v.reshape(H, self.rows // 64, 8, 128, 8).permute(0, 1, 2, 4, 3).reshape(H, self.rows, 128)


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
             scale: float = 0.0, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Step 1 over the layout; lse (optional fp32 [H][S]) receives each row's log-sum-exp."""
        if self.ws_full is None:
            self.ws_full = _ws(self.ws_full_bytes, self.device)
        o = out if out is not None else torch.empty((self.L.S, self.H, 128), dtype=q.dtype, device=self.device)
        if lse is not None:
            assert lse.dtype == torch.float32 and lse.is_contiguous() and lse.shape == (self.H, self.L.S)
        io = Q.make_qkv(q, k, v, o, self.dtype, self.L.S, self.H, self._stride(q), lse)
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
               scale: float = 0.0, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None) -> torch.Tensor:
        """A cached target step; lse (optional fp32 [H][T]) receives each row's log-sum-exp."""
        if self.ws_cached is None:
            self.ws_cached = _ws(self.ws_cached_bytes, self.device)
        T = q_t.shape[0]
        o = out if out is not None else torch.empty((T, self.H, 128), dtype=q_t.dtype, device=self.device)
        if lse is not None:
            assert lse.dtype == torch.float32 and lse.is_contiguous() and lse.shape == (self.H, T)
        io = Q.make_qkv(q_t, k_t, v_t, o, self.dtype, T, self.H, self._stride(q_t), lse)
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


# ------------------------------------------------------------------------------------------------
# one single-stream DiT layer and the sampling loop around the attention
# ------------------------------------------------------------------------------------------------

def pack_swiglu(w_gate: torch.Tensor, w_up: torch.Tensor) -> torch.Tensor:
    """Interleave gate and up weights [F][D] into the [2F][D] layout the SwiGLU epilogue reads:
    blocks of 64 rows, 32 gate rows then the 32 up rows of the same features."""
    F, D = w_gate.shape
    assert w_up.shape == (F, D) and F % 32 == 0
    return torch.stack([w_gate.reshape(F // 32, 32, D), w_up.reshape(F // 32, 32, D)], dim=1).reshape(2 * F, D).contiguous()


class LayerWeights:
    """Device weights of one layer: fp32 norm weights, bf16 Linear weights [out][in]."""

    def __init__(self, norm1, norm2, q_norm, k_norm, w_qkv, w_out, w_gate, w_up, w_down):
        self.norm1, self.norm2 = norm1.contiguous(), norm2.contiguous()
        self.q_norm, self.k_norm = q_norm.contiguous(), k_norm.contiguous()
        self.w_qkv, self.w_out, self.w_down = w_qkv.contiguous(), w_out.contiguous(), w_down.contiguous()
        self.w_gu = pack_swiglu(w_gate, w_up)
        self.D = self.w_out.shape[0]
        self.F = w_gate.shape[0]


class SharedWeights:
    """Device weights shared by all layers: timestep MLP, shared modulation, head, img_in."""

    def __init__(self, t_w1, t_w2, w_mod, w_scale, w_head, w_in):
        self.t_w1, self.t_w2, self.w_mod = t_w1.contiguous(), t_w2.contiguous(), w_mod.contiguous()
        self.w_scale, self.w_head, self.w_in = w_scale.contiguous(), w_head.contiguous(), w_in.contiguous()
        self.D = self.w_mod.shape[1]
        self.t_dim = self.t_w1.shape[1]
        self.latent_ch = self.w_head.shape[0]


def gemm(x: torch.Tensor, w: torch.Tensor, out: torch.Tensor, epilogue: int, gate=None, row0: int = 0, P: int = 0,
         tile_n: int = 0, bias=None):
    M, K = x.shape
    N = w.shape[0]
    assert x.dtype == torch.bfloat16 and w.dtype == torch.bfloat16 and w.shape[1] == K and x.stride(1) == 1
    assert out.stride(1) == 1 and out.shape[0] == M
    if bias is not None:
        assert tile_n == 0 and bias.dtype == torch.float32 and bias.is_contiguous() and bias.numel() == N
        Q.check(Q.qi_gemm_bf16_bias(x, x.stride(0), w, bias, out, out.stride(0), M, N, K, epilogue, gate, row0, P,
                                    stream_handle(x.device)), "qi_gemm_bf16_bias")
        return out
    Q.check(Q.qi_gemm_bf16_ex(x, x.stride(0), w, out, out.stride(0), M, N, K, epilogue, gate, row0, P, tile_n,
                              stream_handle(x.device)), "qi_gemm_bf16_ex")
    return out


def norm_mod(x: torch.Tensor, out: torch.Tensor, w=None, scale=None, shift=None, row0: int = 0, P: int = 0,
             eps: float = 1e-6):
    M, D = x.shape
    assert x.dtype == torch.float32 and out.dtype == torch.bfloat16 and x.stride(1) == 1 and out.stride(1) == 1
    Q.check(Q.qi_zc_rmsnorm_mod(x, x.stride(0), out, out.stride(0), M, D, w, scale, shift, row0, P, eps,
                                stream_handle(x.device)), "qi_zc_rmsnorm_mod")
    return out


def layernorm_mod(x: torch.Tensor, out: torch.Tensor, scale=None, shift=None, row0: int = 0, P: int = 0,
                  eps: float = 1e-6):
    M, D = x.shape
    assert x.dtype == torch.float32 and out.dtype == torch.bfloat16 and x.stride(1) == 1 and out.stride(1) == 1
    Q.check(Q.qi_layernorm_mod(x, x.stride(0), out, out.stride(0), M, D, scale, shift, row0, P, eps,
                               stream_handle(x.device)), "qi_layernorm_mod")
    return out


class TextProjection:
    """The context path of [1B] sections 1-3: ZeroCenterRMSNorm (weights stored as scale - 1),
    Linear, GELU(tanh), Linear; vision-language context rows (fp32 [n][D]) in, the DiT's text
    rows (fp32 [n][D]) out.  Three library calls: the norm, a GEMM with the GELU epilogue, a GEMM
    with the fp32 store."""

    def __init__(self, norm_w: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, eps: float = 1e-6):
        self.norm_w, self.w1, self.w2, self.eps = norm_w.contiguous(), w1.contiguous(), w2.contiguous(), eps
        self.D = self.w1.shape[1]
        assert self.w1.shape == (self.D, self.D) and self.w2.shape == (self.D, self.D)

    def __call__(self, x_ctx: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        n, D = x_ctx.shape
        assert D == self.D and x_ctx.dtype == torch.float32
        dev = x_ctx.device
        h = torch.empty((n, D), dtype=torch.bfloat16, device=dev)
        a = torch.empty((n, D), dtype=torch.bfloat16, device=dev)
        out = torch.empty((n, D), dtype=torch.float32, device=dev) if out is None else out
        norm_mod(x_ctx, h, self.norm_w, None, None, 0, 0, self.eps)
        gemm(h, self.w1, a, Q.QI_EPI_GELU)
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

    def __init__(self, layout: Layout, shared: SharedWeights, layers, device="cuda", eps: float = 1e-6):
        self.L, self.sw, self.layers, self.device, self.eps = layout, shared, list(layers), device, eps
        self.D = shared.D
        self.H = self.D // 128
        self.F = self.layers[0].F if self.layers else 0
        self.attn = Attention(layout, self.H, Q.QI_BF16, device)
        self.cache = KVCache(len(self.layers), self.H, layout.P, Q.QI_BF16, device)
        S, D = layout.S, self.D
        bf, f32 = torch.bfloat16, torch.float32
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

    # -- one layer ---------------------------------------------------------------------------
    def layer(self, li: int, rows: slice, cached: bool):
        """Layer li over residual rows [rows): the whole sequence at step 1, the target rows after."""
        W, D, F, eps = self.layers[li], self.D, self.F, self.eps
        r0, n, P = rows.start, rows.stop - rows.start, self.L.P
        x, h, qkv, o, a = self.x[rows], self.h[:n], self.qkv[:n], self.o[:n], self.a[:n]
        m = self.mods
        norm_mod(x, h, W.norm1, m[1], m[0], r0, P, eps)
        gemm(h, W.w_qkv, qkv, Q.QI_EPI_STORE)
        q = qkv[:, :D].view(n, self.H, 128)
        k = qkv[:, D:2 * D].view(n, self.H, 128)
        v = qkv[:, 2 * D:].view(n, self.H, 128)
        if cached:
            self.attn.cached(q, k, v, self.cache, li, W.q_norm, W.k_norm, eps, out=o)
        else:
            self.attn.full(q, k, v, W.q_norm, W.k_norm, eps, cache=self.cache, layer=li, out=o)
        gemm(o.view(n, D), W.w_out, x, Q.QI_EPI_GATED_RESIDUAL, m[2], r0, P)
        norm_mod(x, h, W.norm2, m[4], m[3], r0, P, eps)
        gemm(h, W.w_gu, a, Q.QI_EPI_SWIGLU)
        gemm(a, W.w_down, x, Q.QI_EPI_GATED_RESIDUAL, m[5], r0, P)

    # -- inputs, head, Euler -----------------------------------------------------------------
    def embed(self, lat: torch.Tensor, out: torch.Tensor):
        """img_in: fp32 latents [n][64] -> bf16 -> fp32 tokens [n][D]."""
        n = lat.shape[0]
        Q.check(Q.qi_cast_bf16(lat, self.lat_bf, lat.numel(), stream_handle(self.device)), "qi_cast_bf16")
        gemm(self.lat_bf[:n], self.sw.w_in, out, Q.QI_EPI_STORE_F32)

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
        norm_mod(self.x[P:], h, None, self.hscale, None, P, P, self.eps)
        gemm(h, self.sw.w_head, self.vel, Q.QI_EPI_STORE_F32)
        euler_step(lat, self.vel, sigma_k, sigma_k1)

    def step(self, k: int, lat: torch.Tensor, sig, x_text=None, lat_ref=None):
        """Euler step k (0-based) of the loop: step 0 runs the whole sequence and fills the caches."""
        S, P = self.L.S, self.L.P
        self.condition(float(sig[k]))
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

    def __init__(self, W: V1BlockWeights, layout: Layout, n_head: int, device="cuda", eps: float = 1e-6):
        assert layout.attention == Q.QI_ATTN_FULL
        assert W.D == n_head * 128
        self.W, self.L, self.H, self.eps, self.device = W, layout, n_head, eps, device
        self.att = Attention(layout, n_head, Q.QI_BF16, device)

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
        # modulation: chunk i of a stream for both conditioning rows, [2][D] each
        mods = {}
        for name, *_ in streams:
            m = torch.empty((6, 2, D), dtype=torch.float32, device=dev)
            for i in range(6):
                linear_small(cond, W[name + "_mod_w"][i * D:(i + 1) * D], m[i], True,
                             W[name + "_mod_b"][i * D:(i + 1) * D])
            mods[name] = m
        h = torch.empty((S, D), dtype=torch.bfloat16, device=dev)
        qkv = torch.empty((S, 3, H, 128), dtype=torch.bfloat16, device=dev)
        for name, x, r0, n, P, nq, nk in streams:
            m = mods[name]
            layernorm_mod(x, h[r0:r0 + n], m[1], m[0], 0, P, eps)
            gemm(h[r0:r0 + n], W[name + "_qkv_w"], qkv[r0:r0 + n].view(n, 3 * D), Q.QI_EPI_STORE,
                 bias=W[name + "_qkv_b"])
            rope3d_apply(qkv[r0:r0 + n, 0], None, None, W[nq], eps)
            rope3d_apply(qkv[r0:r0 + n, 1], None, None, W[nk], eps)
        o = self.att.full(qkv[:, 0], qkv[:, 1], qkv[:, 2])
        a = torch.empty((max(Lt, Li), W.F), dtype=torch.bfloat16, device=dev)
        for name, x, r0, n, P, nq, nk in streams:
            m = mods[name]
            gemm(o[r0:r0 + n].view(n, D), W[name + "_out_w"], x, Q.QI_EPI_GATED_RESIDUAL_LINEAR, m[2], 0, P,
                 bias=W[name + "_out_b"])
            layernorm_mod(x, h[r0:r0 + n], m[4], m[3], 0, P, eps)
            gemm(h[r0:r0 + n], W[name + "_fc1_w"], a[:n], Q.QI_EPI_GELU, bias=W[name + "_fc1_b"])
            gemm(a[:n], W[name + "_fc2_w"], x, Q.QI_EPI_GATED_RESIDUAL_LINEAR, m[5], 0, P, bias=W[name + "_fc2_b"])
        return x_txt, x_img
