"""fp64 CPU oracle for block-causal 3D-RoPE joint attention with a prefix KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library (no kernels,
headers, tables or helpers): every step below is the plain definition, written
out from the pages, in NumPy float64, slow and obvious on purpose.

Sources (cited by page title and section):
  [OV]   "Qwen-Image-2.1: how an image is made from noise" course overview
         (OpenArchLab), lesson list and block cards 1A, 2A, 3A, 3B, 3C, 4A, 5A, 6A, 6B.
  [1B]   "1B - Qwen3-VL Context & Zero-Center RMSNorm" (OpenArchLab), sections 1-4
         (ZeroCenterRMSNorm; the context TextProjection Linear -> GELU(tanh) -> Linear).
  [3A]   "3A - 3D Axial RoPE (16, 56, 56) & Zero-Centered Grid" (OpenArchLab), sections 1-4.
  [EDIT] "QwenImageTransformer2DModel source reading (Qwen-Image-Edit)", sections
         5.1 (timestep embedding), 5.2 (modulation), 6 (attention processor),
         7.1-7.3 (three-axis RoPE), 8.2 (shape walk-through).

Readings taken where the pages are silent or disagree are listed in the
repository's design notes; each is also stated at the function that uses it.
Parity status: every function here is pinned by the CPU tests in
tests/test_oracle_pins.py (closed forms, worked values from the pages,
invariants and brute force on tiny inputs).
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

SEG_TEXT, SEG_IMAGE, SEG_TEXT_BIDIR = 0, 1, 2
HEAD_DIM = 128
BANDS = (16, 56, 56)
THETA = 10000.0


# ------------------------------------------------------------------------------------------------
# sequence layout
# ------------------------------------------------------------------------------------------------

def segment_ids(segments) -> np.ndarray:
    """Segment index of every token of the joint sequence [text | refs | target]
    ([OV] block card 2A: one sequence, target appended last, each token labelled)."""
    return np.concatenate([np.full(s.n_tokens, i, dtype=np.int64) for i, s in enumerate(segments)])


def split_counts(segments) -> Tuple[int, int, int]:
    """(S, P, T): all tokens, prefix tokens (text + references), target tokens (the last segment)."""
    S = sum(s.n_tokens for s in segments)
    T = segments[-1].n_tokens
    return S, S - T, T


# ------------------------------------------------------------------------------------------------
# 3D axial positions and rotation tables
# ------------------------------------------------------------------------------------------------

def text_start(segments, text_pos0: Optional[int] = None) -> int:
    """First text position.  [3A] section 1 only says text steps +1 on all axes; the start
    follows [EDIT] section 7.2 with centred grids: text continues after max over images of
    max(H//2, W//2).  An explicit override wins."""
    if text_pos0 is not None and text_pos0 >= 0:
        return int(text_pos0)
    best = 0
    for s in segments:
        if s.kind == SEG_IMAGE:
            best = max(best, s.grid_h // 2, s.grid_w // 2)
    return best


def positions(segments, text_pos0: Optional[int] = None) -> np.ndarray:
    """Per-token (frame, height, width) integer coordinates, shape [S, 3].

    Text ([3A] section 1): every text token advances all three axes by one.
    Image ([3A] section 1; [EDIT] section 7.3): frame fixed for the whole image,
    height runs -(H - H//2) .. H//2 - 1 and width -(W - W//2) .. W//2 - 1,
    row-major (height outer, width inner)."""
    p0 = text_start(segments, text_pos0)
    out: List[Tuple[int, int, int]] = []
    n_text = 0
    for s in segments:
        if s.kind in (SEG_TEXT, SEG_TEXT_BIDIR):
            for _ in range(s.n_tokens):
                p = p0 + n_text
                out.append((p, p, p))
                n_text += 1
        elif s.kind == SEG_IMAGE:
            H, W = s.grid_h, s.grid_w
            assert H * W == s.n_tokens
            for y in range(H):
                for x in range(W):
                    out.append((s.frame, y - (H - H // 2), x - (W - W // 2)))
        else:
            raise ValueError(s.kind)
    return np.array(out, dtype=np.int64).reshape(-1, 3)


def inv_freq(bands: Sequence[int] = BANDS, theta: float = THETA) -> Tuple[np.ndarray, np.ndarray]:
    """Rotation frequency of each of the 64 complex pairs and the axis it belongs to.

    Band a of width d_a owns d_a/2 pairs with frequency theta^(-2i/d_a), i < d_a/2
    ([EDIT] section 7.1, one frequency table per axis; [3A] section 1 band split
    16 | 56 | 56 for frame | height | width).  Returns (freq[64] fp64, axis[64] int)."""
    freqs, axes = [], []
    for a, d in enumerate(bands):
        assert d % 2 == 0
        for i in range(d // 2):
            freqs.append(1.0 / math.pow(theta, (2 * i) / d))
            axes.append(a)
    return np.array(freqs, dtype=np.float64), np.array(axes, dtype=np.int64)


def angles(pos: np.ndarray, bands=BANDS, theta=THETA) -> np.ndarray:
    """phi[s, k] = pos[s, axis(k)] * freq[k], fp64, shape [S, 64]."""
    f, ax = inv_freq(bands, theta)
    out = np.empty((pos.shape[0], f.shape[0]), dtype=np.float64)
    for k in range(f.shape[0]):
        out[:, k] = pos[:, ax[k]].astype(np.float64) * f[k]
    return out


def rope_tables(pos: np.ndarray, bands=BANDS, theta=THETA) -> Tuple[np.ndarray, np.ndarray]:
    """cos(phi), sin(phi) in fp64, shape [S, 64]."""
    phi = angles(pos, bands, theta)
    return np.cos(phi), np.sin(phi)


def rope_tables_f32(pos: np.ndarray, bands=BANDS, theta=THETA) -> Tuple[np.ndarray, np.ndarray]:
    """The same tables computed one value at a time with the C library's double cos/sin and
    rounded once to fp32 (the stored form of the device tables)."""
    f, ax = inv_freq(bands, theta)
    c = np.empty((pos.shape[0], f.shape[0]), dtype=np.float32)
    s = np.empty_like(c)
    cache = {}
    for r in range(pos.shape[0]):
        for k in range(f.shape[0]):
            key = (int(pos[r, ax[k]]), k)
            v = cache.get(key)
            if v is None:
                a = float(key[0]) * float(f[k])
                v = (np.float32(math.cos(a)), np.float32(math.sin(a)))
                cache[key] = v
            c[r, k], s[r, k] = v
    return c, s


def rotate(x: np.ndarray, cos_t: np.ndarray, sin_t: np.ndarray) -> np.ndarray:
    """Rotate adjacent pairs (x[2k], x[2k+1]) by phi[k]: the pair read as a complex number
    times e^{i phi} ([3A] section 1: RoPE rotates pairs of Q/K dims by an angle proportional
    to position; [EDIT] section 7.1: the tables hold the complex factors, 64 per token).
    x: [S, ..., 128]; cos_t/sin_t: [S, 64]."""
    x = np.asarray(x, dtype=np.float64)
    extra = (slice(None),) + (None,) * (x.ndim - 2)
    c = cos_t[extra]
    s = sin_t[extra]
    a = x[..., 0::2]
    b = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


# ------------------------------------------------------------------------------------------------
# norms
# ------------------------------------------------------------------------------------------------

def rms_norm(x: np.ndarray, w: Optional[np.ndarray], eps: float = 1e-6) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * w (the per-head QK-norm of
    [EDIT] section 6; [OV] card 4A names QK-RMSNorm)."""
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    y = x * r
    return y if w is None else y * w


def zero_center_rms_norm(x: np.ndarray, w: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """ZeroCenterRMSNorm: x * rrms * (w + 1), weights stored as scale - 1 ([1B] sections 1-3)."""
    x = np.asarray(x, dtype=np.float64)
    rrms = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * rrms * (np.asarray(w, dtype=np.float64) + 1.0)


# ------------------------------------------------------------------------------------------------
# block-causal mask
# ------------------------------------------------------------------------------------------------

def mask_dense(segments, full: bool = False) -> np.ndarray:
    """visible[q, k] for the Block-Causal mask ([OV] card 3C and lesson 3C: text reads only
    what precedes it, tokens of one image see each other both ways; [OV] learning goals: the
    prefix never sees the target).  Reading: a query sees every key of earlier segments, all
    keys of its own segment if that segment is an image (or bidirectional text), keys k <= q
    of its own text segment, and nothing of later segments.  full=True: the joint attention of
    the v1 / Edit model ([EDIT] section 6), every token sees every token."""
    sid = segment_ids(segments)
    if full:
        return np.ones((sid.shape[0], sid.shape[0]), dtype=bool)
    kinds = np.array([s.kind for s in segments])
    S = sid.shape[0]
    q = np.arange(S)[:, None]
    k = np.arange(S)[None, :]
    sq, sk = sid[:, None], sid[None, :]
    same = sq == sk
    causal_text = kinds[sid][:, None] == SEG_TEXT
    return (sk < sq) | (same & ~causal_text) | (same & causal_text & (k <= q))


def mask_rows(segments, rows, full: bool = False) -> np.ndarray:
    """The same visibility rule as mask_dense, evaluated only for the given query rows
    (shape [len(rows), S]); used to check sampled rows of full-size sequences."""
    sid = segment_ids(segments)
    if full:
        return np.ones((len(rows), sid.shape[0]), dtype=bool)
    kinds = np.array([s.kind for s in segments])
    rows = np.asarray(rows, dtype=np.int64)
    k = np.arange(sid.shape[0])[None, :]
    sq, sk = sid[rows][:, None], sid[None, :]
    same = sq == sk
    causal_text = kinds[sid[rows]][:, None] == SEG_TEXT
    return (sk < sq) | (same & ~causal_text) | (same & causal_text & (k <= rows[:, None]))


def blockmap(mask: np.ndarray, tile_q: int, tile_k: int) -> np.ndarray:
    """Tile classes over in-range pairs: 0 = no visible pair (skip), 1 = all visible (full),
    2 = mixed (partial).  Shape [ceil(S/tile_q), ceil(S/tile_k)], uint8."""
    Sq, Sk = mask.shape
    nq, nk = -(-Sq // tile_q), -(-Sk // tile_k)
    out = np.zeros((nq, nk), dtype=np.uint8)
    for i in range(nq):
        for j in range(nk):
            sub = mask[i * tile_q:(i + 1) * tile_q, j * tile_k:(j + 1) * tile_k]
            if sub.all():
                out[i, j] = 1
            elif sub.any():
                out[i, j] = 2
    return out


# ------------------------------------------------------------------------------------------------
# attention
# ------------------------------------------------------------------------------------------------

def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: Optional[np.ndarray] = None,
              scale: Optional[float] = None, chunk: int = 512) -> np.ndarray:
    """Masked softmax attention per head, O = softmax(Q K^T * scale, masked to -inf) V.
    q: [Nq, H, d], k, v: [Nk, H, d], mask: [Nq, Nk] bool or None.  Scale defaults to
    1/sqrt(d), the scaled-dot-product default used by the attention dispatch in [EDIT]
    section 6 (no scale is passed there).  Query rows are processed in chunks to bound memory."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Nq, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.empty((Nq, H, v.shape[2]), dtype=np.float64)
    for h in range(H):
        kh = np.ascontiguousarray(k[:, h, :])
        vh = np.ascontiguousarray(v[:, h, :])
        for c0 in range(0, Nq, chunk):
            c1 = min(Nq, c0 + chunk)
            s = (q[c0:c1, h, :] @ kh.T) * scale
            if mask is not None:
                s = np.where(mask[c0:c1], s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            out[c0:c1, h, :] = (p @ vh) / p.sum(axis=1, keepdims=True)
    return out


def attention_lse(q: np.ndarray, k: np.ndarray, mask: Optional[np.ndarray] = None,
                  scale: Optional[float] = None) -> np.ndarray:
    """Per query row and head, the log-sum-exp of the scaled scores over the visible keys,
    ln(sum_k exp(scale q.k)): the softmax denominator of the attention above, in natural log.
    q: [Nq, H, d], k: [Nk, H, d], mask: [Nq, Nk] bool or None.  Returns [H, Nq]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    Nq, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.empty((H, Nq), dtype=np.float64)
    for h in range(H):
        s = (q[:, h, :] @ k[:, h, :].T) * scale
        if mask is not None:
            s = np.where(mask, s, -np.inf)
        mx = s.max(axis=1, keepdims=True)
        out[h] = (mx + np.log(np.exp(s - mx).sum(axis=1, keepdims=True)))[:, 0]
    return out


def prep_qk(x: np.ndarray, cos_t, sin_t, w=None, eps: float = 1e-6) -> np.ndarray:
    """Optional per-head QK-RMSNorm, then the 3D rotation (norm before RoPE, as in [EDIT]
    section 6: QK normalisation, then RoPE, then the joint concat)."""
    y = np.asarray(x, dtype=np.float64)
    if w is not None:
        y = rms_norm(y, w, eps)
    return rotate(y, cos_t, sin_t) if cos_t is not None else y


def step1(q, k, v, segments, cos_t, sin_t, q_w=None, k_w=None, eps: float = 1e-6,
          scale: Optional[float] = None, full: bool = False):
    """Denoising step 1: full block-causal attention over the whole sequence; the prefix's
    K (normalised and rotated) and V are kept as the cache ([OV] card 6A: step 1 computes
    prefix and target and stores the prefix K/V).  Returns (O [S,H,d], (K_cache, V_cache)).
    full=True: the unmasked joint attention of the v1 / Edit model instead."""
    S, P, T = split_counts(segments)
    qr = prep_qk(q, cos_t, sin_t, q_w, eps)
    kr = prep_qk(k, cos_t, sin_t, k_w, eps)
    o = attention(qr, kr, v, mask_dense(segments, full), scale)
    return o, (kr[:P].copy(), np.asarray(v, dtype=np.float64)[:P].copy())


def cached_step(q_t, k_t, v_t, cache, cos_t, sin_t, q_w=None, k_w=None, eps: float = 1e-6,
                scale: Optional[float] = None) -> np.ndarray:
    """Euler steps 2..N: only target queries, against [cached prefix K/V ; fresh target K/V].
    The target sees every token ([OV] card 3C / 6A), so no mask.  cos_t/sin_t are the
    target rows of the tables."""
    kc, vc = cache
    qr = prep_qk(q_t, cos_t, sin_t, q_w, eps)
    kr = prep_qk(k_t, cos_t, sin_t, k_w, eps)
    keys = np.concatenate([kc, kr], axis=0)
    vals = np.concatenate([vc, np.asarray(v_t, dtype=np.float64)], axis=0)
    return attention(qr, keys, vals, None, scale)


def euler(x: np.ndarray, v: np.ndarray, sigma_k: float, sigma_k1: float) -> np.ndarray:
    """x_{k+1} = x_k + (sigma_{k+1} - sigma_k) * v ([OV] learning goals and card 6B)."""
    return np.asarray(x, dtype=np.float64) + (float(sigma_k1) - float(sigma_k)) * np.asarray(v, dtype=np.float64)


# ------------------------------------------------------------------------------------------------
# flop / byte accounting (used by the benchmark's reporting, not by the device path)
# ------------------------------------------------------------------------------------------------

def visible_pairs(segments, full: bool = False) -> int:
    """Number of visible (query, key) pairs per head for step 1, counted from the dense mask."""
    return int(mask_dense(segments, full).sum())


# ------------------------------------------------------------------------------------------------
# one single-stream DiT layer around the attention (the full-layer workload)
# ------------------------------------------------------------------------------------------------

def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def timestep_embedding(t, dim: int = 256, max_period: float = 10000.0) -> np.ndarray:
    """Sinusoidal timestep embedding ([EDIT] section 5.1: 256 channels, frequencies
    max_period^(-i/(dim/2)), cos half first).  t: array of timesteps (1000 * sigma here)."""
    t = np.atleast_1d(np.asarray(t, dtype=np.float64))
    half = dim // 2
    freqs = np.array([math.exp(-math.log(max_period) * i / half) for i in range(half)])
    arg = t[:, None] * freqs[None, :]
    return np.concatenate([np.cos(arg), np.sin(arg)], axis=1)


def linear(x, w):
    """y = x W^T with W in the Linear layout [out][in]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def time_condition(sigma, w1, w2) -> np.ndarray:
    """temb = W2 SiLU(W1 emb(1000 sigma)) ([EDIT] section 5.1: timestep embedding, Linear, SiLU,
    Linear; no biases in this random-init reading)."""
    return linear(silu(linear(timestep_embedding(1000.0 * np.atleast_1d(sigma)), w1)), w2)


def modulation(temb, wm, d: int):
    """Shared modulation ([OV] card 3B, one modulator for all layers): W_mod SiLU(temb) split into
    (shift1, scale1, gate1, shift2, scale2, gate2), each [n, d] ([EDIT] section 5.2 order)."""
    m = linear(silu(temb), wm)
    return tuple(m[:, i * d:(i + 1) * d] for i in range(6))


def norm_mod(x, w, scale, shift, eps: float = 1e-6):
    """ZeroCenterRMSNorm then x (1 + scale) + shift ([1B] sections 1-3; [EDIT] section 5.2)."""
    y = zero_center_rms_norm(x, w, eps) if w is not None else rms_norm(x, None, eps)
    if scale is not None:
        y = y * (1.0 + scale)
    if shift is not None:
        y = y + shift
    return y


def per_row(vec_prefix, vec_target, n_rows: int, row0: int, P: int):
    """Per-row parameters: rows with global index < P (prefix) take the t = 0 values, the rest the
    current step's ([OV] card 3B: prefix at t = 0, target at t)."""
    rows = np.arange(row0, row0 + n_rows)
    return np.where((rows < P)[:, None], np.asarray(vec_prefix)[None, :], np.asarray(vec_target)[None, :])


def gelu_tanh(x):
    """GELU in its tanh form, 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))): the activation
    the TextProjection of [1B] sections 1-3 names GELU(tanh)."""
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def text_projection(x_ctx, w_norm, w1, w2, eps: float = 1e-6):
    """The context path of [1B] sections 1-3: ZeroCenterRMSNorm, Linear, GELU(tanh), Linear
    (no biases: random-init weights; widths D -> D -> D)."""
    h = zero_center_rms_norm(np.asarray(x_ctx, np.float64), w_norm, eps)
    return linear(gelu_tanh(linear(h, w1)), w2)


def swiglu(g, u):
    """SiLU(gate) * up ([OV] card 5A)."""
    return silu(g) * np.asarray(u, dtype=np.float64)


def dit_layer(x, L, mods, segments, cos_t, sin_t, cache=None, eps: float = 1e-6,
              tanh_gate: bool = True):
    """One single-stream DiT layer ([OV] cards 4A, 5A; [EDIT] sections 5.2 and 6 for the order):
        h  = ZeroCenterRMSNorm(x) (1 + scale1) + shift1
        q, k, v = h W_qkv^T, per-head QK-RMSNorm, 3D RoPE
        x += tanh(gate1) * (Attention(q, k, v) W_out^T)
        h2 = ZeroCenterRMSNorm(x) (1 + scale2) + shift2
        x += tanh(gate2) * ((SiLU(h2 W_gate^T) * (h2 W_up^T)) W_down^T)
    Step 1 (cache None): x holds all S tokens, block-causal attention, returns (x_out, (K, V)) with
    the prefix K (normalised, rotated) and V.  Cached step: x holds the T target tokens, cache the
    prefix K/V; returns (x_out, None).  mods: (prefix_params, target_params), each the six
    modulation vectors; L: dict of layer weights; tanh_gate False gives the plain gate of the
    v1 model."""
    x = np.asarray(x, dtype=np.float64)
    S, P, T = split_counts(segments)
    n = x.shape[0]
    row0 = 0 if cache is None else P
    D = x.shape[1]
    H = D // HEAD_DIM
    (sh1p, sc1p, g1p, sh2p, sc2p, g2p), (sh1t, sc1t, g1t, sh2t, sc2t, g2t) = mods
    pr = lambda a, b: per_row(a, b, n, row0, P)
    gate = (lambda g: np.tanh(g)) if tanh_gate else (lambda g: g)
    h = norm_mod(x, L["norm1"], pr(sc1p, sc1t), pr(sh1p, sh1t), eps)
    qkv = linear(h, L["w_qkv"]).reshape(n, 3, H, HEAD_DIM)
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    c, s = cos_t[row0:row0 + n], sin_t[row0:row0 + n]
    if cache is None:
        o, new_cache = step1(q, k, v, segments, c, s, L["q_norm"], L["k_norm"], eps)
    else:
        o = cached_step(q, k, v, cache, c, s, L["q_norm"], L["k_norm"], eps)
        new_cache = None
    x = x + gate(pr(g1p, g1t)) * linear(o.reshape(n, D), L["w_out"])
    h2 = norm_mod(x, L["norm2"], pr(sc2p, sc2t), pr(sh2p, sh2t), eps)
    a = swiglu(linear(h2, L["w_gate"]), linear(h2, L["w_up"]))
    x = x + gate(pr(g2p, g2t)) * linear(a, L["w_down"])
    return x, new_cache


# ------------------------------------------------------------------------------------------------
# the v1 / Edit dual-stream block around the unmasked joint attention
# ------------------------------------------------------------------------------------------------

def layer_norm(x, eps: float = 1e-6):
    """LayerNorm over the last axis without affine parameters: (x - mean) / sqrt(var + eps) with
    the biased variance ([EDIT] section 5.2: the v1 block's norm1 / norm2 have elementwise_affine
    off, eps 1e-6)."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def linear_bias(x, w, b):
    """y = x W^T + b (a Linear with its bias: every Linear of the v1 block carries one, as the
    per-block parameter table of [EDIT] counts them)."""
    y = linear(x, w)
    return y if b is None else y + np.asarray(b, np.float64)


def v1_block(x_txt, x_img, temb, B, cos_t, sin_t, temb0=None, n_noise: Optional[int] = None,
             eps: float = 1e-6, rows_txt=None, rows_img=None):
    """One dual-stream block of the v1 / Edit model ([EDIT] section 5.2 for the block's forward,
    section 6 for the attention processor), both streams in fp64.

    x_txt [Lt, D], x_img [Li, D]: the text stream and the image stream (the noisy target's rows
    first, then the references').  temb [D]: the conditioning of the current t.  Each stream has
    its own modulation, SiLU then a Linear(D, 6 D) with bias, cut into (shift1, scale1, gate1,
    shift2, scale2, gate2).  With temb0 (the optional per-token modulation of the Edit model),
    image rows [0, n_noise) take temb's parameters and the rest temb0's; the text always takes
    temb's.  Per stream:
        h = LayerNorm(x) (1 + scale1) + shift1
        q, k, v = h W^T + b (image: to_q / to_k / to_v; text: add_q_proj / add_k_proj /
                  add_v_proj, stacked q | k | v as [3 D][D]), per-head RMSNorm of q and k with the
                  stream's weights (norm_q / norm_k, norm_added_q / norm_added_k), RoPE
    then the joint sequence [text | image] under unmasked softmax attention, the text rows through
    to_add_out and the image rows through to_out (both with bias), and per stream
        x += gate1 * out
        h2 = LayerNorm(x) (1 + scale2) + shift2
        x += gate2 * (GELU_tanh(h2 W1^T + b1) W2^T + b2)        (img_mlp / txt_mlp, D -> 4 D -> D)
    cos_t / sin_t: rotation tables of the joint sequence [Lt + Li, 64] (text positions first).
    B: dict of the block's weights (keys as read below).  Returns (x_txt, x_img).  With rows_txt
    and rows_img (index arrays), only those output rows are formed (the keys and values still
    come from every row): returns (x_txt[rows_txt], x_img[rows_img]) of the block's output."""
    xt = np.asarray(x_txt, np.float64)
    xi = np.asarray(x_img, np.float64)
    Lt, D = xt.shape
    Li = xi.shape[0]
    H = D // HEAD_DIM

    def mods(which, t):
        m = linear_bias(silu(np.atleast_2d(t)), B[which + "_mod_w"], B[which + "_mod_b"])[0]
        return [m[i * D:(i + 1) * D] for i in range(6)]

    mt, mi = mods("txt", temb), mods("img", temb)
    if temb0 is not None:
        mi0 = mods("img", temb0)
        nn_ = Li if n_noise is None else n_noise
        sel = (np.arange(Li) < nn_)[:, None]
        mi = [np.where(sel, a[None, :], b[None, :]) for a, b in zip(mi, mi0)]
    sh1t, sc1t, g1t, sh2t, sc2t, g2t = mt
    sh1i, sc1i, g1i, sh2i, sc2i, g2i = mi

    def qkv(x, sc, sh, pre, nq, nk):
        h = layer_norm(x, eps) * (1.0 + sc) + sh
        y = linear_bias(h, B[pre + "_qkv_w"], B[pre + "_qkv_b"]).reshape(x.shape[0], 3, H, HEAD_DIM)
        return rms_norm(y[:, 0], B[nq], eps), rms_norm(y[:, 1], B[nk], eps), y[:, 2]

    qt, kt, vt = qkv(xt, sc1t, sh1t, "txt", "norm_added_q", "norm_added_k")
    qi, ki, vi = qkv(xi, sc1i, sh1i, "img", "norm_q", "norm_k")
    q = rotate(np.concatenate([qt, qi]), cos_t, sin_t)
    k = rotate(np.concatenate([kt, ki]), cos_t, sin_t)
    v = np.concatenate([vt, vi])
    if rows_txt is not None:
        rt_ = np.asarray(rows_txt, np.int64)
        ri_ = np.asarray(rows_img, np.int64)
        q = q[np.concatenate([rt_, Lt + ri_])]
        xt, xi = xt[rt_], xi[ri_]
        pick = lambda a, r: a[r] if np.ndim(a) == 2 else a
        sc2t, sh2t, g1t, g2t = (pick(a, rt_) for a in (sc2t, sh2t, g1t, g2t))
        sc2i, sh2i, g1i, g2i = (pick(a, ri_) for a in (sc2i, sh2i, g1i, g2i))
        Lt = len(rt_)
    o = attention(q, k, v).reshape(q.shape[0], D)
    xt = xt + g1t * linear_bias(o[:Lt], B["txt_out_w"], B["txt_out_b"])
    xi = xi + g1i * linear_bias(o[Lt:], B["img_out_w"], B["img_out_b"])

    def mlp(x, sc, sh, g, pre):
        h = layer_norm(x, eps) * (1.0 + sc) + sh
        a = gelu_tanh(linear_bias(h, B[pre + "_fc1_w"], B[pre + "_fc1_b"]))
        return x + g * linear_bias(a, B[pre + "_fc2_w"], B[pre + "_fc2_b"])

    return mlp(xt, sc2t, sh2t, g2t, "txt"), mlp(xi, sc2i, sh2i, g2i, "img")


def v1_output_head(x_img, temb, Hd, eps: float = 1e-6):
    """The v1 / Edit model's exit ([EDIT] section 5.3): norm_out, an AdaLN with a single Linear
    on SiLU(temb) giving 2 D values cut into (scale, shift) in that order, applied as
    LayerNorm(x) (1 + scale) + shift (no affine, eps 1e-6); then proj_out, a Linear(D -> 64)
    with bias, on the image stream.  Hd: norm_out_w [2D][D], norm_out_b [2D], proj_out_w [64][D],
    proj_out_b [64]."""
    xi = np.asarray(x_img, np.float64)
    D = xi.shape[1]
    emb = linear_bias(silu(np.atleast_2d(temb)), Hd["norm_out_w"], Hd["norm_out_b"])[0]
    scale, shift = emb[:D], emb[D:]
    return linear_bias(layer_norm(xi, eps) * (1.0 + scale) + shift, Hd["proj_out_w"], Hd["proj_out_b"])


def v1_forward(x_txt, x_img, temb, blocks, Hd, cos_t, sin_t, eps: float = 1e-6):
    """Dual-stream blocks in sequence, then the exit on the image stream ([EDIT] section 5.3: only
    the image part leaves through norm_out and proj_out).  Returns [Li, 64]."""
    xt, xi = x_txt, x_img
    for B in blocks:
        xt, xi = v1_block(xt, xi, temb, B, cos_t, sin_t, eps=eps)
    return v1_output_head(xi, temb, Hd, eps)


def velocity_head(x_t, temb, w_scale, w_head, eps: float = 1e-6):
    """Scale-only final AdaLN and the 64-channel velocity projection ([OV] card 6B):
    v = (RMSNorm(x) (1 + W_scale SiLU(temb))) W_head^T."""
    scale = linear(silu(temb), w_scale)
    return linear(rms_norm(x_t, None, eps) * (1.0 + scale), w_head)


def img_in(latent, w_in):
    """Latent cell (64 channels) -> one DiT token ([OV] card 1A; no bias in this reading)."""
    return linear(latent, w_in)


def prefix_states(segments, x_text, ref_tokens):
    """Hidden states of the prefix in sequence order: text segments take consecutive rows of
    x_text, reference images consecutive rows of ref_tokens ([OV] card 2A joint packing)."""
    rows, it, ir = [], 0, 0
    for g in segments[:-1]:
        if g.kind == SEG_IMAGE:
            rows.append(ref_tokens[ir:ir + g.n_tokens])
            ir += g.n_tokens
        else:
            rows.append(x_text[it:it + g.n_tokens])
            it += g.n_tokens
    return np.concatenate(rows, axis=0) if rows else np.zeros((0, x_text.shape[1]))


def denoise(segments, x_text, lat_ref, lat0, shared, layers, n_steps: int, eps: float = 1e-6,
            return_velocities: bool = False):
    """The Euler sampling loop with the prefix KV cache ([OV] cards 3B, 6A, 6B): step 1 runs every
    layer over the whole sequence (prefix at t = 0, target at t = 1000 sigma_0) and keeps each
    layer's prefix K/V; steps 2..n run only the target tokens against those caches.  After each
    step the target's velocity (scale-only final norm, 64-channel head) moves the latent by
    (sigma_{k+1} - sigma_k) v.  shared: t_w1, t_w2, w_mod, w_scale, w_head, w_in (fp64 arrays);
    layers: list of per-layer weight dicts.  Returns the final latent (and the velocities)."""
    S, P, T = split_counts(segments)
    D = shared["w_mod"].shape[1]
    c, s = rope_tables(positions(segments))
    sig = np.array([1.0 - k / n_steps for k in range(n_steps + 1)])
    lat = np.asarray(lat0, dtype=np.float64).copy()
    caches = [None] * len(layers)
    vels = []
    for k in range(n_steps):
        temb = time_condition(np.array([0.0, sig[k]]), shared["t_w1"], shared["t_w2"])
        mod = modulation(temb, shared["w_mod"], D)
        mods = (tuple(m[0] for m in mod), tuple(m[1] for m in mod))
        xt = img_in(lat, shared["w_in"])
        if k == 0:
            x = np.concatenate([prefix_states(segments, x_text, img_in(lat_ref, shared["w_in"])), xt], axis=0)
            for li, L in enumerate(layers):
                x, caches[li] = dit_layer(x, L, mods, segments, c, s, eps=eps)
            x_t = x[P:]
        else:
            x_t = xt
            for li, L in enumerate(layers):
                x_t, _ = dit_layer(x_t, L, mods, segments, c, s, cache=caches[li], eps=eps)
        v = velocity_head(x_t, temb[1:2], shared["w_scale"], shared["w_head"], eps)
        vels.append(v)
        lat = euler(lat, v, sig[k], sig[k + 1])
    return (lat, vels) if return_velocities else lat
