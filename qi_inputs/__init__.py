"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

This module holds workload shapes and random draws only.  It contains none of
the method's arithmetic (no positions, rotations, masks, norms or attention):
it says which token segments a workload has, draws N(0,1) numbers from a
counter-style seed ``[cfg_id, tensor_id, step, layer]`` and rounds them to the
storage type the device path consumes (bf16 by round-to-nearest-even, via
fp32).  Both the fp64 oracle and the HIP path receive exactly these bits.

Workloads (joint sequence order: text first, then reference images, target
image last; the 1024x1024 latent grid is 64x64 tokens, "Qwen-Image-Edit"
page, section 8.2 shape table):

  tiny_f32  fp32, 2 heads; text 16 + ref 4x4 (frame 1) + target 4x4 (frame 0)
  txt256_ref32_tgt32  bf16, 24 heads; text 256 + ref 32x32 (frame 1) + target 32x32
  txt512_tgt64  bf16, 24 heads; text 512 + target 64x64
  txt1024_4ref64_tgt64  bf16, 24 heads; text 1024 + 4 refs 64x64 (frames 1..4) + target 64x64
        (17,408 prefix tokens, 21,504 keys)
  txt512_4ref64_tgt64  the same with 512 text tokens (16,896 prefix, 20,992 keys)
  txt512_10ref32_tgt64  bf16, 24 heads; text 512 + 10 refs 32x32 (frames 1..10) + target 64x64
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Sequence, Tuple

import numpy as np

# segment kinds (same numbering as the C header's qi_seg_kind)
SEG_TEXT = 0          # text, token-causal inside the segment
SEG_IMAGE = 1         # one image: all its tokens see each other
SEG_TEXT_BIDIR = 2    # text read as one bidirectional block

# tensor ids for the seed tuple
T_Q, T_K, T_V, T_QW, T_KW, T_X0, T_VEL, T_QT, T_KT, T_VT = range(10)
T_WEIGHT_BASE = 100   # model weights of the full-layer workload: 100 + index


@dataclasses.dataclass(frozen=True)
class Segment:
    kind: int
    n_tokens: int
    frame: int = 0
    grid_h: int = 0
    grid_w: int = 0


def text(n: int, bidir: bool = False) -> Segment:
    return Segment(SEG_TEXT_BIDIR if bidir else SEG_TEXT, n)


def image(h: int, w: int, frame: int) -> Segment:
    return Segment(SEG_IMAGE, h * w, frame, h, w)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    segments: Tuple[Segment, ...]
    n_head: int = 24
    head_dim: int = 128
    dtype: str = "bf16"          # storage type of q/k/v/o ("bf16" or "f32")
    theta: float = 10000.0
    bands: Tuple[int, int, int] = (16, 56, 56)
    qk_rmsnorm: bool = False     # q/k pass a per-head RMSNorm with weights 1+N(0,0.02)
    n_steps: int = 8             # Euler steps (step 1 full + cached steps)
    latent_ch: int = 64          # channels of the velocity / latent per target token

    @property
    def S(self) -> int:
        return sum(s.n_tokens for s in self.segments)

    @property
    def T(self) -> int:
        return self.segments[-1].n_tokens

    @property
    def P(self) -> int:
        return self.S - self.T


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 0, (text(16), image(4, 4, 1), image(4, 4, 0)), n_head=2, dtype="f32",
                     n_steps=2),
    "txt256_ref32_tgt32": Workload("txt256_ref32_tgt32", 1, (text(256), image(32, 32, 1), image(32, 32, 0)), qk_rmsnorm=True),
    "txt512_tgt64": Workload("txt512_tgt64", 2, (text(512), image(64, 64, 0))),
    "txt1024_4ref64_tgt64": Workload("txt1024_4ref64_tgt64", 3, (text(1024),) + tuple(image(64, 64, f) for f in (1, 2, 3, 4))
                     + (image(64, 64, 0),)),
    "txt512_4ref64_tgt64": Workload("txt512_4ref64_tgt64", 3, (text(512),) + tuple(image(64, 64, f) for f in (1, 2, 3, 4))
                          + (image(64, 64, 0),)),
    "txt512_10ref32_tgt64": Workload("txt512_10ref32_tgt64", 4, (text(512),) + tuple(image(32, 32, f) for f in range(1, 11))
                     + (image(64, 64, 0),)),
}

# The v1 / Edit joint attention (full, unmasked) on the Edit shapes of the source-reading page:
# [text | noisy 1024^2 target (64x64 tokens, frame 0) | references (frame 1..)] -- Edit with one
# reference, Edit-Plus with two.  Run with the QI_ATTN_FULL layout.
V1_WORKLOADS = {
    "edit_v1": Workload("edit_v1", 5, (text(512), image(64, 64, 0), image(64, 64, 1))),
    "editplus_v1": Workload("editplus_v1", 6, (text(512), image(64, 64, 0), image(64, 64, 1), image(64, 64, 2))),
}


# Joint packing with text between the images (the prompt may interleave text with up to ten
# reference images): text 64, then ten (reference 32x32, text 16) pairs, then the target 64x64.
INTERLEAVED_WORKLOADS = {
    "interleaved10": Workload("interleaved10", 7, (text(64),) + tuple(s for f in range(1, 11)
                                                                      for s in (image(32, 32, f), text(16)))
                              + (image(64, 64, 0),)),
}


def small_workload(name: str, segments: Sequence[Segment], n_head: int = 2, dtype: str = "bf16",
                   cfg_id: int = 90, qk_rmsnorm: bool = False) -> Workload:
    """An ad-hoc workload for edge-case tests (ragged tiles, odd grids, several text runs)."""
    return Workload(name, cfg_id, tuple(segments), n_head=n_head, dtype=dtype, qk_rmsnorm=qk_rmsnorm)


# ----------------------------------------------------------------------------------------------
# random draws and storage rounding
# ----------------------------------------------------------------------------------------------

def rng(cfg_id: int, tensor_id: int, step: int = 0, layer: int = 0) -> np.random.Generator:
    return np.random.default_rng([cfg_id, tensor_id, step, layer])


def normal(cfg_id: int, tensor_id: int, shape, step: int = 0, layer: int = 0,
           mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """fp64 draws N(mean, std^2) from the seed tuple [cfg_id, tensor_id, step, layer]."""
    x = rng(cfg_id, tensor_id, step, layer).standard_normal(size=shape)
    return x * std + mean


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    r = np.where(nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Stored:
    """One input tensor: the bits handed to the device and the same values as fp64."""
    bits: np.ndarray      # uint16 (bf16) or float32 array, as stored
    f64: np.ndarray       # the stored values, exactly, as fp64
    dtype: str


def stored(x64: np.ndarray, dtype: str) -> Stored:
    if dtype == "bf16":
        b = f32_to_bf16_bits(x64.astype(np.float32))
        return Stored(b, bf16_bits_to_f64(b), dtype)
    if dtype == "f32":
        f = x64.astype(np.float32)
        return Stored(f, f.astype(np.float64), dtype)
    if dtype == "f16":   # by way of fp32, nearest even (values beyond fp16's range become infinite)
        h = x64.astype(np.float32).astype(np.float16)
        return Stored(h.view(np.uint16), h.astype(np.float64), dtype)
    raise ValueError(dtype)


def qkv(wl: Workload, n_tok: int, step: int = 0, layer: int = 0, ids=(T_Q, T_K, T_V)) -> List[Stored]:
    """Q, K, V of shape [n_tok, n_head, head_dim], N(0,1), stored in the workload dtype."""
    shape = (n_tok, wl.n_head, wl.head_dim)
    return [stored(normal(wl.cfg_id, t, shape, step, layer), wl.dtype) for t in ids]


def qk_norm_weights(wl: Workload, layer: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Per-head RMSNorm weights 1 + N(0, 0.02^2), fp32 (shared by all heads), as fp64 arrays."""
    wq = normal(wl.cfg_id, T_QW, (wl.head_dim,), 0, layer, 1.0, 0.02).astype(np.float32)
    wk = normal(wl.cfg_id, T_KW, (wl.head_dim,), 0, layer, 1.0, 0.02).astype(np.float32)
    return wq.astype(np.float64), wk.astype(np.float64)


def sigmas(n_steps: int) -> np.ndarray:
    """Euler sigma schedule sigma_k = 1 - k/n_steps, k = 0..n_steps (fp64), the linspace(1, 0, n+1) grid."""
    return np.array([1.0 - k / n_steps for k in range(n_steps + 1)], dtype=np.float64)


# ----------------------------------------------------------------------------------------------
# random-init weights and inputs of the full single-stream layer workload
# ----------------------------------------------------------------------------------------------

# weight indices (tensor id = T_WEIGHT_BASE + index); per layer:
W_NORM1, W_NORM2, W_QNORM, W_KNORM, W_QKV, W_OUT, W_GATE, W_UP, W_DOWN = range(9)
# shared (layer 0): timestep MLP, modulation, head scale, velocity head, img_in, prefix inputs
W_T1, W_T2, W_MOD, W_HSCALE, W_HEAD, W_IN, X_TEXT, LAT_REF, LAT_TGT = range(20, 29)
# context TextProjection (ZeroCenterRMSNorm weight, two Linears) and its synthetic VLM context
W_TPN, W_TP1, W_TP2, X_CTX = range(29, 33)


def linear_weight(cfg_id: int, index: int, n_out: int, n_in: int, layer: int = 0) -> Stored:
    """A Linear weight [n_out][n_in] ~ N(0, 1/n_in), stored bf16."""
    return stored(normal(cfg_id, T_WEIGHT_BASE + index, (n_out, n_in), 0, layer, 0.0, 1.0 / math.sqrt(n_in)), "bf16")


def f32_vector(cfg_id: int, index: int, shape, layer: int = 0, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """fp32-stored draws, returned as fp64 values."""
    return normal(cfg_id, T_WEIGHT_BASE + index, shape, 0, layer, mean, std).astype(np.float32).astype(np.float64)


def layer_weights(cfg_id: int, D: int, F: int, layer: int) -> dict:
    """Random-init weights of one single-stream layer: ZeroCenterRMSNorm weights N(0, 0.02^2)
    (stored as scale - 1), QK-RMSNorm weights 1 + N(0, 0.02^2), Linear weights N(0, 1/fan_in) in
    bf16 (QKV [3D][D] in q | k | v order, out [D][D], gate and up [F][D], down [D][F])."""
    return {
        "norm1": f32_vector(cfg_id, W_NORM1, (D,), layer, 0.0, 0.02),
        "norm2": f32_vector(cfg_id, W_NORM2, (D,), layer, 0.0, 0.02),
        "q_norm": f32_vector(cfg_id, W_QNORM, (128,), layer, 1.0, 0.02),
        "k_norm": f32_vector(cfg_id, W_KNORM, (128,), layer, 1.0, 0.02),
        "w_qkv": linear_weight(cfg_id, W_QKV, 3 * D, D, layer),
        "w_out": linear_weight(cfg_id, W_OUT, D, D, layer),
        "w_gate": linear_weight(cfg_id, W_GATE, F, D, layer),
        "w_up": linear_weight(cfg_id, W_UP, F, D, layer),
        "w_down": linear_weight(cfg_id, W_DOWN, D, F, layer),
    }


def shared_weights(cfg_id: int, D: int, t_dim: int = 256, latent_ch: int = 64) -> dict:
    """Random-init conditioning and projection weights shared by all layers (bf16)."""
    return {
        "t_w1": linear_weight(cfg_id, W_T1, D, t_dim),
        "t_w2": linear_weight(cfg_id, W_T2, D, D),
        "w_mod": linear_weight(cfg_id, W_MOD, 6 * D, D),
        "w_scale": linear_weight(cfg_id, W_HSCALE, D, D),
        "w_head": linear_weight(cfg_id, W_HEAD, latent_ch, D),
        "w_in": linear_weight(cfg_id, W_IN, D, latent_ch),
    }


def text_projection_weights(cfg_id: int, D: int) -> dict:
    """Random-init context TextProjection: ZeroCenterRMSNorm weight N(0, 0.02^2) (stored as
    scale - 1, fp32) and two Linear weights [D][D] ~ N(0, 1/D) in bf16."""
    return {
        "tp_norm": f32_vector(cfg_id, W_TPN, (D,), 0, 0.0, 0.02),
        "tp_w1": linear_weight(cfg_id, W_TP1, D, D),
        "tp_w2": linear_weight(cfg_id, W_TP2, D, D),
    }


# the v1 / Edit dual-stream block: weights (bf16 Linears, fp32 biases and QK-norm weights) and inputs
V1_LINEARS = ("img_mod", "txt_mod", "img_qkv", "txt_qkv", "img_out", "txt_out", "img_fc1", "img_fc2", "txt_fc1",
              "txt_fc2")
W_V1_BASE = 33                                # ids 33 .. 52: each Linear's weight, then its bias
W_V1_QN, W_V1_KN, W_V1_AQN, W_V1_AKN = range(53, 57)
X_V1_TXT, X_V1_IMG, X_V1_TEMB, X_V1_TEMB0 = range(57, 61)


def v1_block_weights(cfg_id: int, D: int, F: int, layer: int = 0) -> dict:
    """Random-init weights of one v1 dual-stream block: every Linear W ~ N(0, 1/fan_in) in bf16
    with a bias N(0, 0.1^2) in fp32 (modulation [6D][D], QKV [3D][D] in q | k | v order, out
    [D][D], MLP [F][D] then [D][F]); QK-RMSNorm weights 1 + N(0, 0.02^2)."""
    shapes = {"img_mod": (6 * D, D), "txt_mod": (6 * D, D), "img_qkv": (3 * D, D), "txt_qkv": (3 * D, D),
              "img_out": (D, D), "txt_out": (D, D), "img_fc1": (F, D), "img_fc2": (D, F), "txt_fc1": (F, D),
              "txt_fc2": (D, F)}
    out = {}
    for i, name in enumerate(V1_LINEARS):
        n_out, n_in = shapes[name]
        out[name + "_w"] = linear_weight(cfg_id, W_V1_BASE + 2 * i, n_out, n_in, layer)
        out[name + "_b"] = f32_vector(cfg_id, W_V1_BASE + 2 * i + 1, (n_out,), layer, 0.0, 0.1)
    for key, idx in (("norm_q", W_V1_QN), ("norm_k", W_V1_KN), ("norm_added_q", W_V1_AQN),
                     ("norm_added_k", W_V1_AKN)):
        out[key] = f32_vector(cfg_id, idx, (128,), layer, 1.0, 0.02)
    return out


W_V1_NOUT, W_V1_NOUTB, W_V1_POUT, W_V1_POUTB = range(61, 65)


def v1_head_weights(cfg_id: int, D: int, out_ch: int = 64) -> dict:
    """Random-init exit of the v1 model: norm_out's Linear [2D][D] and proj_out [out_ch][D], both
    N(0, 1/D) in bf16 with fp32 biases N(0, 0.1^2)."""
    return {"norm_out_w": linear_weight(cfg_id, W_V1_NOUT, 2 * D, D),
            "norm_out_b": f32_vector(cfg_id, W_V1_NOUTB, (2 * D,), 0, 0.0, 0.1),
            "proj_out_w": linear_weight(cfg_id, W_V1_POUT, out_ch, D),
            "proj_out_b": f32_vector(cfg_id, W_V1_POUTB, (out_ch,), 0, 0.0, 0.1)}


def v1_block_inputs(cfg_id: int, n_txt: int, n_img: int, D: int):
    """Residual streams (fp32 N(0, 1)) of the text and image rows and two conditioning vectors
    (temb, temb0; fp32 N(0, 1)) of one v1 block."""
    f = lambda idx, shape: normal(cfg_id, idx, shape).astype(np.float32).astype(np.float64)
    return f(X_V1_TXT, (n_txt, D)), f(X_V1_IMG, (n_img, D)), f(X_V1_TEMB, (D,)), f(X_V1_TEMB0, (D,))


def context_inputs(cfg_id: int, n_ctx: int, D: int) -> np.ndarray:
    """Synthetic vision-language context rows [n_ctx][D] (fp32, N(0,1)): the stand-in for the
    Qwen3-VL hidden states that the TextProjection maps into the DiT's text rows."""
    return f32_vector(cfg_id, X_CTX, (n_ctx, D))


def prefix_inputs(cfg_id: int, n_text: int, n_ref: int, D: int, latent_ch: int = 64):
    """Text hidden states [n_text][D] (fp32, N(0,1): stand-in for the projected VLM context) and
    clean reference latents [n_ref][latent_ch] (fp32, N(0,1))."""
    xt = f32_vector(cfg_id, X_TEXT, (n_text, D))
    lr = f32_vector(cfg_id, LAT_REF, (n_ref, latent_ch))
    return xt, lr


def target_noise(cfg_id: int, T: int, latent_ch: int = 64) -> np.ndarray:
    """The target latent at sigma = 1: N(0,1) fp32 [T][latent_ch]."""
    return f32_vector(cfg_id, LAT_TGT, (T, latent_ch))
