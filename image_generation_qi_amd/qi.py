"""ctypes binding of libqi.so: the C ABI of include/qi.h under the same names.

Argument marshalling only.  Every computation of the path runs in the library's HIP kernels
(device calls) or its C++ host helpers; nothing here computes part of the method.  Device
pointers are plain integers (``tensor.data_ptr()``); streams are ``hipStream_t`` handles as
integers (``torch.cuda.current_stream().cuda_stream``) or None for the null stream.

If libqi.so has not been built, loading raises ``QiLibraryMissing``: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int, c_int32, c_int64, c_uint8, c_void_p
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
# QI_LIBRARY names another build of the same library (the host-sanitized libqi_san.so of the CPU
# sanitizer tests); it must export the same ABI version.
LIB_PATH = os.environ.get("QI_LIBRARY") or os.path.join(_HERE, "libqi.so")

QI_OK, QI_ERR_ARG, QI_ERR_DTYPE, QI_ERR_SHAPE, QI_ERR_ALIGN, QI_ERR_LAYOUT, QI_ERR_HIP, QI_ERR_CAPACITY = \
    0, -1, -2, -3, -4, -5, -6, -7
QI_F32, QI_BF16, QI_F16 = 0, 1, 2
QI_SEG_TEXT, QI_SEG_IMAGE, QI_SEG_TEXT_BIDIR = 0, 1, 2
QI_EPI_STORE, QI_EPI_STORE_F32, QI_EPI_GATED_RESIDUAL, QI_EPI_SWIGLU, QI_EPI_GELU = 0, 1, 2, 3, 4
QI_EPI_GATED_RESIDUAL_LINEAR = 5
QI_MAX_SOURCE_KEYS = 8388607   # keys per source of the bf16 attention (include/qi.h)
QI_ABI_VERSION = 9             # the qi_version() these bindings are written against
QI_NOALLOC_SCRATCH_BYTES = 96 << 20   # scratch array of qi_attn_target_cached_noalloc (include/qi.h)
QI_ATTN_BLOCK_CAUSAL, QI_ATTN_FULL = 0, 1
QI_RANGE_Q, QI_RANGE_K, QI_RANGE_V, QI_RANGE_OUT = 1, 2, 4, 8   # range flags of fp16 values (include/qi.h)
QI_HEAD_DIM = 128


class QiLibraryMissing(RuntimeError):
    pass


class QiError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = status
        msg = f"{where}: {qi_status_str(status)} ({status})"
        if status == QI_ERR_HIP:
            code = lib().qi_last_hip_error()
            msg += f" [HIP error {code}: {lib().qi_hip_error_name(code).decode()}]"
        super().__init__(msg)


class qi_segment(ctypes.Structure):
    _fields_ = [("kind", c_int32), ("n_tokens", c_int32), ("frame", c_int32), ("grid_h", c_int32),
                ("grid_w", c_int32)]


class qi_layout(ctypes.Structure):
    _fields_ = [("n_seg", c_int32), ("seg", POINTER(qi_segment)), ("head_dim", c_int32),
                ("bands", c_int32 * 3), ("theta", c_double), ("text_pos0", c_int32), ("attention", c_int32)]


class qi_kvcache(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("dtype", c_int), ("n_layers", c_int32),
                ("n_head", c_int32), ("p_cap", c_int64)]


class qi_qkv(ctypes.Structure):
    _fields_ = [("q", c_void_p), ("k", c_void_p), ("v", c_void_p), ("o", c_void_p), ("dtype", c_int),
                ("n_tok", c_int64), ("n_head", c_int32), ("tok_stride", c_int64), ("lse", c_void_p),
                ("range_flags", c_void_p)]


class qi_qkprep(ctypes.Structure):
    _fields_ = [("cos_t", c_void_p), ("sin_t", c_void_p), ("q_rms_w", c_void_p), ("k_rms_w", c_void_p),
                ("eps", c_float)]


class qi_kvtiles(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("n_head", c_int32), ("rows", c_int64)]


class qi_norm_fold(ctypes.Structure):
    _fields_ = [("sumsq", c_void_p), ("eps", c_float), ("bias_t", c_void_p), ("xc", c_void_p), ("ldxc", c_int64),
                ("next_w", c_void_p), ("next_scale", c_void_p), ("sumsq_out", c_void_p)]


_SIGS = {
    "qi_status_str": (c_char_p, [c_int]),
    "qi_last_hip_error": (c_int, []),
    "qi_hip_error_name": (c_char_p, [c_int]),
    "qi_version": (c_int, []),
    "qi_layout_tokens": (c_int, [POINTER(qi_layout), POINTER(c_int64), POINTER(c_int64), POINTER(c_int64)]),
    "qi_rope3d_positions": (c_int, [POINTER(qi_layout), c_void_p]),
    "qi_rope3d_tables": (c_int, [POINTER(qi_layout), c_void_p, c_void_p]),
    "qi_blockmap": (c_int, [POINTER(qi_layout), c_int32, c_int32, c_void_p]),
    "qi_attn_tile_shape": (c_int, [c_int, POINTER(c_int32), POINTER(c_int32)]),
    "qi_attn_schedule": (c_int, [c_int64, c_int32, c_int64, c_int64, POINTER(c_int32), POINTER(c_int32),
                                 POINTER(c_int32)]),
    "qi_attn_full_workspace_bytes": (c_int64, [POINTER(qi_layout), c_int, c_int32]),
    "qi_attn_cached_workspace_bytes": (c_int64, [c_int, c_int64, c_int32]),
    "qi_kvcache_bytes": (c_int64, [c_int, c_int32, c_int32, c_int64]),
    "qi_rope3d_apply": (c_int, [c_void_p, c_int, c_int64, c_int32, c_int64, c_void_p, c_void_p, c_void_p,
                                c_float, c_void_p]),
    "qi_attn_blockcausal_full": (c_int, [POINTER(qi_qkv), POINTER(qi_qkprep), POINTER(qi_layout), c_float,
                                         POINTER(qi_kvcache), c_int32, c_void_p, c_int64, c_void_p]),
    "qi_attn_prefix_store": (c_int, [c_void_p, c_void_p, c_int, c_int64, c_int32, c_int64, POINTER(qi_qkprep),
                                     POINTER(qi_kvcache), c_int32, c_void_p, c_void_p]),
    "qi_attn_target_cached": (c_int, [POINTER(qi_qkv), POINTER(qi_qkprep), POINTER(qi_kvcache), c_int32,
                                      c_int64, c_float, c_void_p, c_int64, c_void_p]),
    "qi_attn_target_cached_noalloc": (c_int, [POINTER(qi_qkv), POINTER(qi_qkprep), POINTER(qi_kvcache), c_int32,
                                              c_int64, c_float, c_void_p]),
    "qi_euler_step": (c_int, [c_void_p, c_void_p, c_int, c_int64, c_float, c_float, c_void_p]),
    "qi_gemm_bf16": (c_int, [c_void_p, c_int64, c_void_p, c_void_p, c_int64, c_int64, c_int64, c_int64, c_int,
                             c_void_p, c_int64, c_int64, c_void_p]),
    "qi_gemm_bf16_ex": (c_int, [c_void_p, c_int64, c_void_p, c_void_p, c_int64, c_int64, c_int64, c_int64, c_int,
                                c_void_p, c_int64, c_int64, c_int32, c_void_p]),
    "qi_gemm_bf16_bias": (c_int, [c_void_p, c_int64, c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_int64,
                                  c_int64, c_int, c_void_p, c_int64, c_int64, c_void_p]),
    "qi_zc_rmsnorm_mod": (c_int, [c_void_p, c_int64, c_void_p, c_int64, c_int64, c_int32, c_void_p, c_void_p,
                                  c_void_p, c_int64, c_int64, c_float, c_void_p]),
    "qi_layernorm_mod": (c_int, [c_void_p, c_int64, c_void_p, c_int64, c_int64, c_int32, c_void_p, c_void_p,
                                 c_int64, c_int64, c_float, c_void_p]),
    "qi_timestep_embed": (c_int, [c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
    "qi_linear_small": (c_int, [c_void_p, c_int32, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
    "qi_linear_small_bias": (c_int, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_int32, c_int32, c_void_p,
                                     c_void_p]),
    "qi_cast_bf16": (c_int, [c_void_p, c_void_p, c_int64, c_void_p]),
    "qi_gemm": (c_int, [c_void_p, c_int64, c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_int64, c_int64, c_int32,
                        c_int32, c_void_p, c_int64, c_int64, c_int32, c_void_p, c_void_p]),
    "qi_norm_mod": (c_int, [c_void_p, c_int64, c_void_p, c_int64, c_int64, c_int32, c_void_p, c_void_p, c_void_p,
                            c_int64, c_int64, c_float, c_int32, c_int32, c_void_p, c_void_p]),
    "qi_cast": (c_int, [c_void_p, c_void_p, c_int64, c_int32, c_void_p, c_void_p]),
    "qi_gemm_norm_fold": (c_int, [c_void_p, c_int64, c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_int64,
                                  c_int64, c_int32, c_int32, c_void_p, c_int64, c_int64, c_int32,
                                  POINTER(qi_norm_fold), c_void_p, c_void_p]),
    "qi_norm_fold_rows": (c_int, [c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64, c_int32, c_void_p,
                                  c_void_p, c_int64, c_int64, c_int32, c_void_p, c_void_p]),
    "qi_linear_multi": (c_int, [c_void_p, c_int32, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
    "qi_attn_tiled_workspace_bytes": (c_int64, [POINTER(qi_layout), c_int32]),
    "qi_gemm_qkv_tiles": (c_int, [c_void_p, c_int64, c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_int32, c_int64,
                                  c_int32, c_int64, c_int64, c_int64, POINTER(qi_norm_fold), POINTER(qi_qkprep),
                                  POINTER(qi_kvcache), c_int32, POINTER(qi_kvtiles), c_void_p, c_void_p]),
    "qi_attn_target_cached_tiled": (c_int, [POINTER(qi_qkv), POINTER(qi_qkprep), POINTER(qi_kvcache), c_int32,
                                            c_int64, c_float, POINTER(qi_kvtiles), c_void_p, c_int64, c_void_p]),
    "qi_attn_blockcausal_full_tiled": (c_int, [POINTER(qi_qkv), POINTER(qi_qkprep), POINTER(qi_layout), c_float,
                                               POINTER(qi_kvcache), c_int32, POINTER(qi_kvtiles), c_void_p, c_int64,
                                               c_void_p]),
    "qi_kernel_timing": (c_int, [c_int]),
    "qi_kernel_timing_read": (c_int, [POINTER(c_double), POINTER(c_int64)]),
    "qi_kernel_timing_read_each": (c_int, [POINTER(c_float), c_int64, POINTER(c_int64)]),
}

_lib = None


def lib():
    """Load libqi.so (once).  Raises QiLibraryMissing when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise QiLibraryMissing(f"{LIB_PATH} not found: build it with `python -m image_generation_qi_amd.build`"
                                   " (or __graft_entry__.build())")
        # PyTorch bundles its own HIP runtime (same soname as the system one, but its libraries
        # ask for it by another name).  Loaded first, it is the one this library binds to;
        # loaded after this library, the process would hold two runtimes and launches made
        # through this one fail with hipErrorNoDevice.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if L.qi_version() != QI_ABI_VERSION:
            raise QiLibraryMissing(f"{LIB_PATH} has ABI version {L.qi_version()}, these bindings need "
                                   f"{QI_ABI_VERSION}: rebuild it")
        _lib = L
    return _lib


def exported_symbols() -> Sequence[str]:
    return list(_SIGS)


def _p(x) -> Optional[int]:
    """Device/host pointer of a tensor-like (``data_ptr()``), an int, or None."""
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):        # numpy array
        return x.ctypes.data
    return int(x)


def _ref(s):
    return None if s is None else ctypes.byref(s)


def check(status: int, where: str = "qi") -> int:
    if status != QI_OK:
        raise QiError(status, where)
    return status


# ------------------------------------------------------------------------------------------------
# struct builders
# ------------------------------------------------------------------------------------------------

def make_layout(segments, head_dim: int = 128, bands=(16, 56, 56), theta: float = 10000.0,
                text_pos0: int = -1, attention: int = 0) -> qi_layout:
    """qi_layout from a sequence of objects with kind/n_tokens/frame/grid_h/grid_w attributes;
    attention is QI_ATTN_BLOCK_CAUSAL (default) or QI_ATTN_FULL."""
    arr = (qi_segment * len(segments))()
    for i, s in enumerate(segments):
        arr[i] = qi_segment(s.kind, s.n_tokens, s.frame, s.grid_h, s.grid_w)
    L = qi_layout(len(segments), ctypes.cast(arr, POINTER(qi_segment)), head_dim, (c_int32 * 3)(*bands),
                  theta, text_pos0, attention)
    L._keep = arr
    return L


def make_qkv(q, k, v, o, dtype: int, n_tok: int, n_head: int, tok_stride: int, lse=None,
             range_flags=None) -> qi_qkv:
    return qi_qkv(_p(q), _p(k), _p(v), _p(o), dtype, n_tok, n_head, tok_stride, _p(lse), _p(range_flags))


def make_prep(cos_t=None, sin_t=None, q_rms_w=None, k_rms_w=None, eps: float = 1e-6) -> qi_qkprep:
    return qi_qkprep(_p(cos_t), _p(sin_t), _p(q_rms_w), _p(k_rms_w), eps)


def make_cache(k, v, dtype: int, n_layers: int, n_head: int, p_cap: int) -> qi_kvcache:
    return qi_kvcache(_p(k), _p(v), dtype, n_layers, n_head, p_cap)


def make_tiles(k, v, n_head: int, rows: int) -> qi_kvtiles:
    return qi_kvtiles(_p(k), _p(v), n_head, rows)


# ------------------------------------------------------------------------------------------------
# the C ABI, same names
# ------------------------------------------------------------------------------------------------

def qi_status_str(status: int) -> str:
    return lib().qi_status_str(status).decode()


def qi_version() -> int:
    return lib().qi_version()


def qi_layout_tokens(layout: qi_layout):
    S, P, T = c_int64(), c_int64(), c_int64()
    check(lib().qi_layout_tokens(ctypes.byref(layout), ctypes.byref(S), ctypes.byref(P), ctypes.byref(T)),
          "qi_layout_tokens")
    return S.value, P.value, T.value


def qi_rope3d_positions(layout: qi_layout, pos) -> int:
    return lib().qi_rope3d_positions(ctypes.byref(layout), _p(pos))


def qi_rope3d_tables(layout: qi_layout, cos_t, sin_t) -> int:
    return lib().qi_rope3d_tables(ctypes.byref(layout), _p(cos_t), _p(sin_t))


def qi_blockmap(layout: qi_layout, tile_q: int, tile_k: int, out_map) -> int:
    return lib().qi_blockmap(ctypes.byref(layout), tile_q, tile_k, _p(out_map))


def qi_attn_tile_shape(dtype: int):
    tq, tk = c_int32(), c_int32()
    check(lib().qi_attn_tile_shape(dtype, ctypes.byref(tq), ctypes.byref(tk)), "qi_attn_tile_shape")
    return tq.value, tk.value


def qi_attn_schedule(n_q: int, n_head: int, n_keys_a: int = 0, n_keys_b: int = 0):
    """(key chunks per cut query tile, whole tiles per XCD run, cut tiles) of a bf16 launch over
    key sources of n_keys_a and n_keys_b keys (0, 0: the key-independent bound the workspace
    queries size for)."""
    s, w, c = c_int32(), c_int32(), c_int32()
    check(lib().qi_attn_schedule(n_q, n_head, n_keys_a, n_keys_b, ctypes.byref(s), ctypes.byref(w), ctypes.byref(c)),
          "qi_attn_schedule")
    return s.value, w.value, c.value


def qi_attn_full_workspace_bytes(layout: qi_layout, dtype: int, n_head: int) -> int:
    return lib().qi_attn_full_workspace_bytes(ctypes.byref(layout), dtype, n_head)


def qi_attn_cached_workspace_bytes(dtype: int, T: int, n_head: int) -> int:
    return lib().qi_attn_cached_workspace_bytes(dtype, T, n_head)


def qi_kvcache_bytes(cache_dtype: int, n_layers: int, n_head: int, p_cap: int) -> int:
    return lib().qi_kvcache_bytes(cache_dtype, n_layers, n_head, p_cap)


def qi_rope3d_apply(x, dtype: int, n_tok: int, n_head: int, tok_stride: int, cos_t, sin_t, rms_w, eps: float,
                    stream=None) -> int:
    return lib().qi_rope3d_apply(_p(x), dtype, n_tok, n_head, tok_stride, _p(cos_t), _p(sin_t), _p(rms_w), eps,
                                 _p(stream))


def qi_attn_blockcausal_full(io: qi_qkv, prep: Optional[qi_qkprep], layout: qi_layout, scale: float,
                             cache: Optional[qi_kvcache], layer: int, workspace, workspace_bytes: int,
                             stream=None) -> int:
    return lib().qi_attn_blockcausal_full(ctypes.byref(io), _ref(prep), ctypes.byref(layout), scale, _ref(cache),
                                          layer, _p(workspace), workspace_bytes, _p(stream))


def qi_attn_prefix_store(k, v, dtype: int, P: int, n_head: int, tok_stride: int, prep: Optional[qi_qkprep],
                         cache: qi_kvcache, layer: int, range_flags=None, stream=None) -> int:
    return lib().qi_attn_prefix_store(_p(k), _p(v), dtype, P, n_head, tok_stride, _ref(prep), _ref(cache), layer,
                                      _p(range_flags), _p(stream))


def qi_attn_target_cached(io: qi_qkv, prep: Optional[qi_qkprep], cache: qi_kvcache, layer: int, P: int,
                          scale: float, workspace, workspace_bytes: int, stream=None) -> int:
    return lib().qi_attn_target_cached(ctypes.byref(io), _ref(prep), _ref(cache), layer, P, scale, _p(workspace),
                                       workspace_bytes, _p(stream))


def qi_attn_target_cached_noalloc(io: qi_qkv, prep: Optional[qi_qkprep], cache: qi_kvcache, layer: int, P: int,
                                  scale: float, stream=None) -> int:
    return lib().qi_attn_target_cached_noalloc(ctypes.byref(io), _ref(prep), _ref(cache), layer, P, scale,
                                               _p(stream))


def qi_attn_tiled_workspace_bytes(layout: qi_layout, n_head: int) -> int:
    return lib().qi_attn_tiled_workspace_bytes(ctypes.byref(layout), n_head)


def qi_gemm_qkv_tiles(x, ldx: int, w, bias, q_out, ldq: int, M: int, n_head: int, K: int, dtype: int, row0: int,
                      P: int, T: int, fold: Optional[qi_norm_fold], prep: Optional[qi_qkprep],
                      cache: Optional[qi_kvcache], layer: int, target: Optional[qi_kvtiles], range_flags=None,
                      stream=None) -> int:
    return lib().qi_gemm_qkv_tiles(_p(x), ldx, _p(w), _p(bias), _p(q_out), ldq, M, n_head, K, dtype, row0, P, T,
                                   _ref(fold), _ref(prep), _ref(cache), layer, _ref(target), _p(range_flags),
                                   _p(stream))


def qi_attn_target_cached_tiled(io: qi_qkv, prep: Optional[qi_qkprep], cache: qi_kvcache, layer: int, P: int,
                                scale: float, target: qi_kvtiles, workspace, workspace_bytes: int, stream=None) -> int:
    return lib().qi_attn_target_cached_tiled(ctypes.byref(io), _ref(prep), _ref(cache), layer, P, scale,
                                             _ref(target), _p(workspace), workspace_bytes, _p(stream))


def qi_attn_blockcausal_full_tiled(io: qi_qkv, prep: Optional[qi_qkprep], layout: qi_layout, scale: float,
                                   cache: qi_kvcache, layer: int, target: qi_kvtiles, workspace,
                                   workspace_bytes: int, stream=None) -> int:
    return lib().qi_attn_blockcausal_full_tiled(ctypes.byref(io), _ref(prep), ctypes.byref(layout), scale,
                                                _ref(cache), layer, _ref(target), _p(workspace), workspace_bytes,
                                                _p(stream))


def qi_euler_step(x, v, v_dtype: int, n: int, sigma_k: float, sigma_k1: float, stream=None) -> int:
    return lib().qi_euler_step(_p(x), _p(v), v_dtype, n, sigma_k, sigma_k1, _p(stream))


def qi_gemm_bf16(x, ldx: int, w, out, ldo: int, M: int, N: int, K: int, epilogue: int, gate=None, row0: int = 0,
                 P: int = 0, stream=None) -> int:
    return lib().qi_gemm_bf16(_p(x), ldx, _p(w), _p(out), ldo, M, N, K, epilogue, _p(gate), row0, P, _p(stream))


def qi_gemm_bf16_ex(x, ldx: int, w, out, ldo: int, M: int, N: int, K: int, epilogue: int, gate=None, row0: int = 0,
                    P: int = 0, tile_n: int = 0, stream=None) -> int:
    return lib().qi_gemm_bf16_ex(_p(x), ldx, _p(w), _p(out), ldo, M, N, K, epilogue, _p(gate), row0, P, tile_n,
                                 _p(stream))


def qi_gemm_bf16_bias(x, ldx: int, w, bias, out, ldo: int, M: int, N: int, K: int, epilogue: int, gate=None,
                      row0: int = 0, P: int = 0, stream=None) -> int:
    return lib().qi_gemm_bf16_bias(_p(x), ldx, _p(w), _p(bias), _p(out), ldo, M, N, K, epilogue, _p(gate), row0, P,
                                   _p(stream))


def qi_layernorm_mod(x, ldx: int, out, ldo: int, M: int, D: int, scale=None, shift=None, row0: int = 0, P: int = 0,
                     eps: float = 1e-6, stream=None) -> int:
    return lib().qi_layernorm_mod(_p(x), ldx, _p(out), ldo, M, D, _p(scale), _p(shift), row0, P, eps, _p(stream))


def qi_linear_small_bias(x, n_vec: int, I: int, w, bias, O: int, silu_in: bool, y, stream=None) -> int:
    return lib().qi_linear_small_bias(_p(x), n_vec, I, _p(w), _p(bias), O, 1 if silu_in else 0, _p(y), _p(stream))


def qi_zc_rmsnorm_mod(x, ldx: int, out, ldo: int, M: int, D: int, w=None, scale=None, shift=None, row0: int = 0,
                      P: int = 0, eps: float = 1e-6, stream=None) -> int:
    return lib().qi_zc_rmsnorm_mod(_p(x), ldx, _p(out), ldo, M, D, _p(w), _p(scale), _p(shift), row0, P, eps,
                                   _p(stream))


def qi_timestep_embed(t, n: int, dim: int, out, stream=None) -> int:
    return lib().qi_timestep_embed(_p(t), n, dim, _p(out), _p(stream))


def qi_linear_small(x, n_vec: int, I: int, w, O: int, silu_in: bool, y, stream=None) -> int:
    return lib().qi_linear_small(_p(x), n_vec, I, _p(w), O, 1 if silu_in else 0, _p(y), _p(stream))


def qi_cast_bf16(x, y, n: int, stream=None) -> int:
    return lib().qi_cast_bf16(_p(x), _p(y), n, _p(stream))


def qi_gemm(x, ldx: int, w, bias, out, ldo: int, M: int, N: int, K: int, dtype: int, epilogue: int, gate=None,
            row0: int = 0, P: int = 0, tile_n: int = 0, range_flags=None, stream=None) -> int:
    return lib().qi_gemm(_p(x), ldx, _p(w), _p(bias), _p(out), ldo, M, N, K, dtype, epilogue, _p(gate), row0, P,
                         tile_n, _p(range_flags), _p(stream))


def qi_norm_mod(x, ldx: int, out, ldo: int, M: int, D: int, w=None, scale=None, shift=None, row0: int = 0,
                P: int = 0, eps: float = 1e-6, center: int = 0, out_dtype: int = QI_BF16, range_flags=None,
                stream=None) -> int:
    return lib().qi_norm_mod(_p(x), ldx, _p(out), ldo, M, D, _p(w), _p(scale), _p(shift), row0, P, eps, center,
                             out_dtype, _p(range_flags), _p(stream))


def qi_cast(x, y, n: int, dtype: int, range_flags=None, stream=None) -> int:
    return lib().qi_cast(_p(x), _p(y), n, dtype, _p(range_flags), _p(stream))


def make_norm_fold(sumsq=None, eps: float = 1e-6, bias_t=None, xc=None, ldxc: int = 0, next_w=None,
                   next_scale=None, sumsq_out=None) -> qi_norm_fold:
    return qi_norm_fold(_p(sumsq), eps, _p(bias_t), _p(xc), ldxc, _p(next_w), _p(next_scale), _p(sumsq_out))


def qi_gemm_norm_fold(x, ldx: int, w, bias, out, ldo: int, M: int, N: int, K: int, dtype: int, epilogue: int,
                      gate=None, row0: int = 0, P: int = 0, tile_n: int = 0, fold: Optional[qi_norm_fold] = None,
                      range_flags=None, stream=None) -> int:
    return lib().qi_gemm_norm_fold(_p(x), ldx, _p(w), _p(bias), _p(out), ldo, M, N, K, dtype, epilogue, _p(gate),
                                   row0, P, tile_n, ctypes.byref(fold) if fold is not None else None,
                                   _p(range_flags), _p(stream))


def qi_norm_fold_rows(x, ldx: int, xc, ldxc: int, sumsq_out, M: int, D: int, w=None, scale=None, row0: int = 0,
                      P: int = 0, dtype: int = QI_F16, range_flags=None, stream=None) -> int:
    return lib().qi_norm_fold_rows(_p(x), ldx, _p(xc), ldxc, _p(sumsq_out), M, D, _p(w), _p(scale), row0, P, dtype,
                                   _p(range_flags), _p(stream))


def qi_linear_multi(x, n_vec: int, I: int, w, w_dtype: int, O: int, y, stream=None) -> int:
    return lib().qi_linear_multi(_p(x), n_vec, I, _p(w), w_dtype, O, _p(y), _p(stream))


def qi_kernel_timing(enable: bool) -> int:
    return lib().qi_kernel_timing(1 if enable else 0)


def qi_kernel_timing_read():
    ms, n = c_double(), c_int64()
    check(lib().qi_kernel_timing_read(ctypes.byref(ms), ctypes.byref(n)), "qi_kernel_timing_read")
    return ms.value, n.value


def qi_kernel_timing_read_each():
    """Per-call elapsed milliseconds of the recorded attention calls, in launch order."""
    n = c_int64()
    check(lib().qi_kernel_timing_read_each(None, 0, ctypes.byref(n)), "qi_kernel_timing_read_each")
    buf = (c_float * max(n.value, 1))()
    check(lib().qi_kernel_timing_read_each(buf, n.value, ctypes.byref(n)), "qi_kernel_timing_read_each")
    return [buf[i] for i in range(n.value)]
