"""CPU tests of libqi's host side: exports, host helpers bit-exact against the oracle, and
argument checks that must fail before anything is launched (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import qi_inputs as qin
from oracle import qi_oracle as O

Q = pytest.importorskip("image_generation_qi_amd.qi")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

try:
    Q.lib()
    HAVE_LIB = True
except Q.QiLibraryMissing:
    HAVE_LIB = False

pytestmark = pytest.mark.skipif(not HAVE_LIB, reason="libqi.so not built")

EDGE_LAYOUTS = {
    "odd_grids": (qin.text(5), qin.image(5, 3, 1), qin.image(3, 7, 0)),
    "one_token_segments": (qin.text(1), qin.image(1, 1, 2), qin.image(1, 1, 0)),
    "target_only": (qin.image(9, 11, 0),),
    "two_text_runs": (qin.text(7), qin.image(4, 6, 1), qin.text(13), qin.image(2, 2, 2), qin.image(6, 5, 0)),
    "bidir_text": (qin.text(70, bidir=True), qin.image(8, 8, 1), qin.image(10, 12, 0)),
    "ragged_tiles": (qin.text(77), qin.image(13, 9, 1), qin.image(15, 17, 0)),
}


def header_functions():
    src = open(os.path.join(ROOT, "include", "qi.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int64_t|int)\s+(qi_\w+)\s*\(", src, re.M)))


def all_layouts():
    out = {k: w.segments for k, w in qin.WORKLOADS.items()}
    out.update(EDGE_LAYOUTS)
    return out


def test_every_declared_symbol_is_exported_and_bound():
    names = header_functions()
    assert len(names) >= 17
    lib = ctypes.CDLL(Q.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in qi.h but not exported"
    assert sorted(Q.exported_symbols()) == names


def test_status_strings_and_version():
    assert Q.qi_version() == Q.QI_ABI_VERSION
    for st in range(0, -8, -1):
        assert Q.qi_status_str(st).startswith("QI_")
    assert "unknown" in Q.qi_status_str(-99)


@pytest.mark.parametrize("name", sorted(all_layouts()))
def test_positions_bit_exact(name):
    segs = all_layouts()[name]
    L = Q.make_layout(segs)
    S, P, T = Q.qi_layout_tokens(L)
    assert (S, P, T) == O.split_counts(segs)
    pos = np.zeros((S, 3), np.int32)
    Q.check(Q.qi_rope3d_positions(L, pos))
    assert np.array_equal(pos.astype(np.int64), O.positions(segs))


def test_positions_text_pos0_override():
    segs = EDGE_LAYOUTS["two_text_runs"]
    L = Q.make_layout(segs, text_pos0=100)
    S, _, _ = Q.qi_layout_tokens(L)
    pos = np.zeros((S, 3), np.int32)
    Q.check(Q.qi_rope3d_positions(L, pos))
    assert np.array_equal(pos.astype(np.int64), O.positions(segs, text_pos0=100))


@pytest.mark.parametrize("name", ["tiny_f32", "txt256_ref32_tgt32", "txt512_tgt64", "txt1024_4ref64_tgt64", "odd_grids", "two_text_runs", "bidir_text"])
def test_rope_tables_bit_exact(name):
    segs = all_layouts()[name]
    L = Q.make_layout(segs)
    S, _, _ = Q.qi_layout_tokens(L)
    c = np.empty((S, 64), np.float32)
    s = np.empty((S, 64), np.float32)
    Q.check(Q.qi_rope3d_tables(L, c, s))
    rc, rs = O.rope_tables_f32(O.positions(segs))
    bad = np.count_nonzero(c.view(np.uint32) != rc.view(np.uint32)) + np.count_nonzero(s.view(np.uint32) != rs.view(np.uint32))
    assert bad == 0, f"{bad} table entries differ from the oracle's once-rounded values"


def test_rope_tables_other_theta_and_bands():
    segs = EDGE_LAYOUTS["odd_grids"]
    L = Q.make_layout(segs, bands=(32, 48, 48), theta=500.0)
    S, _, _ = Q.qi_layout_tokens(L)
    c = np.empty((S, 64), np.float32)
    s = np.empty((S, 64), np.float32)
    Q.check(Q.qi_rope3d_tables(L, c, s))
    rc, rs = O.rope_tables_f32(O.positions(segs), bands=(32, 48, 48), theta=500.0)
    assert np.array_equal(c.view(np.uint32), rc.view(np.uint32)) and np.array_equal(s.view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("name", ["tiny_f32", "txt256_ref32_tgt32", "txt512_tgt64"] + sorted(EDGE_LAYOUTS))
@pytest.mark.parametrize("tiles", [(128, 64), (1, 64), (7, 5), (64, 64), (2, 2)])
def test_blockmap_bit_exact(name, tiles):
    segs = all_layouts()[name]
    tq, tk = tiles
    L = Q.make_layout(segs)
    S, _, _ = Q.qi_layout_tokens(L)
    if S > 3000 and tiles in ((7, 5), (2, 2)):
        pytest.skip("dense oracle map too slow at this tile count")
    out = np.zeros(((S + tq - 1) // tq, (S + tk - 1) // tk), np.uint8)
    Q.check(Q.qi_blockmap(L, tq, tk, out))
    assert np.array_equal(out, O.blockmap(O.mask_dense(segs), tq, tk))


def _oracle_blockmap_by_rows(segs, tq, tk):
    """The oracle's tile map of a full-size layout, one query tile at a time: O.blockmap over the
    rows of O.mask_rows (the dense mask of 21,504 tokens would take 460 MB)."""
    S = sum(g.n_tokens for g in segs)
    rows = []
    for i in range(0, S, tq):
        m = O.mask_rows(segs, np.arange(i, min(i + tq, S)))
        rows.append(O.blockmap(m, tq, tk))
    return np.concatenate(rows, axis=0)


@pytest.mark.parametrize("name", ["txt1024_4ref64_tgt64", "txt512_4ref64_tgt64", "txt512_10ref32_tgt64"])
@pytest.mark.parametrize("tiles", [(256, 64), (64, 64)])
def test_blockmap_bit_exact_full_size(name, tiles):
    # the Block-Causal tile map ([OV] card 3C) of the headline and full-layer workloads, at the
    # attention kernel's tile and at a square tile, bit for bit against the oracle's mask
    segs = qin.WORKLOADS[name].segments
    tq, tk = tiles
    L = Q.make_layout(segs)
    S, _, _ = Q.qi_layout_tokens(L)
    out = np.zeros(((S + tq - 1) // tq, (S + tk - 1) // tk), np.uint8)
    Q.check(Q.qi_blockmap(L, tq, tk, out))
    ref = _oracle_blockmap_by_rows(segs, tq, tk)
    assert np.array_equal(out, ref)
    # all three classes occur: skipped tiles above the diagonal blocks, full and mixed tiles
    assert set(np.unique(ref).tolist()) == {0, 1, 2}


def test_tile_shape_and_sizes():
    assert Q.qi_attn_tile_shape(Q.QI_BF16) == (256, 64)
    assert Q.qi_attn_tile_shape(Q.QI_F16) == (256, 64)     # fp16 I/O runs the same kernels
    for T in (64, 1024, 4096, 5000):
        assert Q.qi_attn_cached_workspace_bytes(Q.QI_F16, T, 24) == Q.qi_attn_cached_workspace_bytes(Q.QI_BF16, T, 24)
    assert Q.qi_attn_tile_shape(Q.QI_F32) == (1, 64)
    # schedules: (key chunks, whole tiles per XCD run, chunked tiles)
    assert Q.qi_attn_schedule(4096, 24) == (2, 32, 128)     # 384 tiles: 48 per XCD
    assert Q.qi_attn_schedule(1024, 24) == (5, 0, 96)       # 96 tiles: 12 per XCD, all chunked
    assert Q.qi_attn_schedule(16384, 24) == (1, 192, 0)     # six whole rounds
    assert Q.qi_attn_schedule(8704, 24) == (5, 96, 48)      # 816 tiles: 102 per XCD
    assert Q.qi_attn_schedule(101 * 256, 5) == (1, 32, 0)   # 505 tiles: the remaining 32 / 31 run whole
    assert Q.qi_attn_schedule(0, 24) == (1, 0, 0)
    # with the key counts: a chunk round costs about 8.5 key tiles more, so short key ranges take
    # fewer chunks (never more than the key-independent count the workspaces are sized for)
    assert Q.qi_attn_schedule(4096, 24, 17408, 4096) == (2, 32, 128)   # 336 key tiles: unchanged
    assert Q.qi_attn_schedule(1024, 24, 1280, 1024) == (2, 0, 96)      # 36 key tiles: 1 round of 2 chunks, not 2 of 5
    assert Q.qi_attn_schedule(512, 24, 0, 512) == (5, 0, 48)           # 8 key tiles: 5 chunks still fit one round
    assert Q.qi_attn_schedule(1024, 24, 0, 0) == Q.qi_attn_schedule(1024, 24)
    L3 = Q.make_layout(qin.WORKLOADS["txt1024_4ref64_tgt64"].segments)
    PART = 256 * (128 * 2 + 4 * 4)   # partials of one chunk of one query tile: 256 rows x (128 fp16 + fp32 max, sum, scale, pad)
    # 4096-token target: 16 x 24 = 384 query tiles (48 per XCD): per XCD 32 whole, 16 in 2 key
    # chunks: K/V fp16 rows plus the partials of the 128 chunked tiles
    # (the block-causal prefix rows of step 1 run whole)
    assert Q.qi_attn_full_workspace_bytes(L3, Q.QI_BF16, 24) == 2 * 24 * 21504 * 128 * 2 + 128 * 2 * PART
    assert Q.qi_attn_cached_workspace_bytes(Q.QI_BF16, 4096, 24) == 2 * 24 * 4096 * 128 * 2 + 128 * 2 * PART
    # text 256 + 32x32 reference + 32x32 target: 4 x 24 = 96 units (12 per XCD, none whole) -> all in 5 key chunks
    L1 = Q.make_layout(qin.WORKLOADS["txt256_ref32_tgt32"].segments)
    assert Q.qi_attn_cached_workspace_bytes(Q.QI_BF16, 1024, 24) == 2 * 24 * 1024 * 128 * 2 + 96 * 5 * PART
    assert Q.qi_attn_full_workspace_bytes(L1, Q.QI_BF16, 24) == 2 * 24 * 2304 * 128 * 2 + 96 * 5 * PART
    # unmasked Edit-Plus (text 512 + target + 2 references of 64 x 64): the 8,704 prefix rows
    # (34 x 24 = 816 tiles, 102 per XCD: 96 whole, 6 in 5 chunks) share the partials with the
    # target rows, which need more
    Lv = Q.make_layout(qin.V1_WORKLOADS["editplus_v1"].segments, attention=Q.QI_ATTN_FULL)
    assert Q.qi_layout_tokens(Lv)[1:] == (8704, 4096)
    assert Q.qi_attn_full_workspace_bytes(Lv, Q.QI_BF16, 24) == 2 * 24 * 12800 * 128 * 2 + 128 * 2 * PART
    # with 2 heads the prefix partials are the larger: 68 tiles (8 or 9 per XCD, all in 7 chunks)
    assert Q.qi_attn_full_workspace_bytes(Lv, Q.QI_BF16, 2) == 2 * 2 * 12800 * 128 * 2 + 68 * 7 * PART
    # long targets stay whole: 16384 tokens x 24 heads = 1536 query tiles (six rounds)
    assert Q.qi_attn_cached_workspace_bytes(Q.QI_BF16, 16384, 24) == 2 * 24 * 16384 * 128 * 2
    # workspace rows are padded to whole 64-key tiles for both dtypes
    assert Q.qi_attn_cached_workspace_bytes(Q.QI_F32, 16, 2) == 2 * 2 * 64 * 128 * 4
    assert Q.qi_attn_full_workspace_bytes(L3, Q.QI_F32, 2) == 2 * 2 * 21504 * 128 * 4
    assert Q.qi_kvcache_bytes(Q.QI_F16, 32, 24, 17408) == 32 * 24 * 17408 * 128 * 2
    # fp16 caches hold whole 64-key tiles (V transposed per tile); fp32 caches are unpadded
    assert Q.qi_kvcache_bytes(Q.QI_F16, 2, 3, 100) == 2 * 3 * 128 * 128 * 2
    assert Q.qi_kvcache_bytes(Q.QI_F32, 2, 3, 100) == 2 * 3 * 100 * 128 * 4
    # ragged prefix and target: each padded to whole tiles in the workspace
    Lr = Q.make_layout((qin.text(77), qin.image(13, 9, 1), qin.image(15, 17, 0)))
    assert Q.qi_attn_full_workspace_bytes(Lr, Q.QI_BF16, 2) >= 2 * 2 * (256 + 256) * 128 * 2
    assert Q.qi_kvcache_bytes(Q.QI_BF16, 1, 1, 1) == Q.QI_ERR_DTYPE


# ---------------------------------------------------------------------------------------------
# argument checks forced from the host: each returns its status before any launch
# ---------------------------------------------------------------------------------------------
FAKE = 0x7F0000000000  # aligned, never dereferenced (every case below fails a check first)


def _good(T=64, H=2, dtype=Q.QI_BF16):
    io = Q.qi_qkv(FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000, dtype, T, H, H * 128)
    prep = Q.make_prep(FAKE + 0x4000, FAKE + 0x5000)
    cache = Q.qi_kvcache(FAKE + 0x6000, FAKE + 0x7000, Q.QI_F16 if dtype == Q.QI_BF16 else Q.QI_F32, 4, H, 100)
    return io, prep, cache


def _cached(io, prep, cache, layer=0, P=50, ws=FAKE + 0x8000, wsb=1 << 40):
    return Q.qi_attn_target_cached(io, prep, cache, layer, P, 0.0, ws, wsb, None)


@pytest.mark.parametrize("case,want", [
    ("null_q", Q.QI_ERR_ARG), ("null_o", Q.QI_ERR_ARG), ("bad_dtype", Q.QI_ERR_DTYPE),
    ("f16_io_f32_cache", Q.QI_ERR_DTYPE), ("stride_small", Q.QI_ERR_SHAPE), ("zero_tokens", Q.QI_ERR_SHAPE),
    ("misaligned", Q.QI_ERR_ALIGN), ("stride_not8", Q.QI_ERR_ALIGN), ("layer_oob", Q.QI_ERR_CAPACITY),
    ("layer_neg", Q.QI_ERR_CAPACITY), ("P_over_cap", Q.QI_ERR_CAPACITY), ("cache_dtype", Q.QI_ERR_DTYPE),
    ("cache_heads", Q.QI_ERR_SHAPE), ("ws_small", Q.QI_ERR_CAPACITY), ("ws_null", Q.QI_ERR_ARG),
    ("cos_without_sin", Q.QI_ERR_ARG), ("null_cache", Q.QI_ERR_ARG), ("bad_eps", Q.QI_ERR_ARG),
    ("prefix_over_max", Q.QI_ERR_SHAPE), ("target_over_max", Q.QI_ERR_SHAPE), ("lse_misaligned", Q.QI_ERR_ALIGN),
])
def test_target_cached_rejects(case, want):
    io, prep, cache = _good()
    kw = {}
    if case == "null_q": io.q = None
    elif case == "null_o": io.o = None
    elif case == "bad_dtype": io.dtype = 7
    elif case == "f16_io_f32_cache":   # fp16 I/O takes the fp16 cache
        io.dtype = Q.QI_F16
        cache.dtype = Q.QI_F32
    elif case == "stride_small": io.tok_stride = 128
    elif case == "zero_tokens": io.n_tok = 0
    elif case == "misaligned": io.k = FAKE + 0x1008
    elif case == "stride_not8": io.tok_stride = 2 * 128 + 4
    elif case == "layer_oob": kw["layer"] = 4
    elif case == "layer_neg": kw["layer"] = -1
    elif case == "P_over_cap": kw["P"] = 101
    elif case == "cache_dtype": cache.dtype = Q.QI_BF16
    elif case == "cache_heads": cache.n_head = 3
    elif case == "ws_small": kw["wsb"] = 10
    elif case == "ws_null": kw["ws"] = None
    elif case == "cos_without_sin": prep.sin_t = None
    elif case == "null_cache": cache = None
    elif case == "bad_eps":
        prep.q_rms_w = FAKE + 0x9000
        prep.eps = float("nan")
    elif case == "prefix_over_max":   # within the cache's capacity, past what 32-bit offsets reach
        cache.p_cap = 1 << 24
        kw["P"] = Q.QI_MAX_SOURCE_KEYS + 1
    elif case == "target_over_max":
        io.n_tok = Q.QI_MAX_SOURCE_KEYS + 1
    elif case == "lse_misaligned":
        io.lse = FAKE + 0xA002
    if case == "null_cache":
        st = Q.lib().qi_attn_target_cached(ctypes.byref(io), ctypes.byref(prep), None, 0, 50, 0.0, FAKE, 1 << 40, None)
    else:
        st = _cached(io, prep, cache, **kw)
    assert st == want, (case, Q.qi_status_str(st))


@pytest.mark.parametrize("case,want", [
    ("head_dim", Q.QI_ERR_LAYOUT), ("bands_sum", Q.QI_ERR_LAYOUT), ("bands_odd", Q.QI_ERR_LAYOUT),
    ("text_last", Q.QI_ERR_LAYOUT), ("grid_mismatch", Q.QI_ERR_LAYOUT), ("bad_kind", Q.QI_ERR_LAYOUT),
    ("empty_seg", Q.QI_ERR_LAYOUT), ("wrong_S", Q.QI_ERR_SHAPE), ("theta_neg", Q.QI_ERR_LAYOUT),
])
def test_full_rejects_bad_layouts(case, want):
    segs = [qin.text(16), qin.image(4, 4, 1), qin.image(4, 4, 0)]
    bands, hd, theta = (16, 56, 56), 128, 10000.0
    S = 48
    if case == "head_dim": hd = 64
    elif case == "bands_sum": bands = (16, 56, 48)
    elif case == "bands_odd": bands = (15, 57, 56)
    elif case == "text_last": segs = segs + [qin.text(3)]; S = 51
    elif case == "grid_mismatch": segs[1] = qin.Segment(qin.SEG_IMAGE, 15, 1, 4, 4); S = 47
    elif case == "bad_kind": segs[0] = qin.Segment(9, 16)
    elif case == "empty_seg": segs[0] = qin.Segment(qin.SEG_TEXT, 0); S = 32
    elif case == "wrong_S": S = 47
    elif case == "theta_neg": theta = -1.0
    L = Q.make_layout(segs, hd, bands, theta)
    io = Q.qi_qkv(FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000, Q.QI_BF16, S, 2, 256)
    st = Q.qi_attn_blockcausal_full(io, None, L, 0.0, None, 0, FAKE + 0x8000, 1 << 40, None)
    assert st == want, (case, Q.qi_status_str(st))
    if want == Q.QI_ERR_LAYOUT:
        assert Q.lib().qi_layout_tokens(ctypes.byref(L), None, None, None) == Q.QI_ERR_LAYOUT


def test_full_rejects_sources_over_the_key_limit():
    # a prefix one key past the bf16 path's limit (fp32 I/O has no such limit, but this is bf16)
    n = Q.QI_MAX_SOURCE_KEYS + 1 - 16
    L = Q.make_layout([qin.text(n, bidir=True), qin.image(4, 4, 1), qin.image(4, 4, 0)])
    S = n + 32
    io = Q.qi_qkv(FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000, Q.QI_BF16, S, 2, 256)
    assert Q.qi_attn_blockcausal_full(io, None, L, 0.0, None, 0, FAKE + 0x8000, 1 << 40, None) == Q.QI_ERR_SHAPE
    assert Q.qi_layout_tokens(L)[1] == Q.QI_MAX_SOURCE_KEYS + 1
    # the header's limit is the binding's
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "qi.h")).read()
    assert re.search(r"#define QI_MAX_SOURCE_KEYS (\d+)", hdr).group(1) == str(Q.QI_MAX_SOURCE_KEYS)


def test_other_entry_points_reject():
    io, prep, cache = _good()
    # prefix store
    assert Q.qi_attn_prefix_store(FAKE, FAKE, Q.QI_BF16, 10, 2, 256, prep, cache, 7, None) == Q.QI_ERR_CAPACITY
    assert Q.qi_attn_prefix_store(FAKE, None, Q.QI_BF16, 10, 2, 256, prep, cache, 0, None) == Q.QI_ERR_ARG
    assert Q.qi_attn_prefix_store(FAKE, FAKE, Q.QI_BF16, -1, 2, 256, prep, cache, 0, None) == Q.QI_ERR_SHAPE
    assert Q.qi_attn_prefix_store(FAKE, FAKE, Q.QI_F32, 10, 2, 256, prep, cache, 0, None) == Q.QI_ERR_DTYPE
    # rope apply
    assert Q.qi_rope3d_apply(FAKE, Q.QI_BF16, 8, 2, 256, None, None, None, 1e-6, None) == Q.QI_ERR_ARG
    assert Q.qi_rope3d_apply(FAKE, Q.QI_BF16, 8, 2, 256, FAKE, None, None, 1e-6, None) == Q.QI_ERR_ARG
    assert Q.qi_rope3d_apply(FAKE + 2, Q.QI_BF16, 8, 2, 256, FAKE, FAKE, None, 1e-6, None) == Q.QI_ERR_ALIGN
    assert Q.qi_rope3d_apply(FAKE, 5, 8, 2, 256, FAKE, FAKE, None, 1e-6, None) == Q.QI_ERR_DTYPE
    # euler
    assert Q.qi_euler_step(None, FAKE, Q.QI_F32, 8, 1.0, 0.875, None) == Q.QI_ERR_ARG
    assert Q.qi_euler_step(FAKE, FAKE, Q.QI_F16, 8, 1.0, 0.875, None) == Q.QI_ERR_DTYPE
    assert Q.qi_euler_step(FAKE, FAKE, Q.QI_F32, -1, 1.0, 0.875, None) == Q.QI_ERR_SHAPE
    assert Q.qi_euler_step(FAKE + 1, FAKE, Q.QI_F32, 8, 1.0, 0.875, None) == Q.QI_ERR_ALIGN
    assert Q.qi_euler_step(FAKE, FAKE, Q.QI_F32, 8, float("inf"), 0.875, None) == Q.QI_ERR_ARG
    # host helpers
    L = Q.make_layout([qin.image(2, 2, 0)])
    assert Q.qi_rope3d_positions(L, None) == Q.QI_ERR_ARG
    assert Q.qi_blockmap(L, 0, 64, np.zeros(4, np.uint8)) == Q.QI_ERR_ARG
    assert Q.lib().qi_attn_tile_shape(9, ctypes.byref(ctypes.c_int32()), ctypes.byref(ctypes.c_int32())) == Q.QI_ERR_DTYPE
    i32 = lambda: ctypes.byref(ctypes.c_int32())
    assert Q.lib().qi_attn_schedule(-1, 24, 0, 0, i32(), i32(), i32()) == Q.QI_ERR_ARG
    assert Q.lib().qi_attn_schedule(4096, 0, 0, 0, i32(), i32(), i32()) == Q.QI_ERR_ARG
    assert Q.lib().qi_attn_schedule(4096, 24, -1, 0, i32(), i32(), i32()) == Q.QI_ERR_ARG
    assert Q.lib().qi_attn_schedule(4096, 24, 0, -64, i32(), i32(), i32()) == Q.QI_ERR_ARG
    assert Q.lib().qi_attn_schedule(4096, 24, 0, 0, None, i32(), i32()) == Q.QI_ERR_ARG


def test_full_attention_layout_maps_and_positions():
    segs = (qin.text(77), qin.image(13, 9, 0), qin.image(15, 17, 1), qin.image(4, 4, 2))
    Lf = Q.make_layout(segs, attention=Q.QI_ATTN_FULL)
    Lb = Q.make_layout(segs)
    S, P, T = Q.qi_layout_tokens(Lf)
    assert (S, P, T) == Q.qi_layout_tokens(Lb)
    for tq, tk in ((256, 64), (7, 5), (64, 64)):
        out = np.zeros(((S + tq - 1) // tq, (S + tk - 1) // tk), np.uint8)
        Q.check(Q.qi_blockmap(Lf, tq, tk, out))
        assert np.all(out == 1)
        assert np.array_equal(out, O.blockmap(O.mask_dense(segs, full=True), tq, tk))
    pf, pb = (np.zeros((S, 3), np.int32) for _ in range(2))
    Q.check(Q.qi_rope3d_positions(Lf, pf))
    Q.check(Q.qi_rope3d_positions(Lb, pb))
    assert np.array_equal(pf, pb)
    bad = Q.make_layout(segs, attention=7)
    n = [ctypes.c_int64() for _ in range(3)]
    assert Q.lib().qi_layout_tokens(ctypes.byref(bad), *(ctypes.byref(x) for x in n)) == Q.QI_ERR_LAYOUT


def test_layer_entry_points_reject():
    """Argument checks of the layer pieces run before any launch, so they answer without a GPU."""
    G = Q.lib().qi_gemm_bf16_ex
    big = 1 << 40
    ok = (FAKE, 256, FAKE, FAKE, 256, 64, 256, 256)
    assert G(None, *ok[1:], Q.QI_EPI_STORE, None, 0, 0, 0, None) == Q.QI_ERR_ARG
    assert G(*ok, 9, None, 0, 0, 0, None) == Q.QI_ERR_ARG
    assert G(*ok, Q.QI_EPI_GATED_RESIDUAL, None, 0, 0, 0, None) == Q.QI_ERR_ARG
    assert G(*ok, Q.QI_EPI_GATED_RESIDUAL_LINEAR, None, 0, 0, 0, None) == Q.QI_ERR_ARG
    assert G(*ok, Q.QI_EPI_STORE, None, 0, 0, 64, None) == Q.QI_ERR_ARG
    assert G(*ok, Q.QI_EPI_SWIGLU, None, 0, 0, 192, None) == Q.QI_ERR_ARG
    assert G(FAKE, 256, FAKE, FAKE, 256, 64, 256, 200, Q.QI_EPI_STORE, None, 0, 0, 0, None) == Q.QI_ERR_SHAPE
    assert G(FAKE, 128, FAKE, FAKE, 256, 64, 256, 256, Q.QI_EPI_STORE, None, 0, 0, 0, None) == Q.QI_ERR_SHAPE
    # 32-bit buffer offsets: the checks may not overflow for huge sizes either
    assert G(FAKE, 256, FAKE, FAKE, 256, 1 << 22, 256, 256, Q.QI_EPI_STORE, None, 0, 0, 0, None) == Q.QI_ERR_SHAPE
    assert G(FAKE, big, FAKE, FAKE, 256, big, 256, 256, Q.QI_EPI_STORE, None, 0, 0, 0, None) == Q.QI_ERR_SHAPE
    assert G(FAKE, 256, FAKE, FAKE, big, 64, big, 256, Q.QI_EPI_STORE, None, 0, 0, 0, None) == Q.QI_ERR_SHAPE
    assert G(FAKE + 8, *ok[1:], Q.QI_EPI_STORE, None, 0, 0, 0, None) == Q.QI_ERR_ALIGN
    assert G(FAKE, 260, FAKE, FAKE, 256, 64, 256, 256, Q.QI_EPI_STORE, None, 0, 0, 0, None) == Q.QI_ERR_ALIGN
    assert G(*ok, Q.QI_EPI_GATED_RESIDUAL, FAKE + 4, 0, 0, 0, None) == Q.QI_ERR_ALIGN
    assert Q.lib().qi_gemm_bf16_bias(FAKE, 256, FAKE, FAKE + 4, FAKE, 256, 64, 256, 256, Q.QI_EPI_STORE, None, 0, 0,
                                     None) == Q.QI_ERR_ALIGN  # bias
    # M == 0 is a no-op that launches nothing
    assert Q.lib().qi_gemm_bf16(FAKE, 256, FAKE, FAKE, 256, 0, 256, 256, Q.QI_EPI_STORE, None, 0, 0, None) == Q.QI_OK
    # norms
    N = Q.lib().qi_zc_rmsnorm_mod
    assert N(None, 256, FAKE, 256, 8, 256, None, None, None, 0, 0, 1e-6, None) == Q.QI_ERR_ARG
    assert N(FAKE, 256, FAKE, 256, 8, 258, None, None, None, 0, 0, 1e-6, None) == Q.QI_ERR_SHAPE
    assert N(FAKE, 128, FAKE, 256, 8, 256, None, None, None, 0, 0, 1e-6, None) == Q.QI_ERR_SHAPE
    assert N(FAKE, 256, FAKE, 256, -1, 256, None, None, None, 0, 0, 1e-6, None) == Q.QI_ERR_SHAPE
    assert N(FAKE, 256, FAKE, 256, 8, 256, None, None, None, 0, 0, -1.0, None) == Q.QI_ERR_ARG
    assert N(FAKE, 256, FAKE + 4, 256, 8, 256, None, None, None, 0, 0, 1e-6, None) == Q.QI_ERR_ALIGN
    assert N(FAKE, 256, FAKE, 256, 8, 256, FAKE + 4, None, None, 0, 0, 1e-6, None) == Q.QI_ERR_ALIGN
    LN = Q.lib().qi_layernorm_mod
    assert LN(None, 256, FAKE, 256, 8, 256, None, None, 0, 0, 1e-6, None) == Q.QI_ERR_ARG
    assert LN(FAKE, 256, FAKE, 256, 8, 6, None, None, 0, 0, 1e-6, None) == Q.QI_ERR_SHAPE
    assert LN(FAKE, 256, FAKE, 256, 8, 256, FAKE + 4, None, 0, 0, 1e-6, None) == Q.QI_ERR_ALIGN
    assert LN(FAKE, 256, FAKE, 256, 8, 256, None, None, 0, 0, float("nan"), None) == Q.QI_ERR_ARG
    # conditioning vectors and the latent cast
    T = Q.lib().qi_timestep_embed
    assert T(None, 2, 256, FAKE, None) == Q.QI_ERR_ARG
    assert T(FAKE, 2, 255, FAKE, None) == Q.QI_ERR_SHAPE
    assert T(FAKE, -1, 256, FAKE, None) == Q.QI_ERR_SHAPE
    assert T(FAKE, 1 << 30, 256, FAKE, None) == Q.QI_ERR_SHAPE
    assert T(FAKE + 2, 2, 256, FAKE, None) == Q.QI_ERR_ALIGN
    LS = Q.lib().qi_linear_small_bias
    assert LS(FAKE, 2, 256, None, None, 64, 1, FAKE, None) == Q.QI_ERR_ARG
    assert LS(FAKE, 5, 256, FAKE, None, 64, 1, FAKE, None) == Q.QI_ERR_SHAPE
    assert LS(FAKE, 2, 260, FAKE, None, 64, 1, FAKE, None) == Q.QI_ERR_SHAPE
    assert LS(FAKE, 2, 256, FAKE + 8, None, 64, 1, FAKE, None) == Q.QI_ERR_ALIGN
    assert LS(FAKE, 2, 256, FAKE, FAKE + 2, 64, 1, FAKE, None) == Q.QI_ERR_ALIGN
    assert LS(FAKE + 2, 2, 256, FAKE, None, 64, 1, FAKE, None) == Q.QI_ERR_ALIGN
    C = Q.lib().qi_cast_bf16
    assert C(None, FAKE, 8, None) == Q.QI_ERR_ARG
    assert C(FAKE, FAKE, -1, None) == Q.QI_ERR_SHAPE
    assert C(FAKE + 2, FAKE, 8, None) == Q.QI_ERR_ALIGN
    assert C(FAKE, FAKE + 1, 8, None) == Q.QI_ERR_ALIGN


def test_schedule_invariants_over_shapes():
    """For every shape: whole tiles come in whole rounds of the 32 CUs of an XCD and never exceed
    an XCD's share, a launch cuts tiles into 1..8 key chunks only when some remain after the whole
    rounds, exactly those remaining tiles are chunked, and the cached workspace holds the prepared
    K/V rows plus exactly their partials."""
    PART = 256 * (128 * 2 + 4 * 4)
    rng = np.random.default_rng(7)
    shapes = [(int(n), int(h)) for n, h in zip(rng.integers(1, 70000, 200), rng.integers(1, 48, 200))]
    shapes += [(256 * t, h) for t in (1, 2, 31, 32, 33) for h in (1, 8, 24, 40)]
    for n_q, heads in shapes:
        units = -(-n_q // 256) * heads
        chunks, whole, chunked = Q.qi_attn_schedule(n_q, heads)
        assert 1 <= chunks <= 8, (n_q, heads)
        assert whole % 32 == 0 and 8 * whole <= units, (n_q, heads)
        assert whole == 32 * ((units // 8) // 32), (n_q, heads)
        rest = units - 8 * whole
        assert chunked == (rest if chunks > 1 else 0), (n_q, heads)
        if rest == 0:
            assert chunks == 1
        rows = -(-n_q // 64) * 64
        assert Q.qi_attn_cached_workspace_bytes(Q.QI_BF16, n_q, heads) == 2 * heads * rows * 128 * 2 + chunked * chunks * PART, (n_q, heads)
        # with key counts: the same whole rounds, at most as many chunks, partials within the workspace's
        for n_keys_a in (0, 64, 1280, int(rng.integers(0, 40000))):
            kc, kw, kch = Q.qi_attn_schedule(n_q, heads, n_keys_a, n_q)
            assert 1 <= kc <= chunks and kw == whole, (n_q, heads, n_keys_a)
            assert kch == (rest if kc > 1 else 0), (n_q, heads, n_keys_a)
            assert kch * kc <= chunked * chunks, (n_q, heads, n_keys_a)


def test_norm_fold_entry_points_reject():
    # qi_gemm_norm_fold, qi_norm_fold_rows and qi_linear_multi: every case fails a check before
    # any launch (include/qi.h documents each status)
    G, F16 = Q.QI_EPI_GATED_RESIDUAL, Q.QI_F16

    def gemm(fold, epi=G, M=256, N=256, K=256, gate=FAKE):
        return Q.qi_gemm_norm_fold(FAKE, K, FAKE + 0x10000, None, FAKE + 0x20000, N, M, N, K, F16, epi, gate, 0, 0,
                                   0, fold, None, None)

    mk = Q.make_norm_fold
    prod = dict(xc=FAKE + 0x30000, ldxc=256, sumsq_out=FAKE + 0x40000)
    assert gemm(mk(**prod), epi=Q.QI_EPI_STORE, gate=None) == Q.QI_ERR_ARG          # producer on a store epilogue
    assert gemm(mk(xc=FAKE + 0x30000, ldxc=256)) == Q.QI_ERR_ARG                    # xc without sumsq_out
    assert gemm(mk(sumsq_out=FAKE + 0x40000)) == Q.QI_ERR_ARG                       # producer fields without xc
    assert gemm(mk(next_w=FAKE + 0x50000)) == Q.QI_ERR_ARG
    assert gemm(mk(sumsq=FAKE + 0x60000, eps=-1.0)) == Q.QI_ERR_ARG                 # negative eps
    assert gemm(mk(sumsq=FAKE + 0x60000, eps=float("nan"))) == Q.QI_ERR_ARG
    assert gemm(mk(xc=FAKE + 0x30000, ldxc=128, sumsq_out=FAKE + 0x40000)) == Q.QI_ERR_SHAPE   # ldxc < N
    assert gemm(mk(xc=FAKE + 0x30000, ldxc=260, sumsq_out=FAKE + 0x40000)) == Q.QI_ERR_ALIGN   # ldxc % 8
    assert gemm(mk(xc=FAKE + 0x30008, ldxc=256, sumsq_out=FAKE + 0x40000)) == Q.QI_ERR_ALIGN   # xc alignment
    assert gemm(mk(sumsq=FAKE + 0x60004)) == Q.QI_ERR_ALIGN
    assert gemm(mk(sumsq=FAKE + 0x60000, bias_t=FAKE + 0x70004)) == Q.QI_ERR_ALIGN
    assert gemm(mk(**prod, next_scale=FAKE + 0x50008)) == Q.QI_ERR_ALIGN
    assert gemm(mk(xc=FAKE + 0x30000, ldxc=256, sumsq_out=FAKE + 0x40002)) == Q.QI_ERR_ALIGN
    assert gemm(mk(), N=96) == Q.QI_ERR_SHAPE                                       # the plain checks still apply
    # the producing side for fp32 rows
    nf = Q.qi_norm_fold_rows
    assert nf(None, 256, FAKE, 256, FAKE, 8, 256) == Q.QI_ERR_ARG
    assert nf(FAKE, 256, FAKE, 256, None, 8, 256) == Q.QI_ERR_ARG
    assert nf(FAKE, 256, FAKE, 256, FAKE, 8, 256, dtype=Q.QI_F32) == Q.QI_ERR_DTYPE
    assert nf(FAKE, 256, FAKE, 256, FAKE, 8, 240) == Q.QI_ERR_SHAPE                 # D % 32
    assert nf(FAKE, 8192, FAKE, 8192, FAKE, 8, 8192) == Q.QI_ERR_SHAPE              # D > 4096
    assert nf(FAKE, 128, FAKE, 256, FAKE, 8, 256) == Q.QI_ERR_SHAPE                 # ldx < D
    assert nf(FAKE, 256, FAKE, 256, FAKE, -1, 256) == Q.QI_ERR_SHAPE
    assert nf(FAKE + 4, 256, FAKE, 256, FAKE, 8, 256) == Q.QI_ERR_ALIGN
    assert nf(FAKE, 256, FAKE + 4, 256, FAKE, 8, 256) == Q.QI_ERR_ALIGN
    assert nf(FAKE, 256, FAKE, 256, FAKE + 2, 8, 256) == Q.QI_ERR_ALIGN
    assert nf(FAKE, 256, FAKE, 256, FAKE, 8, 256, w=FAKE + 8) == Q.QI_ERR_ALIGN
    assert nf(FAKE, 256, FAKE, 256, FAKE, 0, 256) == Q.QI_OK                        # nothing to do, no launch
    # bias tables
    lm = Q.qi_linear_multi
    assert lm(None, 2, 256, FAKE, Q.QI_F16, 8, FAKE) == Q.QI_ERR_ARG
    assert lm(FAKE, 2, 256, FAKE, Q.QI_F32, 8, FAKE) == Q.QI_ERR_DTYPE
    assert lm(FAKE, 0, 256, FAKE, Q.QI_F16, 8, FAKE) == Q.QI_ERR_SHAPE
    assert lm(FAKE, 17, 256, FAKE, Q.QI_F16, 8, FAKE) == Q.QI_ERR_SHAPE
    assert lm(FAKE, 2, 260, FAKE, Q.QI_F16, 8, FAKE) == Q.QI_ERR_SHAPE
    assert lm(FAKE, 2, 256, FAKE, Q.QI_F16, -1, FAKE) == Q.QI_ERR_SHAPE
    assert lm(FAKE + 4, 2, 256, FAKE, Q.QI_F16, 8, FAKE) == Q.QI_ERR_ALIGN
    assert lm(FAKE, 2, 256, FAKE + 8, Q.QI_BF16, 8, FAKE) == Q.QI_ERR_ALIGN
    assert lm(FAKE, 2, 256, FAKE, Q.QI_BF16, 0, FAKE) == Q.QI_OK                    # no outputs, no launch


def test_norm_fold_producer_tile_and_width():
    # the producing side runs 256 x 192 tiles only; the header's partial-sum width is the binding's
    f = Q.make_norm_fold(xc=FAKE + 0x30000, ldxc=256, sumsq_out=FAKE + 0x40000)
    for tile in (128, 256):
        assert Q.qi_gemm_norm_fold(FAKE, 256, FAKE + 0x10000, None, FAKE + 0x20000, 256, 256, 256, 256, Q.QI_F16,
                                   Q.QI_EPI_GATED_RESIDUAL, FAKE, 0, 0, tile, f, None, None) == Q.QI_ERR_ARG
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "qi.h")).read()
    from image_generation_qi_amd import runtime as rt
    assert int(re.search(r"#define QI_FOLD_W (\d+)", hdr).group(1)) == rt.FOLD_W


def test_fused_qkv_entry_points_reject():
    # the fused QKV path's checks, all before any launch
    io, prep, cache = _good()
    L = Q.make_layout((qin.text(16), qin.image(4, 4, 0)))
    tiles = Q.qi_kvtiles(FAKE + 0x10000, FAKE + 0x20000, 2, 64)
    base = dict(x=FAKE, ldx=64, w=FAKE, bias=None, q_out=FAKE, ldq=256, M=32, n_head=2, K=64, dtype=Q.QI_F16,
                row0=0, P=16, T=16, fold=None, prep=None, cache=cache, layer=0, target=tiles)
    g = lambda **kw: Q.qi_gemm_qkv_tiles(**dict(base, **kw))
    assert g(x=None) == Q.QI_ERR_ARG
    assert g(dtype=Q.QI_F32) == Q.QI_ERR_DTYPE
    assert g(K=96, ldx=96) == Q.QI_ERR_SHAPE                 # K % 64
    assert g(M=33) == Q.QI_ERR_SHAPE                         # rows past P + T
    assert g(T=0) == Q.QI_ERR_SHAPE
    assert g(ldq=248) == Q.QI_ERR_SHAPE                      # below 128 n_head
    assert g(ldx=68, K=64) == Q.QI_ERR_ALIGN                 # ldx % 8
    assert g(q_out=FAKE + 8) == Q.QI_ERR_ALIGN
    assert g(cache=None) == Q.QI_ERR_ARG                     # prefix rows need the cache
    assert g(target=None) == Q.QI_ERR_ARG                    # target rows need the tile buffer
    assert g(target=Q.qi_kvtiles(FAKE, FAKE, 3, 64)) == Q.QI_ERR_SHAPE   # head count
    assert g(target=Q.qi_kvtiles(FAKE, FAKE, 2, 0)) == Q.QI_ERR_SHAPE    # rows below the key count
    assert g(layer=5) == Q.QI_ERR_CAPACITY
    assert g(fold=Q.make_norm_fold(None, 1e-6, None, FAKE, 64)) == Q.QI_ERR_ARG   # a producing side
    assert g(M=0) == Q.QI_OK                                 # nothing to do: no launch
    # the tiled attention entry points
    q1 = Q.qi_qkv(FAKE, None, None, FAKE + 0x3000, Q.QI_BF16, 16, 2, 256)
    ws = Q.qi_attn_tiled_workspace_bytes(L, 2)
    assert ws >= 0
    assert Q.qi_attn_target_cached_tiled(q1, None, cache, 0, 16, 0.0, None, FAKE, ws, None) == Q.QI_ERR_ARG
    assert Q.qi_attn_target_cached_tiled(q1, None, cache, 0, 16, 0.0, Q.qi_kvtiles(FAKE, FAKE, 2, 0), FAKE, ws,
                                         None) == Q.QI_ERR_SHAPE
    q32 = Q.qi_qkv(FAKE, None, None, FAKE + 0x3000, Q.QI_F32, 16, 2, 256)
    assert Q.qi_attn_target_cached_tiled(q32, None, cache, 0, 16, 0.0, tiles, FAKE, ws, None) == Q.QI_ERR_DTYPE
    qs = Q.qi_qkv(FAKE, None, None, FAKE + 0x3000, Q.QI_BF16, 31, 2, 256)   # n_tok != S
    assert Q.qi_attn_blockcausal_full_tiled(qs, None, L, 0.0, cache, 0, tiles, FAKE, ws, None) == Q.QI_ERR_SHAPE
    qf = Q.qi_qkv(FAKE, None, None, FAKE + 0x3000, Q.QI_BF16, 32, 2, 256)
    assert Q.qi_attn_blockcausal_full_tiled(qf, None, L, 0.0, None, 0, tiles, FAKE, ws, None) == Q.QI_ERR_ARG
    assert Q.qi_attn_tiled_workspace_bytes(L, 0) == Q.QI_ERR_SHAPE
