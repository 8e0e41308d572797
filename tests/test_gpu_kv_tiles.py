"""GPU parity of the fused QKV path: the QKV projection whose epilogue writes Q rows and K (per-head
RMSNorm, 3D rotation) and V as the attention's fp16 tiles, the prefix tokens into the cache and the
target tokens into a tile buffer (qi_gemm_qkv_tiles), and the attention entry points that take
those tiles (qi_attn_target_cached_tiled, qi_attn_blockcausal_full_tiled).  Called through the C
ABI; checked against the fp64 oracle on the same seeded inputs, and against the unfused entry
points bit for bit where both see the same tiles.

Tolerances (written here): Q, K and V are fp16 values of an fp32-accumulated projection, rounded
once: max|d| <= 1e-2 * max|ref| and sum|d| / sum|ref| <= 2e-3 (the 16-bit bar of the layer
tests).  Key slots past a source's last key in its last tile: exactly zero.  The tiles of a token
do not depend on which rows a call covers (step 1 against the cached step): bit-identical.
"""
import sys

import numpy as np
import pytest

import qi_inputs as qin
from oracle import qi_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from image_generation_qi_amd import qi as Q  # noqa: E402
from image_generation_qi_amd import runtime as rt  # noqa: E402

DEV = "cuda:0"
CFG = 93   # seed id of the ad-hoc shapes here


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    d = np.abs(got - ref)
    max_rel = d.max() / max(np.abs(ref).max(), 1e-300)
    mean_rel = d.sum() / max(np.abs(ref).sum(), 1e-300)
    say(f"  {what}: max_rel={max_rel:.3e} mean_rel={mean_rel:.3e}")
    assert max_rel <= 1e-2 and mean_rel <= 2e-3, (what, max_rel, mean_rel)


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def sync():
    torch.cuda.synchronize()


def dev16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).to(DEV)


def oracle_qkv(x64, w64, H, cos, sin, k_w, eps=1e-6):
    """Q, then K after the per-head RMSNorm (k_w None: none) and the rotation (cos None: none),
    then V, each [rows][H][128], from x W^T in fp64 (W in the Q | K | V row order)."""
    D = 128 * H
    y = O.linear(x64, w64)
    q = y[:, :D].reshape(-1, H, 128)
    k = O.prep_qk(y[:, D:2 * D].reshape(-1, H, 128), cos, sin, k_w, eps)
    v = y[:, 2 * D:].reshape(-1, H, 128)
    return q, k, v


def inputs(S, H, Kd, tag):
    x = qin.stored(qin.normal(CFG, 300 + tag, (S, Kd)), "f16")
    w = qin.linear_weight(CFG, 60 + tag, 3 * 128 * H, Kd)            # bf16-stored, N(0, 1/Kd)
    kw = qin.normal(CFG, 320 + tag, (128,), 0, 0, 1.0, 0.1).astype(np.float32)
    return x, w, kw


LAYOUTS = [
    # text 37 + 9 x 7 reference + 11 x 13 target: P = 100, T = 143 (both ragged), 3 heads
    ((qin.text(37), qin.image(9, 7, 1), qin.image(11, 13, 0)), 3, 192),
    # P = 64 (whole tiles), T = 128, 2 heads, the reduction over 3 slices
    ((qin.text(64), qin.image(8, 16, 0)), 2, 192),
    # 300 prefix tokens over two text runs, a 1-token target (one key, 63 zero slots), 4 heads
    ((qin.text(100), qin.image(10, 10, 1), qin.text(100), qin.image(1, 1, 0)), 4, 128),
]


@pytest.mark.parametrize("case", range(len(LAYOUTS)))
@pytest.mark.parametrize("norm,rot,dt", [(True, True, "f16"), (False, True, "f16"), (True, False, "f16"),
                                         (True, True, "bf16")])
def test_gemm_qkv_tiles_vs_oracle(case, norm, rot, dt):
    segments, H, Kd = LAYOUTS[case]
    L = rt.Layout(segments, DEV)
    S, P, T = L.S, L.P, L.T
    say(f"[qkv tiles] S={S} P={P} T={T} H={H} K={Kd} norm={norm} rot={rot} {dt}")
    x, w, kw = inputs(S, H, Kd, case)
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    if dt == "bf16":   # bf16 activations and weights: the operands as stored (bf16 MFMA), Q rows bf16
        x = qin.stored(x.f64, "bf16")
        xd = rt.from_bits(x.bits, "bf16", DEV)
    else:
        xd = dev16(x.f64)
    wt = rt.pack_qkv_tiles(rt.from_bits(w.bits, "bf16", DEV).to(tdt), H)
    cache = rt.KVCache(2, H, P, Q.QI_BF16, DEV)
    cache.k.fill_(float("nan"))
    cache.v.fill_(float("nan"))
    kvt = rt.KVTiles(T, H, DEV)
    kvt.k.fill_(float("nan"))
    kvt.v.fill_(float("nan"))
    q = torch.full((S, 128 * H), float("nan"), dtype=tdt, device=DEV)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    kwd = torch.from_numpy(kw).to(DEV) if norm else None
    rt.gemm_qkv_tiles(xd, wt, q, H, 0, P, T, cache, 1, kvt, L.rows(0, S) if rot else None, kwd, 1e-6, flags=flags)
    sync()
    c, s = O.rope_tables(O.positions(segments))
    # the weights the GPU multiplies (fp16 copies of the bf16 weights, or the bf16 weights as stored)
    wf16 = w.f64.astype(np.float16).astype(np.float64) if dt == "f16" else w.f64
    rq, rk, rv = oracle_qkv(x.f64, wf16, H, c if rot else None, s if rot else None,
                            kw.astype(np.float64) if norm else None)
    check(host(q).reshape(S, H, 128), rq, "Q")
    k_all = np.concatenate([host(cache.k_rows(1))[:, :P], host(kvt.k_rows())[:, :T]], axis=1)
    v_all = np.concatenate([host(cache.v_rows(1))[:, :P], host(kvt.v_rows())[:, :T]], axis=1)
    check(k_all.transpose(1, 0, 2), rk, "K")
    check(v_all.transpose(1, 0, 2), rv, "V")
    # the padding slots of both sources' last tiles are zero, layer 0 of the cache is untouched
    assert torch.all(cache.k_rows(1)[:, P:] == 0) and torch.all(cache.v_rows(1)[:, P:] == 0)
    assert torch.all(kvt.k_rows()[:, T:] == 0) and torch.all(kvt.v_rows()[:, T:] == 0)
    assert torch.all(torch.isnan(cache.k[0])) and torch.all(torch.isnan(cache.v[0]))
    assert int(flags.item()) == 0
    # the cached step's call over the target rows only writes the same target tiles, bit for bit
    k1, v1 = kvt.k.clone(), kvt.v.clone()
    kvt.k.fill_(float("nan"))
    kvt.v.fill_(float("nan"))
    q2 = torch.empty((T, 128 * H), dtype=tdt, device=DEV)
    rt.gemm_qkv_tiles(xd[P:], wt, q2, H, P, P, T, None, 0, kvt, L.rows(P, S) if rot else None, kwd, 1e-6)
    sync()
    assert torch.equal(kvt.k, k1) and torch.equal(kvt.v, v1)
    assert torch.equal(q2, q[P:])


def test_gemm_qkv_tiles_with_norm_fold_and_bias():
    # the consuming side of the norm fold (rrms from the partial sums, the class bias) ahead of the
    # K norm and the rotation: the Q, K and V of Linear(norm_mod(x)) + bias
    segments, H, Kd = (qin.text(40), qin.image(6, 6, 1), qin.image(8, 9, 0)), 2, 256
    L = rt.Layout(segments, DEV)
    S, P, T = L.S, L.P, L.T
    x_in = qin.normal(CFG, 340, (S, Kd)).astype(np.float32)
    nw = qin.normal(CFG, 341, (Kd,), 0, 0, 0.0, 0.1).astype(np.float32)
    sc = qin.normal(CFG, 342, (2, Kd), 0, 0, 0.0, 0.1).astype(np.float32)
    bias = qin.normal(CFG, 343, (2, 3 * 128 * H), 0, 0, 0.0, 0.3).astype(np.float32)
    _, w, kw = inputs(S, H, Kd, 7)
    wt = rt.pack_qkv_tiles(rt.from_bits(w.bits, "bf16", DEV).to(torch.float16), H)
    D3 = 3 * 128 * H
    perm = host(rt.pack_qkv_tiles(torch.arange(D3, dtype=torch.float32, device=DEV)[:, None], H))[:, 0].astype(int)
    xd = torch.from_numpy(x_in).to(DEV)
    xc = torch.empty((S, Kd), dtype=torch.float16, device=DEV)
    sq = torch.empty((S, rt.fold_parts(Kd)), dtype=torch.float32, device=DEV)
    rt.norm_fold_rows(xd, xc, sq, torch.from_numpy(nw).to(DEV), torch.from_numpy(sc).to(DEV), 0, P)
    bp = torch.from_numpy(bias[0][perm]).to(DEV)
    bt = torch.from_numpy(bias[1][perm]).to(DEV)
    cache = rt.KVCache(1, H, P, Q.QI_BF16, DEV)
    kvt = rt.KVTiles(T, H, DEV)
    q = torch.empty((S, 128 * H), dtype=torch.float16, device=DEV)
    rt.gemm_qkv_tiles(xc, wt, q, H, 0, P, T, cache, 0, kvt, L.rows(0, S), torch.from_numpy(kw).to(DEV), 1e-6,
                      bias=bp, fold=rt.NormFold(sq, 1e-6, bt))
    sync()
    h = O.norm_mod(x_in.astype(np.float64), nw.astype(np.float64), O.per_row(sc[0], sc[1], S, 0, P), 0.0 * sc[0])
    c, s = O.rope_tables(O.positions(segments))
    wf16 = w.f64.astype(np.float16).astype(np.float64)
    y = O.linear(h, wf16) + O.per_row(bias[0], bias[1], S, 0, P)
    D = 128 * H
    rq = y[:, :D].reshape(S, H, 128)
    rk = O.prep_qk(y[:, D:2 * D].reshape(S, H, 128), c, s, kw.astype(np.float64))
    rv = y[:, 2 * D:].reshape(S, H, 128)
    check(host(q).reshape(S, H, 128), rq, "Q (fold, bias)")
    k_all = np.concatenate([host(cache.k_rows(0))[:, :P], host(kvt.k_rows())[:, :T]], axis=1)
    v_all = np.concatenate([host(cache.v_rows(0))[:, :P], host(kvt.v_rows())[:, :T]], axis=1)
    check(k_all.transpose(1, 0, 2), rk, "K (fold, bias)")
    check(v_all.transpose(1, 0, 2), rv, "V (fold, bias)")


def test_gemm_qkv_tiles_range_flags():
    segments, H, Kd = (qin.text(16), qin.image(4, 4, 0)), 1, 64
    L = rt.Layout(segments, DEV)
    S, P, T = L.S, L.P, L.T
    x = torch.zeros((S, Kd), dtype=torch.float16, device=DEV)
    x[3, 0] = 256.0          # a prefix token
    w = torch.zeros((384, Kd), dtype=torch.float16, device=DEV)
    w[0, 0] = 512.0          # K_0 dim 0 (tile order): 131072, beyond fp16
    cache = rt.KVCache(1, H, P, Q.QI_BF16, DEV)
    kvt = rt.KVTiles(T, H, DEV)
    q = torch.empty((S, 128), dtype=torch.float16, device=DEV)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    rt.gemm_qkv_tiles(x, w, q, H, 0, P, T, cache, 0, kvt, None, None, flags=flags)
    sync()
    assert int(flags.item()) == Q.QI_RANGE_K
    w.zero_()
    w[128, 0] = 512.0        # V_0 dim 0
    flags.zero_()
    rt.gemm_qkv_tiles(x, w, q, H, 0, P, T, cache, 0, kvt, None, None, flags=flags)
    sync()
    assert int(flags.item()) == Q.QI_RANGE_V
    w.zero_()
    w[256, 0] = 0.25         # Q dim 0: in range
    flags.zero_()
    rt.gemm_qkv_tiles(x, w, q, H, 0, P, T, cache, 0, kvt, None, None, flags=flags)
    sync()
    assert int(flags.item()) == 0 and float(q[3, 0]) == 64.0


def _tiles_of(k_t, v_t, H, T, tables, k_w, eps=1e-6):
    """Target tiles prepared by the library's own K/V preparation (qi_attn_prefix_store into a
    one-layer cache of T keys, which has the tile buffer's layout)."""
    c = rt.KVCache(1, H, T, Q.QI_BF16, DEV)
    Q.check(Q.qi_attn_prefix_store(k_t, v_t, Q.QI_BF16, T, H, k_t.stride(0),
                                   Q.make_prep(tables[0], tables[1], None, k_w, eps), c.c, 0, None,
                                   rt.stream_handle(DEV)), "qi_attn_prefix_store")
    kvt = rt.KVTiles(T, H, DEV)
    kvt.k.copy_(c.k[0])
    kvt.v.copy_(c.v[0])
    return kvt


@pytest.mark.parametrize("name", ["txt256_ref32_tgt32", "txt512_tgt64"])
def test_attention_tiled_equals_unfused_bitwise(name):
    # given the same K/V tiles, the tiled entry points give the unfused ones' outputs bit for bit
    wl = qin.WORKLOADS[name]
    H = wl.n_head
    L = rt.Layout(wl.segments, DEV)
    S, P, T = L.S, L.P, L.T
    say(f"[attn tiled] {name} S={S} P={P} T={T}")
    q, k, v = (rt.from_bits(t.bits, "bf16", DEV) for t in qin.qkv(wl, S))
    qw, kw = (torch.from_numpy(a.astype(np.float32)).to(DEV) for a in qin.qk_norm_weights(wl))
    att = rt.Attention(L, H, Q.QI_BF16, DEV)
    cache = rt.KVCache(1, H, P, Q.QI_BF16, DEV)
    o_ref = att.full(q, k, v, qw, kw, cache=cache, layer=0)
    kvt = _tiles_of(k[P:], v[P:], H, T, L.rows(P, S), kw)
    o_t = att.full_tiled(q, cache, 0, kvt, qw)
    sync()
    assert torch.equal(o_t, o_ref)
    o_c = att.cached(q[P:], k[P:], v[P:], cache, 0, qw, kw)
    o_ct = att.cached_tiled(q[P:], cache, 0, kvt, qw)
    sync()
    assert torch.equal(o_ct, o_c)
    assert torch.equal(o_ct, o_ref[P:])   # the target rows of step 1 and of the cached step
    assert att.range_flags() == 0


def test_tiled_entry_points_refuse_bad_tiles():
    L = rt.Layout((qin.text(16), qin.image(4, 4, 0)), DEV)
    H = 2
    q = torch.zeros((L.S, H, 128), dtype=torch.bfloat16, device=DEV)
    o = torch.empty_like(q)
    cache = rt.KVCache(1, H, L.P, Q.QI_BF16, DEV)
    io = Q.make_qkv(q[L.P:], None, None, o, Q.QI_BF16, L.T, H, q.stride(0))
    small = Q.make_tiles(cache.k, cache.v, H, 0)               # rows below the key count
    other = Q.make_tiles(cache.k, cache.v, H + 1, 64)          # another head count
    st = rt.stream_handle(DEV)
    assert Q.qi_attn_target_cached_tiled(io, None, cache.c, 0, L.P, 0.0, small, None, 0, st) == Q.QI_ERR_SHAPE
    assert Q.qi_attn_target_cached_tiled(io, None, cache.c, 0, L.P, 0.0, other, None, 0, st) == Q.QI_ERR_SHAPE
    assert Q.qi_attn_target_cached_tiled(io, None, cache.c, 0, L.P, 0.0, None, None, 0, st) == Q.QI_ERR_ARG
    io32 = Q.make_qkv(q[L.P:], None, None, o, Q.QI_F32, L.T, H, q.stride(0))
    assert Q.qi_attn_target_cached_tiled(io32, None, cache.c, 0, L.P, 0.0, small, None, 0, st) == Q.QI_ERR_DTYPE
    x = torch.zeros((L.S, 64), dtype=torch.float16, device=DEV)
    w = torch.zeros((384 * H, 64), dtype=torch.float16, device=DEV)
    qo = torch.empty((L.S, 128 * H), dtype=torch.float16, device=DEV)
    kvt = rt.KVTiles(L.T, H, DEV)
    args = lambda **kw: dict(dict(x=x, ldx=64, w=w, bias=None, q_out=qo, ldq=128 * H, M=L.S, n_head=H, K=64,
                                  dtype=Q.QI_F16, row0=0, P=L.P, T=L.T, fold=None, prep=None, cache=cache.c, layer=0,
                                  target=kvt.c), **kw)
    g = lambda **kw: Q.qi_gemm_qkv_tiles(**args(**kw), stream=st)
    assert g(row0=1) == Q.QI_ERR_SHAPE                      # rows past the sequence
    assert g(cache=None) == Q.QI_ERR_ARG                    # prefix rows with no cache
    assert g(target=None) == Q.QI_ERR_ARG                   # target rows with no tile buffer
    assert g(row0=L.P, M=L.T, cache=None) == Q.QI_OK        # target rows only: no cache needed
    assert g(dtype=Q.QI_F32) == Q.QI_ERR_DTYPE
    assert g(ldq=128 * H - 8) == Q.QI_ERR_SHAPE
    assert g(K=96, ldx=96) == Q.QI_ERR_SHAPE
    prod = Q.make_norm_fold(None, 1e-6, None, qo, 128 * H, None, None, None)
    assert g(fold=prod) == Q.QI_ERR_ARG                     # a producing side
    sync()


@pytest.mark.parametrize("cached", [False, True])
def test_full_size_qkv_tiles_sampled(cached):
    # the 14,848-token workload (D = 3072, 24 heads, K = 3072): step 1 (every row) or the cached
    # step (the 4,096 target rows), Q, K and V of sampled tokens against the oracle
    wl = qin.WORKLOADS["txt512_10ref32_tgt64"]
    H, Kd = 24, 3072
    L = rt.Layout(wl.segments, DEV)
    S, P, T = L.S, L.P, L.T
    r0 = P if cached else 0
    n = S - r0
    say(f"[qkv tiles full] S={S} P={P} T={T} cached={cached}")
    x = qin.stored(qin.normal(CFG, 350, (n, Kd)), "f16")
    w = qin.linear_weight(CFG, 70, 3 * 128 * H, Kd)
    kw = qin.normal(CFG, 351, (128,), 0, 0, 1.0, 0.1).astype(np.float32)
    wt = rt.pack_qkv_tiles(rt.from_bits(w.bits, "bf16", DEV).to(torch.float16), H)
    cache = rt.KVCache(1, H, P, Q.QI_BF16, DEV)
    kvt = rt.KVTiles(T, H, DEV)
    q = torch.empty((n, 128 * H), dtype=torch.float16, device=DEV)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    rt.gemm_qkv_tiles(dev16(x.f64), wt, q, H, r0, P, T, None if cached else cache, 0, kvt, L.rows(r0, S),
                      torch.from_numpy(kw).to(DEV), 1e-6, flags=flags)
    sync()
    rows = np.unique(np.concatenate([[0, n - 1], qin.rng(CFG, 352 + int(cached)).integers(0, n, 30)]))
    if not cached:
        rows = np.unique(np.concatenate([rows, [P - 1, P]]))
    c, s = O.rope_tables(O.positions(wl.segments))
    wf16 = w.f64.astype(np.float16).astype(np.float64)
    rq, rk, rv = oracle_qkv(x.f64[rows], wf16, H, c[r0 + rows], s[r0 + rows], kw.astype(np.float64))
    check(host(q[torch.from_numpy(rows).to(DEV)]).reshape(-1, H, 128), rq, "Q")
    tok = r0 + rows
    kc, vc = (host(cache.k_rows(0)), host(cache.v_rows(0))) if not cached else (None, None)
    kt, vt = host(kvt.k_rows()), host(kvt.v_rows())
    gk = np.stack([kc[:, t] if t < P else kt[:, t - P] for t in tok])
    gv = np.stack([vc[:, t] if t < P else vt[:, t - P] for t in tok])
    check(gk, rk, "K")
    check(gv, rv, "V")
    assert int(flags.item()) == 0


def test_v_store_paths_agree_bitwise():
    # calls whose rows are whole 64-key tiles write V as 16-byte pieces (a lane transpose); other
    # calls write element by element.  The same tokens through both give the same tile bytes.
    segments, H, Kd = (qin.text(64), qin.image(12, 16, 1), qin.image(10, 10, 0)), 2, 128
    L = rt.Layout(segments, DEV)
    S, P, T = L.S, L.P, L.T
    assert P % 64 == 0 and T % 64 != 0
    x, w, kw = inputs(S, H, Kd, 9)
    xd = dev16(x.f64)
    wt = rt.pack_qkv_tiles(rt.from_bits(w.bits, "bf16", DEV).to(torch.float16), H)
    kwd = torch.from_numpy(kw).to(DEV)
    out = []
    for splits in ([0, S], [0, 100, 250, S]):        # one call (whole tiles), or three ragged calls
        cache = rt.KVCache(1, H, P, Q.QI_BF16, DEV)
        kvt = rt.KVTiles(T, H, DEV)
        for t in (cache.k, cache.v, kvt.k, kvt.v):
            t.fill_(float("nan"))
        q = torch.empty((S, 128 * H), dtype=torch.float16, device=DEV)
        for a, b in zip(splits[:-1], splits[1:]):
            rt.gemm_qkv_tiles(xd[a:b], wt, q[a:b], H, a, P, T, cache, 0, kvt, L.rows(a, b), kwd, 1e-6)
        sync()
        out.append((cache.k.clone(), cache.v.clone(), kvt.k.clone(), kvt.v.clone(), q))
    for u, v in zip(out[0], out[1]):
        assert torch.equal(u, v)
    assert not torch.isnan(out[0][3]).any() and torch.all(kvt.v_rows()[:, T:] == 0)


def test_attention_tiled_equals_unfused_bitwise_headline_shape():
    # the 21,504-token layout (text 1024 + four 64 x 64 references + the 64 x 64 target), 24 heads:
    # the tiled entry points against the unfused ones on the same tiles, every output bit
    wl = qin.WORKLOADS["txt1024_4ref64_tgt64"]
    H = wl.n_head
    L = rt.Layout(wl.segments, DEV)
    S, P, T = L.S, L.P, L.T
    say(f"[attn tiled, headline shape] S={S} P={P} T={T} H={H}")
    g = torch.Generator(device=DEV).manual_seed(11)
    q, k, v = (torch.randn((S, H, 128), generator=g, device=DEV).to(torch.bfloat16) for _ in range(3))
    kw = 1.0 + 0.02 * torch.randn(128, generator=g, device=DEV)
    qw = 1.0 + 0.02 * torch.randn(128, generator=g, device=DEV)
    att = rt.Attention(L, H, Q.QI_BF16, DEV)
    cache = rt.KVCache(1, H, P, Q.QI_BF16, DEV)
    o_ref = att.full(q, k, v, qw, kw, cache=cache, layer=0)
    kvt = _tiles_of(k[P:], v[P:], H, T, L.rows(P, S), kw)
    o_t = att.full_tiled(q, cache, 0, kvt, qw)
    o_c = att.cached(q[P:], k[P:], v[P:], cache, 0, qw, kw)
    o_ct = att.cached_tiled(q[P:], cache, 0, kvt, qw)
    sync()
    assert torch.equal(o_t, o_ref)
    assert torch.equal(o_ct, o_c)
    assert torch.equal(o_ct, o_ref[P:])
    assert att.range_flags() == 0
