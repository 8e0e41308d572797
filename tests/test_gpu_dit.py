"""GPU parity of the single-stream layer pieces around the attention (projection GEMMs with their
epilogues on bf16 and on fp16 operands, ZeroCenterRMSNorm + modulation, timestep embedding,
conditioning linears, bf16 and fp16 casts), of one whole layer (step 1 and cached step), and of a
small sampling loop, all called through the C ABI and checked against the fp64 oracle on the same
seeded inputs.  The composed layer path runs fp16 activations and fp16 copies of the bf16
weights.

Tolerances (written here, per output tensor):
  16-bit outputs, and every result of the composed layer path (layer outputs, their residual
  increments, the velocities of the sampling loop, the TextProjection):
        max|d| <= 1e-2 * max|ref|  and  sum|d| / sum|ref| <= 2e-3
  fp32 outputs of one fp32-accumulated step on stored inputs:
        max|d| <= 1e-5 * max|ref|  and  sum|d| / sum|ref| <= 1e-5
  timestep embedding (fp64 in the kernel, one fp32 rounding): max|d| <= 2e-7
  bf16 and fp16 casts: bit-exact (round to nearest even)
The one-layer parity feeds the oracle the GPU's layer input (and the GPU's modulation vectors),
so errors of earlier layers do not count twice.
"""
import math
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
CFG = 91   # seed id of the ad-hoc shapes here


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(got, ref, bar, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    d = np.abs(got - ref)
    max_rel = d.max() / max(np.abs(ref).max(), 1e-300)
    mean_rel = d.sum() / max(np.abs(ref).sum(), 1e-300)
    lim_max, lim_mean = {"bf16": (1e-2, 2e-3), "f16": (1e-2, 2e-3), "f32": (1e-5, 1e-5)}[bar]
    say(f"  {what}: max_rel={max_rel:.3e} mean_rel={mean_rel:.3e}")
    assert max_rel <= lim_max and mean_rel <= lim_mean, (what, max_rel, mean_rel)
    return max_rel, mean_rel


def bf(st: qin.Stored) -> torch.Tensor:
    return rt.from_bits(st.bits, "bf16", DEV)


TD = {"bf16": torch.bfloat16, "f16": torch.float16}


def dv(st: qin.Stored) -> torch.Tensor:
    """A stored 16-bit input on the device, in its own type."""
    return rt.from_bits(st.bits, st.dtype, DEV)


def wdev(st: qin.Stored, dt: str) -> torch.Tensor:
    """A bf16-stored weight on the device in the operand type (fp16: converted, as the runtime
    converts the model's weights)."""
    return bf(st).to(TD[dt])


def f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------------------------------------------
# GEMM epilogues
# ------------------------------------------------------------------------------------------------

GEMM_SHAPES = [(300, 192, 320), (1, 64, 64), (257, 256, 64), (600, 448, 192), (513, 640, 128)]
TILES = [128, 192, 256]   # feature width of the 256-token workgroup tiles (0 = automatic)


def gemm_inputs(M, N, K, tag=0, dt="bf16"):
    x = qin.stored(qin.normal(CFG, 200 + tag, (M, K)), dt)
    w = qin.linear_weight(CFG, 40 + tag, N, K)
    return x, w


def padded(rows, cols, ld, dtype, fill):
    """A [rows][cols] view with leading dimension ld inside a buffer with 3 spare rows, all
    filled with `fill` so that writes outside the view can be detected."""
    buf = torch.full((rows + 3, ld), fill, dtype=dtype, device=DEV)
    return buf, buf[:rows, :cols]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_store_and_store_f32(M, N, K, tile, dt):
    say(f"[gemm store] M={M} N={N} K={K} tile={tile} {dt}")
    x, w = gemm_inputs(M, N, K, dt=dt)
    ref = O.linear(x.f64, w.f64)
    # x with a wider leading dimension, outputs padded to catch stray writes
    xbuf = torch.zeros((M, K + 64), dtype=TD[dt], device=DEV)
    xbuf[:, :K] = dv(x)
    xv = xbuf[:, :K]
    for epi, odt, bar in ((Q.QI_EPI_STORE, TD[dt], dt), (Q.QI_EPI_STORE_F32, torch.float32, "f32")):
        buf, out = padded(M, N, N + 8, odt, 7.0)
        rt.gemm(xv, wdev(w, dt), out, epi, tile_n=tile)
        sync()
        check(host(out), ref, bar, f"epi {epi}")
        assert torch.all(buf[:M, N:] == 7.0) and torch.all(buf[M:] == 7.0), "write outside the output view"


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_gated_residual(M, N, K, tile, dt):
    say(f"[gemm gated residual] M={M} N={N} K={K} tile={tile} {dt}")
    x, w = gemm_inputs(M, N, K, 1, dt)
    x0 = qin.normal(CFG, 210, (M, N)).astype(np.float32).astype(np.float64)
    gate = qin.normal(CFG, 211, (2, N), std=0.7).astype(np.float32).astype(np.float64)
    for row0, P in ((0, M // 3), (50, 60), (0, 0), (M, M)):
        y = O.linear(x.f64, w.f64)
        g = O.per_row(gate[0], gate[1], M, row0, P)
        ref = x0 + np.tanh(g) * y
        buf, out = padded(M, N, N + 8, torch.float32, 5.0)
        out.copy_(f32(x0))
        rt.gemm(dv(x), wdev(w, dt), out, Q.QI_EPI_GATED_RESIDUAL, f32(gate), row0, P, tile_n=tile)
        sync()
        check(host(out), ref, "f32", f"row0={row0} P={P}")
        assert torch.all(buf[:M, N:] == 5.0) and torch.all(buf[M:] == 5.0)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("tile", [128, 256])
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_swiglu(M, N, K, tile, dt):
    say(f"[gemm swiglu] M={M} 2F={N} K={K} tile={tile} {dt}")
    F = N // 2
    x = qin.stored(qin.normal(CFG, 220, (M, K)), dt)
    wg = qin.linear_weight(CFG, 50, F, K)
    wu = qin.linear_weight(CFG, 51, F, K)
    ref = O.swiglu(O.linear(x.f64, wg.f64), O.linear(x.f64, wu.f64))
    buf, out = padded(M, F, F + 8, TD[dt], 3.0)
    rt.gemm(dv(x), rt.pack_swiglu(wdev(wg, dt), wdev(wu, dt)), out, Q.QI_EPI_SWIGLU, tile_n=tile)
    sync()
    check(host(out), ref, dt, "swiglu")
    assert torch.all(buf[:M, F:] == 3.0) and torch.all(buf[M:] == 3.0)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_gelu(M, N, K, tile, dt):
    say(f"[gemm gelu] M={M} N={N} K={K} tile={tile} {dt}")
    x, w = gemm_inputs(M, N, K, 3, dt)
    ref = O.gelu_tanh(O.linear(x.f64, w.f64))
    buf, out = padded(M, N, N + 8, TD[dt], 9.0)
    rt.gemm(dv(x), wdev(w, dt), out, Q.QI_EPI_GELU, tile_n=tile)
    sync()
    check(host(out), ref, dt, "gelu")
    assert torch.all(buf[:M, N:] == 9.0) and torch.all(buf[M:] == 9.0), "write outside the output view"


@pytest.mark.parametrize("dtn", ["bf16", "f16"])
@pytest.mark.parametrize("epi", [Q.QI_EPI_STORE, Q.QI_EPI_STORE_F32, Q.QI_EPI_GATED_RESIDUAL, Q.QI_EPI_SWIGLU,
                                 Q.QI_EPI_GELU])
def test_gemm_tiles_give_identical_bits(epi, dtn):
    # every output is the same fp32 sum in the same order whatever the tile, so the bits agree
    M, N, K = 600, 448, 192
    x, w = gemm_inputs(M, N, K, 2, dtn)
    gate = f32(qin.normal(CFG, 212, (2, N), std=0.7))
    F = N // 2 if epi == Q.QI_EPI_SWIGLU else N
    dt = TD[dtn] if epi in (Q.QI_EPI_STORE, Q.QI_EPI_SWIGLU, Q.QI_EPI_GELU) else torch.float32
    outs = []
    for tile in ([0, 128, 256] if epi == Q.QI_EPI_SWIGLU else [0, 128, 192, 256]):
        out = torch.zeros((M, F), dtype=dt, device=DEV) + 0.5
        rt.gemm(dv(x), wdev(w, dtn), out, epi, gate, 0, 100, tile_n=tile)
        outs.append(out)
    sync()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_gemm_argument_errors():
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((64, 64), dtype=torch.bfloat16, device=DEV)
    o = torch.zeros((8, 64), dtype=torch.float32, device=DEV)
    s = rt.stream_handle(DEV)
    assert Q.qi_gemm_bf16(x, 64, w, o, 64, 8, 64, 64, Q.QI_EPI_GATED_RESIDUAL, None, 0, 0, s) == Q.QI_ERR_ARG
    assert Q.qi_gemm_bf16(x, 64, w, o, 64, 8, 64, 64, Q.QI_EPI_GELU + 1, None, 0, 0, s) == Q.QI_ERR_ARG
    assert Q.qi_gemm_bf16(x, 64, w, o, 64, 8, 96, 64, Q.QI_EPI_STORE_F32, None, 0, 0, s) == Q.QI_ERR_SHAPE
    assert Q.qi_gemm_bf16(x, 64, w, o, 64, 8, 64, 32, Q.QI_EPI_STORE_F32, None, 0, 0, s) == Q.QI_ERR_SHAPE
    assert Q.qi_gemm_bf16(x, 60, w, o, 64, 8, 64, 64, Q.QI_EPI_STORE_F32, None, 0, 0, s) == Q.QI_ERR_SHAPE
    assert Q.qi_gemm_bf16(x, 64, w, o, 64, 8, 64, 64, 9, None, 0, 0, s) == Q.QI_ERR_ARG
    assert Q.qi_gemm_bf16(x, 64, w, o, 64, 0, 64, 64, Q.QI_EPI_STORE_F32, None, 0, 0, s) == Q.QI_OK
    assert Q.qi_gemm_bf16_ex(x, 64, w, o, 64, 8, 64, 64, Q.QI_EPI_STORE_F32, None, 0, 0, 64, s) == Q.QI_ERR_ARG
    assert Q.qi_gemm_bf16_ex(x, 64, w, o, 64, 8, 64, 64, Q.QI_EPI_SWIGLU, None, 0, 0, 192, s) == Q.QI_ERR_ARG
    # x beyond 2^30 elements (32-bit byte offsets), checked before any launch
    assert Q.qi_gemm_bf16(x, 1 << 20, w, o, 64, 1 << 10, 64, 64, Q.QI_EPI_STORE_F32, None, 0, 0, s) == Q.QI_ERR_SHAPE
    # the dtype-generic form: 16-bit operand types only, a 4-byte aligned flag word
    xh, wh = x.half(), w.half()
    assert Q.qi_gemm(xh, 64, wh, None, o, 64, 8, 64, 64, Q.QI_F16, Q.QI_EPI_STORE_F32, stream=s) == Q.QI_OK
    assert Q.qi_gemm(xh, 64, wh, None, o, 64, 8, 64, 64, Q.QI_F32, Q.QI_EPI_STORE_F32, stream=s) == Q.QI_ERR_DTYPE
    assert Q.qi_gemm(xh, 64, wh, None, o, 64, 8, 64, 64, 7, Q.QI_EPI_STORE_F32, stream=s) == Q.QI_ERR_DTYPE
    fl = torch.zeros(2, dtype=torch.int32, device=DEV)
    assert Q.qi_gemm(xh, 64, wh, None, o, 64, 8, 64, 64, Q.QI_F16, Q.QI_EPI_STORE_F32, range_flags=fl.data_ptr() + 2,
                     stream=s) == Q.QI_ERR_ALIGN


# full-size projections of one layer of the 14,848-token workload (hidden 3072, FFN 8192), on
# sampled rows: the cached-step row count (4096) and the step-1 row count (14,848)
FULL = [("qkv", 4096, 9216, 3072, Q.QI_EPI_STORE), ("out", 4096, 3072, 3072, Q.QI_EPI_GATED_RESIDUAL),
        ("gate_up", 4096, 16384, 3072, Q.QI_EPI_SWIGLU), ("down", 4096, 3072, 8192, Q.QI_EPI_GATED_RESIDUAL),
        ("qkv_step1", 14848, 9216, 3072, Q.QI_EPI_STORE)]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("name,M,N,K,epi", FULL)
def test_gemm_full_size_sampled(name, M, N, K, epi, dt):
    say(f"[gemm full] {name} M={M} N={N} K={K} {dt}")
    x = qin.stored(qin.normal(CFG, 230, (M, K)), dt)
    rows = np.unique(np.concatenate([[0, M - 1], qin.rng(CFG, 231).integers(0, M, 40)]))
    if epi == Q.QI_EPI_SWIGLU:
        F = N // 2
        wg, wu = qin.linear_weight(CFG, 52, F, K), qin.linear_weight(CFG, 53, F, K)
        out = torch.empty((M, F), dtype=TD[dt], device=DEV)
        rt.gemm(dv(x), rt.pack_swiglu(wdev(wg, dt), wdev(wu, dt)), out, epi)
        ref = O.swiglu(O.linear(x.f64[rows], wg.f64), O.linear(x.f64[rows], wu.f64))
        bar = dt
    else:
        w = qin.linear_weight(CFG, 54, N, K)
        y = O.linear(x.f64[rows], w.f64)
        if epi == Q.QI_EPI_STORE:
            out = torch.empty((M, N), dtype=TD[dt], device=DEV)
            rt.gemm(dv(x), wdev(w, dt), out, epi)
            ref, bar = y, dt
        else:
            P = M // 4
            x0 = qin.normal(CFG, 232, (M, N)).astype(np.float32).astype(np.float64)
            gate = qin.normal(CFG, 233, (2, N), std=0.7).astype(np.float32).astype(np.float64)
            out = f32(x0)
            rt.gemm(dv(x), wdev(w, dt), out, epi, f32(gate), 0, P)
            ref = x0[rows] + np.tanh(O.per_row(gate[0], gate[1], M, 0, P)[rows]) * y
            bar = "f32"
    sync()
    check(host(out)[rows], ref, bar, name)


# ------------------------------------------------------------------------------------------------
# norm + modulation, timestep embedding, conditioning linears, cast
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("M,D,row0,P,parts", [(300, 3072, 0, 170, "wss"), (129, 256, 40, 100, "wss"),
                                              (77, 132, 0, 0, "w"), (5, 3072, 10, 0, "s"),
                                              (64, 512, 0, 64, ""), (9, 4104, 0, 5, "wss")])
def test_zc_rmsnorm_mod(M, D, row0, P, parts, dt):
    say(f"[norm mod] M={M} D={D} row0={row0} P={P} parts={parts!r} {dt}")
    x = qin.normal(CFG, 240, (M, D), std=3.0).astype(np.float32).astype(np.float64)
    w = qin.normal(CFG, 241, (D,), std=0.02).astype(np.float32).astype(np.float64) if "w" in parts else None
    sc = qin.normal(CFG, 242, (2, D), std=0.3).astype(np.float32).astype(np.float64) if "s" in parts else None
    sh = qin.normal(CFG, 243, (2, D), std=0.3).astype(np.float32).astype(np.float64) if parts.count("s") > 1 else None
    ref = O.norm_mod(x, w, None if sc is None else O.per_row(sc[0], sc[1], M, row0, P),
                     None if sh is None else O.per_row(sh[0], sh[1], M, row0, P))
    buf, out = padded(M, D, D + 4, TD[dt], 9.0)
    rt.norm_mod(f32(x), out, None if w is None else f32(w), None if sc is None else f32(sc),
                None if sh is None else f32(sh), row0, P)
    sync()
    check(host(out), ref, dt, "norm_mod")
    assert torch.all(buf[:M, D:] == 9.0) and torch.all(buf[M:] == 9.0)


def test_timestep_embed():
    t = np.concatenate([1000.0 * qin.sigmas(8), [0.5, 999.9, 123.456]]).astype(np.float32)
    out = torch.empty((len(t), 256), dtype=torch.float32, device=DEV)
    Q.check(Q.qi_timestep_embed(f32(t), len(t), 256, out, rt.stream_handle(DEV)), "qi_timestep_embed")
    sync()
    ref = O.timestep_embedding(t.astype(np.float64))
    err = np.abs(host(out) - ref).max()
    say(f"  timestep embed max abs err {err:.2e}")
    assert err <= 2e-7


@pytest.mark.parametrize("nv,I,O_,silu", [(2, 256, 3072, False), (2, 3072, 3072, True), (1, 8, 5, True),
                                           (4, 520, 70, False), (3, 3072, 18432, True),
                                           # rows of several 3,072-element batches, the last ragged
                                           (2, 8200, 70, True), (1, 3080, 33, False), (4, 6144, 130, True)])
def test_linear_small(nv, I, O_, silu):
    say(f"[linear small] nv={nv} I={I} O={O_} silu={silu}")
    x = qin.normal(CFG, 250, (nv, I), std=2.0).astype(np.float32).astype(np.float64)
    w = qin.linear_weight(CFG, 60, O_, I)
    y = torch.empty((nv, O_), dtype=torch.float32, device=DEV)
    rt.linear_small(f32(x), bf(w), y, silu)
    sync()
    ref = O.linear(O.silu(x) if silu else x, w.f64)
    check(host(y), ref, "f32", "linear_small")


def test_linear_small_rows_independent_of_vector_count():
    # each vector's sums take the same order whatever the number of vectors in the call
    x = qin.normal(CFG, 251, (4, 3072), std=2.0).astype(np.float32)
    w = bf(qin.linear_weight(CFG, 61, 200, 3072))
    y4 = torch.empty((4, 200), dtype=torch.float32, device=DEV)
    rt.linear_small(f32(x), w, y4, True)
    for v in range(4):
        y1 = torch.empty((1, 200), dtype=torch.float32, device=DEV)
        rt.linear_small(f32(x[v:v + 1]), w, y1, True)
        sync()
        assert torch.equal(y1[0], y4[v])


def test_cast_bf16_bit_exact():
    vals = np.concatenate([
        qin.normal(CFG, 260, (5000,), std=100.0),
        [0.0, -0.0, np.inf, -np.inf, 1e-40, -1e-42, 3.0e38, 3.3961776e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
         1.0 + 2 ** -8 + 2 ** -20, 65504.0, 2 ** -126, 2 ** -133]]).astype(np.float32)
    n = len(vals)
    y = torch.empty(n + 5, dtype=torch.bfloat16, device=DEV)
    y.fill_(1.0)
    Q.check(Q.qi_cast_bf16(f32(vals), y, n, rt.stream_handle(DEV)), "qi_cast_bf16")
    sync()
    got = y.cpu().view(torch.int16).numpy().view(np.uint16)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got[:n], ref)
    assert np.all(got[n:] == 0x3F80)
    nanv = np.array([np.nan, -np.nan], dtype=np.float32)
    yn = torch.empty(2, dtype=torch.bfloat16, device=DEV)
    Q.check(Q.qi_cast_bf16(f32(nanv), yn, 2, rt.stream_handle(DEV)), "qi_cast_bf16")
    sync()
    assert torch.all(torch.isnan(yn.float().cpu()))


def test_cast_f16_bit_exact_and_range_flag():
    vals = np.concatenate([
        qin.normal(CFG, 261, (5000,), std=100.0),
        [0.0, -0.0, 1e-8, -3e-7, 6.0e-5, 65504.0, 65519.0, -65504.0, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11,
         2 ** -24, 2 ** -25, 3 * 2 ** -26]]).astype(np.float32)
    n = len(vals)
    y = torch.empty(n + 5, dtype=torch.float16, device=DEV)
    y.fill_(1.0)
    fl = torch.zeros(1, dtype=torch.int32, device=DEV)
    rt.cast(f32(vals), y[:n], fl)
    sync()
    got = y.cpu().view(torch.int16).numpy().view(np.uint16)
    ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got[:n], ref)
    assert np.all(got[n:] == 0x3C00)
    assert int(fl.item()) == 0
    rt.cast(f32(np.array([65520.0, 1.0], dtype=np.float32)), y[:2], fl)
    sync()
    assert int(fl.item()) == Q.QI_RANGE_OUT and np.isinf(float(y[0]))


# ------------------------------------------------------------------------------------------------
# the context TextProjection ([1B] sections 1-3)
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("n,D", [(37, 256), (1, 128), (512, 3072)])
def test_text_projection(n, D):
    say(f"[text projection] n={n} D={D}")
    tw = qin.text_projection_weights(CFG, D)
    x = qin.context_inputs(CFG, n, D)
    tp = rt.TextProjection(f32(tw["tp_norm"]), bf(tw["tp_w1"]), bf(tw["tp_w2"]))
    y = tp(f32(x))
    sync()
    ref = O.text_projection(x, tw["tp_norm"], tw["tp_w1"].f64, tw["tp_w2"].f64)
    # fp16 normed rows and GELU output (weights converted to fp16 once)
    check(host(y), ref, "f16", "text projection")
    assert int(tp.flags.item()) == 0


# ------------------------------------------------------------------------------------------------
# one whole layer, the conditioning, and a small sampling loop
# ------------------------------------------------------------------------------------------------

def make_model(segments, D, F, n_layers, cfg=CFG, fold=True, kv_tiles=True):
    layout = rt.Layout(segments, DEV)
    sw_np = qin.shared_weights(cfg, D)
    lw_np = [qin.layer_weights(cfg, D, F, l) for l in range(n_layers)]
    sw = rt.SharedWeights(*(bf(sw_np[k]) for k in ("t_w1", "t_w2", "w_mod", "w_scale", "w_head", "w_in")))
    layers = [rt.LayerWeights(f32(L["norm1"]), f32(L["norm2"]), f32(L["q_norm"]), f32(L["k_norm"]),
                              bf(L["w_qkv"]), bf(L["w_out"]), bf(L["w_gate"]), bf(L["w_up"]), bf(L["w_down"]))
              for L in lw_np]
    model = rt.DiT(layout, sw, layers, DEV, fold=fold, kv_tiles=kv_tiles)
    shared64 = {k: v.f64 for k, v in sw_np.items()}
    layers64 = [{k: (v.f64 if isinstance(v, qin.Stored) else v) for k, v in L.items()} for L in lw_np]
    return model, shared64, layers64


SMALL = (qin.text(37), qin.image(9, 7, 1), qin.image(11, 13, 0))


@pytest.mark.parametrize("sigma", [1.0, 0.375])
def test_condition(sigma):
    model, sh, _ = make_model(SMALL, 256, 512, 1)
    model.condition(sigma)
    sync()
    temb = O.time_condition(np.array([0.0, sigma]), sh["t_w1"], sh["t_w2"])
    mods = O.modulation(temb, sh["w_mod"], 256)
    for c in range(6):
        check(host(model.mods[c]), mods[c], "f32", f"mod chunk {c}")
    check(host(model.hscale), O.linear(O.silu(temb), sh["w_scale"]), "f32", "head scale")


def gpu_mods(model):
    m = host(model.mods)
    return tuple(m[c][0] for c in range(6)), tuple(m[c][1] for c in range(6))


# (norm fold, fused QKV path writing the K/V tiles)
MODES = [(True, True), (True, False), (False, False), (False, True)]


@pytest.mark.parametrize("fold,kv", MODES)
@pytest.mark.parametrize("segments,D,F", [(SMALL, 256, 512), ((qin.text(130), qin.image(8, 16, 1), qin.text(3),
                                                             qin.image(10, 10, 2), qin.image(16, 9, 0)), 384, 320)])
def test_layer_step1_and_cached(segments, D, F, fold, kv):
    say(f"[layer] S={sum(g.n_tokens for g in segments)} D={D} F={F} fold={fold} kv_tiles={kv}")
    model, sh, layers64 = make_model(segments, D, F, 1, fold=fold, kv_tiles=kv)
    L = model.L
    S, P, T = L.S, L.P, L.T
    c, s = O.rope_tables(O.positions(segments))
    model.condition(1.0)
    x_in = qin.normal(CFG, 270, (S, D)).astype(np.float32)
    model.x.copy_(f32(x_in))
    model.layer(0, slice(0, S), False)
    sync()
    mods = gpu_mods(model)
    ref, cache = O.dit_layer(x_in.astype(np.float64), layers64[0], mods, segments, c, s)
    check(host(model.x), ref, "bf16", "step-1 layer output")
    check(host(model.x) - x_in, ref - x_in, "f16", "step-1 layer increment")
    # cached step: new target rows, the prefix K/V from step 1
    model.condition(0.625)
    xt_in = qin.normal(CFG, 271, (T, D)).astype(np.float32)
    model.x[P:].copy_(f32(xt_in))
    model.layer(0, slice(P, S), True)
    sync()
    mods = gpu_mods(model)
    ref_t, _ = O.dit_layer(xt_in.astype(np.float64), layers64[0], mods, segments, c, s, cache=cache)
    check(host(model.x[P:]), ref_t, "bf16", "cached layer output")
    check(host(model.x[P:]) - xt_in, ref_t - xt_in, "f16", "cached layer increment")
    assert model.attn.range_flags() == 0


@pytest.mark.parametrize("fold,kv", MODES)
def test_cached_layer_equals_step1_target_rows_bitwise(fold, kv):
    # the same target input through step 1 (whole sequence) and through the cached path gives the
    # same target rows, bit for bit: the prefix K/V in the cache are the ones step 1 used
    model, _, _ = make_model(SMALL, 256, 512, 1, fold=fold, kv_tiles=kv)
    S, P = model.L.S, model.L.P
    model.condition(0.5)
    x_in = f32(qin.normal(CFG, 272, (S, 256)))
    model.x.copy_(x_in)
    model.layer(0, slice(0, S), False)
    full_t = model.x[P:].clone()
    model.x.copy_(x_in)
    model.layer(0, slice(P, S), True)
    sync()
    assert torch.equal(model.x[P:], full_t)


@pytest.mark.parametrize("fold,prepared,kv", [(True, True, True), (True, False, True), (False, True, False),
                                               (True, True, False)])   # (step() prepares itself)
def test_sampling_loop_small(fold, prepared, kv):
    segments = (qin.text(20), qin.image(6, 5, 1), qin.image(7, 6, 0))
    D, F, n_layers, n_steps = 256, 512, 2, 3
    say(f"[sampling loop] fold={fold} prepared={prepared} kv_tiles={kv}")
    model, sh, layers64 = make_model(segments, D, F, n_layers, fold=fold, kv_tiles=kv)
    L = model.L
    n_text = 20
    x_text, lat_ref = qin.prefix_inputs(CFG, n_text, 30, D)
    lat0 = qin.target_noise(CFG, L.T)
    sig = qin.sigmas(n_steps)
    lat = f32(lat0)
    vels = []
    xt, lr = f32(x_text), f32(lat_ref)
    if prepared:
        model.prepare(sig)
    for k in range(n_steps):
        model.step(k, lat, sig, xt, lr)
        vels.append(host(model.vel))
    sync()
    ref_lat, ref_vels = O.denoise(segments, x_text, lat_ref, lat0, sh, layers64, n_steps, return_velocities=True)
    for k in range(n_steps):
        check(vels[k], ref_vels[k], "f16", f"velocity step {k + 1}")
    check(host(lat), ref_lat, "bf16", "final latent")
    model.check_range()


# ------------------------------------------------------------------------------------------------
# a full-size layer of the 14,848-token workload, stage by stage on sampled rows
# ------------------------------------------------------------------------------------------------

def test_full_size_layer_stages_sampled():
    wl = qin.WORKLOADS["txt512_10ref32_tgt64"]
    D, F, H = 3072, 8192, 24
    say(f"[layer full] S={wl.S} P={wl.P} T={wl.T}")
    model, sh, layers64 = make_model(wl.segments, D, F, 1, cfg=wl.cfg_id, kv_tiles=False)
    W = layers64[0]
    Lw = model.layers[0]
    S, P, T = wl.S, wl.P, wl.T
    c, s = O.rope_tables(O.positions(wl.segments))
    rows = np.unique(np.concatenate([[0, P - 1, P, S - 1], qin.rng(CFG, 280).integers(0, S, 28)]))
    model.condition(1.0)
    x_in = qin.normal(CFG, 281, (S, D)).astype(np.float32)
    model.x.copy_(f32(x_in))
    mods = gpu_mods(model)
    m = model.mods
    sel = lambda i, r: O.per_row(mods[0][i], mods[1][i], S, 0, P)[r]
    # norm1 + modulation
    h = model.h
    rt.norm_mod(model.x, h, Lw.norm1, m[1], m[0], 0, P)
    sync()
    x64 = x_in.astype(np.float64)
    ref_h = O.norm_mod(x64[rows], W["norm1"], sel(1, rows), sel(0, rows))
    check(host(h[rows]), ref_h, "bf16", "norm1+mod")
    # QKV projection
    rt.gemm(h, Lw.w_qkv, model.qkv, Q.QI_EPI_STORE)
    sync()
    h64 = host(h)
    check(host(model.qkv[rows]), O.linear(h64[rows], W["w_qkv"]), "bf16", "qkv")
    # attention over the GPU's q/k/v (QK-RMSNorm + RoPE fused)
    qkv64 = host(model.qkv).reshape(S, 3, H, 128)
    q = model.qkv[:, :D].view(S, H, 128)
    k = model.qkv[:, D:2 * D].view(S, H, 128)
    v = model.qkv[:, 2 * D:].view(S, H, 128)
    model.attn.full(q, k, v, Lw.q_norm, Lw.k_norm, 1e-6, cache=model.cache, layer=0, out=model.o)
    sync()
    qr = O.prep_qk(qkv64[rows, 0], c[rows], s[rows], W["q_norm"], 1e-6)
    kr = O.prep_qk(qkv64[:, 1], c, s, W["k_norm"], 1e-6)
    ref_o = O.attention(qr, kr, qkv64[:, 2], O.mask_rows(wl.segments, rows))
    check(host(model.o[rows]), ref_o, "bf16", "attention")
    # out-projection, gated residual
    o64 = host(model.o).reshape(S, D)
    rt.gemm(model.o.view(S, D), Lw.w_out, model.x, Q.QI_EPI_GATED_RESIDUAL, m[2], 0, P)
    sync()
    ref_x1 = x64[rows] + np.tanh(sel(2, rows)) * O.linear(o64[rows], W["w_out"])
    check(host(model.x[rows]), ref_x1, "f32", "out-proj residual")
    # norm2, SwiGLU, down-projection
    x1 = host(model.x)
    rt.norm_mod(model.x, h, Lw.norm2, m[4], m[3], 0, P)
    rt.gemm(h, Lw.w_gu, model.a, Q.QI_EPI_SWIGLU)
    sync()
    h2 = host(h)
    check(h2[rows], O.norm_mod(x1[rows], W["norm2"], sel(4, rows), sel(3, rows)), "bf16", "norm2+mod")
    ref_a = O.swiglu(O.linear(h2[rows], W["w_gate"]), O.linear(h2[rows], W["w_up"]))
    check(host(model.a[rows]), ref_a, "bf16", "swiglu")
    a64 = host(model.a)
    rt.gemm(model.a, Lw.w_down, model.x, Q.QI_EPI_GATED_RESIDUAL, m[5], 0, P)
    sync()
    ref_x2 = x1[rows] + np.tanh(sel(5, rows)) * O.linear(a64[rows], W["w_down"])
    check(host(model.x[rows]), ref_x2, "f32", "down-proj residual")


@pytest.mark.parametrize("cached", [False, True])
def test_full_size_layer_norm_fold_sampled(cached):
    # the layer's norm fold at the 14,848-token shape (step 1: every row; cached: the 4,096 target
    # rows) through the launches the denoiser makes, each stage against the oracle on sampled rows
    wl = qin.WORKLOADS["txt512_10ref32_tgt64"]
    D, F = 3072, 8192
    say(f"[layer fold full] S={wl.S} P={wl.P} T={wl.T} cached={cached}")
    model, sh, layers64 = make_model(wl.segments, D, F, 1, cfg=wl.cfg_id, kv_tiles=False)
    W, Lw = layers64[0], model.layers[0]
    S, P = wl.S, wl.P
    r0 = P if cached else 0
    n = S - r0
    rows = np.unique(np.concatenate([[0, n - 1, max(P - r0 - 1, 0), P - r0 if P > r0 else 0],
                                     qin.rng(CFG, 290 + int(cached)).integers(0, n, 24)]))
    model.condition(0.625)
    mods = gpu_mods(model)
    m = model.mods
    sel = lambda i, r: O.per_row(mods[0][i], mods[1][i], n, r0, P)[r]
    x_in = qin.normal(CFG, 291, (n, D)).astype(np.float32)
    x = model.x[r0:]
    x.copy_(f32(x_in))
    x64 = x_in.astype(np.float64)
    h, sq = model.h[:n], model.sq[:n]
    bq = model.bq[0]
    # norm1 folded: xc, partial sums, then the QKV projection with rrms and the shift bias
    rt.norm_fold_rows(x, h, sq, Lw.norm1, m[1], r0, P)
    qkv = model.qkv[:n]
    rt.gemm(h, Lw.w_qkv, qkv, Q.QI_EPI_STORE, None, r0, P, bias=bq[0], fold=rt.NormFold(sq, 1e-6, bq[1]))
    sync()
    check(host(bq[1]), O.linear(mods[1][0][None, :], host(Lw.w_qkv))[0], "f32", "QKV bias table (target)")
    h1 = O.norm_mod(x64[rows], W["norm1"], sel(1, rows), sel(0, rows))
    check(host(qkv[rows]), O.linear(h1, W["w_qkv"]), "bf16", "qkv (norm1 folded)")
    # out-projection (a synthetic attention output) producing norm2's operand
    o = torch.from_numpy(qin.normal(CFG, 292, (n, D)).astype(np.float16)).to(DEV)
    rt.gemm(o, Lw.w_out, x, Q.QI_EPI_GATED_RESIDUAL, m[2], r0, P,
            fold=rt.NormFold(xc=h, next_w=Lw.norm2, next_scale=m[4], sumsq_out=sq))
    sync()
    o64 = host(o)
    ref_x1 = x64[rows] + np.tanh(sel(2, rows)) * O.linear(o64[rows], W["w_out"])
    check(host(x[rows]), ref_x1, "f32", "out-proj residual")
    x1 = host(x)
    check(host(h[rows]), x1[rows] * (1.0 + W["norm2"]) * (1.0 + sel(4, rows)), "f16", "xc for norm2")
    check(host(sq[rows]), (x1[rows] ** 2).reshape(len(rows), D // 96, 96).sum(axis=2), "f32", "norm2 partial sums")
    # gate|up with norm2 folded
    bg = model.bgu[0]
    a = model.a[:n]
    rt.gemm(h, Lw.w_gu, a, Q.QI_EPI_SWIGLU, None, r0, P, bias=bg[0], fold=rt.NormFold(sq, 1e-6, bg[1]))
    sync()
    h2 = O.norm_mod(x1[rows], W["norm2"], sel(4, rows), sel(3, rows))
    check(host(a[rows]), O.swiglu(O.linear(h2, W["w_gate"]), O.linear(h2, W["w_up"])), "bf16", "swiglu (norm2 folded)")
    # down-projection producing the next layer's norm1 operand
    a64 = host(a)
    rt.gemm(a, Lw.w_down, x, Q.QI_EPI_GATED_RESIDUAL, m[5], r0, P,
            fold=rt.NormFold(xc=h, next_w=Lw.norm1, next_scale=m[1], sumsq_out=sq))   # (as a next layer's)
    sync()
    ref_x2 = x1[rows] + np.tanh(sel(5, rows)) * O.linear(a64[rows], W["w_down"])
    check(host(x[rows]), ref_x2, "f32", "down-proj residual")
    x2 = host(x[rows])
    check(host(h[rows]), x2 * (1.0 + W["norm1"]) * (1.0 + sel(1, rows)), "f16", "xc for the next norm1")
    assert model.attn.range_flags() == 0


def test_prepared_schedule_equals_per_step_conditioning():
    # the prepared conditioning of a 17-step schedule (bias tables in two passes of at most 16
    # vectors) equals the conditioning computed for each step on its own, bit for bit
    model, _, _ = make_model(SMALL, 256, 512, 2)
    sig = qin.sigmas(17)
    model.prepare(sig)
    for k in (0, 9, 16):
        assert model._use_step(k, sig)
        mods = model.mods.clone()
        tabs = [t.clone() for li in range(2) for t in model._biases(li)]
        model.condition(float(sig[k]))
        assert torch.equal(model.mods, mods)
        assert all(torch.equal(a, b) for a, b in zip(tabs, [t for li in range(2) for t in model._biases(li)]))
