"""GPU parity of the norm fold (include/qi.h, qi_norm_fold): the layer's ZeroCenterRMSNorm with
modulation folded into the GEMMs around it ([1B] sections 1-3; [EDIT] section 5.2; "Qwen-Image-2.1"
course overview, cards 4A and 5A), called through the C ABI and checked against the fp64 oracle's
plain composition, norm then Linear, on the same seeded inputs.

  - qi_norm_fold_rows: xc = x (1 + w)(1 + scale) (one rounding to the 16-bit type) and the sums of
    x^2 over each 96 features;
  - the producing side of the gated residual epilogues: the updated residual, its xc and sums;
  - the consuming side: rrms(x) * (xc W^T) + shift W^T against Linear(norm_mod(x)) of the oracle,
    on every epilogue it serves (16-bit store, SwiGLU, fp32 store), both row classes;
  - qi_linear_multi (the bias tables) against the oracle's Linear;
  - tile independence: every output of either side has the same bits at every tile width, which
    keeps the cached layer equal to step 1's target rows bit for bit.

Tolerances (written here, per output tensor):
  16-bit outputs, and results that pass a 16-bit operand (xc, the consuming GEMM's outputs):
        max|d| <= 1e-2 * max|ref|  and  sum|d| / sum|ref| <= 2e-3
  fp32 results of fp32 arithmetic on stored inputs (residual, sums of squares, bias tables, the
  fp32 store on the stored operand):
        max|d| <= 1e-5 * max|ref|  and  sum|d| / sum|ref| <= 1e-5
The consuming GEMM is compared with the oracle on its stored operand (rrms(x) xc + shift, with the
device's xc) for both types, and with the plain composition Linear(norm_mod(x)) on fp16 operands;
with bf16 operands one rounding of the operand alone moves the composition by about the 2e-3 bar
(the reason the layer chain runs fp16).
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
CFG = 93   # seed id of the shapes here
TD = {"bf16": torch.bfloat16, "f16": torch.float16}


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
    lim_max, lim_mean = {"16": (1e-2, 2e-3), "f32": (1e-5, 1e-5)}[bar]
    say(f"  {what}: max_rel={max_rel:.3e} mean_rel={mean_rel:.3e}")
    assert max_rel <= lim_max and mean_rel <= lim_mean, (what, max_rel, mean_rel)


def f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def sync():
    torch.cuda.synchronize()


def rows32(x):
    """fp32 values as the device holds them, in fp64."""
    return np.asarray(x, dtype=np.float32).astype(np.float64)


W_PART = 96   # features per partial sum of squares


def n_parts(D):
    return -(-D // W_PART)


def sums96(x):
    """Sums of x^2 over each 96 features, the last group ragged (fp64)."""
    M, D = x.shape
    return np.stack([(x[:, j:j + W_PART] ** 2).sum(axis=1) for j in range(0, D, W_PART)], axis=1)


def params(D, tag):
    w = rows32(qin.normal(CFG, 300 + tag, (D,), std=0.02))
    scale = rows32(qin.normal(CFG, 301 + tag, (2, D), std=0.3))
    shift = rows32(qin.normal(CFG, 302 + tag, (2, D), std=0.5))
    return w, scale, shift


def weight(N, K, tag, dt):
    st = qin.linear_weight(CFG, 60 + tag, N, K)
    return st, rt.from_bits(st.bits, "bf16", DEV).to(TD[dt])


SHAPES = [(300, 192, 320), (1, 64, 64), (257, 256, 64), (600, 448, 192), (513, 640, 128)]
# consuming shapes whose partial sums take the kernel's vector loads (ceil(K / 96) % 8 == 0)
WIDE_K = [(257, 256, 768), (129, 192, 3072)]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("M,D,row0,P", [(5, 256, 0, 2), (257, 3072, 10, 100), (33, 4096, 0, 0), (64, 32, 0, 64),
                                        (70, 992, 3, 40)])
def test_norm_fold_rows(M, D, row0, P, dt):
    say(f"[norm fold rows] M={M} D={D} row0={row0} P={P} {dt}")
    x = rows32(qin.normal(CFG, 310, (M, D), std=2.0))
    w, scale, _ = params(D, 0)
    xc_buf = torch.full((M + 2, D + 8), 7.0, dtype=TD[dt], device=DEV)
    xc = xc_buf[:M, :D]
    sq = torch.full((M + 2, n_parts(D)), 7.0, dtype=torch.float32, device=DEV)
    rt.norm_fold_rows(f32(x), xc, sq[:M], f32(w), f32(scale), row0, P)
    sync()
    sc = O.per_row(scale[0], scale[1], M, row0, P)
    check(host(xc), x * (1.0 + w) * (1.0 + sc), "16", "xc")
    check(host(sq[:M]), sums96(x), "f32", "sums of squares")
    assert torch.all(xc_buf[:M, D:] == 7.0) and torch.all(xc_buf[M:] == 7.0) and torch.all(sq[M:] == 7.0)
    # without the optional factors
    rt.norm_fold_rows(f32(x), xc, sq[:M])
    sync()
    check(host(xc), x, "16", "xc, no factors")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("tile", [0, 192])   # (the producing side runs 256 x 192 tiles)
@pytest.mark.parametrize("M,N,K", SHAPES + WIDE_K)
def test_fold_producer(M, N, K, tile, dt):
    say(f"[fold producer] M={M} N={N} K={K} tile={tile} {dt}")
    a = qin.stored(qin.normal(CFG, 320, (M, K)), dt)
    wst, wd = weight(N, K, 0, dt)
    x0 = rows32(qin.normal(CFG, 321, (M, N)))
    gate = rows32(qin.normal(CFG, 322, (2, N), std=0.7))
    nw, nscale, _ = params(N, 1)
    for row0, P in ((0, M // 3), (0, 0), (M, M)):
        x = f32(x0)
        xc_buf = torch.full((M + 2, N + 8), 5.0, dtype=TD[dt], device=DEV)
        xc = xc_buf[:M, :N]
        sq = torch.full((M + 2, n_parts(N)), 5.0, dtype=torch.float32, device=DEV)
        fold = rt.NormFold(xc=xc, next_w=f32(nw), next_scale=f32(nscale), sumsq_out=sq[:M])
        rt.gemm(rt.from_bits(a.bits, dt, DEV), wd, x, Q.QI_EPI_GATED_RESIDUAL, f32(gate), row0, P, tile_n=tile,
                fold=fold)
        sync()
        g = O.per_row(gate[0], gate[1], M, row0, P)
        ref_x = x0 + np.tanh(g) * O.linear(a.f64, wst.f64)
        check(host(x), ref_x, "f32", f"residual row0={row0} P={P}")
        xg = host(x)    # the residual as updated: xc and the sums are taken of it
        sc = O.per_row(nscale[0], nscale[1], M, row0, P)
        check(host(xc), xg * (1.0 + nw) * (1.0 + sc), "16", "xc")
        check(host(sq[:M]), sums96(xg), "f32", "sums of squares")
        assert torch.all(xc_buf[:M, N:] == 5.0) and torch.all(xc_buf[M:] == 5.0) and torch.all(sq[M:] == 5.0)


def consumer_case(M, N, K, dt, row0, P, epi, tile, tag=0):
    """x fp32 rows -> qi_norm_fold_rows -> the consuming GEMM with the bias tables of linear_multi.
    Returns the output, the oracle's Linear(norm_mod(x)) composition (SwiGLU: on gate and up
    weights), and the same Linear on the operand as stored, rrms(x) xc + shift (which isolates the
    GEMM from the rounding of xc to the 16-bit type: one bf16 rounding of the operand alone moves
    the composed result by about the 2e-3 bar)."""
    x = rows32(qin.normal(CFG, 330 + tag, (M, K), std=1.5))
    w, scale, shift = params(K, 2 + tag)
    if epi == Q.QI_EPI_SWIGLU:
        gst, gd = weight(N // 2, K, 1, dt)
        ust, ud = weight(N // 2, K, 2, dt)
        wd = rt.pack_swiglu(gd, ud)
    else:
        wst, wd = weight(N, K, 3, dt)
    xc = torch.empty((M, K), dtype=TD[dt], device=DEV)
    sq = torch.empty((M, n_parts(K)), dtype=torch.float32, device=DEV)
    rt.norm_fold_rows(f32(x), xc, sq, f32(w), f32(scale), row0, P)
    bias = torch.empty((2, wd.shape[0]), dtype=torch.float32, device=DEV)
    rt.linear_multi(f32(shift), wd, bias)
    odt = torch.float32 if epi == Q.QI_EPI_STORE_F32 else TD[dt]
    out = torch.full((M, N // 2 if epi == Q.QI_EPI_SWIGLU else N), 3.0, dtype=odt, device=DEV)
    rt.gemm(xc, wd, out, epi, None, row0, P, tile_n=tile, bias=bias[0], fold=rt.NormFold(sq, 1e-6, bias[1]))
    sync()
    sh = O.per_row(shift[0], shift[1], M, row0, P)
    h = O.norm_mod(x, w, O.per_row(scale[0], scale[1], M, row0, P), sh)
    hs = host(xc) / np.sqrt(np.mean(x * x, axis=1) + 1e-6)[:, None] + sh
    if epi == Q.QI_EPI_SWIGLU:
        ref, ref_s = (O.swiglu(O.linear(a, gst.f64), O.linear(a, ust.f64)) for a in (h, hs))
    else:
        ref, ref_s = (O.linear(a, wst.f64) for a in (h, hs))
    return out, ref, ref_s


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("tile", [128, 192, 256])
@pytest.mark.parametrize("M,N,K", SHAPES + WIDE_K)
def test_fold_consumer_store(M, N, K, tile, dt):
    say(f"[fold consumer store] M={M} N={N} K={K} tile={tile} {dt}")
    for row0, P in ((0, M // 2), (0, 0), (M, M)):
        out, ref, ref_s = consumer_case(M, N, K, dt, row0, P, Q.QI_EPI_STORE, tile)
        check(host(out), ref_s, "16", f"row0={row0} P={P}, on the stored operand")
        if dt == "f16":
            check(host(out), ref, "16", f"row0={row0} P={P}")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("tile", [128, 256])
@pytest.mark.parametrize("M,N,K", SHAPES + WIDE_K)
def test_fold_consumer_swiglu(M, N, K, tile, dt):
    say(f"[fold consumer swiglu] M={M} 2F={N} K={K} tile={tile} {dt}")
    out, ref, ref_s = consumer_case(M, N, K, dt, 0, M // 3, Q.QI_EPI_SWIGLU, tile)
    check(host(out), ref_s, "16", "swiglu, on the stored operand")
    if dt == "f16":
        check(host(out), ref, "16", "swiglu")


@pytest.mark.parametrize("M,N,K", [(300, 192, 320), (600, 448, 192)])
def test_fold_consumer_store_f32(M, N, K):
    out, ref, ref_s = consumer_case(M, N, K, "f16", 0, 100, Q.QI_EPI_STORE_F32, 0)
    check(host(out), ref_s, "f32", "fp32 store, on the stored operand")
    check(host(out), ref, "16", "fp32 store")


@pytest.mark.parametrize("nv,I,O_", [(1, 64, 5), (2, 3072, 9216), (9, 3072, 1000), (16, 520, 77)])
@pytest.mark.parametrize("wdt", ["bf16", "f16"])
def test_linear_multi(nv, I, O_, wdt):
    say(f"[linear multi] nv={nv} I={I} O={O_} {wdt}")
    x = rows32(qin.normal(CFG, 340, (nv, I)))
    wst, wd = weight(O_, I, 4, wdt)
    y = torch.full((nv, O_), 2.0, dtype=torch.float32, device=DEV)
    rt.linear_multi(f32(x), wd, y)
    sync()
    check(host(y), O.linear(x, host(wd)), "f32", "y")


def test_fold_tiles_give_identical_bits():
    # each row's partial sums and each output are the same fp32 sums in the same order at every
    # tile width of the consuming GEMM (the producing side always runs 256 x 192 tiles), which
    # keeps the cached layer equal to step 1's target rows bit for bit
    M, N, K = 600, 448, 192
    a = qin.stored(qin.normal(CFG, 350, (M, K)), "f16")
    _, wd = weight(N, K, 5, "f16")
    x0 = f32(qin.normal(CFG, 351, (M, N)))
    gate = f32(qin.normal(CFG, 352, (2, N), std=0.7))
    nw, nscale, shift = params(N, 4)
    prod = []
    for tile in (0, 192):
        x = x0.clone()
        xc = torch.zeros((M, N), dtype=torch.float16, device=DEV)
        sq = torch.zeros((M, n_parts(N)), dtype=torch.float32, device=DEV)
        rt.gemm(rt.from_bits(a.bits, "f16", DEV), wd, x, Q.QI_EPI_GATED_RESIDUAL, gate, 0, 100, tile_n=tile,
                fold=rt.NormFold(xc=xc, next_w=f32(nw), next_scale=f32(nscale), sumsq_out=sq))
        prod.append((x, xc, sq))
    _, w2 = weight(320, N, 6, "f16")
    bias = torch.empty((2, 320), dtype=torch.float32, device=DEV)
    rt.linear_multi(f32(shift), w2, bias)
    outs = []
    for tile in (0, 128, 192, 256):
        y = torch.zeros((M, 320), dtype=torch.float16, device=DEV)
        rt.gemm(prod[0][1], w2, y, Q.QI_EPI_STORE, None, 0, 100, tile_n=tile, bias=bias[0],
                fold=rt.NormFold(prod[0][2], 1e-6, bias[1]))
        outs.append(y)
    sync()
    for t, t0 in zip(prod[1], prod[0]):
        assert torch.equal(t, t0)
    for y in outs[1:]:
        assert torch.equal(y, outs[0])
    # other tile widths are refused for the producing side
    x = x0.clone()
    with pytest.raises(Q.QiError):
        rt.gemm(rt.from_bits(a.bits, "f16", DEV), wd, x, Q.QI_EPI_GATED_RESIDUAL, gate, 0, 100, tile_n=128,
                fold=rt.NormFold(xc=prod[0][1], sumsq_out=prod[0][2]))


def test_fold_range_flag():
    # an xc value beyond the fp16 range raises QI_RANGE_OUT in the caller's word
    M, N, K = 64, 64, 64
    a = torch.zeros((M, K), dtype=torch.float16, device=DEV)
    w = torch.zeros((N, K), dtype=torch.float16, device=DEV)
    x = torch.ones((M, N), dtype=torch.float32, device=DEV)
    x[5, 7] = 70000.0
    gate = torch.zeros((2, N), dtype=torch.float32, device=DEV)
    xc = torch.empty((M, N), dtype=torch.float16, device=DEV)
    sq = torch.empty((M, n_parts(N)), dtype=torch.float32, device=DEV)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    rt.gemm(a, w, x, Q.QI_EPI_GATED_RESIDUAL, gate, flags=flags, fold=rt.NormFold(xc=xc, sumsq_out=sq))
    sync()
    assert int(flags.item()) == Q.QI_RANGE_OUT
    flags.zero_()
    x[5, 7] = 60000.0
    rt.gemm(a, w, x, Q.QI_EPI_GATED_RESIDUAL, gate, flags=flags, fold=rt.NormFold(xc=xc, sumsq_out=sq))
    sync()
    assert int(flags.item()) == 0
