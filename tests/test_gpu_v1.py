"""GPU parity of the v1 / Edit dual-stream block ("QwenImageTransformer2DModel source reading
(Qwen-Image-Edit)", sections 5.2 and 6) and of the library pieces it adds: LayerNorm +
modulation, GEMM epilogues with a bias and the plain (untanh'd) residual gate, the conditioning
linear with a bias.  Everything is called through the C ABI and checked against the fp64 oracle on
the same seeded inputs.

Tolerances (written here, per output tensor), as for the single-stream layer:
  16-bit outputs, the block's outputs and its residual increments (the block runs fp16
  activations and fp16 copies of its bf16 weights): max|d| <= 1e-2 * max|ref| and
  sum|d| / sum|ref| <= 2e-3
  fp32 outputs of one fp32-accumulated step on stored inputs: max and mean <= 1e-5
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
CFG = 92   # seed id of the shapes here


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


def bf(st: qin.Stored) -> torch.Tensor:
    return rt.from_bits(st.bits, "bf16", DEV)


TD = {"bf16": torch.bfloat16, "f16": torch.float16}


def f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def f32v(idx, shape, std=1.0):
    return qin.normal(CFG, idx, shape, std=std).astype(np.float32).astype(np.float64)


# ------------------------------------------------------------------------------------------------
# the pieces
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("M,D,row0,P,mod", [(300, 3072, 0, 170, True), (129, 256, 40, 100, True), (77, 132, 0, 0, False),
                                            (64, 768, 0, 64, True), (9, 4104, 0, 5, True)])
def test_layernorm_mod(M, D, row0, P, mod, dt):
    say(f"[layernorm mod] M={M} D={D} row0={row0} P={P} mod={mod} {dt}")
    x = f32v(300, (M, D), 3.0) + 1.7   # rows with a large common offset: the mean matters
    sc = f32v(301, (2, D), 0.3) if mod else None
    sh = f32v(302, (2, D), 0.3) if mod else None
    ref = O.layer_norm(x)
    if mod:
        ref = ref * (1.0 + O.per_row(sc[0], sc[1], M, row0, P)) + O.per_row(sh[0], sh[1], M, row0, P)
    buf = torch.full((M + 3, D + 4), 9.0, dtype=TD[dt], device=DEV)
    out = buf[:M, :D]
    rt.layernorm_mod(f32(x), out, None if sc is None else f32(sc), None if sh is None else f32(sh), row0, P)
    torch.cuda.synchronize()
    check(host(out), ref, dt, "layernorm_mod")
    assert torch.all(buf[:M, D:] == 9.0) and torch.all(buf[M:] == 9.0), "write outside the output view"


@pytest.mark.parametrize("dtn", ["bf16", "f16"])
@pytest.mark.parametrize("M,N,K", [(300, 192, 320), (257, 256, 64), (70, 640, 256)])
def test_gemm_bias_epilogues(M, N, K, dtn):
    say(f"[gemm bias] M={M} N={N} K={K} {dtn}")
    x = qin.stored(qin.normal(CFG, 310, (M, K)), dtn)
    xd, wd = rt.from_bits(x.bits, dtn, DEV), None
    w = qin.linear_weight(CFG, 70, N, K)
    b = f32v(311, (N,), 0.5)
    y = O.linear_bias(x.f64, w.f64, b)
    x0 = f32v(312, (M, N))
    gate = f32v(313, (2, N), 0.7)
    g = O.per_row(gate[0], gate[1], M, 0, M // 3)
    wd = bf(w).to(TD[dtn])
    cases = [(Q.QI_EPI_STORE, TD[dtn], dtn, None, y),
             (Q.QI_EPI_STORE_F32, torch.float32, "f32", None, y),
             (Q.QI_EPI_GELU, TD[dtn], dtn, None, O.gelu_tanh(y)),
             (Q.QI_EPI_GATED_RESIDUAL_LINEAR, torch.float32, "f32", x0, x0 + g * y),
             (Q.QI_EPI_GATED_RESIDUAL, torch.float32, "f32", x0, x0 + np.tanh(g) * y)]
    for epi, dt, bar, init, ref in cases:
        out = torch.zeros((M, N), dtype=dt, device=DEV) if init is None else f32(init)
        rt.gemm(xd, wd, out, epi, f32(gate), 0, M // 3, bias=f32(b))
        torch.cuda.synchronize()
        check(host(out), ref, bar, f"epilogue {epi}")
    # the linear gate without a bias
    out = f32(x0)
    rt.gemm(xd, wd, out, Q.QI_EPI_GATED_RESIDUAL_LINEAR, f32(gate), 0, M // 3)
    torch.cuda.synchronize()
    check(host(out), x0 + g * O.linear(x.f64, w.f64), "f32", "linear gate, no bias")


def test_gemm_bias_argument_errors():
    z = torch.zeros((64, 64), dtype=torch.bfloat16, device=DEV)
    o = torch.zeros((64, 64), dtype=torch.float32, device=DEV)
    s = rt.stream_handle(DEV)
    # the linear gate needs its gate vector; a misaligned bias is refused
    assert Q.qi_gemm_bf16_bias(z, 64, z, None, o, 64, 64, 64, 64, Q.QI_EPI_GATED_RESIDUAL_LINEAR, None, 0, 0, s) \
        == Q.QI_ERR_ARG
    b = torch.zeros(80, dtype=torch.float32, device=DEV)
    assert Q.qi_gemm_bf16_bias(z, 64, z, b[1:], o, 64, 64, 64, 64, Q.QI_EPI_STORE_F32, None, 0, 0, s) == Q.QI_ERR_ALIGN
    assert Q.qi_gemm_bf16_bias(z, 64, z, b, o, 64, 64, 64, 64, 6, None, 0, 0, s) == Q.QI_ERR_ARG
    assert Q.qi_layernorm_mod(None, 64, o, 64, 4, 64, None, None, 0, 0, 1e-6, s) == Q.QI_ERR_ARG


@pytest.mark.parametrize("nv,I,O_", [(2, 256, 256), (2, 3072, 3072), (1, 8, 5)])
def test_linear_small_bias(nv, I, O_):
    say(f"[linear small bias] nv={nv} I={I} O={O_}")
    x = f32v(320, (nv, I), 2.0)
    w = qin.linear_weight(CFG, 80, O_, I)
    b = f32v(321, (O_,), 0.5)
    y = torch.empty((nv, O_), dtype=torch.float32, device=DEV)
    rt.linear_small(f32(x), bf(w), y, True, f32(b))
    torch.cuda.synchronize()
    check(host(y), O.linear_bias(O.silu(x), w.f64, b), "f32", "linear_small_bias")


# ------------------------------------------------------------------------------------------------
# the whole block
# ------------------------------------------------------------------------------------------------

V1_CASES = [
    ("edit_small", 256, 1024, (qin.text(37), qin.image(9, 7, 0), qin.image(9, 7, 1)), None),
    ("edit_small_per_token", 256, 1024, (qin.text(37), qin.image(9, 7, 0), qin.image(9, 7, 1)), 63),
    ("editplus_medium", 768, 3072, (qin.text(77), qin.image(16, 16, 0), qin.image(12, 16, 1), qin.image(8, 8, 2)),
     None),
]


@pytest.mark.parametrize("name,D,F,segs,n_noise", V1_CASES)
def test_v1_block(name, D, F, segs, n_noise):
    H = D // 128
    Lt = segs[0].n_tokens
    Li = sum(s.n_tokens for s in segs[1:])
    say(f"[v1 block] {name}: D={D} F={F} text {Lt} image {Li} n_noise={n_noise}")
    Wh = qin.v1_block_weights(CFG, D, F)
    xt, xi, temb, temb0 = qin.v1_block_inputs(CFG, Lt, Li, D)
    Wd = {k: (bf(v) if isinstance(v, qin.Stored) else f32(v)) for k, v in Wh.items()}
    Bo = {k: (v.f64 if isinstance(v, qin.Stored) else v) for k, v in Wh.items()}
    L = rt.Layout(segs, DEV, attention=Q.QI_ATTN_FULL)
    blk = rt.V1Block(rt.V1BlockWeights(Wd), L, H, DEV)
    cond = np.stack([temb, temb0 if n_noise is not None else temb])
    gt, gi = f32(xt), f32(xi)
    blk(gt, gi, f32(cond), n_noise)
    torch.cuda.synchronize()
    cos, sin = O.rope_tables(O.positions(segs))
    rt_, ri = O.v1_block(xt, xi, temb, Bo, cos, sin, temb0 if n_noise is not None else None, n_noise)
    check(host(gt) - xt, rt_ - xt, "f16", f"{name} text increment")
    check(host(gi) - xi, ri - xi, "f16", f"{name} image increment")
    assert blk.att.range_flags() == 0
    check(host(gt), rt_, "bf16", f"{name} text stream")
    check(host(gi), ri, "bf16", f"{name} image stream")


def v1_device_weights(Wh):
    return {k: (bf(v) if isinstance(v, qin.Stored) else f32(v)) for k, v in Wh.items()}


def host_weights(Wh):
    return {k: (v.f64 if isinstance(v, qin.Stored) else v) for k, v in Wh.items()}


def test_v1_two_blocks_and_output_head():
    # two dual-stream blocks in sequence, then the exit (norm_out + proj_out, [EDIT] section 5.3)
    # on the image stream, against the oracle's v1_forward
    D, F = 256, 1024
    segs = (qin.text(37), qin.image(9, 7, 0), qin.image(9, 7, 1))
    Lt = segs[0].n_tokens
    Li = sum(s.n_tokens for s in segs[1:])
    say(f"[v1 two blocks + head] D={D} text {Lt} image {Li}")
    Wh = [qin.v1_block_weights(CFG, D, F, layer=l) for l in range(2)]
    Hh = qin.v1_head_weights(CFG, D)
    xt, xi, temb, _ = qin.v1_block_inputs(CFG, Lt, Li, D)
    L = rt.Layout(segs, DEV, attention=Q.QI_ATTN_FULL)
    blocks = [rt.V1Block(rt.V1BlockWeights(v1_device_weights(W)), L, D // 128, DEV) for W in Wh]
    Hd = v1_device_weights(Hh)
    head = rt.V1Head(Hd["norm_out_w"], Hd["norm_out_b"], Hd["proj_out_w"], Hd["proj_out_b"])
    gt, gi = f32(xt), f32(xi)
    cond = f32(np.stack([temb, temb]))
    for b in blocks:
        b(gt, gi, cond)
    v = head(gi, f32(temb))
    torch.cuda.synchronize()
    cos, sin = O.rope_tables(O.positions(segs))
    ref = O.v1_forward(xt, xi, temb, [host_weights(W) for W in Wh], host_weights(Hh), cos, sin)
    check(host(v), ref, "f16", "two blocks + output head")
    assert int(head.flags.item()) == 0 and all(b.att.range_flags() == 0 for b in blocks)


def test_v1_block_model_width_sampled():
    # the block at the model's width (D 3072 = 24 x 128 heads, MLP 12288, [EDIT] section 2) on the
    # Edit-Plus sequence (text 512 + noisy target 64x64 + two references 64x64, 12,800 tokens,
    # [EDIT] section 10), compared on sampled rows of every segment (the oracle forms every row's
    # keys and values, and the outputs of the sampled rows only)
    wl = qin.V1_WORKLOADS["editplus_v1"]
    D, F = 3072, 12288
    segs = wl.segments
    Lt = segs[0].n_tokens
    Li = wl.S - Lt
    say(f"[v1 block model width] D={D} F={F} text {Lt} image {Li}")
    Wh = qin.v1_block_weights(CFG, D, F)
    xt, xi, temb, _ = qin.v1_block_inputs(CFG, Lt, Li, D)
    L = rt.Layout(segs, DEV, attention=Q.QI_ATTN_FULL)
    blk = rt.V1Block(rt.V1BlockWeights(v1_device_weights(Wh)), L, D // 128, DEV)
    gt, gi = f32(xt), f32(xi)
    blk(gt, gi, f32(np.stack([temb, temb])))
    torch.cuda.synchronize()
    assert blk.att.range_flags() == 0
    rng = np.random.default_rng(5)
    rows_t = np.unique(np.concatenate([[0, Lt - 1], rng.integers(0, Lt, 10)]))
    bounds = np.cumsum([0] + [s.n_tokens for s in segs[1:]])
    rows_i = np.unique(np.concatenate([np.concatenate([[a, b - 1], rng.integers(a, b, 8)])
                                       for a, b in zip(bounds[:-1], bounds[1:])]))
    cos, sin = O.rope_tables(O.positions(segs))
    Bo = host_weights(Wh)
    del Wh
    rt_, ri = O.v1_block(xt, xi, temb, Bo, cos, sin, rows_txt=rows_t, rows_img=rows_i)
    gt_h, gi_h = host(gt)[rows_t], host(gi)[rows_i]
    check(gt_h - xt[rows_t], rt_ - xt[rows_t], "f16", "text increment, sampled rows")
    check(gi_h - xi[rows_i], ri - xi[rows_i], "f16", "image increment, sampled rows")
    check(gt_h, rt_, "bf16", "text stream, sampled rows")
    check(gi_h, ri, "bf16", "image stream, sampled rows")
