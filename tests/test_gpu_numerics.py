"""GPU parity on inputs that N(0,1) draws never reach, through the C ABI, against the fp64 oracle.

- Every row of two heads of the 21,504-key cached step: head 0 runs as whole query tiles, head 2
  as tiles cut into two key chunks merged afterwards (the launch's schedule, checked here).
- Peaked softmax: Q and K scaled by 6 and by 20, step 1 and the cached step.
- A rising maximum: key scores that grow along the key sequence, so each row's softmax reference
  moves on most tiles (the kernel's rescale branch), in step 1 (masked tiles) and in the cached
  step (whole and chunked tiles).
- V scaled by 1e-3: chunk partials far below fp16's normal range before their per-row scale.
- The range flags of the fp16 operands (values of 65520 and more are reported, 65280 is not).

Bars.  Against the plain oracle (fp64 on the stored bf16 inputs): mean relative error
sum|d| / sum|ref| <= 2e-3 always, and max|d| <= 1e-2 max|ref| where the inputs are N(0,1)-like.
For peaked and rising scores the output is ill-conditioned in the scores: the fp16 rounding of
the rotated operands alone (at most 2^-11 relative per entry) moves a score by up to ~1e-3 of
its magnitude, and where a row's top scores nearly tie that moves the output by more than
1e-2 max|ref| (a NumPy model of that rounding alone gives 1.2e-2 at scale 6 and 0.14 at
scale 20).  There the max bar is applied against the oracle evaluated on the same operands
rounded to fp16 (rotated K; rotated Q times scale * log2(e)), which isolates the online softmax,
its moving reference and the chunk merge from the operand rounding, and the mean bar is still
applied against the plain oracle.
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
LOG2E = 1.4426950408889634
HEADLINE = "txt1024_4ref64_tgt64"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_errors(got, ref):
    d = np.abs(np.asarray(got, np.float64) - ref)
    return d.max() / max(np.abs(ref).max(), 1e-300), d.sum() / max(np.abs(ref).sum(), 1e-300)


def check(got, ref, what, max_bar=1e-2, mean_bar=2e-3):
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape and np.all(np.isfinite(got)), what
    mx, mn = rel_errors(got, ref)
    say(f"  {what}: max_rel={mx:.3e} mean_rel={mn:.3e}")
    if max_bar is not None:
        assert mx <= max_bar, (what, mx)
    assert mn <= mean_bar, (what, mn)


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def f16(x):
    """Round to fp16 (nearest even) by way of fp32, as the kernels convert their fp32 values."""
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float16).astype(np.float64)


def operands_f16(qr, kr):
    """The rotated operands at the kernels' fp16 precision: K as is, Q times scale * log2(e)
    (returned divided by that factor again, so the oracle's own scale applies)."""
    c = np.float32(LOG2E / math.sqrt(128))
    qs = f16(np.asarray(qr, np.float64).astype(np.float32) * c) / float(c)
    return qs, f16(kr)


def stored_bf16(x64):
    return qin.stored(x64, "bf16")


def dev(st):
    return rt.from_bits(st.bits, "bf16", DEV)


# ---------------------------------------------------------------------------------------------
# the 21,504-key cached step, every row of a whole-tile head and a chunked-tile head
# ---------------------------------------------------------------------------------------------

def headline_heads():
    """(whole head, chunked head) of the 4,096-query, 24-head launch: 384 query tiles, 48 per
    XCD run; a run's first 32 tiles (two heads) run whole and its last 16 (the third head) in
    two key chunks."""
    assert Q.qi_attn_schedule(4096, 24, 17408, 4096) == (2, 32, 128)
    return 0, 2


def headline_case(q_scale=1.0, k_scale=1.0, v_scale=1.0, seed=0):
    wl = qin.WORKLOADS[HEADLINE]
    S, P, T = wl.S, wl.P, wl.T
    H = wl.n_head
    base = [qin.normal(wl.cfg_id, t, (S, H, 128), seed) for t in (qin.T_Q, qin.T_K, qin.T_V)]
    q, k, v = (stored_bf16(x * s) for x, s in zip(base, (q_scale, k_scale, v_scale)))
    del base
    return wl, q, k, v


def run_headline_cached(wl, q, k, v):
    S, P, T = wl.S, wl.P, wl.T
    L = rt.Layout(wl.segments, DEV)
    att = rt.Attention(L, wl.n_head, Q.QI_BF16, DEV)
    qd, kd, vd = dev(q), dev(k), dev(v)
    cache = rt.KVCache(1, wl.n_head, P, Q.QI_BF16, DEV)
    att.store(kd[:P], vd[:P], cache, 0)
    ot = att.cached(qd[P:], kd[P:], vd[P:], cache, 0)
    torch.cuda.synchronize()
    assert att.range_flags() == 0
    out = to_np(ot)
    del cache, qd, kd, vd, ot
    torch.cuda.empty_cache()
    return out


def oracle_heads(wl, q, k, v, heads, rows=None, f16_operands=False):
    S, P, T = wl.S, wl.P, wl.T
    c, s = O.rope_tables(O.positions(wl.segments))
    hs = list(heads)
    qt = q.f64[P:][:, hs] if rows is None else q.f64[P:][rows][:, hs]
    ct, st = (c[P:], s[P:]) if rows is None else (c[P:][rows], s[P:][rows])
    qr = O.rotate(qt, ct, st)
    kr = O.rotate(k.f64[:, hs], c, s)
    if f16_operands:
        qr, kr = operands_f16(qr, kr)
    return O.attention(qr, kr, v.f64[:, hs])


def test_headline_cached_every_row_of_a_whole_and_a_chunked_head():
    wl, q, k, v = headline_case()
    hw, hc = headline_heads()
    say(f"{HEADLINE} cached step, every row of head {hw} (whole tiles) and head {hc} (two key chunks)")
    got = run_headline_cached(wl, q, k, v)
    ref = oracle_heads(wl, q, k, v, (hw, hc))
    check(got[:, hw], ref[:, 0], f"head {hw} whole tiles")
    check(got[:, hc], ref[:, 1], f"head {hc} chunked tiles")


def test_headline_cached_small_v_chunk_partials():
    # V ~ 1e-3 N(0,1): a chunk's normalised output is ~1e-5, below fp16's normal range (6.1e-5)
    # until the per-row power-of-two scale lifts it; whole rows never pass through fp16 partials
    wl, q, k, v = headline_case(v_scale=1e-3)
    hw, hc = headline_heads()
    say(f"{HEADLINE} cached step, V scaled by 1e-3")
    got = run_headline_cached(wl, q, k, v)
    ref = oracle_heads(wl, q, k, v, (hw, hc))
    assert np.abs(ref[:, 1]).max() < 2e-4
    check(got[:, hw], ref[:, 0], f"head {hw} whole tiles, small V")
    check(got[:, hc], ref[:, 1], f"head {hc} chunked tiles, small V")


@pytest.mark.parametrize("scale", [6.0, 20.0])
def test_headline_cached_peaked(scale):
    wl, q, k, v = headline_case(q_scale=scale, k_scale=scale, seed=1)
    hw, hc = headline_heads()
    say(f"{HEADLINE} cached step, Q and K scaled by {scale}")
    got = run_headline_cached(wl, q, k, v)
    ref = oracle_heads(wl, q, k, v, (hw, hc))
    ref16 = oracle_heads(wl, q, k, v, (hw, hc), f16_operands=True)
    for i, h in enumerate((hw, hc)):
        mx, mn = rel_errors(got[:, h], ref[:, i])
        say(f"  head {h} vs plain oracle: max_rel={mx:.3e} mean_rel={mn:.3e}")
        assert mn <= 2e-3, (h, mn)
        check(got[:, h], ref16[:, i], f"head {h} vs oracle on fp16 operands")


def test_headline_step1_peaked_sampled_rows():
    # block-causal step 1 at the 21,504-token shape with Q and K scaled by 6, rows from every
    # segment (masked diagonal tiles, the longest and the shortest rows)
    wl, q, k, v = headline_case(q_scale=6.0, k_scale=6.0, seed=2)
    say(f"{HEADLINE} step 1, Q and K scaled by 6, sampled rows")
    L = rt.Layout(wl.segments, DEV)
    att = rt.Attention(L, wl.n_head, Q.QI_BF16, DEV)
    o = att.full(dev(q), dev(k), dev(v))
    torch.cuda.synchronize()
    assert att.range_flags() == 0
    bounds = np.cumsum([0] + [g.n_tokens for g in wl.segments])
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([rng.integers(bounds[i], bounds[i + 1], 6) for i in range(len(bounds) - 1)]
                                    + [bounds[:-1], bounds[1:] - 1]))
    hs = [0, 5]
    c, s = O.rope_tables(O.positions(wl.segments))
    qr = O.rotate(q.f64[rows][:, hs], c[rows], s[rows])
    kr = O.rotate(k.f64[:, hs], c, s)
    m = O.mask_rows(wl.segments, rows)
    ref = O.attention(qr, kr, v.f64[:, hs], m)
    ref16 = O.attention(*operands_f16(qr, kr), v.f64[:, hs], m)
    got = to_np(o[rows][:, hs])
    mx, mn = rel_errors(got, ref)
    say(f"  vs plain oracle: max_rel={mx:.3e} mean_rel={mn:.3e}")
    assert mn <= 2e-3
    check(got, ref16, "step-1 rows vs oracle on fp16 operands")


# ---------------------------------------------------------------------------------------------
# rising maximum: the softmax reference moves on most key tiles
# ---------------------------------------------------------------------------------------------

def rising_inputs(n_tok, n_head, key_index, seed, rise=3.0):
    """Pre-rotated q, k and v (no rotation tables are passed): k_j = 0.5 N(0,1) + a(j) u with a
    common unit direction u per head and a(j) growing by `rise` log2 units of score per 64-key
    tile of the key order (key_index[j] = position of token j among the keys); q_i = 0.5 N(0,1)
    + b_i u with b_i from 0.5 to 4, so rows see their scores climb at different rates."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((n_head, 128))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    b = rng.uniform(0.5, 4.0, (n_tok, n_head, 1))
    c = math.sqrt(128) / LOG2E      # q.k * scale * log2(e) = b * a for unit u
    a = (rise * c / 2.0) * (np.asarray(key_index) // 64)[:, None, None]
    q = 0.5 * rng.standard_normal((n_tok, n_head, 128)) + b * u[None]
    k = 0.5 * rng.standard_normal((n_tok, n_head, 128)) + a * u[None]
    v = rng.standard_normal((n_tok, n_head, 128))
    return stored_bf16(q), stored_bf16(k), stored_bf16(v)


def test_rising_max_step1_block_causal():
    segs = (qin.text(200), qin.image(12, 16, 1), qin.image(16, 20, 2), qin.image(17, 19, 0))
    S, P, T = O.split_counts(segs)
    H = 3
    q, k, v = rising_inputs(S, H, np.arange(S), seed=21)
    say(f"rising maximum, step 1 block-causal, S={S}")
    L = rt.Layout(segs, DEV)
    att = rt.Attention(L, H, Q.QI_BF16, DEV)
    o = att.full(dev(q), dev(k), dev(v), rotate=False)
    torch.cuda.synchronize()
    assert att.range_flags() == 0
    m = O.mask_dense(segs)
    ref = O.attention(q.f64, k.f64, v.f64, m)
    ref16 = O.attention(*operands_f16(q.f64, k.f64), v.f64, m)
    got = to_np(o)
    mx, mn = rel_errors(got, ref)
    say(f"  vs plain oracle: max_rel={mx:.3e} mean_rel={mn:.3e}")
    assert mn <= 2e-3
    check(got, ref16, "step 1 vs oracle on fp16 operands")


def test_rising_max_headline_cached_whole_and_chunked():
    wl = qin.WORKLOADS[HEADLINE]
    S, P, T = wl.S, wl.P, wl.T
    H = wl.n_head
    hw, hc = headline_heads()
    q, k, v = rising_inputs(S, H, np.arange(S), seed=22)
    say(f"rising maximum, {HEADLINE} cached step, heads {hw} and {hc}")
    L = rt.Layout(wl.segments, DEV)
    att = rt.Attention(L, H, Q.QI_BF16, DEV)
    qd, kd, vd = dev(q), dev(k), dev(v)
    cache = rt.KVCache(1, H, P, Q.QI_BF16, DEV)
    att.store(kd[:P], vd[:P], cache, 0, rotate=False)
    ot = att.cached(qd[P:], kd[P:], vd[P:], cache, 0, rotate=False)
    torch.cuda.synchronize()
    assert att.range_flags() == 0
    got = to_np(ot)
    hs = [hw, hc]
    qh, kh = q.f64[P:][:, hs], k.f64[:, hs]
    ref = O.attention(qh, kh, v.f64[:, hs])
    ref16 = O.attention(*operands_f16(qh, kh), v.f64[:, hs])
    # scores reach ~2,000 (log2 units) by the last of the 336 key tiles, so the fp16 rounding
    # of the operands moves them by ~0.1: only the oracle on the same fp16 operands can gate
    # the softmax machinery here (the plain comparison is printed)
    for i, h in enumerate(hs):
        mx, mn = rel_errors(got[:, h], ref[:, i])
        say(f"  head {h} vs plain oracle (not gated): max_rel={mx:.3e} mean_rel={mn:.3e}")
        check(got[:, h], ref16[:, i], f"head {h} vs oracle on fp16 operands")


# ---------------------------------------------------------------------------------------------
# the perturbed target of the prefix bit-identity test, against the oracle
# ---------------------------------------------------------------------------------------------

def test_perturbed_target_rows_match_oracle():
    wl = qin.WORKLOADS["txt256_ref32_tgt32"]
    S, P, T = wl.S, wl.P, wl.T
    q, k, v = qin.qkv(wl, S)
    qw, kw = qin.qk_norm_weights(wl)
    qwd = torch.tensor(qw, dtype=torch.float32, device=DEV)
    kwd = torch.tensor(kw, dtype=torch.float32, device=DEV)
    L = rt.Layout(wl.segments, DEV)
    att = rt.Attention(L, wl.n_head, Q.QI_BF16, DEV)
    q2, k2, v2 = dev(q).clone(), dev(k).clone(), dev(v).clone()
    g = torch.Generator(device=DEV).manual_seed(5)
    for t in (q2, k2, v2):
        t[P:] = (torch.randn(t[P:].shape, generator=g, device=DEV) * 4).to(t.dtype)
    o2 = att.full(q2, k2, v2, qwd, kwd)
    torch.cuda.synchronize()
    c, s = O.rope_tables(O.positions(wl.segments))
    ref, _ = O.step1(to_np(q2), to_np(k2), to_np(v2), wl.segments, c, s, qw, kw)
    say("txt256_ref32_tgt32 step 1 with the target's Q, K, V redrawn at 4 N(0,1)")
    check(to_np(o2)[P:], ref[P:], "perturbed target rows")
    check(to_np(o2)[:P], ref[:P], "prefix rows")


# ---------------------------------------------------------------------------------------------
# fp16 I/O (the layer chain's activation type): the same kernels with fp16 loads and stores
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("segs,heads,qk", [((qin.text(77), qin.image(13, 9, 1), qin.image(15, 17, 0)), 3, True),
                                           ((qin.text(200), qin.image(12, 16, 1), qin.image(16, 20, 2),
                                             qin.image(17, 19, 0)), 2, False)])
def test_f16_io_step1_and_cached(segs, heads, qk):
    wl = qin.small_workload("f16_io", segs, n_head=heads, dtype="f16", qk_rmsnorm=qk)
    S, P, T = wl.S, wl.P, wl.T
    say(f"fp16 I/O step 1 + cached step: S={S} heads={heads} qk_norm={qk}")
    q, k, v = qin.qkv(wl, S)
    q2, k2, v2 = qin.qkv(wl, S, step=1)
    qw, kw = qin.qk_norm_weights(wl) if qk else (None, None)
    qwd = None if qw is None else torch.tensor(qw, dtype=torch.float32, device=DEV)
    kwd = None if kw is None else torch.tensor(kw, dtype=torch.float32, device=DEV)
    L = rt.Layout(segs, DEV)
    att = rt.Attention(L, heads, Q.QI_F16, DEV)
    cache = rt.KVCache(1, heads, P, Q.QI_F16, DEV)
    qd, kd, vd = (rt.from_bits(t.bits, "f16", DEV) for t in (q, k, v))
    o = att.full(qd, kd, vd, qwd, kwd, cache=cache)
    q2d, k2d, v2d = (rt.from_bits(t.bits, "f16", DEV) for t in (q2, k2, v2))
    ot = att.cached(q2d[P:], k2d[P:], v2d[P:], cache, 0, qwd, kwd)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16 and att.range_flags() == 0
    c, s = O.rope_tables(O.positions(segs))
    ref, oc = O.step1(q.f64, k.f64, v.f64, segs, c, s, qw, kw)
    check(to_np(o), ref, "fp16 I/O step 1")
    ref_t = O.cached_step(q2.f64[P:], k2.f64[P:], v2.f64[P:], oc, c[P:], s[P:], qw, kw)
    check(to_np(ot), ref_t, "fp16 I/O cached step")
    # the cached step equals the full recompute on [prefix | new target], bit for bit
    qn, kn, vn = (torch.cat([a[:P], b[P:]]) for a, b in ((qd, q2d), (kd, k2d), (vd, v2d)))
    of = att.full(qn, kn, vn, qwd, kwd)
    torch.cuda.synchronize()
    assert torch.equal(ot.view(torch.int16), of[P:].view(torch.int16))


# ---------------------------------------------------------------------------------------------
# range flags of the fp16 operands
# ---------------------------------------------------------------------------------------------

def small_case(qk=False, n_head=2):
    segs = (qin.text(77), qin.image(13, 9, 1), qin.image(15, 17, 0))
    wl = qin.small_workload("range", segs, n_head=n_head, dtype="bf16", qk_rmsnorm=qk)
    S, P, T = wl.S, wl.P, wl.T
    q, k, v = (dev(t).clone() for t in qin.qkv(wl, S))
    L = rt.Layout(segs, DEV)
    att = rt.Attention(L, n_head, Q.QI_BF16, DEV)
    return wl, att, q, k, v


def test_range_flags_stay_clear_on_ordinary_inputs():
    wl, att, q, k, v = small_case()
    P = wl.P
    cache = rt.KVCache(1, wl.n_head, P, Q.QI_BF16, DEV)
    att.full(q, k, v, cache=cache)
    att.store(k[:P], v[:P], cache, 0)
    att.cached(q[P:], k[P:], v[P:], cache, 0)
    # 65280, the largest bf16 value below fp16's overflow threshold of 65520, converts exactly
    # and raises nothing
    v[P + 3, 1, 7] = 65280.0
    v[5, 0, 0] = -65280.0
    att.store(k[:P], v[:P], cache, 0)
    att.cached(q[P:], k[P:], v[P:], cache, 0)
    torch.cuda.synchronize()
    assert att.range_flags() == 0
    vc = cache.v_rows(0)
    assert float(vc[0, 5, 0]) == -65280.0


@pytest.mark.parametrize("where", ["target_v", "prefix_v", "k", "q"])
def test_range_flags_raised(where):
    wl, att, q, k, v = small_case()
    P = wl.P
    cache = rt.KVCache(1, wl.n_head, P, Q.QI_BF16, DEV)
    att.store(k[:P], v[:P], cache, 0)
    torch.cuda.synchronize()
    assert att.range_flags() == 0
    if where == "target_v":
        v[P + 10, 1, 100] = 1.0e5
        att.cached(q[P:], k[P:], v[P:], cache, 0)
        want = Q.QI_RANGE_V
    elif where == "prefix_v":
        v[3, 0, 0] = -65536.0            # the first bf16 value that rounds to infinity in fp16
        att.store(k[:P], v[:P], cache, 0)
        want = Q.QI_RANGE_V
    elif where == "k":
        k[P + 1, 0, 5] = 2.0e5           # no QK-norm: the rotated K keeps that magnitude
        att.cached(q[P:], k[P:], v[P:], cache, 0)
        want = Q.QI_RANGE_K
    else:
        q[P + 2, 1, 9] = 6.0e5           # times scale * log2(e) = 0.1275: 76,500 > 65,504
        att.cached(q[P:], k[P:], v[P:], cache, 0)
        want = Q.QI_RANGE_Q
    torch.cuda.synchronize()
    assert att.range_flags() == want
    with pytest.raises(rt.RangeError):
        v[P + 10, 1, 100] = 1.0e5
        att.cached(q[P:], k[P:], v[P:], cache, 0)
        att.check_range()
    # the step-1 call reports as well
    att.full(q, k, v)
    torch.cuda.synchronize()
    assert att.range_flags() & Q.QI_RANGE_V


def test_range_flags_not_raised_by_fp32_io():
    segs = (qin.text(16), qin.image(4, 4, 1), qin.image(4, 4, 0))
    wl = qin.WORKLOADS["tiny_f32"]
    S, P, T = wl.S, wl.P, wl.T
    q, k, v = (rt.from_bits(t.bits, "f32", DEV).clone() for t in qin.qkv(wl, S))
    v[3, 0, 0] = 1.0e6
    L = rt.Layout(segs, DEV)
    att = rt.Attention(L, wl.n_head, Q.QI_F32, DEV)
    att.full(q, k, v)
    torch.cuda.synchronize()
    assert att.range_flags() == 0
