"""The allocation-free cached step (qi_attn_target_cached_noalloc) against the cached step with a
caller workspace (qi_attn_target_cached), through the C ABI: the same output bits on two calls in a
row, the second with a smaller target, and QI_ERR_CAPACITY beyond the scratch array before any
launch.  The smaller case is also held to the oracle at the bf16 bar."""
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


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(wl, step):
    S, P, T = O.split_counts(wl.segments)
    q, k, v = qin.qkv(wl, S, step, 0)
    return (q, k, v), tuple(rt.from_bits(t.bits, wl.dtype, DEV) for t in (q, k, v))


def _prepared(wl):
    """Layout, attention object, filled cache and the step-3 target inputs of a workload."""
    S, P, T = O.split_counts(wl.segments)
    L = rt.Layout(wl.segments, DEV)
    att = rt.Attention(L, wl.n_head, Q.QI_BF16, DEV)
    host0, (q0, k0, v0) = _case(wl, 0)
    cache = rt.KVCache(1, wl.n_head, P, Q.QI_BF16, DEV)
    att.store(k0[:P], v0[:P], cache, 0)
    host3, (q3, k3, v3) = _case(wl, 3)
    return L, att, cache, (host0, host3), (q3[P:], k3[P:], v3[P:])


def _noalloc(att, q_t, k_t, v_t, cache, out):
    T = q_t.shape[0]
    io = Q.make_qkv(q_t, k_t, v_t, out, Q.QI_BF16, T, att.H, q_t.stride(0))
    cos, sin = att.L.rows(att.L.P, att.L.P + T)
    prep = Q.make_prep(cos, sin)
    return Q.qi_attn_target_cached_noalloc(io, prep, cache.c, 0, att.L.P, 0.0, rt.stream_handle(DEV))


def test_noalloc_cached_step_equals_workspace_call_twice():
    # first call: the 21,504-key headline shape (4,096 target queries, 24 heads, 65 MiB of scratch);
    # second call: a smaller target (1,024 queries over 2,304 keys), which reuses the same scratch
    # with another schedule (every query tile in 5 key chunks)
    for name in ("txt1024_4ref64_tgt64", "txt256_ref32_tgt32"):
        wl = qin.WORKLOADS[name]
        say(f"noalloc cached step {name}: T={wl.T} heads={wl.n_head} "
            f"workspace={Q.qi_attn_cached_workspace_bytes(Q.QI_BF16, wl.T, wl.n_head)}")
        L, att, cache, host, (qt, kt, vt) = _prepared(wl)
        ref = att.cached(qt, kt, vt, cache, 0).clone()
        got = torch.full_like(ref, float("nan"))
        Q.check(_noalloc(att, qt, kt, vt, cache, got), "qi_attn_target_cached_noalloc")
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{name}: no-alloc output differs"
        if name == "txt256_ref32_tgt32":
            (q0, k0, v0), (q3, k3, v3) = host
            P = wl.P
            c, s = O.rope_tables(O.positions(wl.segments))
            keys = np.concatenate([O.rotate(k0.f64[:P], c[:P], s[:P]), O.rotate(k3.f64[P:], c[P:], s[P:])])
            vals = np.concatenate([v0.f64[:P], v3.f64[P:]])
            r = O.attention(O.rotate(q3.f64[P:], c[P:], s[P:]), keys, vals)
            g = got.float().cpu().numpy().astype(np.float64)
            d = np.abs(g - r)
            max_rel, mean_rel = d.max() / np.abs(r).max(), d.sum() / np.abs(r).sum()
            say(f"  vs oracle: max_rel={max_rel:.3e} mean_rel={mean_rel:.3e}")
            assert max_rel <= 1e-2 and mean_rel <= 2e-3
        del cache, att


def test_noalloc_refuses_beyond_scratch():
    # 200,000 target tokens of one head need 2 x 200,000 x 256 B of K/V tiles (102 MB) > 96 MiB
    T, H = 200000, 1
    need = Q.qi_attn_cached_workspace_bytes(Q.QI_BF16, T, H)
    assert need > Q.QI_NOALLOC_SCRATCH_BYTES
    segs = (qin.text(64), qin.image(400, 500, 0))
    L = rt.Layout(segs, DEV)
    att = rt.Attention(L, H, Q.QI_BF16, DEV)
    x = torch.zeros((T, H, 128), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros_like(x)
    cache = rt.KVCache(1, H, 64, Q.QI_BF16, DEV)
    assert _noalloc(att, x, x, x, cache, out) == Q.QI_ERR_CAPACITY
    torch.cuda.synchronize()
    assert not torch.any(out.view(torch.int16) != 0), "output touched by a refused call"
