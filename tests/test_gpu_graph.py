"""The library's device calls under HIP graph capture (torch.cuda.CUDAGraph on the launch stream):
the cached attention step with a caller workspace and the allocation-free one
(qi_attn_target_cached_noalloc, for callers that capture), the Euler update, and a whole cached
layer of the single-stream denoiser with the norm fold.  Each graph is replayed several times, with
other eager work and synchronisations between the replays, and every replay's outputs must equal
the eager calls' bit for bit.  No call of the library records a memset: the kernels write every
byte they read."""
import sys

import pytest

import qi_inputs as qin

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from image_generation_qi_amd import qi as Q  # noqa: E402
from image_generation_qi_amd import runtime as rt  # noqa: E402

DEV = "cuda:0"
REPLAYS = 3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def test_cached_attention_and_euler_replay_equal_eager():
    wl = qin.WORKLOADS["txt256_ref32_tgt32"]
    S, P, T, H = wl.S, wl.P, wl.T, wl.n_head
    say(f"[graph] cached attention S={S} P={P} T={T} H={H}")
    g = torch.Generator(device=DEV).manual_seed(7)
    L = rt.Layout(wl.segments, DEV)
    att = rt.Attention(L, H, Q.QI_BF16, DEV)
    cache = rt.KVCache(1, H, P, Q.QI_BF16, DEV)
    kv = torch.randn((P, 2, H, 128), generator=g, device=DEV).to(torch.bfloat16)
    att.store(kv[:, 0], kv[:, 1], cache, 0)
    t = torch.randn((T, 3, H, 128), generator=g, device=DEV).to(torch.bfloat16)
    qw = (1.0 + 0.02 * torch.randn(128, generator=g, device=DEV)).contiguous()
    x0 = torch.randn((T, 64), generator=g, device=DEV)
    vel = torch.randn((T, 64), generator=g, device=DEV).to(torch.bfloat16)
    out_ws = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
    out_na = torch.empty_like(out_ws)
    x = x0.clone()
    cos, sin = L.rows(P, P + T)

    def seq():
        att.cached(t[:, 0], t[:, 1], t[:, 2], cache, 0, qw, qw, out=out_ws)
        io = Q.make_qkv(t[:, 0], t[:, 1], t[:, 2], out_na, Q.QI_BF16, T, H, t.stride(0))
        Q.check(Q.qi_attn_target_cached_noalloc(io, Q.make_prep(cos, sin, qw, qw), cache.c, 0, P, 0.0,
                                                 rt.stream_handle(DEV)), "qi_attn_target_cached_noalloc")
        rt.euler_step(x, vel, 0.875, 0.75)

    seq()   # eager (also creates the workspace outside the capture)
    torch.cuda.synchronize()
    ref = (out_ws.clone(), out_na.clone(), x.clone())
    graph = torch.cuda.CUDAGraph()
    x.copy_(x0)
    with torch.cuda.graph(graph):
        seq()
    for r in range(REPLAYS):
        # eager work between the replays: another call into the same buffers, then a reset
        out_ws.fill_(3.0)
        out_na.fill_(-3.0)
        att.cached(t[:, 0], t[:, 1], t[:, 2], cache, 0, out=out_ws)   # (no norm: other bits)
        x.copy_(x0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want, what in zip((out_ws, out_na, x), ref, ("workspace call", "allocation-free call", "Euler")):
            assert torch.equal(bits(got), bits(want)), f"replay {r}: {what} differs from the eager call"
    assert att.range_flags() == 0


@pytest.mark.parametrize("kv", [True, False])
def test_cached_dit_layer_replay_equals_eager(kv):
    # two cached layers of the single-stream denoiser (norm fold on; with the fused QKV path, QKV with
    # the K/V tiles, else QKV and the K/V preparation; then attention, merge, out-projection,
    # gate-up and down-projection), captured and replayed
    segs = (qin.text(40), qin.image(8, 10, 1), qin.image(12, 10, 0))
    D, F, H = 256, 512, 2
    say(f"[graph] cached DiT layers, kv_tiles={kv}")
    g = torch.Generator(device=DEV).manual_seed(8)

    def lin(n_out, n_in):
        return (torch.randn((n_out, n_in), generator=g, device=DEV) / n_in ** 0.5).to(torch.bfloat16)

    def vec(n, mean=0.0, std=0.02):
        return torch.randn(n, generator=g, device=DEV) * std + mean

    layers = [rt.LayerWeights(vec(D), vec(D), vec(128, 1.0), vec(128, 1.0), lin(3 * D, D), lin(D, D), lin(F, D),
                              lin(F, D), lin(D, F)) for _ in range(2)]
    shared = rt.SharedWeights(lin(D, 256), lin(D, D), lin(6 * D, D), lin(D, D), lin(64, D), lin(D, 64))
    L = rt.Layout(segs, DEV)
    model = rt.DiT(L, shared, layers, DEV, kv_tiles=kv)
    S, P = L.S, L.P
    model.condition(1.0)
    model.x.copy_(torch.randn((S, D), generator=g, device=DEV))
    for li in range(2):
        model.layer(li, slice(0, S), False)          # step 1 fills the caches
    model.condition(0.625)
    xt0 = torch.randn((S - P, D), generator=g, device=DEV)

    def seq():
        for li in range(2):
            model.layer(li, slice(P, S), True)

    model.x[P:].copy_(xt0)
    seq()
    torch.cuda.synchronize()
    ref = model.x[P:].clone()
    graph = torch.cuda.CUDAGraph()
    model.x[P:].copy_(xt0)
    with torch.cuda.graph(graph):
        seq()
    for r in range(REPLAYS):
        model.x[P:].fill_(1.0)
        seq()                                        # eager work between the replays
        model.x[P:].copy_(xt0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(model.x[P:]), bits(ref)), f"replay {r}: the layer output differs"
    assert model.attn.range_flags() == 0
