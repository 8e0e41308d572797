"""Benchmark: target-only cached attention step of the Qwen-Image-2.1 DiT hot path on one MI355X.

Workload (default): 24 heads x 128, bf16 I/O; text 1,024 + 4 reference images 64x64 (frames 1..4)
+ target 64x64 (frame 0): 17,408 cached prefix tokens, 4,096 target queries over 21,504 keys.
One step = the target-only cached attention for each of 32 layers (each layer reads its own
prefix cache, so the 6.85 GB of caches cannot sit in the 256 MB Infinity Cache) followed by
one Euler update of the 4096 x 64 fp32 latent.  Inputs are synthetic (torch RNG, seeded) and
resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload txt1024_4ref64_tgt64|txt512_4ref64_tgt64|txt512_tgt64] [--no-cpu]
    python bench.py --dit [--layers L] [--steps K]     # full single-stream layer steps (see below)
    python bench.py --v1edit [--steps K]                # v1 / Edit-Plus full joint attention
    python bench.py --configs [--steps K]               # the other attention workloads, one line each
    python bench.py --graph                             # also the step replayed from a HIP graph
    python bench.py --data-sensitivity                  # the headline step on inputs of other statistics
    python bench.py --gemm-sweep                        # the layer GEMM over K, each epilogue, hipBLASLt

Prints one JSON line.  value = attention TFLOP/s over the timed steps (visible-pair flops,
4*d per pair); roofline = one attention call's average device time (the attention kernel plus,
when the keys are cut in chunks, the merge kernel) from HIP events recorded around each call on
the launch stream.

--dit times the whole denoiser step of the 14,848-token workload (text 512 + 10 references 32x32
+ target 64x64, hidden 3072, 24x128 heads, SwiGLU 8192, random-init weights): step 1 over the
whole sequence (filling the per-layer prefix caches) and the cached target-only steps, each with
the conditioning, all layers, the head and the Euler update.  It prints its own JSON line.

--v1edit times the unmasked joint attention of the v1 / Edit model at the Edit-Plus shape (text
512 + noisy target 64x64 + two references 64x64, 12,800 tokens), and one whole dual-stream block
of that model at the same shape (random-init weights), and prints its own JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2500.0   # MI355X dense fp16/bf16 MFMA, published
METRIC = "attention TFLOP/s + % bf16 MFMA peak, target-only cached step, 4096 tgt tokens"
N_LAYERS = 32
PROFILE = os.path.join(ROOT, "profiles", "attn_f16_4096q_21504k_counters.md")
KERNEL_SRC = os.path.join(ROOT, "image_generation_qi_amd", "csrc", "qi_attn_f16.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_hash() -> str:
    """Hash of the attention kernel's code lines (// comments and blank lines stripped), so that a
    counter summary stays valid across comment-only edits."""
    lines = []
    for line in open(KERNEL_SRC).read().splitlines():
        line = re.sub(r"//.*", "", line).rstrip()
        if line.strip():
            lines.append(line)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per launch from the committed counter summary, if it was taken on this exact
    kernel source (else None)."""
    if not os.path.exists(PROFILE):
        return None
    txt = open(PROFILE).read()
    m_h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_h or not m_b or m_h.group(1) != kernel_hash():
        return None
    return float(m_b.group(1))


def sclk_from_profile():
    """Median shader clock (GHz) during the attention kernel from the committed counter summary,
    if it was taken on this exact kernel source (else None)."""
    if not os.path.exists(PROFILE):
        return None
    txt = open(PROFILE).read()
    m_h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    m_c = re.search(r"sclk_median_ghz:\s*([0-9.]+)", txt)
    if not m_h or not m_c or m_h.group(1) != kernel_hash():
        return None
    return float(m_c.group(1))


def pct(sorted_vals, q):
    """q-th percentile (nearest rank) of an ascending list."""
    i = min(len(sorted_vals) - 1, max(0, int(round(q / 100.0 * (len(sorted_vals) - 1)))))
    return sorted_vals[i]


def visible_pairs_per_head(segments) -> int:
    """Visible (query, key) pairs of step 1: query q sees keys 0..lim(q) (Block-Causal rows)."""
    total, start = 0, 0
    for s in segments:
        end = start + s.n_tokens
        if s.kind == 0:   # causal text: q sees 0..q
            total += sum(q + 1 for q in range(start, end))
        else:             # image / bidirectional text block: sees everything before its end
            total += s.n_tokens * end
        start = end
    return total


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s: float = 12.0):
    """The fp64 oracle's cached target step, one head at a time on the host (each head of each
    layer with its own seeded inputs), until the budget is used (at least one head).  The inputs
    are fp64 N(0,1) draws used as they are (not rounded to bf16 first): the oracle's time does not
    depend on the values."""
    import numpy as np

    import qi_inputs as qin
    from oracle import qi_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
        blas = sorted({f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info() if i.get("user_api") == "blas"})
    except Exception:
        threads = os.cpu_count() or 1
        blas = []
    S, P, T = wl.S, wl.P, wl.T
    cos, sin = O.rope_tables(O.positions(wl.segments))
    done, elapsed = 0, 0.0
    while done == 0 or elapsed < budget_s:
        rng = np.random.default_rng([wl.cfg_id, 900, done])
        k = rng.standard_normal((S, 1, 128))
        v = rng.standard_normal((S, 1, 128))
        q = rng.standard_normal((T, 1, 128))
        cache = (O.rotate(k[:P], cos[:P], sin[:P]), v[:P])
        t0 = time.perf_counter()
        O.cached_step(q, k[P:], v[P:], cache, cos[P:], sin[P:])
        elapsed += time.perf_counter() - t0
        done += 1
    flops = 4.0 * 128 * T * S * done
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} single-head cached target steps ({done / wl.n_head:.2f} layers of {wl.n_head} "
                      f"heads; {T} queries x {S} keys, fp64 NumPy on unrounded fp64 draws), {elapsed:.1f} s",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(), "blas": blas,
            "thread_env": {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                                          "MKL_NUM_THREADS")}}


def dit_bench(args):
    """Full single-stream layer steps at the 14,848-token shape (random-init weights)."""
    import torch

    import qi_inputs as qin
    from image_generation_qi_amd import runtime as rt

    wl = qin.WORKLOADS["txt512_10ref32_tgt64"]
    dev = "cuda:0"
    D, F, H, NL = 3072, 8192, 24, args.layers
    S, P, T = wl.S, wl.P, wl.T
    log(f"dit workload: S={S} P={P} T={T} layers={NL}")
    g = torch.Generator(device=dev).manual_seed(4321)

    def lin(n_out, n_in):
        return (torch.randn((n_out, n_in), generator=g, device=dev) / n_in ** 0.5).to(torch.bfloat16)

    def vec(n, mean=0.0, std=0.02):
        return torch.randn(n, generator=g, device=dev) * std + mean

    layers = [rt.LayerWeights(vec(D), vec(D), vec(128, 1.0), vec(128, 1.0), lin(3 * D, D), lin(D, D), lin(F, D),
                              lin(F, D), lin(D, F)) for _ in range(NL)]
    shared = rt.SharedWeights(lin(D, 256), lin(D, D), lin(6 * D, D), lin(D, D), lin(64, D), lin(D, 64))
    layout = rt.Layout(wl.segments, dev)
    model = rt.DiT(layout, shared, layers, dev)   # keeps fp16 copies of the projection weights
    del layers
    n_text = wl.segments[0].n_tokens
    # the context path: synthetic vision-language rows through the TextProjection give the text rows
    tp = rt.TextProjection(vec(D), lin(D, D), lin(D, D))
    x_ctx = torch.randn((n_text, D), generator=g, device=dev)
    x_text = tp(x_ctx)
    lat_ref = torch.randn((P - n_text, 64), generator=g, device=dev)
    lat = torch.randn((T, 64), generator=g, device=dev)
    sig = qin.sigmas(8)
    torch.cuda.synchronize()
    # flops: GEMMs 2*M*(3D*D + D*D + 2F*D + D*F) per layer; attention 4*128*H*pairs
    gemm_per_row = 2 * (3 * D * D + D * D + 2 * F * D + D * F)
    pairs1 = visible_pairs_per_head(wl.segments)
    f_step1 = NL * (S * gemm_per_row + 4.0 * 128 * H * pairs1)
    f_cached = NL * (T * gemm_per_row + 4.0 * 128 * H * T * S)

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    model.step(0, lat, sig, x_text, lat_ref)       # warm-up (also fills the caches)
    model.step(1, lat, sig)
    torch.cuda.synchronize()
    # the conditioning of the whole schedule: modulation vectors and, with the norm fold, the bias
    # tables shift W^T of every layer for all steps (once per image; counted in the 8-step loop)
    ms_prep = timed(lambda: model.prepare(sig))
    ms1 = timed(lambda: model.step(0, lat, sig, tp(x_ctx, out=x_text), lat_ref))
    ms_tp = min(timed(lambda: tp(x_ctx, out=x_text)) for _ in range(5))
    # cached steps cycle through the schedule's steps 1..7 (sig holds 8 steps + the end point)
    n_cached = len(sig) - 2
    cached = [timed(lambda k=1 + i % n_cached: model.step(k, lat, sig)) for i in range(args.steps)]
    msc = sum(cached) / len(cached)
    # the same steps with the two norms of each layer launched on their own (no fold)
    model.fold = False
    model.step(1, lat, sig)
    unf = [timed(lambda k=1 + i % n_cached: model.step(k, lat, sig)) for i in range(max(2, args.steps // 2))]
    model.fold = True
    ms_unf = sum(unf) / len(unf)
    # the two forms of the QKV projection side by side, alternating step by step (phases of one run
    # differ by a few tenths of a ms): the K/V tiles written by its epilogue (the default, six
    # launches per cached layer) and plain K/V rows that a launch of their own prepares for the
    # attention (seven); after each switch the schedule is prepared and one step warms up, untimed
    pair = {True: [], False: []}
    pair1 = {True: [], False: []}
    for i in range(max(2, args.steps // 2)):
        for form in (False, True):
            model.use_kv_tiles(form)
            model.prepare(sig)
            model.step(1, lat, sig)
            pair[form].append(timed(lambda k=1 + i % n_cached: model.step(k, lat, sig)))
            if i == 0:
                pair1[form].append(timed(lambda: model.step(0, lat, sig, tp(x_ctx, out=x_text), lat_ref)))
    ms_kv = sum(pair[False]) / len(pair[False])
    ms_kv_on = sum(pair[True]) / len(pair[True])
    ms1_kv, ms1_kv_on = pair1[False][0], pair1[True][0]
    res = {
        "metric": "single-stream DiT denoiser step time (conditioning + layers + head + Euler)",
        "value": round(msc, 3), "unit": "ms per cached step", "higher_is_better": False,
        "n_gpus": 1, "steps": args.steps, "dtype": "f16", "data": "synthetic, random-init weights",
        "config": {"workload": f"text {n_text} (context through the TextProjection) + 10 refs 32x32 + target 64x64 (S={S}, P={P}, T={T}); "
                               f"hidden {D}, {H}x128 heads, SwiGLU {F}; {NL} layers",
                   "step1_ms": round(ms1, 3), "step1_tflops": round(f_step1 / (ms1 * 1e-3) / 1e12, 1),
                   "cached_step_tflops": round(f_cached / (msc * 1e-3) / 1e12, 1),
                   "eight_step_loop_ms": round(ms_prep + ms1 + 7 * msc, 2),
                   "schedule_prepare_ms": round(ms_prep, 3),
                   "norm_fold": True, "kv_tiles": True, "cached_step_ms_without_fold": round(ms_unf, 3),
                   "alternating_cached_step_ms": {"kv_tiles": round(ms_kv_on, 3), "without_kv_tiles": round(ms_kv, 3)},
                   "alternating_step1_ms": {"kv_tiles": round(ms1_kv_on, 3), "without_kv_tiles": round(ms1_kv, 3)},
                   "launches_per_cached_layer": 6,
                   "text_projection_ms": round(ms_tp, 4),
                   "text_projection_tflops": round(2 * 2 * n_text * D * D / (ms_tp * 1e-3) / 1e12, 1)},
    }
    print(json.dumps(res), flush=True)


def v1edit_bench(args):
    """The unmasked joint attention of the v1 / Edit model at the Edit-Plus shape: text 512 +
    noisy 64x64 target + two 64x64 references (12,800 tokens, 24 heads), one call per layer over
    distinct Q/K/V; TFLOP/s per call from the library's HIP-event timing."""
    import torch

    import qi_inputs as qin
    from image_generation_qi_amd import qi as Q
    from image_generation_qi_amd import runtime as rt

    wl = qin.V1_WORKLOADS["editplus_v1"]
    dev = "cuda:0"
    S, H = wl.S, wl.n_head
    layout = rt.Layout(wl.segments, dev, attention=Q.QI_ATTN_FULL)
    att = rt.Attention(layout, H, Q.QI_BF16, dev)
    g = torch.Generator(device=dev).manual_seed(77)
    n_sets = 4
    qkv = [torch.randn((S, 3, H, 128), generator=g, device=dev).to(torch.bfloat16) for _ in range(n_sets)]
    out = torch.empty((S, H, 128), dtype=torch.bfloat16, device=dev)
    for i in range(args.warmup + 1):
        x = qkv[i % n_sets]
        att.full(x[:, 0], x[:, 1], x[:, 2], out=out)
    torch.cuda.synchronize()
    Q.qi_kernel_timing(True)
    for i in range(args.steps):
        x = qkv[i % n_sets]
        att.full(x[:, 0], x[:, 1], x[:, 2], out=out)
    torch.cuda.synchronize()
    per_call = sorted(Q.qi_kernel_timing_read_each())
    Q.qi_kernel_timing(False)
    flops = 4.0 * 128 * H * S * S
    ms = sum(per_call) / len(per_call)
    del qkv
    # the whole dual-stream block at this shape (random-init weights, D = 3072, MLP 4 D)
    D, F = H * 128, 4 * H * 128
    Lt = wl.segments[0].n_tokens
    Li = S - Lt

    def lin(n_out, n_in):
        return (torch.randn((n_out, n_in), generator=g, device=dev) / n_in ** 0.5).to(torch.bfloat16)

    shapes = {"img_mod": (6 * D, D), "txt_mod": (6 * D, D), "img_qkv": (3 * D, D), "txt_qkv": (3 * D, D),
              "img_out": (D, D), "txt_out": (D, D), "img_fc1": (F, D), "img_fc2": (D, F), "txt_fc1": (F, D),
              "txt_fc2": (D, F)}
    Wt = {}
    for name, (n_out, n_in) in shapes.items():
        Wt[name + "_w"] = lin(n_out, n_in)
        Wt[name + "_b"] = 0.1 * torch.randn(n_out, generator=g, device=dev)
    for key in ("norm_q", "norm_k", "norm_added_q", "norm_added_k"):
        Wt[key] = 1.0 + 0.02 * torch.randn(128, generator=g, device=dev)
    blk = rt.V1Block(rt.V1BlockWeights(Wt), layout, H, dev)
    x_txt = torch.randn((Lt, D), generator=g, device=dev)
    x_img = torch.randn((Li, D), generator=g, device=dev)
    cond = torch.randn((2, D), generator=g, device=dev)
    for _ in range(2):
        blk(x_txt, x_img, cond)
    torch.cuda.synchronize()
    n_blk = max(3, args.steps // 2)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_blk):
        blk(x_txt, x_img, cond)
    e1.record()
    torch.cuda.synchronize()
    blk_ms = e0.elapsed_time(e1) / n_blk
    # the same block with both streams' calls on one stream
    blk1 = rt.V1Block(rt.V1BlockWeights(Wt), layout, H, dev, two_streams=False)
    blk1(x_txt, x_img, cond)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n_blk):
        blk1(x_txt, x_img, cond)
    e1.record()
    torch.cuda.synchronize()
    blk1_ms = e0.elapsed_time(e1) / n_blk
    del blk1
    blk_flops = 2.0 * S * D * (3 * D + D + 2 * F) + flops
    res = {"metric": "v1 / Edit-Plus joint full attention TFLOP/s per call", "value": round(flops / (ms * 1e-3) / 1e12, 2),
           "unit": "TFLOP/s", "higher_is_better": True, "n_gpus": 1, "steps": args.steps, "dtype": "f16",
           "data": "synthetic", "ms_per_call": round(ms, 4),
           "per_call_ms": {q: round(pct(per_call, int(q[1:])), 4) for q in ("p50", "p95", "p99")},
           "config": {"workload": f"text 512 + noisy target 64x64 + 2 references 64x64, full attention, S={S}, "
                                  f"{H}x128 heads", "flops_per_call": flops,
                      "pct_of_peak": round(100.0 * flops / (ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 2),
                      # one whole dual-stream block (both streams' modulation, norms, projections and
                      # MLPs with the joint attention), random-init weights, D 3072, MLP 12288
                      "block_ms": round(blk_ms, 3), "block_flops": blk_flops,
                      "block_tflops": round(blk_flops / (blk_ms * 1e-3) / 1e12, 1),
                      "block_attention_share": round(ms / blk_ms, 3),
                      "block_ms_one_stream": round(blk1_ms, 3)}}
    print(json.dumps(res), flush=True)


def configs_bench(args):
    """Per-call timings of the other attention workloads (one JSON line each):
    txt256_ref32_tgt32: the 8-step loop of one layer (step 1 with the prefix store, then 7 cached
      steps, each followed by the Euler update of the 1024 x 64 latent), QK-RMSNorm on;
    txt512_tgt64: step 1 (4,608 tokens) and the cached target step (4,096 over 4,608 keys);
    txt512_4ref64_tgt64: the cached target step (4,096 queries over 20,992 keys).
    call_ms brackets the whole library call (K/V prep included) with events on the launch
    stream; kernel_ms is the attention kernel plus merge from the library's own HIP events."""
    import torch

    import qi_inputs as qin
    from image_generation_qi_amd import qi as Q
    from image_generation_qi_amd import runtime as rt

    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(99)
    n_sets = 4

    def ev_time(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        Q.qi_kernel_timing(True)
        e0.record()
        for i in range(reps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        kern = sorted(Q.qi_kernel_timing_read_each())
        Q.qi_kernel_timing(False)
        return e0.elapsed_time(e1) / reps, kern

    def line(name, what, flops, call_ms, kern, kern_per_unit=None):
        # kern_per_unit: attention-kernel time of one unit of `flops` when a unit is several calls
        # (the 8-step loop); else the median single call
        k50 = pct(kern, 50) if kern_per_unit is None else kern_per_unit
        key = "kernel_ms_p50" if kern_per_unit is None else "kernel_ms_per_loop"
        return {"metric": f"attention TFLOP/s, {what}", "value": round(flops / (call_ms * 1e-3) / 1e12, 1),
                "unit": "TFLOP/s", "higher_is_better": True, "n_gpus": 1, "dtype": "f16", "data": "synthetic",
                "config": {"workload": name, "flops_per_call": flops, "call_ms": round(call_ms, 4),
                           key: round(k50, 4), "kernel_tflops": round(flops / (k50 * 1e-3) / 1e12, 1),
                           "pct_of_peak_kernel": round(100.0 * flops / (k50 * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 2)}}

    reps = max(args.steps, 8)
    # txt256_ref32_tgt32: one layer's 8-step loop
    wl = qin.WORKLOADS["txt256_ref32_tgt32"]
    S, P, T, H = wl.S, wl.P, wl.T, wl.n_head
    L = rt.Layout(wl.segments, dev)
    att = rt.Attention(L, H, Q.QI_BF16, dev)
    cache = rt.KVCache(1, H, P, Q.QI_BF16, dev)
    qw = (1.0 + 0.02 * torch.randn(128, generator=g, device=dev)).contiguous()
    kw = (1.0 + 0.02 * torch.randn(128, generator=g, device=dev)).contiguous()
    full = [torch.randn((S, 3, H, 128), generator=g, device=dev).to(torch.bfloat16) for _ in range(n_sets)]
    tgt = [torch.randn((T, 3, H, 128), generator=g, device=dev).to(torch.bfloat16) for _ in range(n_sets)]
    x = torch.randn((T, 64), generator=g, device=dev)
    vel = torch.randn((T, 64), generator=g, device=dev).to(torch.bfloat16)
    o_full = torch.empty((S, H, 128), dtype=torch.bfloat16, device=dev)
    o_t = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
    sig = qin.sigmas(8)

    def loop(i):
        f = full[i % n_sets]
        att.full(f[:, 0], f[:, 1], f[:, 2], qw, kw, cache=cache, out=o_full)
        rt.euler_step(x, vel, float(sig[0]), float(sig[1]))
        for k in range(1, 8):
            t = tgt[(i + k) % n_sets]
            att.cached(t[:, 0], t[:, 1], t[:, 2], cache, 0, qw, kw, out=o_t)
            rt.euler_step(x, vel, float(sig[k]), float(sig[k + 1]))

    for i in range(2):
        loop(i)
    loop_ms, kern = ev_time(loop, reps)
    f1 = 4.0 * 128 * H * visible_pairs_per_head(wl.segments)
    fc = 4.0 * 128 * H * T * S
    res = line(wl.name, "one layer's 8-step loop (step 1 + 7 cached steps + Euler)", f1 + 7 * fc, loop_ms, kern,
               kern_per_unit=sum(kern) / reps)
    res["config"].update({"step1_flops": f1, "cached_flops": fc, "qk_rmsnorm": True, "heads": H})
    print(json.dumps(res), flush=True)
    del full, tgt, cache, att

    # txt512_tgt64: step 1 and the cached target step
    wl = qin.WORKLOADS["txt512_tgt64"]
    S, P, T, H = wl.S, wl.P, wl.T, wl.n_head
    L = rt.Layout(wl.segments, dev)
    att = rt.Attention(L, H, Q.QI_BF16, dev)
    cache = rt.KVCache(1, H, P, Q.QI_BF16, dev)
    full = [torch.randn((S, 3, H, 128), generator=g, device=dev).to(torch.bfloat16) for _ in range(n_sets)]
    o_full = torch.empty((S, H, 128), dtype=torch.bfloat16, device=dev)
    o_t = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)

    def step1(i):
        f = full[i % n_sets]
        att.full(f[:, 0], f[:, 1], f[:, 2], cache=cache, out=o_full)

    def cached(i):
        f = full[i % n_sets]
        att.cached(f[P:, 0], f[P:, 1], f[P:, 2], cache, 0, out=o_t)

    step1(0)
    cached(0)
    ms1, k1 = ev_time(step1, reps)
    msc, kc = ev_time(cached, reps)
    f1 = 4.0 * 128 * H * visible_pairs_per_head(wl.segments)
    fc = 4.0 * 128 * H * T * S
    print(json.dumps(line(wl.name, "step 1 (block-causal, 4,608 tokens)", f1, ms1, k1)), flush=True)
    print(json.dumps(line(wl.name, "cached target step (4,096 queries over 4,608 keys)", fc, msc, kc)), flush=True)
    del full, cache, att

    # txt512_4ref64_tgt64: the cached target step over 20,992 keys (32 layer caches, round robin)
    wl = qin.WORKLOADS["txt512_4ref64_tgt64"]
    S, P, T, H = wl.S, wl.P, wl.T, wl.n_head
    NL = N_LAYERS
    L = rt.Layout(wl.segments, dev)
    att = rt.Attention(L, H, Q.QI_BF16, dev)
    cache = rt.KVCache(NL, H, P, Q.QI_BF16, dev)
    for layer in range(NL):
        kv = torch.randn((P, 2, H, 128), generator=g, device=dev).to(torch.bfloat16)
        att.store(kv[:, 0], kv[:, 1], cache, layer)
        del kv
    tq = [torch.randn((T, 3, H, 128), generator=g, device=dev).to(torch.bfloat16) for _ in range(n_sets)]
    o_t = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)

    def cached3(i):
        t = tq[i % n_sets]
        att.cached(t[:, 0], t[:, 1], t[:, 2], cache, i % NL, out=o_t)

    for i in range(4):
        cached3(i)
    msc, kc = ev_time(cached3, NL * 4)
    fc = 4.0 * 128 * H * T * S
    print(json.dumps(line(wl.name, "cached target step (4,096 queries over 20,992 keys)", fc, msc, kc)), flush=True)


def data_sensitivity_bench(args):
    """The headline cached step (4,096 queries over 21,504 keys, 24 heads) with the same shapes,
    launches and instruction stream on inputs of different statistics: N(0,1) (the workload's),
    N(0,1) rounded to half-integers (few mantissa bits), all ones and all zeros.  On a
    power-limited chip the clock, and so the kernel time, follows the switching activity of the
    data; one JSON line per input kind."""
    import torch

    import qi_inputs as qin
    from image_generation_qi_amd import qi as Q
    from image_generation_qi_amd import runtime as rt

    dev = "cuda:0"
    wl = qin.WORKLOADS["txt1024_4ref64_tgt64"]
    P, T, H = wl.P, wl.T, wl.n_head
    L = rt.Layout(wl.segments, dev)
    att = rt.Attention(L, H, Q.QI_BF16, dev)
    g = torch.Generator(device=dev).manual_seed(5)
    NL = 4
    flops = 4.0 * 128 * H * T * (P + T)

    def draw(kind, shape):
        if kind == "zeros":
            return torch.zeros(shape, device=dev, dtype=torch.bfloat16)
        if kind == "ones":
            return torch.ones(shape, device=dev, dtype=torch.bfloat16)
        x = torch.randn(shape, generator=g, device=dev)
        if kind == "randn_half_integers":
            x = torch.round(x * 2) / 2
        return x.to(torch.bfloat16)

    for kind in ("randn", "randn_half_integers", "ones", "zeros"):
        cache = rt.KVCache(NL, H, P, Q.QI_BF16, dev)
        for layer in range(NL):
            kv = draw(kind, (P, 2, H, 128))
            att.store(kv[:, 0], kv[:, 1], cache, layer)
            del kv
        qkv = [draw(kind, (T, 3, H, 128)) for _ in range(NL)]
        out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)

        def run(n):
            for _ in range(n):
                for layer in range(NL):
                    t = qkv[layer]
                    att.cached(t[:, 0], t[:, 1], t[:, 2], cache, layer, out=out)

        run(max(args.warmup, 1) * 30)   # long enough for the clock to settle
        torch.cuda.synchronize()
        Q.qi_kernel_timing(True)
        run(max(args.steps, 1) * 4)
        torch.cuda.synchronize()
        kern = sorted(Q.qi_kernel_timing_read_each())
        Q.qi_kernel_timing(False)
        k50 = pct(kern, 50)
        print(json.dumps({"metric": "attention kernel TFLOP/s vs input statistics, cached target step",
                          "value": round(flops / (k50 * 1e-3) / 1e12, 1), "unit": "TFLOP/s", "higher_is_better": True,
                          "n_gpus": 1, "dtype": "f16", "data": kind,
                          "config": {"workload": wl.name, "kernel_ms_p50": round(k50, 4), "launches": len(kern),
                                     "pct_of_peak": round(100.0 * flops / (k50 * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 2)}}),
              flush=True)
        del cache, qkv, out
        torch.cuda.empty_cache()


def gemm_sweep_bench(args):
    """The layer GEMM at 4,096 rows over a sweep of reduction lengths K, with each epilogue the
    denoiser uses at that shape (fp16 store, fp32 store, tanh-gated residual, gated residual with
    the norm fold's producing side), beside hipBLASLt (torch.matmul, fp16, plain store) on the same
    operands.  A line fit over K separates the time that grows with K (per 64-deep slice) from the
    time each launch pays once (launch, first slices' loads, the epilogue's traffic).  One JSON line
    per (N, K) and one per epilogue with the fit."""
    import torch

    from image_generation_qi_amd import qi as Q
    from image_generation_qi_amd import runtime as rt

    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(11)
    M = 4096

    def ev_median(f, n=20):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        for i in range(n):
            ev[i].record()
            f()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(n))[n // 2] * 1000.0

    fits = {}
    for N in (3072, 9216):
        for K in (64, 768, 3072, 8192):
            x = (torch.randn((M, K), generator=g, device=dev) * 0.5).half()
            w = (torch.randn((N, K), generator=g, device=dev) / K ** 0.5).half()
            wt = w.t()
            o16 = torch.empty((M, N), device=dev, dtype=torch.float16)
            o32 = torch.empty((M, N), device=dev)
            cases = {"store_f16": lambda: rt.gemm(x, w, o16, Q.QI_EPI_STORE, tile_n=192),
                     "store_f32": lambda: rt.gemm(x, w, o32, Q.QI_EPI_STORE_F32, tile_n=192),
                     "hipblaslt_f16": lambda: torch.matmul(x, wt, out=o16)}
            if N == 3072:
                gate = torch.randn((2, N), generator=g, device=dev) * 0.1
                nw = torch.randn(N, generator=g, device=dev) * 0.1
                ns = torch.randn((2, N), generator=g, device=dev) * 0.1
                h = torch.empty((M, N), device=dev, dtype=torch.float16)
                sq = torch.empty((M, rt.fold_parts(N)), device=dev)
                fold = rt.NormFold(xc=h, next_w=nw, next_scale=ns, sumsq_out=sq)
                cases["gated"] = lambda: rt.gemm(x, w, o32, Q.QI_EPI_GATED_RESIDUAL, gate, 0, 0, tile_n=192)
                cases["gated_norm_fold"] = lambda: rt.gemm(x, w, o32, Q.QI_EPI_GATED_RESIDUAL, gate, 0, 0, fold=fold)
            us = {name: round(ev_median(f), 1) for name, f in cases.items()}
            for name, t in us.items():
                fits.setdefault((N, name), {})[K] = t
            fl = 2.0 * M * N * K
            print(json.dumps({"metric": "layer GEMM time per launch (HIP events, median of 20)", "unit": "us",
                              "value": us["store_f16"], "higher_is_better": False, "n_gpus": 1, "dtype": "f16",
                              "data": "synthetic",
                              "config": {"workload": f"{M} x {N} x {K}", "us": us,
                                         "tflops": {k: round(fl / (t * 1e-6) / 1e12, 1) for k, t in us.items()}}}),
                  flush=True)
            del x, w, wt, o16, o32
    for (N, name), t in fits.items():
        per_slice = (t[8192] - t[3072]) / ((8192 - 3072) / 64)
        print(json.dumps({"metric": "layer GEMM line fit over K (3,072 and 8,192)", "unit": "us",
                          "value": round(t[3072] - 48 * per_slice, 1), "higher_is_better": False, "n_gpus": 1,
                          "dtype": "f16", "data": "synthetic",
                          "config": {"workload": f"{M} x {N}", "epilogue": name,
                                     "us_per_64_deep_slice": round(per_slice, 3),
                                     "fixed_us_per_launch": round(t[3072] - 48 * per_slice, 1)}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="txt1024_4ref64_tgt64", choices=["txt1024_4ref64_tgt64", "txt512_4ref64_tgt64", "txt512_tgt64"])
    ap.add_argument("--layers", type=int, default=N_LAYERS)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--step1", action="store_true", help="also time one full step-1 attention per layer")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 10 device-to-device copies of MIB MiB (reference kernel for HBM counters)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the same step captured in a HIP graph and replayed (launch overheads)")
    ap.add_argument("--dit", action="store_true", help="time full single-stream layer steps instead")
    ap.add_argument("--v1edit", action="store_true",
                    help="time the v1 / Edit-Plus joint full attention (text 512 + target + 2 references) instead")
    ap.add_argument("--configs", action="store_true",
                    help="time the other attention workloads instead (one JSON line each)")
    ap.add_argument("--gemm-sweep", action="store_true",
                    help="time the layer GEMM at 4,096 rows over a sweep of K with each epilogue, beside hipBLASLt")
    ap.add_argument("--data-sensitivity", action="store_true",
                    help="time the headline cached step on N(0,1), low-mantissa, ones and zeros inputs instead")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.dit:
        from image_generation_qi_amd import qi as Q
        Q.lib()
        dit_bench(args)
        return
    if args.v1edit:
        from image_generation_qi_amd import qi as Q
        Q.lib()
        v1edit_bench(args)
        return
    if args.configs:
        from image_generation_qi_amd import qi as Q
        Q.lib()
        configs_bench(args)
        return
    if args.data_sensitivity:
        from image_generation_qi_amd import qi as Q
        Q.lib()
        data_sensitivity_bench(args)
        return
    if args.gemm_sweep:
        from image_generation_qi_amd import qi as Q
        Q.lib()
        gemm_sweep_bench(args)
        return

    import torch

    import qi_inputs as qin
    from image_generation_qi_amd import qi as Q
    from image_generation_qi_amd import runtime as rt

    Q.lib()
    dev = "cuda:0"
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": n * 4, "launches": 10}), flush=True)
        return
    wl = qin.WORKLOADS[args.workload]
    S, P, T, H = wl.S, wl.P, wl.T, wl.n_head
    NL = args.layers
    log(f"workload {wl.name}: S={S} P={P} T={T} H={H} layers={NL}")
    L = rt.Layout(wl.segments, dev)
    att = rt.Attention(L, H, Q.QI_BF16, dev)
    cache = rt.KVCache(NL, H, P, Q.QI_BF16, dev)
    g = torch.Generator(device=dev).manual_seed(1234)

    # fill every layer's prefix cache (prepared K, V) from synthetic prefix K/V
    for layer in range(NL):
        kv = torch.randn((P, 2, H, 128), generator=g, device=dev).to(torch.bfloat16)
        att.store(kv[:, 0], kv[:, 1], cache, layer)
        del kv
    # per-layer target Q/K/V (fused [T, 3, H, 128] buffers), output, latent and velocity
    qkv = [torch.randn((T, 3, H, 128), generator=g, device=dev).to(torch.bfloat16) for _ in range(NL)]
    out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
    x = torch.randn((T, wl.latent_ch), generator=g, device=dev)
    vel = torch.randn((T, wl.latent_ch), generator=g, device=dev).to(torch.bfloat16)
    sig = qin.sigmas(8)
    torch.cuda.synchronize()
    log("caches filled")

    def one_step(k):
        for layer in range(NL):
            t = qkv[layer]
            att.cached(t[:, 0], t[:, 1], t[:, 2], cache, layer, out=out)
        i = 1 + (k % 7)
        rt.euler_step(x, vel, float(sig[i]), float(sig[i + 1]))

    for k in range(args.warmup):
        one_step(k)
    torch.cuda.synchronize()
    log("warmup done")

    Q.qi_kernel_timing(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        one_step(k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms, n_launch = Q.qi_kernel_timing_read()
    per_call = sorted(Q.qi_kernel_timing_read_each())
    Q.qi_kernel_timing(False)
    log(f"timed {args.steps} steps in {wall:.3f} s; attention kernel {kern_ms / max(n_launch, 1):.4f} ms/launch")

    flops_launch = 4.0 * 128 * H * T * (P + T)
    n_chunks, whole_per_xcd, chunked_tiles = Q.qi_attn_schedule(T, H, P, T)
    value = flops_launch * NL * args.steps / wall / 1e12
    avg_ms = kern_ms / max(n_launch, 1)
    achieved = flops_launch / (avg_ms * 1e-3) / 1e12
    extra = {}
    if args.step1:
        o1 = torch.empty((S, H, 128), dtype=torch.bfloat16, device=dev)
        qkv1 = torch.randn((S, 3, H, 128), generator=g, device=dev).to(torch.bfloat16)
        att.full(qkv1[:, 0], qkv1[:, 1], qkv1[:, 2], cache=cache, layer=0, out=o1)
        torch.cuda.synchronize()
        Q.qi_kernel_timing(True)
        for _ in range(3):
            att.full(qkv1[:, 0], qkv1[:, 1], qkv1[:, 2], cache=cache, layer=0, out=o1)
        torch.cuda.synchronize()
        ms1, n1 = Q.qi_kernel_timing_read()
        Q.qi_kernel_timing(False)
        f1 = 4.0 * 128 * H * visible_pairs_per_head(wl.segments)
        extra["step1_attention_kernel_ms"] = round(ms1 / n1, 4)
        extra["step1_attention_tflops"] = round(f1 / (ms1 / n1 * 1e-3) / 1e12, 1)
        del qkv1, o1

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: target-only cached attention step, {H}x128 heads, text "
                               f"{wl.segments[0].n_tokens} + {len(wl.segments) - 2} refs + target "
                               f"{wl.segments[-1].grid_h}x{wl.segments[-1].grid_w}; {T} queries over {P + T} keys "
                               f"({P} cached); {NL} layers + Euler per step",
                   "io_dtype": "bf16", "cache_dtype": "f16", "mfma": "v_mfma_f32_16x16x32_f16",
                   "layers_per_step": NL, "target_tokens": T, "prefix_tokens": P, "heads": H,
                   "pct_of_peak": round(100.0 * value / PEAK_F16_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_F16_TFLOPS, 4), "traffic": traffic_from_profile(),
                     "kernel": "k_attn_f16<false> + k_combine (one attention call)" if n_chunks > 1 else "k_attn_f16<false>",
                     "schedule": {"query_tiles": -(-T // 256) * H, "whole_tiles_per_xcd": whole_per_xcd,
                                  "chunked_tiles": chunked_tiles, "key_chunks": n_chunks},
                     "kernel_ms_per_launch": round(avg_ms, 4),
                     "flops_per_launch": flops_launch, "launches": n_launch,
                     # per-call duration percentiles (p95/p99: the slow tail) and the TFLOP/s at each
                     "per_call_ms": {q: round(pct(per_call, int(q[1:])), 4) for q in ("p50", "p95", "p99")},
                     "per_call_tflops": {q: round(flops_launch / (pct(per_call, int(q[1:])) * 1e-3) / 1e12, 1)
                                         for q in ("p50", "p95", "p99")}},
    }
    sclk = sclk_from_profile()
    if sclk:
        # context from the committed counter summary (another run, possibly another box), not
        # measured in this run: the shader clock that run held during the kernel, and this run's
        # rate as a fraction of the MFMA rate at that clock (256 CUs x 4,096 flop per clock)
        peak_at_sclk = 256 * 4096 * sclk * 1e9 / 1e12
        res["roofline"]["profile_sclk_ghz"] = sclk
        res["roofline"]["frac_at_profile_sclk"] = round(achieved / peak_at_sclk, 4)
        res["roofline"]["profile"] = os.path.relpath(PROFILE, ROOT)
    if res["roofline"]["traffic"] is not None:
        # the traffic figure also comes from that committed summary (same kernel source)
        res["roofline"]["traffic_source"] = os.path.relpath(PROFILE, ROOT)
    if args.graph:
        # the same step (32 layers' calls + Euler) captured once and replayed: the launch gaps between
        # the 97 kernels of a step are what the graph can remove; the value above stays the eager one
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step(0)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        gms = e0.elapsed_time(e1) / args.steps
        extra["graph_ms_per_step"] = round(gms, 4)
        extra["graph_tflops"] = round(flops_launch * NL / (gms * 1e-3) / 1e12, 2)
        del graph
    res["config"].update(extra)
    if not args.no_cpu:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
