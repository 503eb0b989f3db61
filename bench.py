#!/usr/bin/env python3
"""Decode throughput of the IndexCache / DSA hot path on one MI355X.

Workload (default): long-context decode, a 48-layer stack with F layers at
0,3,7,11,15,19,23,27,31,35,40,44 (S elsewhere), batch 8, context 131072,
indexer 64 heads x 128 fp8 with per-row scales, top-2048, sparse MLA with 128
heads over 576-wide bf16 latent rows.  One step = one decode token for every
sequence through all 48 layers: indexer + top-k on F layers, sparse attention
on every layer.  Inputs are seeded synthetic tensors resident in HBM before
the timed region.

Also reported on the same line:
  * the same stack with all-F and with 'FSSS' x 12, and the configured stack
    captured into one HIP graph and replayed;
  * indexer + top-k time per layer and per 4-layer group (Hq = 0 stacks);
  * per-kernel average durations from HIP events on the launch stream, and the
    roofline of the dominant kernel;
  * the prefill chunk (8192 queries on a 65536-token context, fp8, plus the
    same shape in bf16): indexer scores TFLOP/s and top-k time;
  * the same prefill chunk through a 4-layer stack with sparse attention on
    every layer (all-F against FSSS): chunked prefill under IndexCache;
  * the KV-cache append (latent bf16 + fp8 indexer key rows) at the decode
    and prefill-chunk shapes, which precedes the path in every step;
  * the training-free pattern search (greedy F -> S conversion under a proxy
    loss) on a 48-layer synthetic calibration stack with planted critical
    layers: device cost-matrix time, host search time, the chosen pattern;
  * the fp64 CPU oracle timed on a bounded sample on this host;
  * the pattern sweep at context 196608 (16 layers, batch 4): all-F, FS,
    FSSS, FSSSSSSS, with the overlap between each S layer's reused index set
    and the set its own indexer would select.

python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-prefill]
                [--no-sweep] [--no-search] [--no-kv-append] [--search-only] [--kv-append-only]
                [--stream-probe-only]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode tokens/s + indexer+top-k µs/layer at 128K ctx, FSSS vs all-F"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def event_time_ms(fn, reps: int, warm: int = 2) -> float:
    """Average milliseconds per call of fn() over `reps` back-to-back calls,
    bracketed by HIP events on torch's current stream (the launch stream)."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fn(i)
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def build_decode_workload(s, dev):
    import torch
    from dsa_sparse_attention_lightning_amd import inputs as gen
    t0 = time.time()
    qi = gen.make_indexer_query(s, dev)
    kb = gen.make_key_base(s, dev)
    layers = []
    for l in range(s.n_layers):
        ki = gen.make_indexer_keys(s, l, kb, dev)
        q, kv = gen.make_mla_layer(s, l, dev)
        layers.append(dict(q_idx=qi.q, q_idx_scale=qi.q_scale, w=qi.w, k_idx=ki.k,
                           k_idx_scale=ki.k_scale, q=q, kv=kv,
                           out=torch.empty((s.B, s.T, s.Hq, s.d_v), dtype=torch.bfloat16,
                                           device=dev),
                           lse=torch.empty((s.B, s.T, s.Hq), dtype=torch.float32, device=dev)))
    del kb
    torch.cuda.synchronize()
    log(f"workload built in {time.time() - t0:.1f} s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB on device)")
    return layers


def shape_kw(s, attn=True):
    return dict(B=s.B, T=s.T, H=s.H, D=s.D, Lmax=s.Lmax, k=s.k, Hq=s.Hq if attn else 0,
                idx_dtype=s.idx_dtype, scale=s.scale)


def time_stack(stack, steps, warmup):
    import torch
    for _ in range(warmup):
        stack.run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        stats = stack.run()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / steps, stats


def indexer_bytes(s):
    e = 1 if s.idx_dtype == "fp8" else 2
    per_key = s.D * e + (4 if s.idx_dtype == "fp8" else 0) + 4        # key row (+scale) + score
    per_seq = s.Lmax * per_key + s.H * s.D * e + s.H * 4 * (2 if s.idx_dtype == "fp8" else 1)
    return s.B * s.T * per_seq if s.T == 1 else None


def attn_bytes_flops(s):
    per_row = (s.k * s.d_qk * 2 + s.k * 4 + s.Hq * s.d_qk * 2 + s.Hq * s.d_v * 2 + s.Hq * 4)
    flops = 2.0 * s.Hq * s.k * (s.d_qk + s.d_v)
    return s.B * s.T * per_row, s.B * s.T * flops


def recorded_traffic(kernel: str, source: str):
    """HBM bytes per call measured by hardware counters (two rocprofv3 --pmc
    passes, scaled by a plain copy of known size) as recorded in the
    committed profile summary - or None once the kernel source has changed
    since the counters were taken."""
    import hashlib
    import re
    prof = os.path.join(ROOT, "profiles", "long_context_decode_traffic_pmc.md")
    src = os.path.join(ROOT, "dsa_sparse_attention_lightning_amd", "csrc", source)
    try:
        text = open(prof).read()
        cur = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    m = re.search(rf"- source-sha256: {re.escape(source)} (\w+)", text)
    t = re.search(rf"- traffic: {re.escape(kernel)} (\d+)", text)
    if not m or not t or m.group(1) != cur:
        return None
    return int(t.group(1))


def decode_bench(args, dev):
    import torch
    import dsa_sparse_attention_lightning_amd as dsa
    from dsa_sparse_attention_lightning_amd import inputs as gen

    s = gen.CONFIGS[args.config]
    layers = build_decode_workload(s, dev)
    ctx = gen.ctx_lens(s, dev)
    pats = {"config": s.pattern, "all-F": "F" * s.n_layers,
            "FSSS": gen.tile_pattern("FSSS", s.n_layers)}
    res = {}
    res_fused = dsa.Stack(s.pattern, layers, ctx, **shape_kw(s, attn=False)).fused
    for name, p in pats.items():
        st = dsa.Stack(p, layers, ctx, **shape_kw(s))
        ms, stats = time_stack(st, args.steps, args.warmup)
        st_i = dsa.Stack(p, layers, ctx, **shape_kw(s, attn=False))
        ms_i, _ = time_stack(st_i, args.steps, args.warmup)
        res[name] = dict(pattern=p, ms_per_step=ms, tokens_per_s=s.B / (ms * 1e-3),
                         n_indexer_calls=stats["n_indexer_calls"],
                         indexer_topk_ms_per_step=ms_i,
                         indexer_topk_us_per_layer=ms_i * 1e3 / s.n_layers,
                         indexer_topk_us_per_group4=ms_i * 1e3 / (s.n_layers / 4))
        log(f"{name:7s} {ms:8.3f} ms/step  {s.B / (ms * 1e-3):9.0f} tok/s  "
            f"indexer+topk {ms_i * 1e3 / s.n_layers:7.2f} us/layer  F={stats['n_indexer_calls']}")
    cut = 1.0 - res["FSSS"]["indexer_topk_ms_per_step"] / res["all-F"]["indexer_topk_ms_per_step"]

    # ---- the configured stack captured once into a HIP graph and replayed
    # (same kernels and arguments; the step without host launch overhead)
    st = dsa.Stack(s.pattern, layers, ctx, **shape_kw(s))
    st.run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.run()
    ms_g = event_time_ms(lambda i=0: graph.replay(), args.steps, args.warmup)
    res["config"]["graph_replay_ms_per_step"] = ms_g
    log(f"config   {ms_g:8.3f} ms/step as HIP-graph replays")
    del graph, st

    # ---- the same stack with F layers through the separate indexer (scores
    # to memory, top-k histogram built on the way) and top-k kernels, for
    # comparison with the default fused indexer + top-k
    st = dsa.Stack(s.pattern, layers, ctx, fused_topk=False, **shape_kw(s))
    ms_u, _ = time_stack(st, args.steps, args.warmup)
    st_ui = dsa.Stack(s.pattern, layers, ctx, fused_topk=False, **shape_kw(s, attn=False))
    ms_ui, _ = time_stack(st_ui, args.steps, args.warmup)
    res["config"]["fused_topk"] = bool(res_fused)
    res["config"]["separate_topk_ms_per_step"] = ms_u
    res["config"]["separate_topk_indexer_topk_us_per_layer"] = ms_ui * 1e3 / s.n_layers
    log(f"config   {ms_u:8.3f} ms/step with separate indexer and top-k kernels "
        f"({ms_ui * 1e3 / s.n_layers:.2f} us/layer without attention)")
    del st, st_ui

    # ---- per-kernel durations (events around back-to-back launches)
    f_layers = [l for l, c in enumerate(s.pattern) if c == "F"]
    score = torch.empty((s.B, s.T, dsa.ld_for(s.Lmax)), dtype=torch.float32, device=dev)
    idx = torch.empty((s.B, s.T, s.k), dtype=torch.int32, device=dev)
    reps = max(24, 2 * len(f_layers))

    def run_idx(i=0):
        L = layers[f_layers[i % len(f_layers)]]
        dsa.indexer_scores(L["q_idx"], L["w"], L["k_idx"], ctx, L["q_idx_scale"],
                           L["k_idx_scale"], out=score)

    t_idx = event_time_ms(run_idx, reps)
    tk_ws = torch.zeros(max(1, dsa.topk_workspace_size(s.B, s.T, s.Lmax, s.k)),
                        dtype=torch.uint8, device=dev)
    t_topk = event_time_ms(lambda i=0: dsa.topk(score[..., :s.Lmax], ctx, s.k, out=idx,
                                                workspace=tk_ws), reps)
    fz_ws = torch.zeros(dsa.indexer_topk_workspace_size(s.B, s.T, s.H, s.D, s.Lmax, s.k,
                                                        s.idx_dtype),
                        dtype=torch.uint8, device=dev)

    def run_fused(i=0):
        L = layers[f_layers[i % len(f_layers)]]
        dsa.indexer_topk(L["q_idx"], L["w"], L["k_idx"], ctx, s.k, L["q_idx_scale"],
                         L["k_idx_scale"], out=idx, workspace=fz_ws)

    t_fused = event_time_ms(run_fused, reps)
    at_ws = torch.zeros(max(1, dsa.sparse_attn_workspace_size(s.B, s.T, s.Hq, s.k)),
                        dtype=torch.uint8, device=dev)

    def run_attn(i=0):
        L = layers[i % s.n_layers]
        dsa.sparse_attn(L["q"], L["kv"], idx, ctx, s.scale, out=L["out"], lse=L["lse"],
                        workspace=at_ws)

    t_attn = event_time_ms(run_attn, max(48, reps))
    ib = indexer_bytes(s)
    ab, af = attn_bytes_flops(s)
    nF = s.pattern.count("F")
    # the default stack runs the fused indexer + top-k; the separate kernels
    # run only with fused_topk=False (launches_per_step 0 here)
    fb = ib - s.B * s.T * s.Lmax * 4 + s.B * s.T * s.k * 4  # no score writes; indices out
    kernels = {
        "indexer_topk": dict(us=t_fused * 1e3, launches_per_step=nF if res_fused else 0,
                             bytes=fb, gbs=fb / (t_fused * 1e-3) / 1e9,
                             path="default stack: fused indexer + top-k (kernel + finish)"),
        "indexer_decode": dict(us=t_idx * 1e3, launches_per_step=0 if res_fused else nF,
                               bytes=ib, gbs=ib / (t_idx * 1e-3) / 1e9,
                               path="separate path: indexer writing scores"),
        "topk": dict(us=t_topk * 1e3, launches_per_step=0 if res_fused else nF,
                     bytes=s.B * s.Lmax * 4 + s.B * s.k * 4,
                     gbs=(s.B * s.Lmax * 4 + s.B * s.k * 4) / (t_topk * 1e-3) / 1e9,
                     path="separate path: top-k over the scores"),
        "sparse_mla": dict(us=t_attn * 1e3, launches_per_step=s.n_layers, bytes=ab, flops=af,
                           gbs=ab / (t_attn * 1e-3) / 1e9,
                           tflops=af / (t_attn * 1e-3) / 1e12),
    }
    for k_, v in kernels.items():
        v["us_per_step"] = v["us"] * v["launches_per_step"]
        v.setdefault("path", "")
        log(f"kernel {k_:15s} {v['us']:8.2f} us x {v['launches_per_step']:2d}  "
            f"{v['gbs']:8.1f} GB/s")
    dom = max(kernels, key=lambda n: kernels[n]["us_per_step"])
    kd = kernels[dom]
    srcs = {"indexer_decode": "indexer_decode.hip", "indexer_topk": "indexer_decode.hip",
            "sparse_mla": "sparse_mla.hip", "topk": "topk.hip"}
    src = srcs[dom]
    roof = dict(kernel=dom, bound="hbm", achieved=round(kd["gbs"], 1), peak=HBM_PEAK_GBS,
                unit="GB/s", frac=round(kd["gbs"] / HBM_PEAK_GBS, 4),
                traffic=recorded_traffic(dom, src),
                per_launch_bytes=kd["bytes"], avg_launch_us=round(kd["us"], 3))
    if dom == "sparse_mla":
        roof["mfma_tflops"] = round(kd["tflops"], 1)
        roof["mfma_frac_bf16"] = round(kd["tflops"] / BF16_PEAK_TFLOPS, 4)
    for name, v in kernels.items():
        v["traffic"] = recorded_traffic(name, srcs[name])
    return s, layers, res, cut, kernels, roof


def oracle_layer_seconds(s, layers, kinds, budget_s, b=0):
    """Wall time of the fp64 oracle on sequence b of a decode workload: one
    F layer (indexer + top-k + attention) and one S layer (attention over the
    F layer's set), each repeated while the budget lasts; returns the mean
    seconds per F and per S layer and the host threads the oracle used."""
    import numpy as np
    import oracle
    from dsa_sparse_attention_lightning_amd import inputs as gen

    def real(t, sc=None):
        return (oracle.bf16_bits_to_f64(gen.bits(t)) if sc is None else
                oracle.dequant_fp8_rows(gen.bits(t), sc.cpu().numpy()))

    L = layers[0]
    qs = L["q_idx_scale"][b:b + 1] if L["q_idx_scale"] is not None else None
    ks = L["k_idx_scale"][b:b + 1] if L["k_idx_scale"] is not None else None
    q_idx = real(L["q_idx"][b:b + 1], qs)
    k_idx = real(L["k_idx"][b:b + 1], ks)
    w = L["w"][b:b + 1].cpu().double().numpy()
    q = real(L["q"][b:b + 1])
    kv = real(L["kv"][b:b + 1])
    ctx = [s.ctx]
    t_f, t_s = [], []
    start = time.time()
    idx = None
    while (not t_f or not t_s) or (time.time() - start < budget_s and len(t_f) < 3):
        t0 = time.perf_counter()
        idx = oracle.topk(oracle.indexer_scores(q_idx, w, k_idx, ctx), ctx, s.k)
        oracle.sparse_attn(q, kv, idx, ctx, s.scale, s.d_v)
        t_f.append(time.perf_counter() - t0)
        t0 = time.perf_counter()
        oracle.sparse_attn(q, kv, idx, ctx, s.scale, s.d_v)
        t_s.append(time.perf_counter() - t0)
    return float(np.mean(t_f)), float(np.mean(t_s)), blas_threads()


def batched_decode_bench(dev, steps, warmup, cpu_seconds, cfg=1):
    """The batched decode workload (32 sequences x 32K context, bf16 indexer,
    8 layers): the configured pattern FSSSFSSS against all-F, per-kernel times
    with their roofline fractions, and the fp64 oracle's time per token."""
    import torch
    import dsa_sparse_attention_lightning_amd as dsa
    from dsa_sparse_attention_lightning_amd import inputs as gen
    s = gen.CONFIGS[cfg]
    layers = build_decode_workload(s, dev)
    ctx = gen.ctx_lens(s, dev)
    out = {"workload": f"{s.name}: {s.n_layers} layers, batch {s.B}, context {s.ctx}, indexer "
                       f"{s.H}x{s.D} {s.idx_dtype}, top-{s.k}, MLA {s.Hq} heads x {s.d_qk} bf16"}
    for name, p in (("config", s.pattern), ("all-F", "F" * s.n_layers)):
        st = dsa.Stack(p, layers, ctx, **shape_kw(s))
        ms, stats = time_stack(st, steps, warmup)
        st_i = dsa.Stack(p, layers, ctx, **shape_kw(s, attn=False))
        ms_i, _ = time_stack(st_i, steps, warmup)
        out[name] = dict(pattern=p, ms_per_step=round(ms, 4),
                         tokens_per_s=round(s.B / (ms * 1e-3), 1),
                         n_indexer_calls=stats["n_indexer_calls"],
                         indexer_topk_us_per_layer=round(ms_i * 1e3 / s.n_layers, 3),
                         indexer_topk_us_per_group4=round(ms_i * 1e3 / (s.n_layers / 4), 3))
        log(f"batched decode {name:6s} {ms:7.3f} ms/step {s.B / (ms * 1e-3):8.0f} tok/s  "
            f"indexer+topk {ms_i * 1e3 / s.n_layers:6.2f} us/layer")
        del st, st_i
    out["fsss_vs_allf_indexer_topk_cut"] = round(
        1 - out["config"]["indexer_topk_us_per_layer"] / out["all-F"]["indexer_topk_us_per_layer"],
        4)
    idx = torch.empty((s.B, s.T, s.k), dtype=torch.int32, device=dev)
    f_layers = [l for l, c in enumerate(s.pattern) if c == "F"]
    fz_ws = torch.zeros(dsa.indexer_topk_workspace_size(s.B, s.T, s.H, s.D, s.Lmax, s.k,
                                                        s.idx_dtype), dtype=torch.uint8,
                        device=dev)
    score = torch.empty((s.B, s.T, dsa.ld_for(s.Lmax)), dtype=torch.float32, device=dev)

    def run_fused(i=0):
        L = layers[i % s.n_layers]
        dsa.indexer_topk(L["q_idx"], L["w"], L["k_idx"], ctx, s.k, L["q_idx_scale"],
                         L["k_idx_scale"], out=idx, workspace=fz_ws)

    def run_idx(i=0):
        L = layers[i % s.n_layers]
        dsa.indexer_scores(L["q_idx"], L["w"], L["k_idx"], ctx, L["q_idx_scale"],
                           L["k_idx_scale"], out=score)

    at_ws = torch.zeros(max(1, dsa.sparse_attn_workspace_size(s.B, s.T, s.Hq, s.k)),
                        dtype=torch.uint8, device=dev)

    def run_attn(i=0):
        L = layers[i % s.n_layers]
        dsa.sparse_attn(L["q"], L["kv"], idx, ctx, s.scale, out=L["out"], lse=L["lse"],
                        workspace=at_ws)

    reps = 3 * s.n_layers
    t_f = event_time_ms(run_fused, reps)
    t_i = event_time_ms(run_idx, reps)
    t_a = event_time_ms(run_attn, reps)
    ib = indexer_bytes(s)
    fb = ib - s.B * s.T * s.Lmax * 4 + s.B * s.T * s.k * 4
    ab, af = attn_bytes_flops(s)
    out["kernels"] = {
        "indexer_topk": dict(us=round(t_f * 1e3, 3), bytes=fb,
                             frac_hbm=round(fb / (t_f * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                             launches_per_step=len(f_layers)),
        "indexer_decode": dict(us=round(t_i * 1e3, 3), bytes=ib,
                               frac_hbm=round(ib / (t_i * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                               launches_per_step=0),
        "sparse_mla": dict(us=round(t_a * 1e3, 3), bytes=ab, flops=af,
                           frac_hbm=round(ab / (t_a * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           frac_bf16_mfma=round(af / (t_a * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                           launches_per_step=s.n_layers)}
    for k_, v in out["kernels"].items():
        log(f"batched decode kernel {k_:15s} {v['us']:8.2f} us  {v['frac_hbm']:.1%} of HBM peak")
    del fz_ws, at_ws, score
    if cpu_seconds > 0:
        sf, ss, thr = oracle_layer_seconds(s, layers, s.pattern, cpu_seconds)
        nF = s.pattern.count("F")
        per_token = nF * sf + (s.n_layers - nF) * ss
        out["cpu_oracle"] = dict(seconds_per_F_layer=round(sf, 4), seconds_per_S_layer=round(ss, 4),
                                 tokens_per_s=round(1.0 / per_token, 4), threads=thr,
                                 sample=f"sequence 0 of {s.B}: one F and one S layer timed, "
                                        f"projected to {nF} F + {s.n_layers - nF} S layers")
        log(f"batched decode cpu oracle: {out['cpu_oracle']['tokens_per_s']} tokens/s")
    del layers
    torch.cuda.empty_cache()
    return out


def reuse_overlap(own, reused) -> float:
    """Share of one row's own selection (the set its layer's indexer and
    top-k pick) that the reused set of the nearest F layer also holds:
    |own ∩ reused| / |own|, -1 padding ignored (nan when own is empty).
    Checked against the oracle's pinned overlap_fraction by the CPU tests."""
    import numpy as np
    a = np.asarray(own).reshape(-1)
    b = np.asarray(reused).reshape(-1)
    a = np.unique(a[a >= 0])
    if a.size == 0:
        return math.nan
    return float(np.isin(a, b[b >= 0]).sum()) / a.size


def pattern_sweep(dev, steps, warmup, cfg=4, cpu_seconds=0.0):
    """The pattern sweep near maximum context: step time, indexer+top-k time
    per layer, and the overlap between the index set each S layer reuses and
    the set its own indexer would have produced (rows and S layers averaged)."""
    import numpy as np
    import torch
    import dsa_sparse_attention_lightning_amd as dsa
    from dsa_sparse_attention_lightning_amd import inputs as gen
    s = gen.CONFIGS[cfg]
    layers = build_decode_workload(s, dev)
    ctx = gen.ctx_lens(s, dev)
    own = []
    for L in layers:   # each layer's own selection (what an F layer would compute)
        sc = dsa.indexer_scores(L["q_idx"], L["w"], L["k_idx"], ctx, L["q_idx_scale"],
                                L["k_idx_scale"])
        own.append(dsa.topk(sc, ctx, s.k).cpu().numpy())
    out = {}
    for p in s.patterns:
        st = dsa.Stack(p, layers, ctx, **shape_kw(s))
        ms, stats = time_stack(st, steps, warmup)
        st_i = dsa.Stack(p, layers, ctx, **shape_kw(s, attn=False))
        ms_i, _ = time_stack(st_i, steps, warmup)
        ovs = []
        last_f = 0
        for l, c in enumerate(p):
            if c == "F":
                last_f = l
                continue
            for b in range(s.B):
                ovs.append(reuse_overlap(own[l][b, 0], own[last_f][b, 0]))
        key = "all-F" if set(p) == {"F"} else next(
            p[:n] for n in range(1, len(p) + 1) if gen.tile_pattern(p[:n], len(p)) == p)
        out[key] = dict(ms_per_step=round(ms, 4), tokens_per_s=round(s.B / (ms * 1e-3), 1),
                        n_indexer_calls=stats["n_indexer_calls"],
                        indexer_topk_us_per_layer=round(ms_i * 1e3 / s.n_layers, 3),
                        per_token_latency_ms=round(ms, 4),
                        reuse_overlap=round(float(np.nanmean(ovs)), 4) if ovs else None)
        log(f"sweep {key:9s} {ms:7.3f} ms/step  indexer+topk {ms_i * 1e3 / s.n_layers:7.2f} "
            f"us/layer  overlap {out[key]['reuse_overlap']}")
    cpu = None
    if cpu_seconds > 0:
        sf, ss, thr = oracle_layer_seconds(s, layers, s.pattern, cpu_seconds)
        cpu = dict(seconds_per_F_layer=round(sf, 4), seconds_per_S_layer=round(ss, 4),
                   threads=thr, sample=f"sequence 0 of {s.B}: one F and one S layer timed, "
                                       f"projected to each pattern's F and S layers")
        for key, v in out.items():
            nF = v["n_indexer_calls"]
            cpu[f"tokens_per_s_{key}"] = round(1.0 / (nF * sf + (s.n_layers - nF) * ss), 4)
        log(f"sweep cpu oracle: {sf:.3f} s per F layer, {ss:.3f} s per S layer")
    del layers
    torch.cuda.empty_cache()
    return dict(workload=f"{s.name}: {s.n_layers} layers, batch {s.B}, context {s.ctx}",
                patterns=out, cpu_oracle=cpu)


def prefill_oracle_sample(s, qi, ki, n_rows=8):
    """The fp64 oracle's indexer scores and full-sort top-k for n_rows query
    rows of the prefill chunk (the last rows: the most visible keys), timed
    and projected to the whole chunk by the rows' visible-key counts."""
    import numpy as np
    import oracle
    from dsa_sparse_attention_lightning_amd import inputs as gen
    rows = list(range(s.T - n_rows, s.T))
    q = oracle.dequant_fp8_rows(gen.bits(qi.q[:, rows]), qi.q_scale[:, rows].cpu().numpy())
    w = qi.w[:, rows].cpu().double().numpy()
    k = oracle.dequant_fp8_rows(gen.bits(ki.k), ki.k_scale.cpu().numpy())
    pos0 = s.ctx - s.T
    t0 = time.perf_counter()
    # a context that ends at the last sampled row: rows sit at pos0 + rows[i]
    sc = oracle.indexer_scores(q, w, k, [s.ctx])
    oracle.topk(sc, [s.ctx], s.k)
    dt = time.perf_counter() - t0
    seen = sum(pos0 + r + 1 for r in rows)
    total = sum(pos0 + t + 1 for t in range(s.T))
    return dict(seconds_sample=round(dt, 3), rows_sampled=n_rows,
                projected_seconds_per_chunk=round(dt * total / seen, 1), threads=blas_threads(),
                sample=f"query rows {rows[0]}..{rows[-1]} of the {s.T}-row chunk (fp64 numpy, "
                       f"indexer + full-sort top-k), projected by visible keys")


def prefill_bench(dev, reps=5, cpu=True):
    import torch
    import dsa_sparse_attention_lightning_amd as dsa
    from dsa_sparse_attention_lightning_amd import inputs as gen
    out = {}
    base = gen.CONFIGS[2]
    for dt in ("fp8", "bf16"):
        s = gen.Shape(2, base.name, 1, "F", B=base.B, T=base.T, ctx=base.ctx, H=base.H,
                      D=base.D, idx_dtype=dt, k=base.k)
        qi = gen.make_indexer_query(s, dev)
        ki = gen.make_indexer_keys(s, 0, gen.make_key_base(s, dev), dev)
        ctx = gen.ctx_lens(s, dev)
        score = torch.empty((s.B, s.T, dsa.ld_for(s.Lmax)), dtype=torch.float32, device=dev)
        idx = torch.empty((s.B, s.T, s.k), dtype=torch.int32, device=dev)
        t_i = event_time_ms(lambda i=0: dsa.indexer_scores(qi.q, qi.w, ki.k, ctx, qi.q_scale,
                                                           ki.k_scale, out=score), reps, 1)
        t_k = event_time_ms(lambda i=0: dsa.topk(score[..., :s.Lmax], ctx, s.k, out=idx), reps, 1)
        # the fused form (scores never written; candidate lists per row)
        fz_ws = torch.empty(dsa.indexer_topk_workspace_size(s.B, s.T, s.H, s.D, s.Lmax, s.k, dt),
                            dtype=torch.uint8, device=dev)
        t_f = event_time_ms(lambda i=0: dsa.indexer_topk(qi.q, qi.w, ki.k, ctx, s.k, qi.q_scale,
                                                         ki.k_scale, out=idx, workspace=fz_ws),
                            reps, 1)
        del fz_ws
        pos0 = s.ctx - s.T
        pairs = sum(pos0 + t + 1 for t in range(s.T))
        flops = 2.0 * s.H * s.D * pairs * s.B
        tf = flops / (t_i * 1e-3) / 1e12
        own_peak = FP8_PEAK_TFLOPS if dt == "fp8" else BF16_PEAK_TFLOPS
        out[dt] = dict(indexer_ms=round(t_i, 4), topk_ms=round(t_k, 4),
                       fused_indexer_topk_ms=round(t_f, 4),
                       algorithmic_tflop=round(flops / 1e12, 4), tflops=round(tf, 1),
                       frac_own_dtype_peak=round(tf / own_peak, 4),
                       frac_bf16_peak=round(tf / BF16_PEAK_TFLOPS, 4),
                       frac_fp8_peak=round(tf / FP8_PEAK_TFLOPS, 4))
        target = " (the >= 50% target applies to this bf16 kernel)" if dt == "bf16" else ""
        log(f"prefill {dt}: indexer {t_i:.3f} ms ({tf:.0f} TFLOP/s = {tf / own_peak:.1%} of the "
            f"{dt} MFMA peak{target}), top-k {t_k:.3f} ms, fused indexer + top-k {t_f:.3f} ms")
        if cpu and dt == "fp8":
            out[dt]["cpu_oracle"] = prefill_oracle_sample(s, qi, ki)
            log(f"prefill cpu oracle: {out[dt]['cpu_oracle']}")
        del qi, ki, score, idx
        torch.cuda.empty_cache()
    return out


def prefill_stack_bench(dev, n_layers=4, reps=3):
    """The prefill chunk (8192 queries appended to a 65536-token context, fp8
    indexer) through a short layer stack with sparse MLA attention (128 heads)
    on every layer: chunked prefill under IndexCache, all-F against FSSS."""
    import torch
    import dsa_sparse_attention_lightning_amd as dsa
    from dsa_sparse_attention_lightning_amd import inputs as gen
    base = gen.CONFIGS[2]
    s = gen.Shape(2, "prefill stack", n_layers, "F" * n_layers, B=base.B, T=base.T,
                  ctx=base.ctx, H=base.H, D=base.D, idx_dtype=base.idx_dtype, k=base.k, Hq=128)
    layers = build_decode_workload(s, dev)
    ctx = gen.ctx_lens(s, dev)
    out = {"workload": f"prefill chunk: {n_layers} layers, {s.T} queries on a {s.ctx}-token "
                       f"context, indexer {s.H}x{s.D} {s.idx_dtype}, top-{s.k}, "
                       f"MLA {s.Hq} heads x {s.d_qk} bf16"}
    af = 2.0 * s.Hq * s.k * (s.d_qk + s.d_v) * s.B * s.T
    for name, p in (("all-F", "F" * n_layers), ("FSSS", gen.tile_pattern("FSSS", n_layers))):
        st = dsa.Stack(p, layers, ctx, **shape_kw(s))
        ms, stats = time_stack(st, reps, 1)
        del st
        st_i = dsa.Stack(p, layers, ctx, **shape_kw(s, attn=False))
        ms_i, _ = time_stack(st_i, reps, 1)
        del st_i
        att = (ms - ms_i) / n_layers
        out[name] = dict(pattern=p, ms_per_chunk=round(ms, 3),
                         tokens_per_s=round(s.B * s.T / (ms * 1e-3), 1),
                         n_indexer_calls=stats["n_indexer_calls"],
                         indexer_topk_ms=round(ms_i, 3),
                         attention_ms_per_layer=round(att, 3),
                         attention_tflops=round(af / (att * 1e-3) / 1e12, 1))
        log(f"prefill stack {name}: {ms:.2f} ms per chunk ({s.B * s.T / (ms * 1e-3):.0f} tok/s), "
            f"indexer+top-k {ms_i:.2f} ms, attention {att:.2f} ms/layer")
    out["speedup_fsss_vs_allf"] = round(out["all-F"]["ms_per_chunk"] / out["FSSS"]["ms_per_chunk"], 3)
    del layers
    torch.cuda.empty_cache()
    return out


def prefill_context_bench(dev, ctx_final=196608, chunk=8192):
    """Whole-context chunked prefill under IndexCache: a prompt of ctx_final
    tokens taken in chunks of `chunk` tokens through the 48-layer stack of
    the long-context workload (fp8 indexer 64x128, top-2048, 128-head MLA).
    Each chunk appends its latent rows and indexer keys to every layer's
    caches (KV append, T = chunk), then runs the stack over the grown context.
    The full pass is timed for the 12-F pattern and for all-F, and again
    without attention (indexer + top-k only), which gives the indexer + top-k
    share of prefill time.  One pass each (about 40 s of GPU time in all)."""
    import torch
    import dsa_sparse_attention_lightning_amd as dsa
    from dsa_sparse_attention_lightning_amd import inputs as gen
    base = gen.CONFIGS[3]
    n_chunks = ctx_final // chunk
    s = gen.Shape(6, "chunked prefill", base.n_layers, base.pattern, B=1, T=chunk,
                  ctx=ctx_final, H=base.H, D=base.D, idx_dtype=base.idx_dtype, k=base.k,
                  Hq=base.Hq)
    t0 = time.time()
    qi = gen.make_indexer_query(s, dev)
    kb = gen.randn((s.Lmax, s.D), gen.seed_of(s.cfg_id, 0, "k_base"), dev)
    layers, src = [], []
    for l in range(s.n_layers):
        # fp32 rows a projection would produce: indexer keys correlated across
        # layers as in the other workloads, latent rows N(0,1)
        k_src = 0.95 * kb + 0.31 * gen.randn((s.Lmax, s.D), gen.seed_of(s.cfg_id, l, "k_noise"),
                                            dev)
        kv_src = gen.randn((s.Lmax, s.d_qk), gen.seed_of(s.cfg_id, l, "kv"), dev)
        q = gen.randn((1, chunk, s.Hq, s.d_qk), gen.seed_of(s.cfg_id, l, "q"), dev).to(
            torch.bfloat16)
        src.append((kv_src[None], k_src[None]))
        layers.append(dict(q_idx=qi.q, q_idx_scale=qi.q_scale, w=qi.w,
                           k_idx=torch.zeros((1, s.Lmax, s.D), dtype=torch.float8_e4m3fn,
                                             device=dev),
                           k_idx_scale=torch.ones((1, s.Lmax), dtype=torch.float32, device=dev),
                           q=q, kv=torch.zeros((1, s.Lmax, s.d_qk), dtype=torch.bfloat16,
                                               device=dev),
                           out=torch.empty((1, chunk, s.Hq, s.d_v), dtype=torch.bfloat16,
                                           device=dev)))
    del kb
    torch.cuda.synchronize()
    log(f"chunked prefill workload built in {time.time() - t0:.1f} s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB on device)")
    # one context-length tensor, set on the stream before each chunk (the
    # stack's buffers are sized for the whole prompt)
    ctx_t = torch.zeros((1,), dtype=torch.int32, device=dev)

    def one_pass(pattern, attn):
        st = dsa.Stack(pattern, layers, ctx_t, **shape_kw(s, attn))
        e = [torch.cuda.Event(enable_timing=True) for _ in range(n_chunks + 1)]
        torch.cuda.synchronize()
        e[0].record()
        for c in range(n_chunks):
            rows = slice(c * chunk, (c + 1) * chunk)
            ctx_t.fill_((c + 1) * chunk)
            for l, L in enumerate(layers):
                dsa.kv_append(ctx_t, src[l][0][:, rows], L["kv"], src[l][1][:, rows],
                              L["k_idx"], L["k_idx_scale"])
            st.run()
            e[c + 1].record()
        e[-1].synchronize()
        per = [e[c].elapsed_time(e[c + 1]) for c in range(n_chunks)]
        del st
        return sum(per), per

    # warm-up: the first chunk once
    ctx_t.fill_(chunk)
    warm = dsa.Stack(s.pattern, layers, ctx_t, **shape_kw(s))
    warm.run()
    torch.cuda.synchronize()
    del warm
    out = {"workload": f"{s.name}: prompt of {ctx_final} tokens in {n_chunks} chunks of {chunk}, "
                       f"{s.n_layers} layers, indexer {s.H}x{s.D} {s.idx_dtype}, top-{s.k}, "
                       f"MLA {s.Hq} heads x {s.d_qk} bf16, KV append per chunk"}
    for name, p in (("config", s.pattern), ("all-F", "F" * s.n_layers)):
        ms, per = one_pass(p, True)
        ms_i, _ = one_pass(p, False)
        out[name] = dict(pattern=p, prefill_s=round(ms / 1e3, 3),
                         tokens_per_s=round(ctx_final / (ms * 1e-3), 1),
                         first_chunk_ms=round(per[0], 2), last_chunk_ms=round(per[-1], 2),
                         indexer_topk_append_s=round(ms_i / 1e3, 3),
                         indexer_topk_share=round(ms_i / ms, 4))
        log(f"chunked prefill {name}: {ms / 1e3:.2f} s for {ctx_final} tokens "
            f"(chunks {per[0]:.1f} .. {per[-1]:.1f} ms), indexer+top-k(+append) "
            f"{ms_i / 1e3:.2f} s = {ms_i / ms:.1%}")
    out["speedup_config_vs_allf"] = round(out["all-F"]["prefill_s"] / out["config"]["prefill_s"],
                                          3)
    del layers, src, qi
    torch.cuda.empty_cache()
    return out


def pattern_search_bench(dev, n_layers=48, n_shared=36):
    """Training-free pattern search on a synthetic calibration stack with
    planted structure: layers 0..2 each have an unrelated key cache, layers
    3..23 share one, layers 24..47 another (an early block and a transition,
    the layers the pages name as critical).  The device builds the proxy
    cost matrix (every layer's own index set, every reuse attention, the
    reductions); the host runs the greedy F -> S search to 75% S layers."""
    import torch
    import dsa_sparse_attention_lightning_amd as dsa
    from dsa_sparse_attention_lightning_amd import inputs as gen
    s = gen.Shape(5, "calibration stack", n_layers, "F" * n_layers, B=4, T=1, ctx=32768, H=64,
                  D=128, idx_dtype="fp8", k=2048, Hq=128)
    early, transition = 3, 24
    seg = gen.calibration_segments(n_layers, early, transition)
    qi = gen.make_indexer_query(s, dev)
    bases = {g: gen.make_segment_base(s, g, dev) for g in sorted(set(seg))}
    layers = []
    for l in range(n_layers):
        ki = gen.make_indexer_keys(s, l, bases[seg[l]], dev)
        q, kv = gen.make_mla_layer(s, l, dev)
        layers.append(dict(q_idx=qi.q, q_idx_scale=qi.q_scale, w=qi.w, k_idx=ki.k,
                           k_idx_scale=ki.k_scale, q=q, kv=kv,
                           out=torch.empty((s.B, s.T, s.Hq, s.d_v), dtype=torch.bfloat16,
                                           device=dev)))
    del bases
    ctx = gen.ctx_lens(s, dev)
    planted = sorted({0} | {l for l in range(1, n_layers) if seg[l] != seg[l - 1]})
    kw = dict(B=s.B, T=s.T, H=s.H, D=s.D, Lmax=s.Lmax, k=s.k, Hq=s.Hq, idx_dtype=s.idx_dtype,
              scale=s.scale)
    out = {"workload": f"{s.name}: {n_layers} layers, batch {s.B}, context {s.ctx}, indexer "
                       f"{s.H}x{s.D} {s.idx_dtype}, top-{s.k}, MLA {s.Hq} heads; key caches "
                       f"unrelated across layers {planted}",
           "planted_critical_layers": planted, "n_shared": n_shared}
    for proxy in ("output", "miss"):
        ws = torch.zeros(dsa.reuse_costs_workspace_size(n_layers, proxy=proxy, **kw),
                         dtype=torch.uint8, device=dev)
        dsa.reuse_costs(layers, ctx, proxy=proxy, workspace=ws, **kw)   # warm-up
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cost = dsa.reuse_costs(layers, ctx, proxy=proxy, workspace=ws, **kw)
        e1.record()
        e1.synchronize()
        cost = cost.cpu().numpy()
        t0 = time.perf_counter()
        trace = dsa.greedy_search(cost, n_shared)
        t_host = time.perf_counter() - t0
        best = trace[-1][0]
        kept = [l for l, c in enumerate(best) if c == "F"]
        uniform = gen.tile_pattern("FSSS", n_layers)
        out[proxy] = dict(cost_matrix_ms=round(e0.elapsed_time(e1), 3),
                          search_ms=round(t_host * 1e3, 3), pattern=best,
                          proxy_cost=round(trace[-1][1], 5),
                          proxy_cost_uniform_fsss=round(dsa.pattern_cost(cost, uniform), 5),
                          proxy_cost_fixed_12f=round(dsa.pattern_cost(cost, gen.C3_PATTERN), 5),
                          planted_layers_kept=all(l in kept for l in planted))
        log(f"pattern search ({proxy}): matrix {out[proxy]['cost_matrix_ms']} ms, search "
            f"{out[proxy]['search_ms']} ms -> {best} cost {trace[-1][1]:.4f} "
            f"(uniform FSSS {out[proxy]['proxy_cost_uniform_fsss']:.4f})")
        del ws, cost
    del layers
    torch.cuda.empty_cache()
    return out


def kv_append_bench(dev, reps=200):
    """KV-cache append (latent row bf16 + fp8 indexer key with its row scale)
    at the decode shape (batch 8, one token, 131072-row caches) and the prefill
    chunk (8192 tokens into a 65536-row cache).  Algorithmic bytes per token
    row: fp32 reads of d_qk + D values, bf16 latent write, fp8 key write and
    one fp32 scale."""
    import torch
    import dsa_sparse_attention_lightning_amd as dsa
    d_qk, D = 576, 128
    row_bytes = 4 * (d_qk + D) + 2 * d_qk + D + 4
    out = {"bytes_per_row": row_bytes}
    for name, B, T, Lmax in (("decode", 8, 1, 131072), ("prefill", 1, 8192, 65536)):
        kvc = torch.zeros((B, Lmax, d_qk), dtype=torch.bfloat16, device=dev)
        kc = torch.zeros((B, Lmax, D), dtype=torch.float8_e4m3fn, device=dev)
        ks = torch.ones((B, Lmax), dtype=torch.float32, device=dev)
        g = torch.Generator(device=dev)
        g.manual_seed(1234)
        kvn = torch.randn((B, T, d_qk), generator=g, device=dev)
        kn = torch.randn((B, T, D), generator=g, device=dev)
        ctx = torch.full((B,), Lmax, dtype=torch.int32, device=dev)
        # The decode append is far shorter than one host-side call, so the
        # appends are captured into a HIP graph (20 per replay) and the graph
        # is timed: the figure is device time, not the binding's call rate.
        per = 20
        for _ in range(3):
            dsa.kv_append(ctx, kvn, kvc, kn, kc, ks)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(per):
                dsa.kv_append(ctx, kvn, kvc, kn, kc, ks)
        ms = event_time_ms(lambda i=0: graph.replay(), max(1, reps // per), 1) / per
        del graph
        gbs = B * T * row_bytes / (ms * 1e-3) / 1e9
        out[name] = dict(batch=B, tokens=T, cache_rows=Lmax, us=round(ms * 1e3, 2),
                         gbs=round(gbs, 1), frac_hbm_peak=round(gbs / HBM_PEAK_GBS, 4))
        log(f"kv append {name}: {ms * 1e3:.2f} us ({gbs:.0f} GB/s)")
        del kvc, kc, ks, kvn, kn
    torch.cuda.empty_cache()
    return out



def stream_probe_bench(dev, replays=8):
    """Streaming-read ceiling for the decode indexer: a plain read of the bytes
    one indexer launch moves at batch 8 x 131072 context (142,675,968, rounded
    up to whole 8 KB tiles), in the indexer's own load pattern (256 workgroups
    of eight waves, contiguous runs of 8 KB tiles, two tiles in flight per
    wave) and in other launch shapes.  Twelve copies of the buffer are read in
    turn (1.7 GB, far beyond the L2 and last-level caches), one graph replay
    reading each copy once, so every read comes from HBM."""
    import torch
    import dsa_sparse_attention_lightning_amd as dsa
    nbytes = (142675968 + 8191) // 8192 * 8192
    copies = 12
    bufs = [torch.full((nbytes,), c, dtype=torch.uint8, device=dev) for c in range(copies)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    out = {"bytes": nbytes, "copies": copies}
    for name, form, wgs in (("tiles_256wg", "tiles", 256), ("tiles_512wg", "tiles", 512),
                            ("tiles_1024wg", "tiles", 1024), ("stride_1024wg", "stride", 1024),
                            ("stride_2048wg", "stride", 2048)):
        for b in bufs:
            dsa.probe_stream_read(b, sink, wgs, form)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for b in bufs:
                dsa.probe_stream_read(b, sink, wgs, form)
        ms = event_time_ms(lambda i=0: graph.replay(), replays, 1) / copies
        del graph
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = dict(us=round(ms * 1e3, 2), gbs=round(gbs, 1),
                         frac_hbm_peak=round(gbs / HBM_PEAK_GBS, 4))
        log(f"stream read {name}: {ms * 1e3:.2f} us ({gbs:.0f} GB/s, "
            f"{100 * gbs / HBM_PEAK_GBS:.1f}% of HBM peak)")
    del bufs, sink
    torch.cuda.empty_cache()
    return out

def environment():
    """Where the numbers were taken: GPU, gfx target, ROCm and torch versions,
    the GPU shader clock as rocm-smi reports it, host CPU model and threads."""
    import torch
    env = {}
    try:
        p = torch.cuda.get_device_properties(0)
        env.update(gpu=p.name, gfx_target=getattr(p, "gcnArchName", None),
                   compute_units=p.multi_processor_count,
                   hbm_gib=round(p.total_memory / 2**30, 1))
    except Exception as e:  # pragma: no cover - reported, not fatal
        env["gpu_error"] = str(e)
    try:
        env["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        env["rocm"] = None
    env["torch"] = torch.__version__
    # shader / memory clock levels the driver offers (sysfs text); the clock a
    # kernel actually runs at under load is read from hardware counters
    # (GRBM_GUI_ACTIVE over the dispatch time) in the profile summaries
    clocks = {}
    try:
        import glob
        for dev_dir in sorted(glob.glob("/sys/class/drm/card*/device")):
            for name in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
                path = os.path.join(dev_dir, name)
                if os.path.exists(path):
                    lines = [l.strip().rstrip("*").strip() for l in open(path) if l.strip()]
                    clocks[name[7:] + "_levels"] = [l.split(":", 1)[-1].strip() for l in lines]
            if clocks:
                break
    except OSError as e:  # pragma: no cover
        clocks = {"error": str(e)}
    env["gpu_clocks"] = clocks
    try:
        models = [l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo")
                  if l.startswith("model name")]
        env["host_cpu"] = models[0] if models else None
    except OSError:
        env["host_cpu"] = None
    env["host_cpus"] = os.cpu_count()
    try:
        env["host_cpus_usable"] = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        env["host_cpus_usable"] = None
    return env


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(s, layers, budget_s):
    """The fp64 oracle, as it stands, on sequence 0 of the same workload."""
    import numpy as np
    import oracle
    from dsa_sparse_attention_lightning_amd import inputs as gen
    threads = blas_threads()
    b = 0
    t_f, t_s = [], []
    idx = None
    q_idx = oracle.dequant_fp8_rows(gen.bits(layers[0]["q_idx"][b:b + 1]),
                                    layers[0]["q_idx_scale"][b:b + 1].cpu().numpy())
    w = layers[0]["w"][b:b + 1].cpu().double().numpy()
    ctx = [s.ctx]
    start = time.time()
    for l, c in enumerate(s.pattern):
        if time.time() - start > budget_s and t_f and t_s:
            break
        L = layers[l]
        q = oracle.bf16_bits_to_f64(gen.bits(L["q"][b:b + 1]))
        kv = oracle.bf16_bits_to_f64(gen.bits(L["kv"][b:b + 1]))
        kk = None
        if c == "F":
            kk = oracle.dequant_fp8_rows(gen.bits(L["k_idx"][b:b + 1]),
                                         L["k_idx_scale"][b:b + 1].cpu().numpy())
        t0 = time.perf_counter()
        if c == "F":
            sc = oracle.indexer_scores(q_idx, w, kk, ctx)
            idx = oracle.topk(sc, ctx, s.k)
        oracle.sparse_attn(q, kv, idx, ctx, s.scale, s.d_v)
        dt = time.perf_counter() - t0
        (t_f if c == "F" else t_s).append(dt)
        del q, kv, kk
    nF = s.pattern.count("F")
    per_token = nF * float(np.mean(t_f)) + (s.n_layers - nF) * float(np.mean(t_s))
    return dict(value=round(1.0 / per_token, 4), unit="tokens/s", cores=int(threads),
                kind="oracle",
                sample=(f"sequence 0 of {s.B}, layers 0..{len(t_f) + len(t_s) - 1} of the "
                        f"{s.n_layers}-layer stack ({len(t_f)} F, {len(t_s)} S timed), projected "
                        f"to {nF} F + {s.n_layers - nF} S layers for one token; fp64 numpy, "
                        f"{os.cpu_count()} host cores"),
                seconds_per_F_layer=round(float(np.mean(t_f)), 4),
                seconds_per_S_layer=round(float(np.mean(t_s)), 4))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the 196K-context pattern sweep")
    ap.add_argument("--no-search", action="store_true", help="skip the pattern-search leg")
    ap.add_argument("--no-kv-append", action="store_true", help="skip the KV-append leg")
    ap.add_argument("--no-batched", action="store_true",
                    help="skip the batched-decode leg (32 x 32K, bf16 indexer)")
    ap.add_argument("--no-prefill-context", action="store_true",
                    help="skip the whole-context chunked prefill leg (196608 tokens)")
    ap.add_argument("--prefill-context-only", action="store_true",
                    help="run only the whole-context chunked prefill leg")
    ap.add_argument("--search-only", action="store_true",
                    help="run only the pattern-search leg and print its JSON object")
    ap.add_argument("--kv-append-only", action="store_true",
                    help="run only the KV-cache append leg and print its JSON object")
    ap.add_argument("--no-stream-probe", action="store_true",
                    help="skip the streaming-read ceiling probe")
    ap.add_argument("--stream-probe-only", action="store_true",
                    help="run only the streaming-read ceiling probe and print its JSON object")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the prefill legs (kernels and 4-layer stack) and print "
                         "their JSON object")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size "
                         "reference for hardware traffic counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU's share of the path: --gpus {args.gpus} "
              f"(WORLD_SIZE {world}) is not supported; run with --gpus 1", flush=True)
        sys.exit(2)

    import torch
    import dsa_sparse_attention_lightning_amd as dsa
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", flush=True)
        sys.exit(1)
    dsa.library()  # fail loudly if the HIP library is missing
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.search_only:
        print(json.dumps({"pattern_search": pattern_search_bench(dev)}), flush=True)
        return
    if args.stream_probe_only:
        print(json.dumps({"stream_read_ceiling": stream_probe_bench(dev)}), flush=True)
        return
    if args.kv_append_only:
        print(json.dumps({"kv_append": kv_append_bench(dev)}), flush=True)
        return
    if args.prefill_context_only:
        print(json.dumps({"prefill_context": prefill_context_bench(dev)}), flush=True)
        return
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_bench(dev, cpu=False),
                          "prefill_stack": prefill_stack_bench(dev)}), flush=True)
        return
    env = environment()
    log(f"environment: {json.dumps(env)}")
    s, layers, res, cut, kernels, roof = decode_bench(args, dev)
    main_res = res["config"]
    batched = None
    if not args.no_batched:
        batched = batched_decode_bench(dev, args.steps, args.warmup,
                                       0.0 if args.no_cpu_baseline else args.cpu_seconds / 3)
    sweep = None
    if not args.no_sweep:
        sweep = pattern_sweep(dev, max(5, args.steps // 3), 2,
                              cpu_seconds=0.0 if args.no_cpu_baseline else args.cpu_seconds / 3)
    prefill = None if args.no_prefill else prefill_bench(dev, cpu=not args.no_cpu_baseline)
    prefill_stack = None if args.no_prefill else prefill_stack_bench(dev)
    kv_app = None if args.no_kv_append else kv_append_bench(dev)
    ceiling = None if args.no_stream_probe else stream_probe_bench(dev)
    prefill_ctx = None
    if not (args.no_prefill or args.no_prefill_context):
        prefill_ctx = prefill_context_bench(dev)
    search = None if args.no_search else pattern_search_bench(dev)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(s, layers, args.cpu_seconds)
        log(f"cpu oracle: {cpu['value']} tokens/s on {cpu['cores']} threads")

    line = {
        "metric": METRIC,
        "value": round(main_res["tokens_per_s"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 indexer, bf16 attention, fp32 accumulate",
        "data": "synthetic: seeded N(0,1) queries/keys/latents, U(0,1) head weights, "
                "indexer keys correlated 0.9 across layers",
        "config": {"workload": f"{s.name}: {s.n_layers} layers, batch {s.B}, context {s.ctx}, "
                               f"indexer {s.H}x{s.D} {s.idx_dtype}, top-{s.k}, "
                               f"MLA {s.Hq} heads x {s.d_qk} bf16",
                   "pattern": s.pattern, "batch": s.B, "context": s.ctx},
        "roofline": roof,
        "cpu_baseline": cpu,
        "environment": env,
        "patterns": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                         for kk, vv in v.items()} for k, v in res.items()},
        "fsss_vs_allf_indexer_topk_cut": round(cut, 4),
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv)
                        for kk, vv in v.items()} for k, v in kernels.items()},
        "batched_decode": batched,
        "prefill": prefill,
        "prefill_stack": prefill_stack,
        "prefill_context": prefill_ctx,
        "kv_append": kv_app,
        "stream_read_ceiling": ceiling,
        "pattern_search": search,
        "pattern_sweep": sweep,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
