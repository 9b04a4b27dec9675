#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer on one MI355X.

Headline workload: batch-1 decode of one MoE layer (T=1; hidden 2048, 256 routed
experts top-8 plus one shared expert, SwiGLU intermediate 512, int4 group-64 weights
with bf16 scale and bias; fp32 router). One step is one token through the whole layer
(router GEMV + top-8 + 8+1 expert GEMVs + combine). Weights are cache-cold: 20 seeded
copies of the layer (9.1 GB) rotate per token, so a copy is reused only after 19 other
tokens have streamed 342 MB, more than the 256 MB Infinity Cache plus L2. --warmup tokens
run first; then 20 repetitions of exactly --steps tokens are replayed from HIP graphs (the
host enqueues ahead and never synchronises in between), each timed with events on the
replay stream, and the median repetition gives `value` and `ms_per_step`.

Also reported in the same line:
  - the dominant decode kernel's roofline (durations from HIP events bound to its
    dispatches) and every decode kernel against the spec peak and against its read ceiling:
    the same loads from the same grid with the arithmetic taken out (the page's "fastest
    sustained rate for the access pattern");
  - the cost of one kernel inside a HIP graph, and a dense MFMA loop (the matrix-core rate
    the GPU sustains, on full-mantissa operands like the GEMMs' and on low-entropy ones: the
    part clocks down at its power limit in proportion to the bits the matrix cores switch);
  - prefill of T=4096 tokens with near-uniform routing and with Zipf(1.1)-skewed routing
    (median per call; tokens/s, fraction of the dense bf16 MFMA peak and of the measured
    full-mantissa MFMA ceiling);
  - a stack of 40 such layers (pre-norm residual blocks): batch-1 decode of 256 tokens and a
    32,768-token prompt in chunks of 4096 tokens;
  - moe_prefill with 2, 4 and 8 tokens (the small-T kernels) over the 20 layer copies, and
    the prefill ablations (separate dequantisation pass, host-inspected routing, fixed tile
    heights) at 512, 2048 and 4096 tokens beside the product path;
  - grouped-query decode attention (16 query heads, 2 KV heads, head dimension 256, bf16
    cache) over 3,840 to 131,072 cached positions, packed and unpacked; the Gated DeltaNet
    prompt scan of one layer (2,048 and 8,192 tokens, 32 value heads, fp32 state in
    registers);
  - the CPU oracle on bounded samples (decode alternating with GPU rounds, the tiny layer on
    one thread, a teacher-forced slice of the stack, attention and DeltaNet).
Prefill timings start after about 80 ms of sustained calls, past the lower-clock spell that
follows an idle GPU.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-prefill]
                       [--no-stack] [--no-attention] [--no-gdn]
       python bench.py --profile {decode,prefill_uniform,...}   (fixed work for rocprofv3)
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector (packed FMA), TFLOP/s
H, I, E, K_TOP, S = 2048, 512, 256, 8, 1
N_COPIES = 20
N_TOKENS = 1000


def expert_bytes():
    w13 = 2 * I * H // 2 + 2 * (2 * I * H // 64) * 2
    w2 = H * I // 2 + 2 * (H * I // 64) * 2
    return w13, w2


def decode_bytes_per_token():
    w13, w2 = expert_bytes()
    return E * H * 4 + (K_TOP + S) * (w13 + w2) + H * 2 * 2


def _decode_kernel_bytes():
    w13, w2 = expert_bytes()
    return {
        # router fp32 rows + x
        "k_dec_a": E * H * 4 + H * 2,
        # routed and shared experts' gate/up + logits + x
        "k_dec_b": (K_TOP + S) * w13 + E * 4 + H * 2,
        # all k+1 experts' down projection + h (fp32) + routing + y
        "k_dec_c": (K_TOP + S) * w2 + (K_TOP + S) * I * 4 + K_TOP * 8 + H * 2,
    }


DECODE_KERNEL_BYTES = _decode_kernel_bytes()


def prefill_flops_per_token():
    return (K_TOP + S) * 3 * 2 * H * I + 2 * H * E


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(kernel, src):
    """HBM traffic per launch from a committed rocprofv3 --pmc summary, if the kernel
    source has not changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(src):
        return None
    return rec.get("bytes_per_launch")


def gpu_layer(moe, torch, synth, dev, seed):
    """A layer of the decode shape drawn on the GPU (seeded torch generator) with the
    distributions of synth.make_int4_layer; used only for timing."""
    mag = 0.02 / synth.NIBBLE_STD
    g = torch.Generator(device=dev)
    g.manual_seed(seed)

    def int4(rows, K):
        q = torch.randint(0, 256, (E + S, rows, K // 2), dtype=torch.uint8, device=dev,
                          generator=g)
        s = (torch.rand((E + S, rows, K // 64), device=dev, generator=g) + 0.5) * mag
        s = s.to(torch.bfloat16)
        b = (-s.float() * (6.5 + 2.0 * torch.rand(s.shape, device=dev, generator=g)))
        return q, s, b.to(torch.bfloat16)

    rw = torch.randn((E, H), device=dev, generator=g) * 0.02
    q13, s13, b13 = int4(2 * I, H)
    q2, s2, b2 = int4(H, I)
    return moe.DeviceLayer.from_tensors(H, I, E, K_TOP, S, "int4", router_w=rw, router_b=None,
                                        w13_q=q13, w13_s=s13, w13_b=b13, w2_q=q2, w2_s=s2,
                                        w2_b=b2)


def gpu_copies(moe, torch, synth, dev):
    """Layer copy 0 from the seeded numpy generator; copies 1..19 drawn on the GPU with
    the same distributions, used only for timing."""
    layers = [moe.DeviceLayer.from_host(synth.decode_layer(0), dev)]
    for c in range(1, N_COPIES):
        layers.append(gpu_layer(moe, torch, synth, dev, c))
    return layers


def decode_graphs(moe, torch, layers, xs, ws, y, first, count):
    """HIP graphs replaying decode tokens first .. first+count-1 (token i reads layer copy
    i % N_COPIES and input row i % N_TOKENS), at most 100 tokens per graph."""
    def step(i):
        moe.moe_decode(layers[i % N_COPIES], xs[i % N_TOKENS:i % N_TOKENS + 1], y=y, ws=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(3):
            step(first + i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graphs = []
    for c0 in range(first, first + count, 100):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(c0, min(c0 + 100, first + count)):
                step(i)
        graphs.append(g)
    return graphs, step


def bench_decode(moe, torch, synth, dev, steps, warmup, reps=20):
    """Batch-1 decode over 20 cache-cold layer copies. One repetition replays exactly `steps`
    tokens from HIP graphs; `warmup` tokens run first (untimed), then `reps` repetitions are
    timed one by one with events on the replay stream and the median is reported."""
    import numpy as np
    layers = gpu_copies(moe, torch, synth, dev)
    xs = moe.bf16_from_bits(np.concatenate([synth.decode_token(t) for t in range(N_TOKENS)]),
                            dev)
    ws = moe.workspace(layers[0], 1, dev)
    y = torch.empty((1, H), dtype=torch.bfloat16, device=dev)
    graphs, step = decode_graphs(moe, torch, layers, xs, ws, y, 0, steps)
    if warmup > 0:
        wgraphs, _ = decode_graphs(moe, torch, layers, xs, ws, y, steps, warmup)
        for g in wgraphs:
            g.replay()
        # a graph may only be released once its replays have finished: its executable owns
        # the argument buffers its kernels read
        torch.cuda.synchronize()
        del wgraphs
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        for g in graphs:
            g.replay()
        b.record()
    torch.cuda.synchronize()
    rep_ms = [a.elapsed_time(b) for a, b in ev]
    ms = float(np.median(rep_ms))

    # eager (no graph) rate, for context
    torch.cuda.synchronize()
    e0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    eager_s = time.perf_counter() - e0

    # per-kernel durations from HIP events recorded by the library on its stream
    nprof = max(steps, 200)
    moe.profile_reset()
    moe.profile_enable(True)
    for i in range(nprof):
        step(i)
    torch.cuda.synchronize()
    moe.profile_enable(False)
    kern = {}
    for name in DECODE_KERNEL_BYTES:
        tot, n = moe.profile_query(name)
        if n:
            kern[name] = {"avg_us": 1e3 * tot / n, "launches": n}
    moe.profile_reset()
    ceil = bench_read_ceilings(moe, torch, layers, xs, nprof)
    # a captured graph holds raw pointers, not the tensors: everything its kernels read or
    # write must stay allocated for as long as the graph may be replayed
    keep = {"graphs": graphs, "layers": layers, "xs": xs, "ws": ws, "y": y}

    def gpu_round():
        """One more timed repetition (for the interleaved CPU comparison); ms."""
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for g in keep["graphs"]:
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    return {"ms_rep_median": ms, "rep_ms": rep_ms, "steps": steps, "reps": reps,
            "eager_tok_s": steps / eager_s, "kernels": kern, "ceilings": ceil,
            "gpu_round": gpu_round}


# weight bytes each read-ceiling kernel loads (the decode kernels' weights, no activations)
CEILING_PARTS = {"k_dec_a": (0, "k_read_router"), "k_dec_b": (1, "k_read_gateup"),
                 "k_dec_c": (2, "k_read_down")}


def bench_read_ceilings(moe, torch, layers, xs, n):
    """The page's read ceiling for each decode kernel: the same loads from the same grid with
    the arithmetic taken out (moe_decode_read_ceiling), over the same cache-cold rotation of
    layer copies, each token reading the experts copy 0 routes it to."""
    w13, w2 = expert_bytes()
    nbytes = {"k_dec_a": E * H * 4 + H * 2, "k_dec_b": (K_TOP + S) * w13,
              "k_dec_c": (K_TOP + S) * w2}
    T = min(n, N_TOKENS)
    ids = moe.moe_route(layers[0], xs[:T])["topk_ids"]
    sink = torch.zeros(1, dtype=torch.int32, device=ids.device)
    for i in range(3):
        for part, _ in CEILING_PARTS.values():
            moe.decode_read_ceiling(layers[i % N_COPIES], ids[i % T], part, sink)
    torch.cuda.synchronize()
    moe.profile_reset()
    moe.profile_enable(True)
    for i in range(n):
        for part, _ in CEILING_PARTS.values():
            moe.decode_read_ceiling(layers[i % N_COPIES], ids[i % T], part, sink)
    torch.cuda.synchronize()
    moe.profile_enable(False)
    res = {}
    for kname, (part, rname) in CEILING_PARTS.items():
        tot, cnt = moe.profile_query(rname)
        us = 1e3 * tot / max(cnt, 1)
        res[kname] = {"read_kernel": rname, "avg_us": round(us, 3), "weight_bytes": nbytes[kname],
                      "GB_s": round(nbytes[kname] / (us * 1e-6) / 1e9, 1)}
    moe.profile_reset()
    return res


def bench_mfma_ceiling(moe, torch, dev, iters=1500, reps=20):
    """Dense v_mfma_f32_32x32x16_f16 loop (no memory traffic), 512 workgroups of 4 waves: the
    matrix-core rate this GPU sustains, median of `reps` back-to-back timed launches after a
    warm-up, once on full-mantissa operands (like the GEMMs' data) and once on low-entropy
    ones. The part clocks down at its power limit in proportion to the bits the matrix cores
    switch, so only the second comes near the nominal peak."""
    import numpy as np
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    res = {}
    for name, kind in (("full_mantissa", moe.CEIL_FULL_MANTISSA),
                       ("low_entropy", moe.CEIL_LOW_ENTROPY)):
        flops = moe.mfma_ceiling(iters, sink, kind)
        warm_up(lambda: moe.mfma_ceiling(iters, sink, kind))
        ms = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            moe.mfma_ceiling(iters, sink, kind)
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        med = float(np.median(ms))
        tf = flops / (med * 1e-3) / 1e12
        res[name] = {"tflops": round(tf, 1), "flop_per_launch": flops, "ms_median": round(med, 4),
                     "frac_of_spec": round(tf / BF16_PEAK_TFLOPS, 3)}
    res["tflops"] = res["full_mantissa"]["tflops"]
    return res


def bench_launch_floor(torch, dev, n=30, reps=20):
    """Cost of one kernel inside a HIP graph on this GPU: a graph of n single-workgroup
    elementwise kernels (torch's add on one element), median over reps replays."""
    import numpy as np
    t = torch.zeros(1, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        t.add_(1.0)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            t.add_(1.0)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    return {"us_per_kernel": round(1e3 * float(np.median(ms)) / n, 3), "kernels_per_graph": n}


def warm_up(fn, ms=80.0):
    """Calls fn until about `ms` of sustained GPU work has run: the first tens of
    milliseconds after an idle spell run at lower clocks (up to 15 % slower)."""
    import time
    import torch
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def timed_median(torch, fn, reps):
    """Median milliseconds of `reps` calls of fn, each bracketed by events on the current
    stream (the calls run back to back; the events are read afterwards)."""
    import numpy as np
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


PREFILL_KERNELS = ("k_router_mfma", "k_topk", "k_group", "k_grouped_fused",
                   "k_shared_down_combine")


def bench_prefill(moe, torch, synth, dev, layer_host, reps=30):
    """moe_prefill at T = 4096: median per-call time over `reps` calls after about 80 ms of
    sustained calls (eager, and replayed from a HIP graph), and per-kernel durations."""
    T = 4096
    dl = moe.DeviceLayer.from_host(layer_host, dev)
    x = moe.bf16_from_bits(synth.prefill_x(T, seed=2), dev)
    ws = moe.workspace(dl, T, dev)
    y = torch.empty_like(x)
    call = lambda: moe.moe_prefill(dl, x, y=y, ws=ws)
    warm_up(call)
    ms = timed_median(torch, call, reps)
    # the same call replayed from a HIP graph (no host work between kernels)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    warm_up(g.replay)
    ms_graph = timed_median(torch, g.replay, reps)
    del g
    moe.profile_reset()
    moe.profile_enable(True)
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    moe.profile_enable(False)
    kern = {}
    for name in PREFILL_KERNELS:
        tot, n = moe.profile_query(name)
        kern[name] = {"avg_us": 1e3 * tot / max(n, 1), "launches": n}
    moe.profile_reset()
    buf = moe.moe_route(dl, x, ws=ws)
    rows = int(buf["counts"].sum().item()) + T * S
    flops = prefill_flops_per_token() * T
    tok_s = T / (ms * 1e-3)
    # the persistent expert launch: gate/up of every row (routed and shared), down of the
    # routed rows (the shared expert's down projection runs with the combine)
    fused_flops = rows * 2 * H * 2 * I + (rows - T * S) * 2 * I * H
    fu_us = kern["k_grouped_fused"]["avg_us"]
    del dl, ws, x, y
    torch.cuda.empty_cache()
    return {"tokens_per_s": tok_s, "ms_per_call": ms, "ms_per_call_graph": ms_graph,
            "tokens_per_s_graph": T / (ms_graph * 1e-3), "calls_timed": reps,
            "tflops": flops / (ms * 1e-3) / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "max_group": int(buf["counts"].max().item()),
            "experts_tflops": fused_flops / (fu_us * 1e-6) / 1e12 if fu_us > 0 else None,
            "kernels": kern}


STACK_LAYERS, STACK_DECODE_TOKENS, STACK_PROMPT, STACK_CHUNK = 40, 256, 32768, 4096

# The pages' prefill ablations ("Optimize sparse expert computation") and their reported
# end-to-end gains of the adopted design over each (other hardware, whole model).
PAGE_ABLATION_GAINS = {"separate_dequant": {"tokens": 512, "gain": 0.774},
                       "host_routing": {"tokens": 512, "gain": 0.89},
                       "tile_64": {"tokens": 2048, "gain": 0.132, "note": "16- vs 32-row tile"}}


ATTN_CTXS = (3840, 32768, 65536, 131072)


def bench_attention(moe, torch, synth, dev, ctxs=ATTN_CTXS, rounds=5):
    """Decode attention of one token (16 query heads, 2 KV heads, head dimension 256, bf16
    cache) over caches of the given lengths. Cache-cold: enough seeded cache copies rotate
    that together they exceed 1 GiB (several Infinity Caches); calls replay from HIP graphs.
    Bytes per call = the K and V rows read (2 * 2 * ctx * 256 * 2) + q and out. Also the
    unpacked variant (one workgroup per query head, the page's ablation) for its gain."""
    import numpy as np
    nq, nkv, D = synth.ATTN_Q_HEADS, synth.ATTN_KV_HEADS, synth.ATTN_HEAD_DIM
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    res = {}
    for ctx in ctxs:
        cache_bytes = 2 * nkv * ctx * D * 2
        n = max(4, -(-(1 << 30) // cache_bytes))
        ks = [torch.randn(nkv, ctx, D, device=dev, generator=gen).to(torch.bfloat16)
              for _ in range(n)]
        vs = [torch.randn(nkv, ctx, D, device=dev, generator=gen).to(torch.bfloat16)
              for _ in range(n)]
        q = torch.randn(nq, D, device=dev, generator=gen).to(torch.bfloat16)
        out = torch.empty_like(q)
        ws = moe.attn_workspace(nq, nkv, D, ctx, dev)
        calls = n * max(1, 40 // n)
        graphs = {}
        for packed in (True, False):
            def call(i, packed=packed):
                moe.moe_attn_decode(q, ks[i % n], vs[i % n], out=out, ws=ws, packed=packed)
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for i in range(3):
                    call(i)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(calls):
                    call(i)
            graphs[packed] = g
        warm_up(graphs[True].replay)
        us = {True: [], False: []}
        for _ in range(rounds):
            for packed, g in graphs.items():
                ev0.record()
                for _ in range(3):
                    g.replay()
                ev1.record()
                torch.cuda.synchronize()
                us[packed].append(ev0.elapsed_time(ev1) * 1e3 / (3 * calls))
        del graphs
        moe.profile_reset()
        moe.profile_enable(True)
        for i in range(2 * n):
            moe.moe_attn_decode(q, ks[i % n], vs[i % n], out=out, ws=ws)
        torch.cuda.synchronize()
        moe.profile_enable(False)
        kern = {}
        for name in ("k_attn_split", "k_attn_combine"):
            tot, cnt = moe.profile_query(name)
            kern[name] = round(1e3 * tot / max(cnt, 1), 2)
        moe.profile_reset()
        t_p, t_u = float(np.median(us[True])), float(np.median(us[False]))
        nbytes = cache_bytes + 2 * nq * D * 2
        split_gbs = cache_bytes / (kern["k_attn_split"] * 1e-6) / 1e9
        res[str(ctx)] = {"us_per_call": round(t_p, 2), "GB_s": round(nbytes / (t_p * 1e-6) / 1e9, 1),
                         "hbm_frac": round(nbytes / (t_p * 1e-6) / 1e9 / HBM_PEAK_GBS, 3),
                         "kernels_us": kern, "split_kernel_hbm_frac":
                         round(split_gbs / HBM_PEAK_GBS, 3), "cache_copies": n,
                         "unpacked_us_per_call": round(t_u, 2),
                         "packing_gain": round(t_u / t_p - 1, 3)}
        del ks, vs, ws
        torch.cuda.empty_cache()
    res["pages"] = {"gqa_packing_gain_e2e_32k": 0.238, "note": "whole-model decode, other hardware"}
    return res


GDN_TS = (2048, 8192)


def synth_gdn_dims():
    from routed_expert_amd import synth
    return synth.GDN_K_HEADS, synth.GDN_V_HEADS, synth.GDN_DK, synth.GDN_DV


def gdn_flops_per_token():
    """Algorithmic fp32 FLOP of the DeltaNet recurrence per token (all value heads): per
    state row two dot products with k and q (2 d_k each) and the update alpha S + c k
    (3 d_k), 7 d_k FLOP."""
    _, n_v, d_k, d_v = synth_gdn_dims()
    return 7 * d_k * d_v * n_v


def bench_gdn(moe, torch, synth, dev, Ts=GDN_TS, reps=10):
    """Gated DeltaNet prompt scan of one layer (16 key / 32 value heads of 128, fp32 state
    from zero). Time per call after a warm-up; FLOP/s against the fp32 vector peak; bytes
    per call for reference (q, k, v, gates in, o out, the state read and written once)."""
    res = {}
    n_k, n_v, d_k, d_v = synth_gdn_dims()
    for T in Ts:
        q, k, v, a, b = synth.gdn_inputs(T, seed=3)
        qd, kd, vd = (moe.bf16_from_bits(x, dev) for x in (q, k, v))
        ad, bd = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
        st = torch.zeros((n_v, d_v, d_k), dtype=torch.float32, device=dev)
        out = torch.empty((T, n_v, d_v), dtype=torch.bfloat16, device=dev)
        ws = moe.gdn_chunked_workspace(T, n_k, n_v, dev)
        fn = lambda: moe.moe_gdn_scan(qd, kd, vd, ad, bd, st, out=out)
        fc = lambda: moe.moe_gdn_scan_chunked(qd, kd, vd, ad, bd, st, out=out, ws=ws)
        warm_up(fn)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)

        def timed(f):
            e0.record()
            for _ in range(reps):
                f()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / reps

        us = timed(fn)
        us_chunked = timed(fc)
        flops = gdn_flops_per_token() * T
        nbytes = T * (2 * n_k * d_k * 2 + n_v * d_v * 2 * 2 + n_v * 8) + 2 * n_v * d_v * d_k * 4
        res[str(T)] = {"us_per_call": round(us, 1), "ns_per_token": round(us * 1e3 / T, 1),
                       "tflops": round(flops / (us * 1e-6) / 1e12, 2),
                       "alu_frac": round(flops / (us * 1e-6) / 1e12 / FP32_VECTOR_PEAK_TFLOPS, 3),
                       "bytes_per_call": nbytes, "chunked_us_per_call": round(us_chunked, 1)}
        del qd, kd, vd, ad, bd, st, out, ws
        torch.cuda.empty_cache()
    res["bound"] = "alu"
    res["peak_tflops"] = FP32_VECTOR_PEAK_TFLOPS
    return res


def bench_ablations(moe, torch, synth, dev, Ts=(512, 2048, 4096), rounds=5, calls=20):
    """moe_prefill_ablation on the uniform-routing layer: the product path and each
    rejected design, rounds alternating over the variants after a warm-up; median
    microseconds per call and the product's gain over each (t_variant / t_product - 1)."""
    import numpy as np
    dl = moe.DeviceLayer.from_host(synth.decode_layer(0), dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    res = {}
    for T in Ts:
        x = moe.bf16_from_bits(synth.prefill_x(T, seed=2), dev)
        y = torch.empty_like(x)
        ws = {n: moe.ablation_workspace(dl, T, v, dev) for n, v in moe.ABLATIONS.items()}
        fn = {n: (lambda n=n, v=v: moe.moe_prefill_ablation(dl, x, v, y=y, ws=ws[n]))
              for n, v in moe.ABLATIONS.items()}
        warm_up(fn["none"])
        us = {n: [] for n in fn}
        for _ in range(rounds):
            for n in fn:
                for _ in range(3):
                    fn[n]()
                ev0.record()
                for _ in range(calls):
                    fn[n]()
                ev1.record()
                torch.cuda.synchronize()
                us[n].append(ev0.elapsed_time(ev1) * 1e3 / calls)
        med = {n: float(np.median(v)) for n, v in us.items()}
        res[str(T)] = {"us_per_call": {n: round(v, 1) for n, v in med.items()},
                       "gain_over": {n: round(med[n] / med["none"] - 1, 3)
                                     for n in med if n != "none"}}
        del ws, fn
        torch.cuda.empty_cache()
    del dl
    torch.cuda.empty_cache()
    res["pages"] = PAGE_ABLATION_GAINS
    return res


def bench_small_t(moe, torch, synth, dev, Ts=(2, 4, 8), calls=40, reps=10):
    """moe_prefill with a few tokens (no routing output requested: the small-T kernels),
    graph replays over the 20 cache-cold layer copies. Bytes per call: the router, every
    expert in the union of the tokens' selections (read once) plus the shared expert, x, y;
    the union size comes from the GPU's own routing of the same tokens."""
    import numpy as np
    layers = gpu_copies(moe, torch, synth, dev)
    res = {}
    for T in Ts:
        x = moe.bf16_from_bits(synth.prefill_x(T, seed=3), dev)
        ws = moe.workspace(layers[0], T, dev)
        y = torch.empty_like(x)

        def call(i):
            moe.moe_prefill(layers[i % N_COPIES], x, y=y, ws=ws)

        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(3):
                call(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(calls):
                call(i)
        warm_up(g.replay)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1000 / (reps * calls)
        del g
        # union of the experts these tokens select (same layer copy 0 routing)
        buf = moe.route_buffers(layers[0], T, dev)
        moe.moe_route(layers[0], x, out=buf)
        torch.cuda.synchronize()
        n_union = len(np.unique(buf["topk_ids"].cpu().numpy()))
        nbytes = E * H * 4 + (n_union + S) * sum(expert_bytes()) + 2 * T * H * 2
        res[str(T)] = {"us_per_call": us, "tokens_per_s": T / (us * 1e-6),
                       "union_experts": n_union, "bytes_per_call": nbytes,
                       "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    return res


def bench_stack(moe, torch, synth, dev, eps=1e-6):
    """40 layers of the decode shape (18.3 GB of int4 weights, plus their tiled copies)
    resident in HBM, as pre-norm residual blocks: batch-1 decode of 256 tokens, and a
    32,768-token prompt in chunks of 4096 tokens reusing one workspace."""
    layers = [gpu_layer(moe, torch, synth, dev, 1000 + l) for l in range(STACK_LAYERS)]
    # decode: each token's output is the next token's input; 8 tokens per graph
    ws1 = moe.stack_workspace(layers, 1, dev)
    h = moe.bf16_from_bits(synth.decode_token(0), dev)
    per_graph = 8
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            moe.moe_stack_forward(layers, h, chunk_tokens=1, eps=eps, ws=ws1)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            moe.moe_stack_forward(layers, h, chunk_tokens=1, eps=eps, ws=ws1)
    g.replay()
    torch.cuda.synchronize()
    # median over the 32 replays of 8 tokens (256 tokens)
    dec_ms = timed_median(torch, g.replay, STACK_DECODE_TOKENS // per_graph) * \
        (STACK_DECODE_TOKENS // per_graph)
    del g, ws1
    # prefill: the same prompt each time, restored outside the timed region
    wsp = moe.stack_workspace(layers, STACK_CHUNK, dev)
    x0 = moe.bf16_from_bits(synth.bf16_activations(3, (STACK_PROMPT, H)), dev)
    hp = x0.clone()
    moe.moe_stack_forward(layers, hp, chunk_tokens=STACK_CHUNK, eps=eps, ws=wsp)
    import numpy as np
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(5):
        hp.copy_(x0)
        torch.cuda.synchronize()
        t0.record()
        moe.moe_stack_forward(layers, hp, chunk_tokens=STACK_CHUNK, eps=eps, ws=wsp)
        t1.record()
        torch.cuda.synchronize()
        times.append(t0.elapsed_time(t1))
    pre_ms = float(np.median(times))
    bpt = STACK_LAYERS * decode_bytes_per_token()
    us_tok = 1e3 * dec_ms / STACK_DECODE_TOKENS
    flops = STACK_LAYERS * prefill_flops_per_token() * STACK_PROMPT
    del layers, wsp, x0, hp
    torch.cuda.empty_cache()
    return {"layers": STACK_LAYERS, "decode_tokens": STACK_DECODE_TOKENS,
            "decode_tokens_per_s": 1e6 / us_tok, "decode_us_per_token": us_tok,
            "decode_hbm_frac": bpt / (us_tok * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "decode_timing": "median of 32 graph replays of 8 tokens",
            "prefill_prompt_tokens": STACK_PROMPT, "prefill_chunk": STACK_CHUNK,
            "prefill_ms_per_prompt": pre_ms, "prefill_timing": "median of 5 prompts",
            "prefill_tokens_per_s": STACK_PROMPT / (pre_ms * 1e-3),
            "prefill_mfma_frac": flops / (pre_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "weights": "seeded GPU draws of the decode-layer distributions, layer l seed 1000+l"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(synth, gpu_round=None, rounds=5, chunk=820):
    """The oracle (plain C, fp64, OpenMP over tokens on every host core this process may use)
    on bounded samples of the benchmarked workloads. The decode leg alternates with GPU rounds
    (one timed repetition of the decode benchmark each, when gpu_round is given), so both run
    under the same conditions, in the order the page uses for its comparisons."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    threads = len(os.sched_getaffinity(0))
    cpu = cpu_model()
    layer = synth.decode_layer(0)
    n = rounds * chunk
    xs = np.concatenate([synth.decode_token(t) for t in range(n)])
    olayer = oracle.OracleLayer(layer)
    cpu_s, gpu_ms = 0.0, []
    for r in range(rounds):
        if gpu_round is not None:
            gpu_ms.append(gpu_round())
        t0 = time.perf_counter()
        oracle.moe(olayer, xs[r * chunk:(r + 1) * chunk], nthreads=threads)
        cpu_s += time.perf_counter() - t0
    res = {"value": n / cpu_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{n} decode tokens (seeds 1000000..{1000000 + n - 1}) through layer "
                     f"copy 0, full layer per token, fp64, {cpu_s:.1f} s on {cpu}, in {rounds} "
                     f"rounds of {chunk} alternating with GPU rounds"}
    if gpu_ms:
        res["interleaved_gpu_round_ms"] = [round(v, 4) for v in gpu_ms]
    # the tiny fp32 layer on one thread
    tl, tx = synth.tiny_config(0)
    t0 = time.perf_counter()
    oracle.moe(tl, tx, nthreads=1)
    dt = time.perf_counter() - t0
    res["tiny_1thread"] = {"value": tx.shape[0] / dt, "unit": "tokens/s", "cores": 1,
                           "kind": "oracle", "sample": f"the T=64 fp32 layer (H=128, I=64), "
                                                       f"{dt * 1e3:.1f} ms"}
    # the 40-layer stack: 64 prompt tokens through 4 decode-shaped layers (seeds 0..3), each
    # layer's input normalised and rounded to bf16 as the stack defines it; scaled to 40 layers
    nl, nt = 4, 64
    h = oracle.to_f64(synth.bf16_activations(3, (nt, H)))
    st = 0.0
    for l in range(nl):
        ol = oracle.OracleLayer(synth.decode_layer(l))
        t0 = time.perf_counter()
        h = h + oracle.moe(ol, oracle.stack_layer_input(oracle.round_bf16(h)), nthreads=threads)
        st += time.perf_counter() - t0
        del ol
    res["stack_40"] = {"value": nt / (st / nl * STACK_LAYERS), "unit": "tokens/s", "cores": threads,
                       "kind": "oracle",
                       "sample": f"{nt} tokens through {nl} decode-shaped layers "
                                 f"({st:.1f} s), scaled to {STACK_LAYERS} layers"}
    # the oracle beside the other two workloads (bounded samples of their benchmark shapes)
    ctx = 32768
    q, k, v = synth.attn_inputs(ctx, seed=5)
    t0 = time.perf_counter()
    oracle.attn_decode(q, k, v, synth.ATTN_Q_HEADS, synth.ATTN_KV_HEADS, synth.ATTN_HEAD_DIM ** -0.5)
    dt_a = time.perf_counter() - t0
    res["attention_decode"] = {"value": 1.0 / dt_a, "unit": "calls/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"one decode token over {ctx} cached positions, 16 query "
                                         f"/ 2 KV heads of 256, fp64, {dt_a:.2f} s"}
    T = 2048
    gq, gk, gv, ga, gb = synth.gdn_inputs(T, seed=3)
    t0 = time.perf_counter()
    oracle.gdn_scan(gq, gk, gv, ga, gb, synth.GDN_K_HEADS, synth.GDN_V_HEADS, nthreads=threads)
    dt_g = time.perf_counter() - t0
    res["gdn_scan"] = {"value": T / dt_g, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                       "sample": f"one DeltaNet layer over a {T}-token prompt (32 value heads "
                                 f"of 128), fp64, {dt_g:.2f} s"}
    return res


COPY_BYTES = 256 << 20


def profile_run(moe, torch, synth, dev, what):
    """Fixed work for rocprofv3 (kernel trace or counters): a plain device copy of
    COPY_BYTES (the calibration for FETCH_SIZE / WRITE_SIZE), then a few calls of the
    named path. Prints nothing but a done line."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    if what == "decode":
        layers = [moe.DeviceLayer.from_host(synth.decode_layer(0), dev)] + \
                 [gpu_layer(moe, torch, synth, dev, c) for c in range(1, N_COPIES)]
        import numpy as np
        xs = moe.bf16_from_bits(np.concatenate([synth.decode_token(t) for t in range(64)]), dev)
        ws = moe.workspace(layers[0], 1, dev)
        y = torch.empty((1, H), dtype=torch.bfloat16, device=dev)
        for i in range(200):
            moe.moe_decode(layers[i % N_COPIES], xs[i % 64:i % 64 + 1], y=y, ws=ws)
    elif what == "attn_decode_32k":
        # decode attention over a 32,768-position cache, 16 rotating copies (cache-cold)
        nq, nkv, D, ctx = synth.ATTN_Q_HEADS, synth.ATTN_KV_HEADS, synth.ATTN_HEAD_DIM, 32768
        gen = torch.Generator(device=dev)
        gen.manual_seed(5)
        ks = [torch.randn(nkv, ctx, D, device=dev, generator=gen).to(torch.bfloat16)
              for _ in range(16)]
        vs = [torch.randn(nkv, ctx, D, device=dev, generator=gen).to(torch.bfloat16)
              for _ in range(16)]
        q = torch.randn(nq, D, device=dev, generator=gen).to(torch.bfloat16)
        ws = moe.attn_workspace(nq, nkv, D, ctx, dev)
        out = torch.empty_like(q)
        for i in range(400):
            moe.moe_attn_decode(q, ks[i % 16], vs[i % 16], out=out, ws=ws)
    elif what == "gdn_scan_2k":
        # one DeltaNet layer's scan of a 2,048-token prompt (32 value heads), 20 calls of the
        # token scan, then 20 of the chunked form
        q, k, v, a, b = synth.gdn_inputs(2048, seed=3)
        qd, kd, vd = (moe.bf16_from_bits(x, dev) for x in (q, k, v))
        ad, bd = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
        st = torch.zeros((synth.GDN_V_HEADS, synth.GDN_DV, synth.GDN_DK), dtype=torch.float32,
                         device=dev)
        ws = moe.gdn_chunked_workspace(2048, synth.GDN_K_HEADS, synth.GDN_V_HEADS, dev)
        for _ in range(20):
            moe.moe_gdn_scan(qd, kd, vd, ad, bd, st)
        for _ in range(20):
            moe.moe_gdn_scan_chunked(qd, kd, vd, ad, bd, st, ws=ws)
    elif what == "prefill_separate_dequant":
        # the separate-dequantisation ablation (expansion pass + GEMMs on fp16 weights)
        dl = moe.DeviceLayer.from_host(synth.decode_layer(0), dev)
        x = moe.bf16_from_bits(synth.prefill_x(4096, seed=2), dev)
        ws = moe.ablation_workspace(dl, 4096, moe.ABL_SEPARATE_DEQUANT, dev)
        y = torch.empty_like(x)
        for _ in range(60):
            moe.moe_prefill_ablation(dl, x, moe.ABL_SEPARATE_DEQUANT, y=y, ws=ws)
    else:
        layer = synth.skewed_layer(0) if what == "prefill_skewed" else synth.decode_layer(0)
        dl = moe.DeviceLayer.from_host(layer, dev)
        x = moe.bf16_from_bits(synth.prefill_x(4096, seed=2), dev)
        ws = moe.workspace(dl, 4096, dev)
        y = torch.empty_like(x)
        # 200 calls (about 75 ms): the averages are dominated by the steady clock, not by
        # the slower first tens of milliseconds after the GPU was idle
        for _ in range(200):
            moe.moe_prefill(dl, x, y=y, ws=ws)
    torch.cuda.synchronize()
    print(f"profile run done: {what}", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000,
                    help="decode tokens per timed repetition (20 repetitions, median)")
    ap.add_argument("--warmup", type=int, default=100, help="untimed decode tokens first")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--no-attention", action="store_true")
    ap.add_argument("--no-gdn", action="store_true")
    ap.add_argument("--profile", choices=["decode", "prefill_uniform", "prefill_skewed",
                                          "prefill_separate_dequant", "attn_decode_32k",
                                          "gdn_scan_2k"],
                    help="fixed work for rocprofv3 instead of the benchmark")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from routed_expert_amd import moe, synth
    dev = "cuda:0"
    moe.lib()
    if args.profile:
        profile_run(moe, torch, synth, dev, args.profile)
        return
    dec = bench_decode(moe, torch, synth, dev, args.steps, args.warmup)
    ms_step = dec["ms_rep_median"] / dec["steps"]
    tok_s = dec["steps"] / (dec["ms_rep_median"] * 1e-3)
    bpt = decode_bytes_per_token()

    # dominant kernel: the decode kernel with the longest average duration
    kname = max(dec["kernels"], key=lambda n: dec["kernels"][n]["avg_us"])
    kbytes = DECODE_KERNEL_BYTES[kname]
    k_us = dec["kernels"][kname]["avg_us"]
    achieved = kbytes / (k_us * 1e-6) / 1e9
    src = os.path.join(ROOT, "routed_expert_amd", "csrc", "decode_gemv.hip")
    ceil = dec["ceilings"]
    roofline = {"bound": "hbm", "kernel": kname, "achieved": achieved,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                "traffic": traffic_for(kname, src),
                "algorithmic_bytes_per_launch": kbytes, "avg_launch_us": k_us,
                "read_ceiling_GB_s": ceil[kname]["GB_s"],
                "frac_of_read_ceiling": ceil[kname]["avg_us"] / k_us}
    out = {
        "metric": "MoE-layer tokens/s: prefill T=4096 and decode T=1, % of MFMA/HBM roofline",
        "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": dec["steps"],
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "dtype_detail": "int4 weights rebuilt exactly as fp16 pairs, fp16 products accumulated "
                        "in fp32 (v_dot2_f32_f16 in decode, v_mfma_f32_32x32x16_f16 in "
                        "prefill); fp32 router; bf16 inputs and outputs",
        "data": "synthetic (seeded int4 g64 layer, 20 rotating cache-cold copies)",
        "config": {"workload": "moe_decode_T1", "hidden": H, "inter": I, "experts": E,
                   "top_k": K_TOP, "shared": S, "weights": "int4-g64", "copies": N_COPIES,
                   "parallelism": "single-gpu"},
        "timing": f"median of {dec['reps']} repetitions of {dec['steps']} tokens replayed from "
                  f"HIP graphs (at most 100 tokens per graph), events on the replay stream",
        "roofline": roofline,
        "layer_roofline": {"bound": "hbm", "bytes_per_token": bpt,
                           "achieved": bpt / (ms_step * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": bpt / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "decode_eager_tokens_per_s": dec["eager_tok_s"],
        "decode_kernels": {k: {"avg_us": round(v["avg_us"], 3),
                               "GB_s": round(DECODE_KERNEL_BYTES[k] / (v["avg_us"] * 1e3), 1),
                               "hbm_frac": round(DECODE_KERNEL_BYTES[k] / (v["avg_us"] * 1e3) /
                                                 HBM_PEAK_GBS, 3),
                               "frac_of_read_ceiling": round(ceil[k]["avg_us"] / v["avg_us"], 3)}
                           for k, v in dec["kernels"].items()},
        "decode_read_ceilings": ceil,
        "graph_launch_floor": bench_launch_floor(torch, dev),
    }
    if not args.no_prefill:
        mc = bench_mfma_ceiling(moe, torch, dev)
        out["mfma_ceiling"] = mc
        for key, lay in (("prefill_uniform", synth.decode_layer(0)),
                         ("prefill_skewed", synth.skewed_layer(0))):
            pr = bench_prefill(moe, torch, synth, dev, lay)
            pr["mfma_frac_of_ceiling"] = pr["tflops"] / mc["tflops"]
            out[key] = pr
    if not args.no_stack:
        out["stack_40"] = bench_stack(moe, torch, synth, dev)
    if not args.no_prefill:
        out["small_T"] = bench_small_t(moe, torch, synth, dev)
        out["ablations"] = bench_ablations(moe, torch, synth, dev)
    if not args.no_attention:
        out["attention_decode"] = bench_attention(moe, torch, synth, dev)
    if not args.no_gdn:
        out["gdn_scan"] = bench_gdn(moe, torch, synth, dev)
    if not args.no_cpu:
        cb = cpu_baseline(synth, dec["gpu_round"])
        if "interleaved_gpu_round_ms" in cb:
            import numpy as np
            cb["interleaved_gpu_tokens_per_s"] = dec["steps"] / (
                float(np.median(cb["interleaved_gpu_round_ms"])) * 1e-3)
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
