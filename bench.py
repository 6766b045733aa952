"""Benchmark one tensor-parallel rank's decoder-layer shard on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode] [--no-ffn]

A step is one pass of the whole path for rank 0 of a TP=2 prefill layer
(4096 tokens, hidden 8192, 64 q / 8 KV heads, head_dim 128, intermediate
28672): RMSNorm, fused QKV column-parallel GEMM, causal local attention,
o_proj row-parallel partial, sum of both ranks' partials + residual with the
MLP's RMSNorm in the same pass, gate|up column-parallel GEMM with SwiGLU in its
epilogue, down row-parallel partial, sum of partials + residual.  Rank 1's partials (what the all-reduce would deliver)
are computed once before timing.  Inputs are seeded synthetic tensors already
resident in HBM.  Prints ONE JSON line.

Secondary figures (same line, key "decode"): the decode MLP shard at TP=8
(M = 1, 8, 64), the decode attention shard at TP=4 (contiguous and paged
cache), the same attention at TP=16 with replicated KV heads and the vocab-parallel lm_head shard with its
greedy argmax (TP=8), timed over rotating
copies of the weights/caches so that the 256 MB Infinity Cache cannot hold
the working set between steps (also as HIP-graph replays, "graph_ms", and with the
copies as consecutive layers of one graph, "graph_layers_ms"), with the
HBM bytes the same steps moved by the FETCH_SIZE/WRITE_SIZE counters
(profiles/decode_traffic.md) and their rate relative to the attainable read
rate of a plain read-only stream ("hbm_read_ceiling").
Key "ffn_tp8": rank 0's shard of the GELU FFN at TP=8 (2048 tokens, hidden
12288): fc1 with GELU in its epilogue, fc2, and the sum of 8 partials.
"""
from __future__ import annotations

import argparse
import itertools
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import tensor_transformer_layer_05_amd as tpl  # noqa: E402
from tensor_transformer_layer_05_amd import inputs as I  # noqa: E402
from tensor_transformer_layer_05_amd.shard import LayerShard  # noqa: E402

METRIC = "TFLOP/s + HBM GB/s per TP-rank layer shard (decode M=1..64, prefill M=4096)"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0
DEV = "cuda:0"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def traffic_source_hash(files):
    """SHA-256 (first 16 hex digits) over the kernel's source files, in order."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def profile_data(name):
    """The DATA line of a committed rocprofv3 summary (a JSON object), or None
    if the summary or its DATA line is missing."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        line = [l for l in open(path) if l.startswith("DATA ")][0]
        return json.loads(line[5:])
    except (OSError, IndexError, ValueError):
        return None


def recorded_profile(name):
    """The DATA line of a committed rocprofv3 summary of the dominant kernel
    (HBM traffic from FETCH_SIZE/WRITE_SIZE scaled by a plain copy of known
    size; MFMA and LDS counters), or None once the kernel's sources no longer
    match the hash recorded with the counters."""
    data = profile_data(name)
    try:
        if data is None or traffic_source_hash(data["sources"]) != data["sources_sha256_16"]:
            return None
    except (OSError, KeyError, TypeError):
        return None
    return data


# ---------------------------------------------------------------------------
# prefill layer shard (rank 0 of TP=2)
# ---------------------------------------------------------------------------

def prefill_setup():
    c = I.config("prefill_layer_tp2")
    H, R, D, S = c.hidden, c.tp, c.head_dim, c.tokens[0]
    hq, hkv, il = c.n_q // R, c.n_kv // R, c.inter // R
    seed = c.seed
    t0 = time.time()

    def rank_weights(r):
        wq = I.normal(seed, "wq", (hq * D, H), c.w_std, rank=r)
        wk = I.normal(seed, "wk", (hkv * D, H), c.w_std, rank=r)
        wv = I.normal(seed, "wv", (hkv * D, H), c.w_std, rank=r)
        wo = I.normal(seed, "wo", (H, hq * D), c.w_std, rank=r)
        wg = I.normal(seed, "wg", (il, H), c.w_std, rank=r)
        wu = I.normal(seed, "wu", (il, H), c.w_std, rank=r)
        wd = I.normal(seed, "wd", (H, il), c.w_std, rank=r)
        return dict(wq=wq, wk=wk, wv=wv, wo=wo, wg=wg, wu=wu, wd=wd)

    x = I.normal(seed, "x", (S, H), c.x_std)
    g1 = torch.ones(H, dtype=torch.bfloat16)
    g2 = torch.ones(H, dtype=torch.bfloat16)
    shards, host = [], []
    for r in range(R):
        w = rank_weights(r)
        host.append(w)
        wqkv = torch.cat([w["wq"].dev, w["wk"].dev, w["wv"].dev], 0).to(DEV)
        wgu = torch.cat([w["wg"].dev, w["wu"].dev], 0).to(DEV)
        shards.append(LayerShard(g1.to(DEV), g2.to(DEV), wqkv, w["wo"].dev.to(DEV), wgu,
                                 w["wd"].dev.to(DEV), hq, hkv, D, c.eps, S))
    log(f"prefill inputs generated in {time.time() - t0:.1f}s")
    X = x.dev.to(DEV)
    pa = [torch.empty((S, H), dtype=torch.float32, device=DEV) for _ in range(R)]
    pm = [torch.empty((S, H), dtype=torch.float32, device=DEV) for _ in range(R)]
    # every rank's partials once (rank 1's stay as the all-reduce contribution)
    for r in range(R):
        shards[r].attn_partial(X, pa[r])
    h = tpl.reduce_partials(pa, residual=X, out_dtype=torch.float32)   # float32 residual stream
    for r in range(R):
        shards[r].mlp_partial(h, pm[r])
    y = torch.empty((S, H), dtype=torch.bfloat16, device=DEV)
    torch.cuda.synchronize()
    return dict(c=c, x=x, X=X, shards=shards, host=host, pa=pa, pm=pm, y=y, g1=g1, g2=g2)


def prefill_counts(c):
    H, R, D, S = c.hidden, c.tp, c.head_dim, c.tokens[0]
    hq, hkv, il = c.n_q // R, c.n_kv // R, c.inter // R
    nqkv = (hq + 2 * hkv) * D
    gemm = {  # name: (M, K, N)
        "qkv": (S, H, nqkv), "o_proj": (S, hq * D, H), "gate_up_swiglu": (S, H, 2 * il),
        "down": (S, il, H)}
    flops = {k: 2.0 * m * kk * n for k, (m, kk, n) in gemm.items()}
    flops["attention"] = 4.0 * D * (S * (S + 1) / 2) * hq
    # algorithmic HBM bytes per call: each operand read once, each result written once
    b2, b4 = 2, 4
    byts = {
        "rmsnorm1": S * H * b2 * 2 + H * b2,
        "qkv": (S * H + nqkv * H + S * nqkv) * b2,
        "attention": S * nqkv * b2 + S * hq * D * b2,
        "o_proj": (S * hq * D + H * hq * D) * b2 + S * H * b4,
        # partials + bf16 residual x read, float32 h and bf16 RMSNorm(h) written
        "reduce1_rmsnorm2": R * S * H * b4 + S * H * b2 + S * H * b4 + S * H * b2 + H * b2,
        # activation in the epilogue: only h = act(g) * u ([S, il]) is written
        "gate_up_swiglu": (S * H + 2 * il * H + S * il) * b2,
        "down": (S * il + H * il) * b2 + S * H * b4,
        # partials + float32 h read, bf16 y written
        "reduce2": R * S * H * b4 + S * H * b4 + S * H * b2,
    }
    return gemm, flops, byts


def prefill_step(st, ev=None, only=None):
    """Rank 0's step; ``ev`` (dict name -> list of (start, end) events) times
    each call, or only the call named ``only``."""
    sh, X, pa, pm, y = st["shards"][0], st["X"], st["pa"], st["pm"], st["y"]
    S = X.shape[0]

    def run(name, fn):
        if ev is None or (only is not None and name != only):
            fn()
            return
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        ev.setdefault(name, []).append((e0, e1))

    at, ml = sh.attn, sh.mlp
    xn, h, hn = sh.xn[:S], sh.h[:S], sh.hn[:S]
    qkv, o = at.qkv[:S], at.o[:S]
    q, k, v = at._views(qkv, 1, S)
    a = ml.a[:S]
    run("rmsnorm1", lambda: tpl.rmsnorm(X, sh.g1, sh.eps, out=xn))
    run("qkv", lambda: tpl.column_linear(xn, at.wqkv, out=qkv))
    run("attention", lambda: tpl.local_attention(q, k, v, causal=True,
                                                 out=o.view(1, S, at.n_q, at.D)))
    run("o_proj", lambda: tpl.row_linear_partial(o, at.wo, out=pa[0]))
    run("reduce1_rmsnorm2", lambda: tpl.reduce_partials_rmsnorm(pa, sh.g2, residual=X, eps=sh.eps,
                                                                out=h, out_norm=hn))
    run("gate_up_swiglu", lambda: tpl.column_linear_act(hn, ml.w_in, "swiglu", out=a))
    run("down", lambda: tpl.row_linear_partial(a, ml.w_out, out=pm[0]))
    run("reduce2", lambda: tpl.reduce_partials(pm, residual=h, out=y))


def time_prefill(st, steps, warmup, dominant):
    """Times ``steps`` steps with events around the ``dominant`` call only (an
    event pair around every call adds about 50 us to a 3 ms step), then the
    same number of steps with events around every call for the per-call
    breakdown.  Returns (ms per step, per-call ms, wall seconds of the timed
    steps, ms per step of the breakdown pass)."""
    for _ in range(warmup):
        prefill_step(st)
    torch.cuda.synchronize()
    ev = {}
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t0.record()
    for _ in range(steps):
        prefill_step(st, ev, only=dominant)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = t0.elapsed_time(t1)
    dom = float(np.mean([a.elapsed_time(b) for a, b in ev[dominant]]))
    ev_all = {}
    t0.record()
    for _ in range(steps):
        prefill_step(st, ev_all)
    t1.record()
    torch.cuda.synchronize()
    per = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev_all.items()}
    per[dominant] = dom
    return total_ms / steps, per, wall, t0.elapsed_time(t1) / steps


# ---------------------------------------------------------------------------
# oracle timing on a bounded sample (rank 0's step on a prefix of the sequence)
# ---------------------------------------------------------------------------

def cpu_baseline(st, target_s=15.0):
    import oracle.tp_oracle as O
    try:
        from threadpoolctl import threadpool_info
    except Exception:  # pragma: no cover
        threadpool_info = lambda: []
    c = st["c"]
    w = st["host"][0]
    H, D, eps = c.hidden, c.head_dim, c.eps
    x = st["x"].ref
    g1 = np.ones(H)
    g2 = np.ones(H)
    other_a = np.zeros((1, H))
    other_m = np.zeros((1, H))

    def run(Sp):
        xs = x[:Sp]
        xn = O.rmsnorm(xs, g1, eps)
        pa = O.attention_rank_partial(xn, w["wq"].ref, w["wk"].ref, w["wv"].ref, w["wo"].ref, D, 0, 1)
        h = O.reduce_partials([pa, np.broadcast_to(other_a, pa.shape)], residual=xs)
        hn = O.rmsnorm(h, g2, eps)
        pm = O.mlp_rank_partial(hn, w["wg"].ref, w["wd"].ref, "swiglu", 0, 1, w_up=w["wu"].ref)
        return O.reduce_partials([pm, np.broadcast_to(other_m, pm.shape)], residual=h)

    def flops(Sp):
        R, hq = c.tp, c.n_q // c.tp
        per_tok = 2.0 * ((hq + 2 * c.n_kv // R) * D * H + hq * D * H + 2 * (c.inter // R) * H
                         + (c.inter // R) * H)
        return per_tok * Sp + 4.0 * D * (Sp * (Sp + 1) / 2) * hq

    # The whole 4096-token step if one run fits the budget (repeated to ~10 s),
    # else the longest 32-multiple prefix estimated to take ~target_s.
    S = c.tokens[0]
    t = time.perf_counter(); run(256); dt256 = time.perf_counter() - t
    est_full = dt256 * flops(S) / flops(256)
    if est_full <= 2.0 * target_s:
        Sp, reps, total = S, 0, 0.0
        while total < 10.0 and reps < 8:
            t = time.perf_counter(); run(Sp); total += time.perf_counter() - t
            reps += 1
        what = f"the full rank-0 layer-shard step (4096 tokens), run {reps}x"
    else:
        Sp = int(256 * (target_s / max(dt256, 1e-3)))
        Sp = max(256, min(S, (Sp // 32) * 32))
        t = time.perf_counter(); run(Sp); total = time.perf_counter() - t
        reps = 1
        what = f"rank-0 layer-shard step on the first {Sp} of {S} tokens"
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    return {"value": flops(Sp) * reps / total / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{what} (float64 numpy oracle, {total:.1f}s, {os.cpu_count()} host CPUs visible)",
            "seconds": total}


# ---------------------------------------------------------------------------
# decode figures (secondary)
# ---------------------------------------------------------------------------

def _warm(fn, calls, min_ms=100.0):
    """At least ``calls`` calls and at least ``min_ms`` of back-to-back work:
    after an idle gap (input generation on the host) the GPU takes some tens
    of milliseconds of load to reach its steady clock, during which a 0.3 ms
    GEMM measured 15% slower."""
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(max(calls, 1)):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= min_ms:
            return


def _median_ms(fn, steps, warmup):
    _warm(fn, warmup)
    ts = []
    for i in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn(i)
        e1.record()
        ts.append((e0, e1))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ts]))


def _graph_ms(steps_fns, steps, warmup):
    """Capture each closure of ``steps_fns`` (one per rotating copy) into a HIP
    graph and return the median time of one replay (replays rotate over the
    copies).  Decode steps are launch-bound when issued call by call from the
    host; replaying a captured graph is how a serving loop issues them."""
    for f in steps_fns:          # eager warm-up: allocations happen here, not in capture
        f()
    torch.cuda.synchronize()
    graphs = []
    for f in steps_fns:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            f()
        graphs.append(g)
    torch.cuda.synchronize()
    n = len(graphs)
    return _median_ms(lambda i: graphs[i % n].replay(), steps, warmup)


def _graph_layers_ms(steps_fns, steps, warmup):
    """All closures of ``steps_fns`` captured in order in ONE graph, as a
    serving loop captures a whole decode step (every layer, each with its own
    weights and cache: here the rotating copies); the median replay time
    divided by the number of closures.  The replay's own launch cost is then
    shared by the layers, as it is in such a loop."""
    for f in steps_fns:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in steps_fns:
            f()
    torch.cuda.synchronize()
    return _median_ms(lambda i: g.replay(), steps, warmup) / len(steps_fns)


def _decode_entry(ms_eager, ms_graph, ms_layers, byts, fl):
    """Figures of one decode shard: the three issue modes, and the rates of the
    fastest (a serving loop would use whichever is fastest)."""
    modes = {"eager": ms_eager, "graph": ms_graph, "graph_layers": ms_layers}
    issue = min(modes, key=modes.get)
    ms = modes[issue]
    return {"ms": ms, "issue": issue, "eager_ms": ms_eager, "graph_ms": ms_graph,
            "graph_layers_ms": ms_layers,
            "GB/s": byts / ms / 1e6, "TFLOP/s": fl / ms / 1e9, "hbm_frac": byts / ms / 1e6 / PEAK_HBM_GBPS}


# the kernels (and their dispatch) a decode shard runs: the counter summary
# of their HBM bytes is used only while these sources still hash as recorded
DECODE_SRCS = ["tensor_transformer_layer_05_amd/csrc/gemm_stream.hip",
               "tensor_transformer_layer_05_amd/csrc/gemm_stream_dma.hip",
               "tensor_transformer_layer_05_amd/csrc/gemv_dot.hip",
               "tensor_transformer_layer_05_amd/csrc/attention_decode.hip",
               "tensor_transformer_layer_05_amd/csrc/argmax.hip",
               "tensor_transformer_layer_05_amd/csrc/tplayer_api.hip",
               "tensor_transformer_layer_05_amd/csrc/common.h"]


def read_ceiling(steps=10, warmup=3, nbytes=1 << 30):
    """Attainable HBM read rate on this GPU: the hand-written read-only
    stream of libtpref (16-byte loads per lane, chunks of 4-16 KB per wave with
    the next chunk in flight, like the decode weight streams) over 1 GiB, for
    several grid shapes, with and without non-temporal loads and with a slice
    per wave or chunks interleaved over all waves; the best median rate is the
    ceiling the decode shards are also compared with."""
    from tensor_transformer_layer_05_amd import ref
    buf = torch.ones(nbytes, dtype=torch.uint8, device=DEV)
    out = torch.empty(4096 * 16 * 64, dtype=torch.int32, device=DEV)
    best, rows = None, []
    for (wg, waves, u), fl in itertools.product(
            ((256, 8, 8), (512, 8, 8), (1024, 8, 4), (256, 16, 8), (512, 16, 4), (256, 8, 16),
             (2048, 4, 4)), (0, ref.NONTEMPORAL, ref.SPREAD, ref.NONTEMPORAL | ref.SPREAD)):
        ms = _median_ms(lambda i: ref.stream_read(buf, out, wg, waves, u, fl), steps, warmup)
        gbs = nbytes / ms / 1e6
        rows.append({"workgroups": wg, "waves": waves, "loads_per_lane": u,
                     "nontemporal": bool(fl & ref.NONTEMPORAL), "spread": bool(fl & ref.SPREAD),
                     "GB/s": round(gbs, 1)})
        if best is None or gbs > best["GB/s"]:
            best = rows[-1]
    del buf
    return {"GB/s": best["GB/s"], "frac_of_peak": best["GB/s"] / PEAK_HBM_GBPS, "best": best,
            "configs": rows, "bytes": nbytes}


def stream_ms(nbytes, steps=30, warmup=5):
    """The same read-only stream as ``read_ceiling``, over ``nbytes`` per call
    (enough rotating buffers that the Infinity Cache cannot hold them), issued
    and timed like a decode step: the fastest of four grid shapes.  A decode
    shard moves at least its algorithmic bytes, so this is the time a single
    plain read of that many bytes takes here, fixed launch and first-load
    latency included (the fastest of the stream's load options too)."""
    from tensor_transformer_layer_05_amd import ref
    n = max(4096, int(nbytes) // 4096 * 4096)
    copies = max(2, int(600e6 // n) + 1)
    bufs = [torch.ones(n, dtype=torch.uint8, device=DEV) for _ in range(copies)]
    out = torch.empty(4096 * 16 * 64, dtype=torch.int32, device=DEV)
    best = None
    for (wg, waves, u), fl in itertools.product(
            ((256, 8, 8), (512, 8, 8), (1024, 8, 4), (256, 16, 8)),
            (0, ref.NONTEMPORAL, ref.SPREAD, ref.NONTEMPORAL | ref.SPREAD)):
        ms = _median_ms(lambda i: ref.stream_read(bufs[i % copies], out, wg, waves, u, fl), steps,
                        warmup)
        best = ms if best is None else min(best, ms)
    del bufs
    return best


def decode_figures(steps=30, warmup=5, copies=4, ceiling=None):
    """Decode shards timed over ``copies`` rotating copies of the weights and
    caches (together larger than the 256 MB Infinity Cache).  ``eager_ms`` is
    the step issued call by call, ``graph_ms`` the same step replayed from a
    captured HIP graph, ``graph_layers_ms`` the copies captured one after the
    other in one graph (like the layers of a decode step), per copy; ``ms`` and
    the rates use the fastest of the three.
    ``hbm_frac`` is algorithmic bytes over time; ``counter_hbm_frac`` the HBM
    bytes the same step moved by the FETCH_SIZE/WRITE_SIZE counters (profiles/
    decode_traffic.md, while the decode kernels' sources match) over time;
    ``frac_of_read_ceiling`` algorithmic bytes over time relative to the
    attainable read rate measured by ``read_ceiling``; ``size_stream_ms`` the
    time of one plain read of the shard's algorithmic bytes (``stream_ms``) and
    ``frac_of_size_stream`` that time over the shard's."""
    from tensor_transformer_layer_05_amd.decode_workloads import all_decode
    counted = recorded_profile("decode_traffic.md")
    out = {}
    for build in all_decode(copies):
        w = build()
        n, name, byts = len(w.steps), w.name, w.bytes
        gms = _graph_ms(w.steps, steps, warmup)
        lms = _graph_layers_ms(w.steps, steps, warmup)
        ms = _median_ms(lambda i: w.steps[i % n](), steps, warmup)
        e = _decode_entry(ms, gms, lms, w.bytes, w.flops)
        e.update(w.extra)
        if counted and w.name in counted.get("shards", {}):
            cb = counted["shards"][w.name]["bytes"]
            e["counter_bytes"] = cb
            e["counter_hbm_frac"] = cb / e["ms"] / 1e6 / PEAK_HBM_GBPS
        else:
            e["counter_bytes"] = e["counter_hbm_frac"] = None
        if ceiling:
            e["frac_of_read_ceiling"] = e["GB/s"] / ceiling["GB/s"]
        del w
        e["size_stream_ms"] = stream_ms(byts, steps, warmup)
        e["frac_of_size_stream"] = e["size_stream_ms"] / e["ms"]
        out[name] = e
    return out


def ffn_figures(steps=20, warmup=3):
    """Rank 0's shard of the GELU FFN at TP 8 (hidden 12288, 4x expansion,
    2048 tokens): fc1 with GELU in its epilogue, fc2 to an fp32 partial, and the
    8-rank sum of partials.  The eight partial buffers all sit on this GPU,
    standing in for the peers' buffers of the in-HBM reduction."""
    c = I.config("gelu_mlp_tp8")
    M, H, F, R = c.tokens[0], c.hidden, c.inter, c.tp
    fl_ = F // R
    x = I.normal(c.seed, "x", (M, H), c.x_std).dev.to(DEV)
    w1 = I.normal(c.seed, "w1", (fl_, H), c.w_std, rank=0).dev.to(DEV)
    w2 = I.normal(c.seed, "w2", (H, fl_), c.w_std, rank=0).dev.to(DEV)
    a = torch.empty((M, fl_), dtype=torch.bfloat16, device=DEV)
    parts = [torch.empty((M, H), dtype=torch.float32, device=DEV) for _ in range(R)]
    y = torch.empty((M, H), dtype=torch.bfloat16, device=DEV)
    tpl.column_linear_act(x, w1, "gelu", out=a)
    for p_ in parts:
        tpl.row_linear_partial(a, w2, out=p_)
    ms1 = _median_ms(lambda i: tpl.column_linear_act(x, w1, "gelu", out=a), steps, warmup)
    ms2 = _median_ms(lambda i: tpl.row_linear_partial(a, w2, out=parts[0]), steps, warmup)
    msr = _median_ms(lambda i: tpl.reduce_partials(parts, out=y), steps, warmup)
    f1 = 2.0 * M * H * fl_
    rb = R * M * H * 4 + M * H * 2
    out = {
        "workload": f"gelu_mlp_tp8 rank 0: fc1 [{M},{H}]x[{H},{fl_}] + GELU, fc2 [{M},{fl_}]x[{fl_},{H}] "
                    f"-> fp32, sum of {R} partials -> bf16",
        "fc1_gelu": {"ms": ms1, "TFLOP/s": f1 / ms1 / 1e9, "mfma_frac": f1 / ms1 / 1e9 / PEAK_BF16_TFLOPS},
        "fc2": {"ms": ms2, "TFLOP/s": f1 / ms2 / 1e9, "mfma_frac": f1 / ms2 / 1e9 / PEAK_BF16_TFLOPS},
        "reduce8": {"ms": msr, "GB/s": rb / msr / 1e6, "hbm_frac": rb / msr / 1e6 / PEAK_HBM_GBPS},
    }
    del parts
    return out


# ---------------------------------------------------------------------------

def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-ffn", action="store_true")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}); the multi-GPU all-reduce is "
              "emulated in HBM on one device and runs at N=1.", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 2
    tpl.lib()
    st = prefill_setup()
    gemm, flops, byts = prefill_counts(st["c"])
    log("timing prefill layer shard")
    DK = "gate_up_swiglu"
    ms, per, wall, ms_all_events = time_prefill(st, a.steps, a.warmup, DK)
    tot_flops = sum(flops.values())
    tot_bytes = sum(byts.values())
    m, k, n = gemm[DK]
    dom_ms = per[DK]
    tr = recorded_profile("gate_up_gemm_traffic.md")
    cn = recorded_profile("gate_up_gemm_counters.md")
    dom = {"bound": "mfma",
           "kernel": "column_linear_act gate|up + SwiGLU (gemm_bf16_dma_kernel, 256x256 tiles, "
                     "SwiGLU epilogue)",
           "achieved": flops[DK] / dom_ms / 1e9, "peak": PEAK_BF16_TFLOPS,
           "unit": "TFLOP/s", "frac": flops[DK] / dom_ms / 1e9 / PEAK_BF16_TFLOPS,
           "traffic": tr["traffic_bytes"] if tr else None,
           "traffic_unit": "HBM bytes per launch (profiles/gate_up_gemm_traffic.md)",
           "algorithmic_bytes": byts[DK],
           "counters": ({k: cn[k] for k in ("mfma_util", "sclk_ghz", "lds_idx_active")}
                        | {"source": "profiles/gate_up_gemm_counters.md"}) if cn else None,
           "flop_per_launch": flops[DK], "avg_launch_ms": dom_ms,
           "shape_mkn": [m, k, n]}
    kernels = {}
    for name, t in per.items():
        d = {"ms": round(t, 4)}
        if name in flops:
            d["TFLOP/s"] = round(flops[name] / t / 1e9, 1)
        d["GB/s"] = round(byts[name] / t / 1e6, 1)
        kernels[name] = d
    res = {
        "metric": METRIC, "value": round(tot_flops / ms / 1e9, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) bf16 weights, N(0,1) activations)",
        "config": {"workload": "prefill_layer_tp2 (rank 0 of TP=2: 4096 tokens, hidden 8192, "
                               "32/4 local q/KV heads x 128, local intermediate 14336, SwiGLU, "
                               "RMSNorm pre-norm, 2-rank partial sums in HBM)",
                   "tokens": 4096, "hidden": 8192, "tp": 2, "rank": 0},
        "hbm_gbps": round(tot_bytes / ms / 1e6, 1),
        "flop_per_step": tot_flops, "bytes_per_step": tot_bytes,
        "roofline": dom, "kernels": kernels,
        "kernels_note": "per-call event times from a second pass of the same number of steps "
                        "with an event pair around every call (that pass: "
                        f"{ms_all_events:.4f} ms per step); the dominant call's time is from "
                        "the timed steps, which carry events around that call only",
    }
    if not a.no_decode:
        log("measuring the attainable HBM read rate (reference stream)")
        ceil_ = read_ceiling()
        res["hbm_read_ceiling"] = ceil_
        log("timing decode shards")
        res["decode"] = decode_figures(ceiling=ceil_)
    if not a.no_ffn:
        log("timing the GELU FFN shard at TP=8")
        res["ffn_tp8"] = ffn_figures()
    if not a.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(st)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
