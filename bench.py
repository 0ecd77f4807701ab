#!/usr/bin/env python3
"""Benchmark of the MI355X hybrid-attention hot path (one GPU).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--secondary a,b,...]

Prints ONE JSON line. `value` is the throughput of the headline workload in
algorithmic TFLOP/s: FLOPs of allowed (query, key) pairs only,
B*Hq*pairs(T,W)*2*(Dk+Dv) per layer. The default headline is the largest
single-GPU workload, the 7-layer stack (B=2, T=16384): 5 sliding-window local
layers (W=1024, 16q/8kv, D=256, RoPE theta=1e4), one global layer (32q/4kv,
Dk=512, Dv=256, p-RoPE on 128 of 512 dims, theta=1e6) and one global layer
that reuses the previous layer's K/V. A step is one pass of the whole path
over that batch: seven attn_prefill calls on one stream, each turning K's
rotary dims once (a pre-pass) and running the flash kernel, which forms the
rotation angles of Q itself from pos0.

Timing: HIP events recorded on the stream the kernels run on; W untimed
warm-up steps, then exactly K timed steps between two device
synchronisations; `ms_per_step` is the median step. The roofline entry is
for the dominant kernel (the global layers' flash kernel, ~91 % of the
FLOPs): its algorithmic FLOPs per launch over the mean duration of the
global-layer calls inside the timed steps. `traffic` comes from committed
rocprofv3 FETCH_SIZE / WRITE_SIZE summaries, and is null once the kernel's
source has changed since they were taken.

Secondary workloads (local prefill, global prefill, the small fp32 call,
batched decode, the small models' 4:1 stack) are measured in the same run,
each with its own roofline. The CPU baseline is the fp64 oracle timed on a
seeded row subset of every layer of the headline stack on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published dense peaks (AMD specification, no sparsity).
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
MIN_TIMED_MS = 200.0


def pairs(T: int, W: int) -> int:
    """Allowed (query, key) pairs of one (batch, head): sum_i min(i+1, W)."""
    if W <= 0 or W >= T:
        return T * (T + 1) // 2
    return W * (W + 1) // 2 + (T - W) * W


def prefill_flops(c) -> float:
    return float(c.B * c.Hq * pairs(c.T, c.window) * 2 * (c.Dk + c.Dv))


def prefill_bytes(c) -> float:
    es = 2 if str(c.dtype).endswith("bfloat16") else 4
    return float(c.B * c.T * es * (c.Hq * c.Dk + c.Hkv * c.Dk + c.Hkv * c.Dv + c.Hq * c.Dv))


def rows_flops(c, rows) -> float:
    """Algorithmic FLOPs of a subset of query rows (all batches and heads)."""
    W = c.window if 0 < c.window < c.T else c.T
    return float(sum(min(int(i) + 1, W) for i in rows) * c.B * c.Hq * 2 * (c.Dk + c.Dv))


def _digest(paths):
    """sha256[:16] over the given source files, in order."""
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel sources (else None)."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    srcs = rec.get("sources") or [rec.get("source", "")]
    if not all(os.path.exists(os.path.join(ROOT, s)) for s in srcs):
        return None
    if _digest(srcs) != rec.get("sources_sha256_16", rec.get("source_sha256_16")):
        return None
    return rec.get("bytes_per_launch")


class Events:
    """n_marks events per iteration on the current stream."""

    def __init__(self, torch, iters, n_marks):
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_marks)]
                   for _ in range(iters)]

    def mark(self, i, j):
        self.ev[i][j].record()

    def ms(self, i, a, b):
        return self.ev[i][a].elapsed_time(self.ev[i][b])

    def series(self, a, b):
        return [self.ms(i, a, b) for i in range(len(self.ev))]


def timed(torch, body, iters, warmup, n_marks):
    """Run body(ev, i) for `warmup` untimed and `iters` timed iterations
    (ev None while warming up), with a device synchronisation on both sides
    of the timed ones. Returns (events, wall seconds of the timed ones)."""
    for _ in range(warmup):
        body(None, 0)
    torch.cuda.synchronize()
    ev = Events(torch, iters, n_marks)
    t0 = time.perf_counter()
    for i in range(iters):
        body(ev, i)
    torch.cuda.synchronize()
    return ev, time.perf_counter() - t0


def iters_for(torch, body, n_marks, min_iters=10, min_ms=MIN_TIMED_MS, cap=5000):
    """Timed iterations needed to span >= min_ms (from a short probe)."""
    ev, _ = timed(torch, body, 3, 1, n_marks)
    per = max(statistics.median(ev.series(0, n_marks - 1)), 1e-3)
    return int(min(cap, max(min_iters, -(-min_ms // per) + 1)))


def stats(xs):
    return {"median": statistics.median(xs), "mean": sum(xs) / len(xs), "min": min(xs),
            "max": max(xs)}


def roofline(bound, achieved, peak, unit, traffic):
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


# ---------------------------------------------------------------------------
# Prefill workloads
# ---------------------------------------------------------------------------
def prefill_ws(ar, torch, cases):
    """One workspace large enough for every call of `cases` (reused)."""
    n = max(ar.prefill_workspace_bytes(c.B, c.T, c.Hkv, c.Dk, rotary_dims=c.rotary_dims,
                                       theta=c.theta, dtype=c.dtype) for c in cases)
    return torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")


def bench_prefill(ar, torch, inputs, cfg, warmup, iters=None, graph_burst=0):
    """The attn_prefill call (K rotation pre-pass, flash kernel) and,
    separately, the flash kernel alone: a call with Q-only rotation launches
    the same kernel instantiation with the same DMA volume (K's rotary dims
    then come from k itself) and nothing else.

    graph_burst > 0: the kernel alone is timed as replays of a captured graph
    of that many kernel-only calls (replay time / graph_burst). A kernel of a
    few tens of microseconds is shorter than one call's host-side cost, so
    events around single calls would time the host, not the kernel; in a
    graph the launches run back to back. The replay's output is checked
    against an eager call's."""
    c = cfg["case"]
    q, k, v = inputs.prefill_inputs(c, cfg["seed"], device="cuda")
    o = torch.empty((c.B, c.T, c.Hq, c.Dv), dtype=c.dtype, device="cuda")
    ws = prefill_ws(ar, torch, [c])

    def call(ev, i, mask=ar.ROPE_Q | ar.ROPE_K):
        if ev: ev.mark(i, 0)
        ar.prefill(q, k, v, window=c.window, scale=c.scale, rotary_dims=c.rotary_dims,
                   theta=c.theta, pos0=c.pos0, out=o, workspace=ws, rope_mask=mask)
        if ev: ev.mark(i, 1)

    n = iters or iters_for(torch, call, 2)
    ev, wall = timed(torch, call, n, warmup, 2)
    call_ms = ev.series(0, 1)
    kernel_only = lambda e, i: call(e, i, ar.ROPE_Q)
    timing = "HIP events around each kernel-only call"
    if graph_burst:
        kernel_only(None, 0)
        torch.cuda.synchronize()
        eager = o.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(graph_burst):
                kernel_only(None, 0)

        def replay(e, i):
            if e: e.mark(i, 0)
            g.replay()
            if e: e.mark(i, 1)

        o.zero_()
        evk, _ = timed(torch, replay, max(10, n // graph_burst), 3, 2)
        kern_ms = [x / graph_burst for x in evk.series(0, 1)]
        same = bool(torch.equal(o, eager))
        del g, eager
        timing = (f"HIP events around replays of a captured graph of {graph_burst} "
                  f"kernel-only calls, / {graph_burst}; replay output equal to an eager "
                  f"call's: {same}")
    else:
        evk, _ = timed(torch, kernel_only, n, 3, 2)
        kern_ms = evk.series(0, 1)
    call(None, 0)  # leave o holding the full result
    torch.cuda.synchronize()
    return dict(flops=prefill_flops(c), bytes=prefill_bytes(c), call=stats(call_ms),
                kern=stats(kern_ms), iters=n, wall_s=wall, tensors=(q, k, v, o),
                kern_timing=timing)


def bench_prefill_kv_shared(ar, torch, inputs, cfg, warmup):
    """The global prefill shape as a K = V layer: keys turned once by
    prope_apply and passed as both k and v (RoPE on q only), 512-dim values."""
    c = cfg["case"]
    q, k, _ = inputs.prefill_inputs(c, cfg["seed"], device="cuda")
    pos = torch.arange(c.T, dtype=torch.int32, device="cuda").repeat(c.B)
    kr = ar.prope(k.reshape(c.B * c.T, c.Hkv, c.Dk), pos, rotary_dims=c.rotary_dims,
                  theta=c.theta).reshape(c.B, c.T, c.Hkv, c.Dk)
    del k
    o = torch.empty((c.B, c.T, c.Hq, c.Dk), dtype=c.dtype, device="cuda")
    ws = prefill_ws(ar, torch, [c])

    def call(ev, i):
        if ev: ev.mark(i, 0)
        ar.prefill(q, kr, kr, window=c.window, scale=c.scale, rotary_dims=c.rotary_dims,
                   theta=c.theta, pos0=c.pos0, out=o, rope_mask=ar.ROPE_Q, workspace=ws)
        if ev: ev.mark(i, 1)

    ev, _ = timed(torch, call, 10, warmup, 2)
    ms = statistics.median(ev.series(0, 1))
    flops = float(c.B * c.Hq * pairs(c.T, c.window) * 2 * (c.Dk + c.Dk))
    nbytes = float((q.numel() + kr.numel() + o.numel()) * 2)  # q, keys (as values too), o
    del q, kr, o
    return dict(flops=flops, ms=ms, bytes=nbytes)


def build_stack(ar, torch, inputs, cfg):
    sc = cfg["case"]
    layers = []
    for li, (c, kv_from) in enumerate(sc.layers):
        q, k, v = inputs.prefill_inputs(c, cfg["seed"], device="cuda", layer=li,
                                        draw_kv=kv_from is None)
        if kv_from is not None:
            k, v = layers[kv_from]["k"], layers[kv_from]["v"]
        o = torch.empty((c.B, c.T, c.Hq, c.Dv), dtype=c.dtype, device="cuda")
        layers.append(dict(c=c, q=q, k=k, v=v, o=o, kv_from=kv_from, li=li))
    return layers


def bench_stack(ar, torch, inputs, cfg, steps, warmup):
    """Steps over every layer of the stack on one stream, with an event
    between consecutive layers (per-layer durations come out of the same
    timed steps)."""
    layers = build_stack(ar, torch, inputs, cfg)
    ws = prefill_ws(ar, torch, [L["c"] for L in layers])
    n = len(layers)

    def step(ev, i):
        for li, L in enumerate(layers):
            c = L["c"]
            if ev: ev.mark(i, li)
            ar.prefill(L["q"], L["k"], L["v"], window=c.window, scale=c.scale,
                       rotary_dims=c.rotary_dims, theta=c.theta, pos0=c.pos0, out=L["o"],
                       workspace=ws)
        if ev: ev.mark(i, n)

    ev, wall = timed(torch, step, steps, warmup, n + 1)
    step_ms = ev.series(0, n)
    per_layer = [ev.series(li, li + 1) for li in range(n)]
    flops = [prefill_flops(L["c"]) for L in layers]
    return dict(flops=sum(flops), layer_flops=flops, step=stats(step_ms), step_series=step_ms,
                layer_ms=per_layer, wall_s=wall, layers=layers)


def stack_record(cfg, r):
    """Per-layer detail of a stack run (median call time, TFLOP/s)."""
    out = []
    for L, fl, ms in zip(r["layers"], r["layer_flops"], r["layer_ms"]):
        c = L["c"]
        kind = "local" if c.window else ("global (shared K/V)" if L["kv_from"] is not None
                                        else "global")
        med = statistics.median(ms)
        out.append({"layer": L["li"] + 1, "kind": kind, "ms": round(med, 4),
                    "TFLOP/s": round(fl / med / 1e9, 2)})
    return out


def global_layer_roofline(r, traffic_workload):
    """Dominant kernel of a stack: the global layers' flash kernel. Achieved =
    a global layer's algorithmic FLOPs over the mean duration of the global
    layers' calls in the timed steps (each call also turns K's 128 rotary
    dims in a pre-pass, ~0.1 % of the call)."""
    g = [i for i, L in enumerate(r["layers"]) if not L["c"].window]
    ms = [x for i in g for x in r["layer_ms"][i]]
    mean_ms = sum(ms) / len(ms)
    fl = r["layer_flops"][g[0]]
    rl = roofline("mfma", fl / mean_ms / 1e9, PEAK_BF16_TFLOPS, "TFLOP/s",
                  _traffic("prefill_mfma1w", traffic_workload))
    rl.update(kernel="prefill_mfma1w_kernel", launches_per_step=len(g),
              flops_per_launch=fl, launch_ms_mean=round(mean_ms, 4))
    return rl


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------
def bench_decode(ar, torch, inputs, cfg, warmup, oracle=None):
    seed = cfg["seed"]
    calls = []
    for name in ("glob", "loc"):
        d = cfg["cases"][name]
        kvl = inputs.decode_lengths(d, seed)          # same lengths for both calls
        q, kc, vc, off, kvl = inputs.decode_inputs(d, seed + (0 if name == "glob" else 100),
                                                  device="cuda", kv_len=kvl)
        offd, kvld = off.cuda(), kvl.cuda()
        maxl = int(kvl.max())
        ws = torch.empty(ar.decode_workspace_bytes(d.n_seq, d.Hq, d.Hkv, d.Dv, maxl, d.window),
                         dtype=torch.uint8, device="cuda")
        o = torch.empty((d.n_seq, d.Hq, d.Dv), dtype=d.dtype, device="cuda")
        vis = [min(int(n), d.window) if d.window > 0 else int(n) for n in kvl.tolist()]
        nbytes = sum(vis) * d.Hkv * (d.Dk + d.Dv) * 2 + d.n_seq * d.Hq * (d.Dk + d.Dv) * 2
        calls.append(dict(name=name, d=d, q=q, kc=kc, vc=vc, off=offd, kvl=kvld, maxl=maxl,
                          ws=ws, o=o, bytes=nbytes, kvl_host=kvl, vis=vis))
    # A write larger than the 256 MB last-level (MALL) cache before each timed
    # call, so no call reads cache lines a previous one left behind.
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def run(cl):
        d = cl["d"]
        ar.decode(cl["q"], cl["kc"], cl["vc"], cl["off"], cl["kvl"], window=d.window,
                  scale=d.scale, rotary_dims=d.rotary_dims, theta=d.theta,
                  max_kv_len=cl["maxl"], out=cl["o"], workspace=cl["ws"])

    def time_call(fn, n=10):
        def body(ev, i):
            flush.fill_(i & 0xff)
            if ev: ev.mark(i, 0)
            fn()
            if ev: ev.mark(i, 1)
        ev, _ = timed(torch, body, n, warmup, 2)
        return statistics.median(ev.series(0, 1))

    g_ms = time_call(lambda: run(calls[0]))
    l_ms = time_call(lambda: run(calls[1]), n=40)
    g = calls[0]
    d = g["d"]

    # Keys as values (K = V) on the global shape: the global call's key cache
    # passed as both caches (Dv = Dk = 512), so each row is read once.
    o_kv = torch.empty((d.n_seq, d.Hq, d.Dk), dtype=d.dtype, device="cuda")
    ws_kv = torch.empty(ar.decode_workspace_bytes(d.n_seq, d.Hq, d.Hkv, d.Dk, g["maxl"],
                                                  d.window), dtype=torch.uint8, device="cuda")
    kv_bytes = sum(g["vis"]) * d.Hkv * d.Dk * 2 + d.n_seq * d.Hq * 2 * d.Dk * 2
    kv_ms = time_call(lambda: ar.decode(g["q"], g["kc"], g["kc"], g["off"], g["kvl"],
                                        window=d.window, scale=d.scale,
                                        rotary_dims=d.rotary_dims, theta=d.theta,
                                        max_kv_len=g["maxl"], out=o_kv, workspace=ws_kv))

    # Verify (speculative decoding): the global call with its last 2 cache
    # rows taken as 2 new tokens per sequence (8 heads x 2 tokens fill the 16
    # MFMA columns, so each row is still read once per KV head).
    n_q = 2
    q_v = inputs.normal((d.n_seq, n_q, d.Hq, d.Dk), seed, 90, d.dtype, "cuda")
    o_v = torch.empty((d.n_seq, n_q, d.Hq, d.Dv), dtype=d.dtype, device="cuda")
    ws_v = torch.empty(ar.verify_workspace_bytes(d.n_seq, n_q, d.Hq, d.Hkv, d.Dk, d.Dv,
                                                 g["maxl"], d.window),
                       dtype=torch.uint8, device="cuda")
    v_bytes = (sum(g["vis"]) * d.Hkv * (d.Dk + d.Dv) * 2
               + d.n_seq * n_q * d.Hq * (d.Dk + d.Dv) * 2)
    v_ms = time_call(lambda: ar.verify(q_v, g["kc"], g["vc"], g["off"], g["kvl"],
                                       window=d.window, scale=d.scale,
                                       rotary_dims=d.rotary_dims, theta=d.theta,
                                       max_kv_len=g["maxl"], out=o_v, workspace=ws_v))
    # 4 new tokens: 32 (token, head) pairs per KV head, two 16-column groups,
    # which one workgroup serves from the same cache rows.
    n_q4 = 4
    q_v4 = inputs.normal((d.n_seq, n_q4, d.Hq, d.Dk), seed, 91, d.dtype, "cuda")
    o_v4 = torch.empty((d.n_seq, n_q4, d.Hq, d.Dv), dtype=d.dtype, device="cuda")
    ws_v4 = torch.empty(ar.verify_workspace_bytes(d.n_seq, n_q4, d.Hq, d.Hkv, d.Dk, d.Dv,
                                                  g["maxl"], d.window),
                        dtype=torch.uint8, device="cuda")
    v4_bytes = (sum(g["vis"]) * d.Hkv * (d.Dk + d.Dv) * 2
                + d.n_seq * n_q4 * d.Hq * (d.Dk + d.Dv) * 2)
    v4_ms = time_call(lambda: ar.verify(q_v4, g["kc"], g["vc"], g["off"], g["kvl"],
                                        window=d.window, scale=d.scale,
                                        rotary_dims=d.rotary_dims, theta=d.theta,
                                        max_kv_len=g["maxl"], out=o_v4, workspace=ws_v4))
    del q_v4, o_v4, ws_v4

    # int8 cache: the global call's caches quantised once (outside the timed
    # region), one scale per (row, KV head); the decode reads codes + scales.
    kq, ks = ar.kv_quantize_int8(g["kc"])
    vq, vs = ar.kv_quantize_int8(g["vc"])
    o_i8 = torch.empty((d.n_seq, d.Hq, d.Dv), dtype=d.dtype, device="cuda")
    ws_i8 = torch.empty(ar.decode_int8_workspace_bytes(d.n_seq, d.Hq, d.Hkv, d.Dv, g["maxl"],
                                                       d.window),
                        dtype=torch.uint8, device="cuda")
    i8_bytes = (sum(g["vis"]) * d.Hkv * (d.Dk + d.Dv + 8)
                + d.n_seq * d.Hq * (d.Dk + d.Dv) * 2)
    i8_ms = time_call(lambda: ar.decode_int8(g["q"], kq, ks, vq, vs, g["off"], g["kvl"],
                                             window=d.window, scale=d.scale,
                                             rotary_dims=d.rotary_dims, theta=d.theta,
                                             max_kv_len=g["maxl"], out=o_i8, workspace=ws_i8))
    del kq, vq, flush
    cpu = cpu_baseline_decode(oracle, calls, cfg["seed"]) if oracle is not None else None
    return dict(g_ms=g_ms, l_ms=l_ms, g_bytes=g["bytes"], l_bytes=calls[1]["bytes"],
                kv_ms=kv_ms, kv_bytes=kv_bytes, v_ms=v_ms, v_bytes=v_bytes, v_nq=n_q,
                v4_ms=v4_ms, v4_bytes=v4_bytes, v4_nq=n_q4,
                i8_ms=i8_ms, i8_bytes=i8_bytes, cpu=cpu)


def cpu_baseline_decode(oracle, calls, seed, n_seq=4):
    """The oracle's one-token decode over a seeded sample of whole sequences
    of both calls (their visible cache rows copied to the host); GB/s of the
    visible rows' bf16 bytes, as the GPU legs count them."""
    import numpy as np
    rng = np.random.default_rng(seed)
    tot_b, tot_s, parts = 0, 0.0, []
    for cl in calls:
        d = cl["d"]
        seqs = sorted(rng.choice(d.n_seq, size=n_seq, replace=False).tolist())
        off = cl["off"].cpu().tolist()
        for b in seqs:
            n = int(cl["kvl_host"][b])
            row0 = max(0, n - d.window) if d.window > 0 else 0
            r0 = off[b] + row0
            kr, vr = cl["kc"][r0:off[b] + n].cpu(), cl["vc"][r0:off[b] + n].cpu()
            qh = cl["q"][b].cpu()
            t0 = time.perf_counter()
            oracle.decode_one(qh, kr, vr, kv_len=n, row0=row0, window=d.window, scale=d.scale,
                              rotary_dims=d.rotary_dims, theta=d.theta)
            tot_s += time.perf_counter() - t0
            tot_b += (n - row0) * d.Hkv * (d.Dk + d.Dv) * 2
        parts.append(f"{cl['name']}: sequences {seqs}")
    return {"value": tot_b / tot_s / 1e9, "unit": "GB/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{'; '.join(parts)} (seeded), every visible cache row of each; "
                      f"fp64 incl. query rotation and KV replication; {tot_b / 1e9:.2f} GB "
                      f"of bf16 rows in {tot_s:.1f} s"}


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a seeded row subset of the stack
# ---------------------------------------------------------------------------
def cpu_baseline_stack(oracle, cfg, r, target_s):
    """Time the oracle on every layer of the stack, on seeded query rows
    (the first rows, window and tile edges, the last rows, plus random rows);
    report algorithmic FLOP/s over the rows computed and the time the whole
    stack would take at that rate."""
    import numpy as np
    import torch
    n_rand = max(16, int(280 * target_s / 20.0))
    rng = np.random.default_rng(cfg["seed"])
    tot_fl, tot_s, rows_done, rows_all = 0.0, 0.0, 0, 0
    for L in r["layers"]:
        c = L["c"]
        fixed = {0, 1, 2, 31, 32, 63, 64, c.T - 2, c.T - 1}
        if c.window:
            fixed |= {c.window - 1, c.window, c.window + 1}
        rows = np.array(sorted(fixed | set(rng.choice(c.T, size=n_rand, replace=False)
                                           .tolist())), dtype=np.int32)
        idx = torch.as_tensor(rows, dtype=torch.long, device=L["q"].device)
        qh = L["q"][:, idx].cpu()
        kh, vh = L["k"].cpu(), L["v"].cpu()
        t0 = time.perf_counter()
        oracle.prefill(qh, kh, vh, window=c.window, scale=c.scale,
                       rotary_dims=c.rotary_dims, theta=c.theta, rows=rows)
        tot_s += time.perf_counter() - t0
        tot_fl += rows_flops(c, rows)
        rows_done += len(rows)
        rows_all += c.T
        del qh, kh, vh
    rate = tot_fl / tot_s
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": (f"{rows_done} of {rows_all} query rows over the {len(r['layers'])} layers "
                       f"(~{n_rand} seeded random rows per layer plus first/last/window-edge "
                       f"rows), x B={r['layers'][0]['c'].B} x all heads; fp64 incl. K "
                       f"rotation and KV replication per layer; {tot_s:.1f} s for "
                       f"{tot_fl:.3e} FLOP; the whole stack ({r['flops']:.3e} FLOP) "
                       f"would take ~{r['flops'] / rate / 3600:.1f} h at this rate")}


def cpu_baseline_prefill(oracle, c, tensors, rows=None, seed=0):
    """The oracle on one prefill workload: every query row (rows None), or
    the given rows plus seeded random ones (all batches and heads)."""
    import numpy as np
    import torch
    q, k, v = tensors[:3]
    if rows is not None:
        rng = np.random.default_rng(seed)
        rows = np.array(sorted(set(rows) | set(rng.choice(c.T, size=64, replace=False)
                                                  .tolist())), dtype=np.int32)
        q = q[:, torch.as_tensor(rows, dtype=torch.long, device=q.device)]
    qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
    t0 = time.perf_counter()
    oracle.prefill(qh, kh, vh, window=c.window, scale=c.scale, rotary_dims=c.rotary_dims,
                   theta=c.theta, pos0=c.pos0, rows=rows)
    dt = time.perf_counter() - t0
    fl = rows_flops(c, rows if rows is not None else range(c.T))
    what = (f"all {c.T} query rows" if rows is None else
            f"{len(rows)} of {c.T} query rows (first/last/tile/window edges plus 64 seeded "
            f"random rows)")
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{what} x B={c.B} x Hq={c.Hq}; fp64 incl. rotation and KV "
                      f"replication; {fl:.3e} FLOP in {dt:.3f} s"}


# ---------------------------------------------------------------------------
def secondary_prefill(ar, torch, inputs, name, sc, oracle=None):
    fp32 = not str(sc["case"].dtype).endswith("bfloat16")
    peak = PEAK_FP32_TFLOPS if fp32 else PEAK_BF16_TFLOPS
    warm = 200 if name == "local_prefill" else (3 if name == "global_prefill" else 50)
    rr = bench_prefill(ar, torch, inputs, sc, warm,
                       iters=10 if name == "global_prefill" else None,
                       graph_burst=20 if fp32 else 0)
    c = sc["case"]
    kname = ("prefill_general" if fp32 else "prefill_mfma2g" if c.window and c.Hq // c.Hkv == 2
             else "prefill_mfma1w" if c.Dk == 512 else "prefill_mfma")
    tf_k = rr["flops"] / rr["kern"]["median"] / 1e9
    rec = {"workload": sc["name"], "unit": "TFLOP/s",
           "value": round(rr["flops"] / rr["call"]["median"] / 1e9, 3),
           "ms_per_call": round(rr["call"]["median"], 5), "timed_calls": rr["iters"],
           "what": "attn_prefill call: K rotation pre-pass, flash kernel",
           "roofline": dict(roofline("alu" if fp32 else "mfma", tf_k, peak, "TFLOP/s",
                                     _traffic(kname, name)),
                            kernel=kname + "_kernel",
                            kernel_ms=round(rr["kern"]["median"], 5),
                            kernel_timing=rr["kern_timing"],
                            flops_per_launch=rr["flops"])}
    if not fp32:
        rec["roofline"]["hbm_frac_at_algorithmic_bytes"] = round(
            rr["bytes"] / (rr["kern"]["median"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    if oracle is not None:
        # whole workload where it takes seconds; a row subset for the 32k-token one
        edges = None if rr["flops"] < 1e12 else [0, 1, 2, 31, 32, 63, 64, c.T - 2, c.T - 1]
        rec["cpu_baseline"] = cpu_baseline_prefill(oracle, c, rr["tensors"], edges, sc["seed"])
    del rr
    torch.cuda.empty_cache()
    if name == "global_prefill":
        kv = bench_prefill_kv_shared(ar, torch, inputs, sc, 1)
        tf_kv = kv["flops"] / kv["ms"] / 1e9
        rec["keys_as_values"] = {
            "TFLOP/s": round(tf_kv, 3), "ms": round(kv["ms"], 4),
            "what": "same shape as a K = V layer: rotated keys as both k and v, 512-dim "
                    "values, one pass (the call is the kernel: K does not turn in it); "
                    "TFLOP/s counts the K = V layer's algorithmic FLOPs",
            "roofline": dict(roofline("mfma", tf_kv, PEAK_BF16_TFLOPS, "TFLOP/s",
                                      _traffic("prefill_kv1w", "global_prefill_kv")),
                             kernel="prefill_kv1w_kernel", flops_per_launch=kv["flops"],
                             algorithmic_bytes=kv["bytes"])}
    return rec


def secondary_decode(ar, torch, inputs, sc, oracle=None):
    rr = bench_decode(ar, torch, inputs, sc, 1, oracle)
    g = rr["g_bytes"] / (rr["g_ms"] * 1e-3) / 1e9
    l = rr["l_bytes"] / (rr["l_ms"] * 1e-3) / 1e9
    step_ms = rr["g_ms"] + rr["l_ms"]

    def leg(ms, nbytes, what, prof):
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"GB/s": round(gbs, 1), "ms": round(ms, 4), "bytes": nbytes, "what": what,
                "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", _traffic(*prof))}

    return {"workload": sc["name"], "unit": "GB/s",
            "value": round((rr["g_bytes"] + rr["l_bytes"]) / (step_ms * 1e-3) / 1e9, 1),
            "ms_per_step": round(step_ms, 4),
            "global_call": {"GB/s": round(g, 1), "ms": round(rr["g_ms"], 4),
                            "bytes": rr["g_bytes"]},
            "local_call": {"GB/s": round(l, 1), "ms": round(rr["l_ms"], 4),
                           "bytes": rr["l_bytes"],
                           "roofline": roofline("hbm", l, PEAK_HBM_GBS, "GB/s",
                                                _traffic("decode_ring", "local_decode"))},
            "keys_as_values_call": leg(rr["kv_ms"], rr["kv_bytes"],
                                       "global shape with K = V: one 512-dim cache read "
                                       "once for both products (Dv = Dk = 512)",
                                       ("decode_ring", "kv_shared_global_decode")),
            "verify_call": leg(rr["v_ms"], rr["v_bytes"],
                               f"global call with {rr['v_nq']} new tokens per sequence "
                               "(speculative-decoding verify)",
                               ("decode_ring", "verify_global_decode")),
            "verify4_call": leg(rr["v4_ms"], rr["v4_bytes"],
                                f"global call with {rr['v4_nq']} new tokens per sequence: "
                                "32 (token, head) pairs per KV head, two column groups "
                                "served from the same cache rows",
                                ("decode_ring", "verify4_global_decode")),
            "int8_cache_call": leg(rr["i8_ms"], rr["i8_bytes"],
                                   "global call over int8 codes + fp32 per-row scales "
                                   "(same tokens; bytes counted as read)",
                                   ("decode_i8", "int8_global_decode")),
            "roofline": roofline("hbm", g, PEAK_HBM_GBS, "GB/s",
                                 _traffic("decode_ring", "global_decode")),
            "timing": "median of 10 calls (local: 40), 1 GiB MALL-evicting write before each",
            **({"cpu_baseline": rr["cpu"]} if rr.get("cpu") else {})}


def secondary_stack(ar, torch, inputs, name, sc, oracle=None):
    rr = bench_stack(ar, torch, inputs, sc, 10, 2)
    tf = rr["flops"] / rr["step"]["median"] / 1e9
    rec = {"workload": sc["name"], "unit": "TFLOP/s", "value": round(tf, 3),
           "ms_per_step": round(rr["step"]["median"], 4), "timed_steps": 10,
           "layers": stack_record(sc, rr),
           "roofline": global_layer_roofline(rr, name)}
    if oracle is not None:
        rec["cpu_baseline"] = cpu_baseline_stack(oracle, sc, rr, 5.0)
    del rr
    return rec


def progress(msg):
    """One line per finished leg on stderr (the JSON line stays alone on stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="stack", choices=["stack", "small_stack"])
    ap.add_argument("--secondary",
                    default="local_prefill,global_prefill,small_global_fp32,decode,small_stack",
                    help="other workloads measured in the same run, by name ('' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device copies of MIB MiB (HBM counter scale)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this library runs on one GPU only: the hot path has no "
                          "multi-GPU mode, so --gpus must be 1"}), flush=True)
        sys.exit(2)

    import torch
    import attention_rope_amd as ar
    import inputs
    ar.load()
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}), flush=True)
        return

    cfg = inputs.WORKLOADS[args.workload]
    r = bench_stack(ar, torch, inputs, cfg, args.steps, args.warmup)
    med = r["step"]["median"]
    progress(f"{args.workload}: {med:.3f} ms per step")
    value = r["flops"] / med / 1e9
    timed_ms = sum(r["step_series"])
    out = {
        "metric": "prefill attn TFLOP/s & decode KV GB/s, as % of MI355X MFMA/HBM peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, no weights)",
        "config": {"workload": cfg["name"], "workload_key": args.workload,
                   "seed": cfg["seed"], "flops_per_step": r["flops"],
                   "parallelism": "none (1 GPU)"},
        "roofline": global_layer_roofline(r, args.workload),
        "timing": {"ms_per_step_median": round(med, 4),
                   "ms_per_step_mean": round(r["step"]["mean"], 4),
                   "ms_per_step_min": round(r["step"]["min"], 4),
                   "ms_per_step_max": round(r["step"]["max"], 4),
                   "timed_gpu_ms": round(timed_ms, 2),
                   "timed_wall_ms": round(r["wall_s"] * 1e3, 2),
                   "how": "HIP events on the kernels' stream, one pair per step and per "
                          "layer; median of the timed steps"},
        "layers": stack_record(cfg, r),
    }
    if not args.no_cpu_baseline:
        import oracle
        out["cpu_baseline"] = cpu_baseline_stack(oracle, cfg, r, args.cpu_seconds)
        progress("cpu baseline done")
    del r
    torch.cuda.empty_cache()

    secondary = {}
    orc = None
    if not args.no_cpu_baseline:
        import oracle as orc
    for s in [x.strip() for x in args.secondary.split(",") if x.strip()]:
        if s == args.workload:
            continue
        if s not in inputs.WORKLOADS:
            raise SystemExit(f"--secondary: unknown workload {s!r}")
        sc = inputs.WORKLOADS[s]
        if sc["kind"] == "prefill":
            secondary[s] = secondary_prefill(ar, torch, inputs, s, sc, orc)
        elif sc["kind"] == "decode":
            secondary[s] = secondary_decode(ar, torch, inputs, sc, orc)
        else:
            secondary[s] = secondary_stack(ar, torch, inputs, s, sc, orc)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        progress(f"{s} done")
    if secondary:
        out["secondary"] = secondary
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
