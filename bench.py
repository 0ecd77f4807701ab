#!/usr/bin/env python3
"""Benchmark of the MI355X hybrid-attention hot path (one GPU).

    python bench.py [--steps K] [--warmup W] [--workload NAME]
                    [--secondary global_prefill,decode,stack]

Prints ONE JSON line. `value` is the throughput of the headline workload
(default: the local sliding-window prefill, B=4 T=4096 16q/8kv D=256 W=512,
RoPE theta=1e4), in algorithmic TFLOP/s: FLOPs of allowed (query, key) pairs
only, B*Hq*pairs(T,W)*2*(Dk+Dv). A step is one pass of the hot path over that
batch: the RoPE cos/sin table for the positions, then attn_prefill, which
turns K's rotary dims once into a workspace and runs the flash prefill kernel
(Q rotated on load, window-aware tile skipping, QK^T and PV on bf16 MFMA,
online softmax). The roofline entry times the attention kernel alone. The other workloads (global prefill, batched
decode, the 7-layer local/global/shared-KV stack) are measured in the same
run and reported under "secondary", each with its own roofline.

Inputs are synthetic and seeded (inputs/), resident in HBM before timing.
Kernel durations come from HIP events recorded on the stream the kernels run
on. The CPU baseline is the fp64 oracle timed on a bounded row sample of the
headline workload on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (AMD spec, no sparsity)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")


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
    return float(sum(min(i + 1, W) for i in rows) * c.B * c.Hq * 2 * (c.Dk + c.Dv))


def _traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel source (else None)."""
    import hashlib
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, rec.get("source", ""))
    if not os.path.exists(src):
        return None
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()[:16]
    if digest != rec.get("source_sha256_16"):
        return None
    return rec.get("bytes_per_launch")


class Timer:
    """Event pairs on the current stream, one per step."""

    def __init__(self, torch, n):
        self.torch = torch
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]

    def mark(self, i, j):
        self.ev[i][j].record()

    def ms(self, i, a, b):
        return self.ev[i][a].elapsed_time(self.ev[i][b])


def bench_prefill(ar, torch, inputs, cfg, steps, warmup):
    """Time the step (cos/sin table, then attn_prefill: K rotation pre-pass and
    the attention kernel) and, separately, the attention kernel alone."""
    c = cfg["case"]
    q, k, v = inputs.prefill_inputs(c, cfg["seed"], device="cuda")
    o = torch.empty((c.B, c.T, c.Hq, c.Dv), dtype=c.dtype, device="cuda")
    tab = torch.empty((c.T, max(c.rotary_dims // 2, 1), 2), dtype=torch.float32, device="cuda")
    nws = ar.prefill_workspace_bytes(c.B, c.T, c.Hkv, c.Dk, rotary_dims=c.rotary_dims,
                                     theta=c.theta, dtype=c.dtype)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")

    def step(t=None, i=0):
        if t: t.mark(i, 0)
        ar.rope_table(c.T, head_dim=c.Dk, rotary_dims=c.rotary_dims, theta=c.theta,
                      pos0=c.pos0, out=tab)
        if t: t.mark(i, 1)
        ar.prefill(q, k, v, window=c.window, scale=c.scale, rotary_dims=c.rotary_dims,
                   theta=c.theta, pos0=c.pos0, out=o, table=tab, workspace=ws)
        if t: t.mark(i, 2)

    def kernel_only(t, i):
        # Q-only rotation: the same kernel instantiation and launch with the
        # same DMA volume (K's rotary dims are then read from k itself), and
        # no pre-pass, so the events bracket the attention kernel alone.
        t.mark(i, 0)
        ar.prefill(q, k, v, window=c.window, scale=c.scale, rotary_dims=c.rotary_dims,
                   theta=c.theta, pos0=c.pos0, out=o, table=tab, workspace=ws,
                   rope_mask=ar.ROPE_Q)
        t.mark(i, 1)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t = Timer(torch, steps)
    t0 = time.perf_counter()
    for i in range(steps):
        step(t, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = sum(t.ms(i, 0, 2) for i in range(steps)) / steps
    call_ms = sum(t.ms(i, 1, 2) for i in range(steps)) / steps
    span_ms = t.ev[0][0].elapsed_time(t.ev[-1][2])
    tk = Timer(torch, steps)
    for i in range(steps):
        kernel_only(tk, i)
    torch.cuda.synchronize()
    kern_ms = sum(tk.ms(i, 0, 1) for i in range(steps)) / steps
    step()  # leave o holding the full result
    flops = prefill_flops(c)
    return dict(flops=flops, bytes=prefill_bytes(c), step_ms=step_ms, call_ms=call_ms,
                kern_ms=kern_ms, span_ms=span_ms, wall_s=wall, tensors=(q, k, v, o))


def bench_prefill_kv_shared(ar, torch, inputs, cfg, steps, warmup):
    """The global prefill shape as a K = V layer: keys turned once by
    prope_apply and passed as both k and v (RoPE on q only), 512-dim values.
    Times the attention call (two passes over 256-dim value halves)."""
    c = cfg["case"]
    q, k, _ = inputs.prefill_inputs(c, cfg["seed"], device="cuda")
    pos = torch.arange(c.T, dtype=torch.int32, device="cuda").repeat(c.B)
    kr = ar.prope(k.reshape(c.B * c.T, c.Hkv, c.Dk), pos, rotary_dims=c.rotary_dims,
                  theta=c.theta).reshape(c.B, c.T, c.Hkv, c.Dk)
    o = torch.empty((c.B, c.T, c.Hq, c.Dk), dtype=c.dtype, device="cuda")
    tab = ar.rope_table(c.T, head_dim=c.Dk, rotary_dims=c.rotary_dims, theta=c.theta,
                        pos0=c.pos0)

    def call():
        ar.prefill(q, kr, kr, window=c.window, scale=c.scale, rotary_dims=c.rotary_dims,
                   theta=c.theta, pos0=c.pos0, out=o, table=tab, rope_mask=ar.ROPE_Q)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t = Timer(torch, steps)
    for i in range(steps):
        t.mark(i, 0)
        call()
        t.mark(i, 1)
    torch.cuda.synchronize()
    ms = sum(t.ms(i, 0, 1) for i in range(steps)) / steps
    flops = float(c.B * c.Hq * pairs(c.T, c.window) * 2 * (c.Dk + c.Dk))
    del q, k, kr, o
    return dict(flops=flops, ms=ms)


def bench_decode(ar, torch, inputs, cfg, steps, warmup):
    seed = cfg["seed"]
    calls = []
    total_bytes = 0.0
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
        total_bytes += nbytes
        calls.append(dict(name=name, d=d, q=q, kc=kc, vc=vc, off=offd, kvl=kvld, maxl=maxl,
                          ws=ws, o=o, bytes=nbytes, kvl_host=kvl, off_host=off))
    # A write larger than the 256 MB last-level (MALL) cache between steps, so
    # no step reads cache lines a previous step left behind.
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def run(cl):
        d = cl["d"]
        ar.decode(cl["q"], cl["kc"], cl["vc"], cl["off"], cl["kvl"], window=d.window,
                  scale=d.scale, rotary_dims=d.rotary_dims, theta=d.theta,
                  max_kv_len=cl["maxl"], out=cl["o"], workspace=cl["ws"])

    for _ in range(warmup):
        for cl in calls:
            run(cl)
    torch.cuda.synchronize()
    t = Timer(torch, steps)
    for i in range(steps):
        flush.fill_(i & 0xff)
        t.mark(i, 0)
        run(calls[0])
        t.mark(i, 1)
        run(calls[1])
        t.mark(i, 2)
    torch.cuda.synchronize()
    g_ms = sum(t.ms(i, 0, 1) for i in range(steps)) / steps
    l_ms = sum(t.ms(i, 1, 2) for i in range(steps)) / steps

    # Keys as values (K = V) on the global shape: the global call's key cache
    # passed as both caches (Dv = Dk = 512), so each row is read once.
    g = calls[0]
    d = g["d"]
    o_kv = torch.empty((d.n_seq, d.Hq, d.Dk), dtype=d.dtype, device="cuda")
    ws_kv = torch.empty(ar.decode_workspace_bytes(d.n_seq, d.Hq, d.Hkv, d.Dk, g["maxl"],
                                                  d.window), dtype=torch.uint8, device="cuda")
    vis = [min(int(n), d.window) if d.window > 0 else int(n) for n in g["kvl_host"].tolist()]
    kv_bytes = sum(vis) * d.Hkv * d.Dk * 2 + d.n_seq * d.Hq * 2 * d.Dk * 2

    def run_kv():
        ar.decode(g["q"], g["kc"], g["kc"], g["off"], g["kvl"], window=d.window, scale=d.scale,
                  rotary_dims=d.rotary_dims, theta=d.theta, max_kv_len=g["maxl"], out=o_kv,
                  workspace=ws_kv)

    for _ in range(warmup):
        run_kv()
    tk = Timer(torch, steps)
    for i in range(steps):
        flush.fill_(i & 0xff)
        tk.mark(i, 0)
        run_kv()
        tk.mark(i, 1)
    torch.cuda.synchronize()
    kv_ms = sum(tk.ms(i, 0, 1) for i in range(steps)) / steps

    # Verify (speculative decoding): the global call with its last 2 cache
    # rows taken as 2 new tokens per sequence (8 heads x 2 tokens fill the 16
    # MFMA columns, so each row is still read once per KV head).
    n_q = 2
    q_v = inputs.normal((d.n_seq, n_q, d.Hq, d.Dk), seed, 90, d.dtype, "cuda")
    o_v = torch.empty((d.n_seq, n_q, d.Hq, d.Dv), dtype=d.dtype, device="cuda")
    ws_v = torch.empty(ar.verify_workspace_bytes(d.n_seq, n_q, d.Hq, d.Hkv, d.Dk, d.Dv,
                                                 g["maxl"], d.window),
                       dtype=torch.uint8, device="cuda")
    v_bytes = (sum(vis) * d.Hkv * (d.Dk + d.Dv) * 2
               + d.n_seq * n_q * d.Hq * (d.Dk + d.Dv) * 2)

    def run_v():
        ar.verify(q_v, g["kc"], g["vc"], g["off"], g["kvl"], window=d.window, scale=d.scale,
                  rotary_dims=d.rotary_dims, theta=d.theta, max_kv_len=g["maxl"], out=o_v,
                  workspace=ws_v)

    for _ in range(warmup):
        run_v()
    tv = Timer(torch, steps)
    for i in range(steps):
        flush.fill_(i & 0xff)
        tv.mark(i, 0)
        run_v()
        tv.mark(i, 1)
    torch.cuda.synchronize()
    v_ms = sum(tv.ms(i, 0, 1) for i in range(steps)) / steps

    # int8 cache: the global call's caches quantised once (outside the timed
    # region), one scale per (row, KV head); the decode reads codes + scales.
    kq, ks = ar.kv_quantize_int8(g["kc"])
    vq, vs = ar.kv_quantize_int8(g["vc"])
    o_i8 = torch.empty((d.n_seq, d.Hq, d.Dv), dtype=d.dtype, device="cuda")
    ws_i8 = torch.empty(ar.decode_int8_workspace_bytes(d.n_seq, d.Hq, d.Hkv, d.Dv, g["maxl"],
                                                       d.window),
                        dtype=torch.uint8, device="cuda")
    i8_bytes = (sum(vis) * d.Hkv * (d.Dk + d.Dv + 8)
                + d.n_seq * d.Hq * (d.Dk + d.Dv) * 2)

    def run_i8():
        ar.decode_int8(g["q"], kq, ks, vq, vs, g["off"], g["kvl"], window=d.window,
                       scale=d.scale, rotary_dims=d.rotary_dims, theta=d.theta,
                       max_kv_len=g["maxl"], out=o_i8, workspace=ws_i8)

    for _ in range(warmup):
        run_i8()
    ti = Timer(torch, steps)
    for i in range(steps):
        flush.fill_(i & 0xff)
        ti.mark(i, 0)
        run_i8()
        ti.mark(i, 1)
    torch.cuda.synchronize()
    i8_ms = sum(ti.ms(i, 0, 1) for i in range(steps)) / steps
    del kq, vq
    return dict(bytes=total_bytes, g_ms=g_ms, l_ms=l_ms, step_ms=g_ms + l_ms,
                g_bytes=calls[0]["bytes"], l_bytes=calls[1]["bytes"], calls=calls,
                kv_ms=kv_ms, kv_bytes=kv_bytes, kv_out=o_kv, v_ms=v_ms, v_bytes=v_bytes,
                v_nq=n_q, i8_ms=i8_ms, i8_bytes=i8_bytes)


def bench_stack(ar, torch, inputs, cfg, steps, warmup):
    sc = cfg["case"]
    seed = cfg["seed"]
    layers = []
    for li, (c, kv_from) in enumerate(sc.layers):
        q, k, v = inputs.prefill_inputs(c, seed, device="cuda", layer=li,
                                        draw_kv=kv_from is None)
        if kv_from is not None:
            k, v = layers[kv_from]["k"], layers[kv_from]["v"]
        o = torch.empty((c.B, c.T, c.Hq, c.Dv), dtype=c.dtype, device="cuda")
        layers.append(dict(c=c, q=q, k=k, v=v, o=o, kv_from=kv_from))
    loc, glo = sc.layers[0][0], sc.layers[sc.n_local][0]
    tabs = {}
    for c in (loc, glo):
        tabs[id(c)] = torch.empty((c.T, c.rotary_dims // 2, 2), dtype=torch.float32,
                                  device="cuda")
    nws = max(ar.prefill_workspace_bytes(c.B, c.T, c.Hkv, c.Dk, rotary_dims=c.rotary_dims,
                                         theta=c.theta, dtype=c.dtype) for c in (loc, glo))
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")  # reused layer by layer

    def step(t=None, i=0):
        if t: t.mark(i, 0)
        for c in (loc, glo):  # one table per layer type, shared by its layers
            ar.rope_table(c.T, head_dim=c.Dk, rotary_dims=c.rotary_dims, theta=c.theta,
                          out=tabs[id(c)])
        for L in layers:
            c = L["c"]
            ar.prefill(L["q"], L["k"], L["v"], window=c.window, scale=c.scale,
                       rotary_dims=c.rotary_dims, theta=c.theta, out=L["o"],
                       table=tabs[id(c)], workspace=ws)
        if t: t.mark(i, 2)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t = Timer(torch, steps)
    for i in range(steps):
        step(t, i)
    torch.cuda.synchronize()
    step_ms = sum(t.ms(i, 0, 2) for i in range(steps)) / steps
    flops = sum(prefill_flops(L["c"]) for L in layers)
    return dict(flops=flops, step_ms=step_ms, layers=layers)


def cpu_baseline(oracle, inputs, cfg, res, target_s):
    """Time the fp64 oracle on a growing sample of query rows (all batches and
    heads) of the headline workload until one run takes >= target_s/4."""
    import numpy as np
    c = cfg["case"]
    q, k, v, _ = res["tensors"]
    qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
    rng = np.random.default_rng(0)
    n = 16
    while True:
        rows = np.sort(rng.choice(c.T, size=min(n, c.T), replace=False)).astype(np.int32)
        t0 = time.perf_counter()
        oracle.prefill(qh[:, rows], kh, vh, window=c.window, scale=c.scale,
                       rotary_dims=c.rotary_dims, theta=c.theta, rows=rows)
        dt = time.perf_counter() - t0
        if dt >= target_s / 4 or n >= c.T:
            break
        n = min(c.T, max(2 * n, int(n * target_s / max(dt, 1e-3))))
    fl = rows_flops(c, rows.tolist())
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{len(rows)} of {c.T} query rows x B={c.B} x Hq={c.Hq} "
                      f"(seeded random rows; fp64, incl. K rotation and KV replication), "
                      f"{dt:.1f} s"}


def roofline(bound, achieved, peak, unit, traffic):
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # The GPU's clocks ramp up over the first tens of milliseconds of work: a
    # few warm-up steps leave the headline step measured on a cold part
    # (0.27-0.28 ms against 0.23 ms once warm), so the default warm-up runs
    # ~0.15 s of untimed steps.
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="local_prefill",
                    choices=["local_prefill", "global_prefill", "stack"])
    ap.add_argument("--secondary", default="global_prefill,decode,stack",
                    help="other workloads measured in the same run, by name ('' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device copies of MIB MiB (HBM counter scale)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only: the hot path has no "
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
    # Steps of tens of milliseconds (global prefill, stack) warm the part in
    # a few steps; cap their warm-up so the default run stays short.
    warmup = args.warmup if args.workload == "local_prefill" else min(args.warmup, 10)
    if cfg["kind"] == "stack":
        r = bench_stack(ar, torch, inputs, cfg, args.steps, warmup)
        value, kern_ms = r["flops"] / r["step_ms"] / 1e9, r["step_ms"]
        bound_rl = roofline("mfma", value, PEAK_BF16_TFLOPS, "TFLOP/s", None)
    else:
        r = bench_prefill(ar, torch, inputs, cfg, args.steps, warmup)
        value = r["flops"] / r["step_ms"] / 1e9
        kern = r["flops"] / r["kern_ms"] / 1e9
        # the local layers' kernel (two workgroups per CU); the global shape
        # runs the one-wave kernel
        kname = "prefill_mfma2g" if cfg["case"].window else "prefill_mfma1w"
        wl = "local_prefill" if cfg["case"].window else "global_prefill"
        bound_rl = roofline("mfma", kern, PEAK_BF16_TFLOPS, "TFLOP/s", _traffic(kname, wl))
        bound_rl["kernel"] = kname + "_kernel"
        bound_rl["kernel_ms"] = round(r["kern_ms"], 5)
        bound_rl["prefill_call_ms"] = round(r["call_ms"], 5)  # K rotation + kernel
        bound_rl["hbm_frac_at_algorithmic_bytes"] = round(
            r["bytes"] / (r["kern_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    out = {
        "metric": "prefill attn TFLOP/s & decode KV GB/s, as % of MI355X MFMA/HBM peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": round(r["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) / U(-1,1) inputs, no weights)",
        "config": {"workload": cfg["name"], "workload_key": args.workload,
                   "seed": cfg["seed"], "parallelism": "none (1 GPU)"},
        "roofline": bound_rl,
    }

    secondary = {}
    for s in [x.strip() for x in args.secondary.split(",") if x.strip()]:
        if s == args.workload:
            continue
        if s not in inputs.WORKLOADS or s == "small_global_fp32":
            raise SystemExit(f"--secondary: unknown workload {s!r}")
        sc = inputs.WORKLOADS[s]
        torch.cuda.empty_cache()
        if sc["kind"] == "prefill":
            rr = bench_prefill(ar, torch, inputs, sc, max(3, args.steps // 4), 1)
            tf = rr["flops"] / rr["kern_ms"] / 1e9
            secondary[s] = {"workload": sc["name"], "unit": "TFLOP/s",
                                 "value": round(rr["flops"] / rr["step_ms"] / 1e9, 3),
                                 "ms_per_step": round(rr["step_ms"], 4),
                                 "roofline": dict(roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s",
                                                           _traffic("prefill_mfma1w", "global_prefill")),
                                                  kernel="prefill_mfma1w_kernel")}
            del rr
            torch.cuda.empty_cache()
            kv = bench_prefill_kv_shared(ar, torch, inputs, sc, max(2, args.steps // 8), 1)
            secondary[s]["keys_as_values"] = {
                "TFLOP/s": round(kv["flops"] / kv["ms"] / 1e9, 3), "ms": round(kv["ms"], 4),
                "what": "same shape as a K = V layer: rotated keys as both k and v, 512-dim "
                        "values, attention call only (two passes over 256-dim value halves; "
                        "TFLOP/s counts the K = V layer's algorithmic FLOPs)"}
        elif sc["kind"] == "decode":
            rr = bench_decode(ar, torch, inputs, sc, max(3, args.steps // 4), 1)
            gbs = rr["bytes"] / (rr["step_ms"] * 1e-3) / 1e9
            g = rr["g_bytes"] / (rr["g_ms"] * 1e-3) / 1e9
            l = rr["l_bytes"] / (rr["l_ms"] * 1e-3) / 1e9
            secondary[s] = {"workload": sc["name"], "unit": "GB/s", "value": round(gbs, 1),
                                 "ms_per_step": round(rr["step_ms"], 4),
                                 "global_call": {"GB/s": round(g, 1), "ms": round(rr["g_ms"], 4),
                                                 "bytes": rr["g_bytes"]},
                                 "local_call": {"GB/s": round(l, 1), "ms": round(rr["l_ms"], 4),
                                                "bytes": rr["l_bytes"]},
                                 "keys_as_values_call": {
                                     "GB/s": round(rr["kv_bytes"] / (rr["kv_ms"] * 1e-3) / 1e9, 1),
                                     "ms": round(rr["kv_ms"], 4), "bytes": rr["kv_bytes"],
                                     "what": "global shape with K = V: one 512-dim cache read "
                                             "once for both products (Dv = Dk = 512)",
                                     "roofline": roofline(
                                         "hbm", rr["kv_bytes"] / (rr["kv_ms"] * 1e-3) / 1e9,
                                         PEAK_HBM_GBS, "GB/s",
                                         _traffic("decode_ring", "kv_shared_global_decode"))},
                                 "verify_call": {
                                     "GB/s": round(rr["v_bytes"] / (rr["v_ms"] * 1e-3) / 1e9, 1),
                                     "ms": round(rr["v_ms"], 4), "bytes": rr["v_bytes"],
                                     "what": f"global call with {rr['v_nq']} new tokens per "
                                             "sequence (speculative-decoding verify)",
                                     "roofline": roofline(
                                         "hbm", rr["v_bytes"] / (rr["v_ms"] * 1e-3) / 1e9,
                                         PEAK_HBM_GBS, "GB/s",
                                         _traffic("decode_ring", "verify_global_decode"))},
                                 "int8_cache_call": {
                                     "GB/s": round(rr["i8_bytes"] / (rr["i8_ms"] * 1e-3) / 1e9, 1),
                                     "ms": round(rr["i8_ms"], 4), "bytes": rr["i8_bytes"],
                                     "what": "global call over int8 codes + fp32 per-row scales "
                                             "(same tokens; bytes counted as read)",
                                     "roofline": roofline(
                                         "hbm", rr["i8_bytes"] / (rr["i8_ms"] * 1e-3) / 1e9,
                                         PEAK_HBM_GBS, "GB/s",
                                         _traffic("decode_i8", "int8_global_decode"))},
                                 "roofline": roofline("hbm", g, PEAK_HBM_GBS, "GB/s",
                                                      _traffic("decode_ring", "global_decode"))}
            del rr
        else:
            rr = bench_stack(ar, torch, inputs, sc, max(3, args.steps // 4), 1)
            tf = rr["flops"] / rr["step_ms"] / 1e9
            secondary[s] = {"workload": sc["name"], "unit": "TFLOP/s", "value": round(tf, 3),
                                 "ms_per_step": round(rr["step_ms"], 4),
                                 "roofline": roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s",
                                                      None)}
            del rr
        torch.cuda.synchronize()
    if secondary:
        out["secondary"] = secondary

    if not args.no_cpu_baseline and cfg["kind"] == "prefill":
        import oracle
        out["cpu_baseline"] = cpu_baseline(oracle, inputs, cfg, r, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
