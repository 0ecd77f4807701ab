"""The five workloads at full size, in the launch configuration the bench
times, against the fp64 oracle on sampled outputs.

Sampled rows always include the first rows, 32-row tile edges, window edges
and the last rows, plus seeded random rows; every batch and head of a sampled
row is compared. Decode compares the shortest, the longest and random
sequences.
"""
import numpy as np
import pytest
import torch

import attention_rope_amd as ar
import inputs
import oracle
from parity import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def sample_rows(T, W, n_random, seed):
    fixed = {0, 1, 2, 15, 16, 31, 32, 33, 63, 64, 127, 128, T // 2, T - 33, T - 32,
             T - 2, T - 1}
    if W:
        fixed |= {W - 2, W - 1, W, W + 1, 2 * W}
    rng = np.random.default_rng(seed)
    rows = fixed | set(rng.choice(T, size=n_random, replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < T), dtype=np.int32)


def prefill_case(name, rows_random):
    cfg = inputs.WORKLOADS[name]
    c = cfg["case"]
    q, k, v = inputs.prefill_inputs(c, cfg["seed"], device=DEV)
    o = ar.prefill(q, k, v, window=c.window, scale=c.scale, rotary_dims=c.rotary_dims,
                   theta=c.theta)
    torch.cuda.synchronize()
    rows = None if rows_random is None else sample_rows(c.T, c.window, rows_random, cfg["seed"])
    qh = q.cpu() if rows is None else q.cpu()[:, rows]
    ref = oracle.prefill(qh, k.cpu(), v.cpu(), window=c.window, scale=c.scale,
                         rotary_dims=c.rotary_dims, theta=c.theta, rows=rows)
    got = o if rows is None else o[:, torch.as_tensor(rows, device=DEV, dtype=torch.long)]
    mx, rel = assert_close(got, ref, c.dtype, name)
    print(f"{name}: rows={'all' if rows is None else len(rows)} "
          f"max_abs={mx:.3e} rel_rms={rel:.3e}", flush=True)


def test_small_global_fp32_full():
    prefill_case("small_global_fp32", None)


def test_local_prefill_full_size():
    prefill_case("local_prefill", 96)


def test_global_prefill_full_size():
    prefill_case("global_prefill", 512)
    torch.cuda.empty_cache()


def test_global_prefill_keys_as_values_full_size():
    """The global prefill shape as a K = V layer, as the bench times it: keys
    turned once by prope_apply, passed as both k and v (RoPE on q only), the
    one-pass kernel over 512-dim values; sampled rows against the oracle."""
    cfg = inputs.WORKLOADS["global_prefill"]
    c = cfg["case"]
    q, k, _ = inputs.prefill_inputs(c, cfg["seed"], device=DEV)
    pos = torch.arange(c.T, dtype=torch.int32, device=DEV).repeat(c.B)
    kr = ar.prope(k.reshape(c.B * c.T, c.Hkv, c.Dk), pos, rotary_dims=c.rotary_dims,
                  theta=c.theta).reshape(c.B, c.T, c.Hkv, c.Dk)
    o = ar.prefill(q, kr, kr, window=c.window, scale=c.scale, rotary_dims=c.rotary_dims,
                   theta=c.theta, rope_mask=ar.ROPE_Q)
    torch.cuda.synchronize()
    rows = sample_rows(c.T, c.window, 128, cfg["seed"])
    ref = oracle.prefill_kv_shared(q.cpu()[:, rows], k.cpu(), window=c.window, scale=c.scale,
                                   rotary_dims=c.rotary_dims, theta=c.theta, rows=rows)
    got = o[:, torch.as_tensor(rows, device=DEV, dtype=torch.long)]
    mx, rel = assert_close(got, ref, c.dtype, "global K=V")
    print(f"global K=V: rows={len(rows)} max_abs={mx:.3e} rel_rms={rel:.3e}", flush=True)
    del q, k, kr, o
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kind", ["glob", "loc", "glob_kv", "glob_verify", "glob_int8"])
def test_decode_full_size(kind):
    """glob_kv: the global call with keys as values (its key cache passed as
    both caches, Dv = Dk = 512); glob_verify: the global call with its last 2
    rows as 2 new tokens per sequence; both as the benchmark times them."""
    cfg = inputs.WORKLOADS["decode"]
    d = cfg["cases"]["loc" if kind == "loc" else "glob"]
    seed = cfg["seed"] + (100 if kind == "loc" else 0)
    kvl = inputs.decode_lengths(d, cfg["seed"])
    q, kc, vc, off, kvl = inputs.decode_inputs(d, seed, device=DEV, kv_len=kvl)
    if kind == "glob_kv":
        del vc
        vc = kc
    maxl = int(kvl.max())
    if kind == "glob_verify":
        verify_case(d, q, kc, vc, off, kvl, maxl, cfg["seed"])
        return
    if kind == "glob_int8":
        int8_case(d, q, kc, vc, off, kvl, maxl)
        return
    o = ar.decode(q, kc, vc, off.to(DEV), kvl.to(DEV), window=d.window, scale=d.scale,
                  rotary_dims=d.rotary_dims, theta=d.theta, max_kv_len=maxl)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    lens = kvl.tolist()
    rng = np.random.default_rng(4)
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens))} |
                  set(rng.choice(len(lens), size=4, replace=False).tolist()))
    for b in seqs:
        n = lens[b]
        lo = max(0, n - d.window) if d.window else 0
        a = int(off[b])
        ref = oracle.decode_one(q[b].cpu(), kc[a + lo:a + n].cpu(), vc[a + lo:a + n].cpu(),
                                kv_len=n, row0=lo, window=d.window, scale=d.scale,
                                rotary_dims=d.rotary_dims, theta=d.theta)
        mx, rel = assert_close(o[b], ref, torch.bfloat16, f"decode {kind} seq {b} len {n}")
        print(f"decode {kind}: seq {b} kv_len={n} max_abs={mx:.3e} rel_rms={rel:.3e}",
              flush=True)
    del kc, vc
    torch.cuda.empty_cache()


def verify_case(d, q1, kc, vc, off, kvl, maxl, seed, n_q=2):
    q = inputs.normal((d.n_seq, n_q, d.Hq, d.Dk), seed, 90, d.dtype, DEV)
    o = ar.verify(q, kc, vc, off.to(DEV), kvl.to(DEV), window=d.window, scale=d.scale,
                  rotary_dims=d.rotary_dims, theta=d.theta, max_kv_len=maxl)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    lens = kvl.tolist()
    for b in sorted({int(np.argmin(lens)), int(np.argmax(lens)), 7, 40}):
        n, a = lens[b], int(off[b])
        ref = oracle.verify(q[b:b + 1].cpu(), kc[a:a + n].cpu(), vc[a:a + n].cpu(), [0], [n],
                            window=d.window, scale=d.scale, rotary_dims=d.rotary_dims,
                            theta=d.theta)
        mx, rel = assert_close(o[b:b + 1], ref, torch.bfloat16, f"decode verify seq {b}")
        print(f"decode verify n_q={n_q}: seq {b} kv_len={n} max_abs={mx:.3e} "
              f"rel_rms={rel:.3e}", flush=True)
    del kc, vc
    torch.cuda.empty_cache()


def int8_case(d, q, kc, vc, off, kvl, maxl):
    kq, ks = ar.kv_quantize_int8(kc)
    vq, vs = ar.kv_quantize_int8(vc)
    del kc, vc
    o = ar.decode_int8(q, kq, ks, vq, vs, off.to(DEV), kvl.to(DEV), window=d.window,
                       scale=d.scale, rotary_dims=d.rotary_dims, theta=d.theta, max_kv_len=maxl)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    lens = kvl.tolist()
    for b in sorted({int(np.argmin(lens)), int(np.argmax(lens)), 3, 33}):
        n, a = lens[b], int(off[b])
        ref = oracle.decode_int8(q[b:b + 1].cpu(), kq[a:a + n].cpu(), ks[a:a + n].cpu(),
                                 vq[a:a + n].cpu(), vs[a:a + n].cpu(), [0], [n],
                                 window=d.window, scale=d.scale, rotary_dims=d.rotary_dims,
                                 theta=d.theta)
        mx, rel = assert_close(o[b:b + 1], ref, torch.bfloat16, f"decode int8 seq {b}")
        print(f"decode int8: seq {b} kv_len={n} max_abs={mx:.3e} rel_rms={rel:.3e}",
              flush=True)
    del kq, vq
    torch.cuda.empty_cache()


def stack_case(name, rows_random):
    """Every layer of a stack workload as the benchmark runs it (one
    attn_prefill call per layer, shared-KV layers handed the earlier layer's
    K/V), each against the oracle on sampled rows."""
    cfg = inputs.WORKLOADS[name]
    sc = cfg["case"]
    layers = []
    for li, (c, kv_from) in enumerate(sc.layers):
        q, k, v = inputs.prefill_inputs(c, cfg["seed"], device=DEV, layer=li,
                                        draw_kv=kv_from is None)
        if kv_from is not None:
            k, v = layers[kv_from][1], layers[kv_from][2]
        o = ar.prefill(q, k, v, window=c.window, scale=c.scale, rotary_dims=c.rotary_dims,
                       theta=c.theta)
        layers.append((q, k, v, o, c, kv_from))
    torch.cuda.synchronize()
    for li, (q, k, v, o, c, kv_from) in enumerate(layers):
        if kv_from is None:
            continue
        # a shared-KV layer equals a standalone call on the earlier layer's K/V, bit for bit
        assert k.data_ptr() == layers[kv_from][1].data_ptr()
        alone = ar.prefill(q, k.clone(), v.clone(), window=c.window, scale=c.scale,
                           rotary_dims=c.rotary_dims, theta=c.theta)
        torch.cuda.synchronize()
        assert torch.equal(alone, o)
    for li, (q, k, v, o, c, _) in enumerate(layers):
        rows = sample_rows(c.T, c.window, rows_random, 50 + li)
        ref = oracle.prefill(q.cpu()[:, rows], k.cpu(), v.cpu(), window=c.window,
                             scale=c.scale, rotary_dims=c.rotary_dims, theta=c.theta,
                             rows=rows)
        got = o[:, torch.as_tensor(rows, device=DEV, dtype=torch.long)]
        mx, rel = assert_close(got, ref, c.dtype, f"{name} layer {li + 1}")
        print(f"{name} layer {li + 1}: rows={len(rows)} max_abs={mx:.3e} rel_rms={rel:.3e}",
              flush=True)
    del layers
    torch.cuda.empty_cache()


def test_stack_full_size():
    stack_case("stack", 512)


def test_small_stack_full_size():
    """The small models' 4:1 stack (window 512, 8 query heads per KV head)."""
    stack_case("small_stack", 512)


@pytest.mark.parametrize("shape", ["global", "local_w512", "local_w1024", "small_local_w512"])
def test_full_tensor_T2048(shape):
    """Every output element at T = 2048 against the oracle, in the head shapes
    of the workloads: global (32q/4kv, 512-dim keys, 256-dim values, p-RoPE),
    local (16q/8kv, 256-dim heads, full RoPE) at both windows, and the small
    models' local layer (8q/1kv)."""
    shapes = {"global": (inputs.GLOBAL, 0), "local_w512": (inputs.LOCAL, 512),
              "local_w1024": (inputs.LOCAL, 1024), "small_local_w512": (inputs.SMALL_LOCAL, 512)}
    kw, W = shapes[shape]
    c = inputs.PrefillCase(1, 2048, window=W, dtype=torch.bfloat16, **kw)
    q, k, v = inputs.prefill_inputs(c, 77, device=DEV)
    print(f"T=2048 {shape}", flush=True)
    o = ar.prefill(q, k, v, window=c.window, scale=c.scale, rotary_dims=c.rotary_dims,
                   theta=c.theta)
    torch.cuda.synchronize()
    ref = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), window=c.window, scale=c.scale,
                         rotary_dims=c.rotary_dims, theta=c.theta)
    mx, rel = assert_close(o, ref, c.dtype, f"T=2048 {shape}")
    print(f"T=2048 {shape}: max_abs={mx:.3e} rel_rms={rel:.3e}", flush=True)
