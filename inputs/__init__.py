"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws numbers and lays them out; it holds none of the
attention arithmetic (no rotation, no softmax, no masking). Both the HIP path
and the fp64 oracle consume what it produces.

Every tensor is drawn from its own torch generator seeded from
(config seed, tensor stream id), on the device where it will live, in fp32,
then rounded to the storage dtype (round-to-nearest-even for bf16). The same
(seed, stream, shape, device) always gives the same values. Large tensors are
drawn in fixed-size chunks so fp32 temporaries stay bounded; the chunking is
part of the definition and never depends on free memory.

Workload shapes follow the configurations the pages' hybrid attention implies
(local sliding-window layers with 2 query heads per KV head and 256-dim heads,
global layers with 8 query heads per KV head, 512-dim keys and 256-dim values);
see ``WORKLOADS``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

# Stream ids: tensor t of stack layer `layer` uses stream 16 * layer + t.
STREAM_Q, STREAM_K, STREAM_V = 0, 1, 2
_CHUNK = 1 << 26  # elements per draw (256 MiB of fp32 temporaries)


def _seed(seed: int, stream: int) -> int:
    # Mix the two integers into one 63-bit seed (splitmix64 finaliser).
    z = (seed * 0x9E3779B97F4A7C15 + stream + 0x632BE59BD9B4E019) & (2**64 - 1)
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & (2**64 - 1)
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & (2**64 - 1)
    return (z ^ (z >> 31)) & (2**63 - 1)


def _draw(kind: str, shape, seed: int, stream: int, dtype, device) -> torch.Tensor:
    device = torch.device(device)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, stream))
    n = flat.numel()
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        if kind == "normal":
            x = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        elif kind == "uniform":  # U(-1, 1)
            x = torch.rand(e - s, generator=g, device=device, dtype=torch.float32)
            x.mul_(2.0).sub_(1.0)
        else:
            raise ValueError(kind)
        flat[s:e].copy_(x)  # fp32 -> storage dtype, round to nearest even
    return out


def normal(shape, seed: int, stream: int, dtype=torch.bfloat16, device="cpu"):
    """N(0, 1) draws rounded to ``dtype``."""
    return _draw("normal", shape, seed, stream, dtype, device)


def uniform(shape, seed: int, stream: int, dtype=torch.bfloat16, device="cpu"):
    """U(-1, 1) draws rounded to ``dtype``."""
    return _draw("uniform", shape, seed, stream, dtype, device)


@dataclass
class PrefillCase:
    """One prefill call: shapes, attention type and RoPE settings."""
    B: int
    T: int
    Hq: int
    Hkv: int
    Dk: int
    Dv: int
    window: int            # 0: full causal; W > 0: keys i-W+1 .. i
    rotary_dims: int       # 0: no RoPE
    theta: float
    dtype: torch.dtype
    v_dist: str = "normal"
    pos0: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.Dk)


def prefill_inputs(c: PrefillCase, seed: int, device="cpu", layer: int = 0,
                   draw_kv: bool = True):
    """(q, k, v) of shapes [B,T,Hq,Dk], [B,T,Hkv,Dk], [B,T,Hkv,Dv]."""
    base = 16 * layer
    q = normal((c.B, c.T, c.Hq, c.Dk), seed, base + STREAM_Q, c.dtype, device)
    if not draw_kv:
        return q, None, None
    k = normal((c.B, c.T, c.Hkv, c.Dk), seed, base + STREAM_K, c.dtype, device)
    vdraw = uniform if c.v_dist == "uniform" else normal
    v = vdraw((c.B, c.T, c.Hkv, c.Dv), seed, base + STREAM_V, c.dtype, device)
    return q, k, v


@dataclass
class DecodeCase:
    """A batch of single-token decode calls over a ragged bf16 KV cache."""
    n_seq: int
    Hq: int
    Hkv: int
    Dk: int
    Dv: int
    window: int            # 0: global (all rows); W > 0: last W rows
    rotary_dims: int
    theta: float
    len_lo: int            # pre-append cache lengths L ~ U{len_lo .. len_hi}
    len_hi: int
    dtype: torch.dtype = torch.bfloat16

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.Dk)


def decode_lengths(c: DecodeCase, seed: int) -> torch.Tensor:
    """kv_len = L + 1 per sequence (the new token's row is appended), int32."""
    g = torch.Generator(device="cpu")
    g.manual_seed(_seed(seed, 1000))
    L = torch.randint(c.len_lo, c.len_hi + 1, (c.n_seq,), generator=g)
    return (L + 1).to(torch.int32)


def decode_inputs(c: DecodeCase, seed: int, device="cpu", kv_len=None,
                  poison_outside_window: bool = True):
    """q [n_seq, Hq, Dk]; k_cache [rows, Hkv, Dk]; v_cache [rows, Hkv, Dv];
    row_offset int64 [n_seq]; kv_len int32 [n_seq].

    Sequences are packed back to back. With a window, rows the new token cannot
    see are filled with NaN (never drawn), so a kernel that reads them shows it.
    Cached keys are plain N(0, 1) draws standing for already-rotated keys.
    """
    if kv_len is None:
        kv_len = decode_lengths(c, seed)
    kv_len = torch.as_tensor(kv_len, dtype=torch.int32).cpu()
    lens = kv_len.to(torch.int64)
    row_offset = torch.zeros_like(lens)
    if lens.numel() > 1:
        row_offset[1:] = torch.cumsum(lens, 0)[:-1]
    rows = int(lens.sum())
    q = normal((c.n_seq, c.Hq, c.Dk), seed, STREAM_Q, c.dtype, device)
    if c.window > 0 and poison_outside_window:
        kc = torch.empty((rows, c.Hkv, c.Dk), dtype=c.dtype, device=device)
        vc = torch.empty((rows, c.Hkv, c.Dv), dtype=c.dtype, device=device)
        kc.fill_(float("nan"))
        vc.fill_(float("nan"))
        # Draw only the visible rows of each sequence, one sequence at a time
        # (stream ids per sequence keep the draw independent of the packing).
        for b in range(c.n_seq):
            n = int(lens[b])
            lo = max(0, n - c.window)
            off = int(row_offset[b])
            kc[off + lo: off + n] = normal((n - lo, c.Hkv, c.Dk), seed,
                                           2000 + 2 * b, c.dtype, device)
            vc[off + lo: off + n] = normal((n - lo, c.Hkv, c.Dv), seed,
                                           2001 + 2 * b, c.dtype, device)
    else:
        kc = normal((rows, c.Hkv, c.Dk), seed, STREAM_K, c.dtype, device)
        vc = normal((rows, c.Hkv, c.Dv), seed, STREAM_V, c.dtype, device)
    return q, kc, vc, row_offset, kv_len


# --------------------------------------------------------------------------
# The five workloads. Seeds: 20260402 + config number.
# --------------------------------------------------------------------------
SEED0 = 20260402

LOCAL = dict(Hq=16, Hkv=8, Dk=256, Dv=256, rotary_dims=256, theta=1e4)
GLOBAL = dict(Hq=32, Hkv=4, Dk=512, Dv=256, rotary_dims=128, theta=1e6)


# The small models' layer shapes: 8 query heads share one KV head on both
# layer types, 256-dim local heads, 512-dim global keys, window 512.
SMALL_LOCAL = dict(Hq=8, Hkv=1, Dk=256, Dv=256, rotary_dims=256, theta=1e4)
SMALL_GLOBAL = dict(Hq=8, Hkv=1, Dk=512, Dv=256, rotary_dims=128, theta=1e6)


@dataclass
class StackCase:
    """n_local local layers (sliding window), then one global layer, then (with
    shared_kv) a global layer reusing the previous global layer's K/V (only a
    new Q is drawn). The default is the 5:1 stack with a shared-KV layer."""
    B: int = 2
    T: int = 16384
    n_local: int = 5
    window: int = 1024
    dtype: torch.dtype = torch.bfloat16
    local: dict = field(default_factory=lambda: dict(LOCAL))
    glob: dict = field(default_factory=lambda: dict(GLOBAL))
    shared_kv: bool = True
    layers: list = field(default_factory=list)

    def __post_init__(self):
        if not self.layers:
            loc = PrefillCase(self.B, self.T, window=self.window, dtype=self.dtype, **self.local)
            glo = PrefillCase(self.B, self.T, window=0, dtype=self.dtype, **self.glob)
            # (case, kv_from_layer): kv_from_layer is None when the layer owns K/V.
            self.layers = [(loc, None)] * self.n_local + [(glo, None)]
            if self.shared_kv:
                self.layers.append((glo, self.n_local))


WORKLOADS = {
    "small_global_fp32": dict(kind="prefill", seed=SEED0 + 1,
            case=PrefillCase(1, 256, 8, 1, 128, 128, window=0, rotary_dims=32,
                             theta=1e6, dtype=torch.float32),
            name="global prefill fp32 B=1 T=256 8q/1kv D=128 p-RoPE(32 of 128, 1e6)"),
    "local_prefill": dict(kind="prefill", seed=SEED0 + 2,
            case=PrefillCase(4, 4096, window=512, dtype=torch.bfloat16, **LOCAL),
            name="local sliding-window prefill bf16 B=4 T=4096 16q/8kv D=256 W=512 RoPE(1e4)"),
    "global_prefill": dict(kind="prefill", seed=SEED0 + 3,
            case=PrefillCase(1, 32768, window=0, dtype=torch.bfloat16,
                             v_dist="uniform", **GLOBAL),
            name="global prefill bf16 B=1 T=32768 32q/4kv Dk=512 Dv=256 p-RoPE(128 of 512, 1e6)"),
    "decode": dict(kind="decode", seed=SEED0 + 4,
            cases=dict(
                glob=DecodeCase(64, 32, 4, 512, 256, window=0, rotary_dims=128,
                                theta=1e6, len_lo=1024, len_hi=131072),
                loc=DecodeCase(64, 16, 8, 256, 256, window=1024, rotary_dims=256,
                               theta=1e4, len_lo=1024, len_hi=131072)),
            name="decode bf16 64 seqs L~U[1024,131072]: global 32q/4kv 512/256 + local 16q/8kv 256 W=1024"),
    "stack": dict(kind="stack", seed=SEED0 + 5, case=StackCase(),
            name="stack bf16 B=2 T=16384: 5 local W=1024 + global + shared-KV global"),
    # The small models' 4:1 pattern (4 local layers of window 512, then one
    # global layer), 8 query heads per KV head throughout; same batch and
    # length as the 5:1 stack.
    "small_stack": dict(kind="stack", seed=SEED0 + 6,
            case=StackCase(n_local=4, window=512, local=dict(SMALL_LOCAL),
                           glob=dict(SMALL_GLOBAL), shared_kv=False),
            name="small-model stack bf16 B=2 T=16384: 4 local W=512 8q/1kv D=256 + "
                 "global 8q/1kv Dk=512 Dv=256"),
}
