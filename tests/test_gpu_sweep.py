"""Seeded random shapes through the HIP path against the fp64 oracle.

The other GPU tests pick their cases by hand (tile edges, window edges,
every GQA ratio). This sweep draws combinations instead, from a fixed seed,
over what the MFMA kernels instantiate: the local head shape (256/256), the
global one (512/256), keys as values (512/512, k == v), and 128-dim heads;
batch 1 or 2, 1..259 tokens, windows from none through 1 and short to
longer than the sequence, rotated dims none / a quarter / all, a RoPE mask
of q, k, both or neither, and positions starting at 0 or far out. Decode
draws ragged cache lengths the same way. Every case prints its parameters
before the GPU call.
"""
import numpy as np
import pytest
import torch

import inputs
import oracle
from parity import assert_close
from test_gpu_decode import run as run_decode

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF = torch.bfloat16

# name, KV-head choices, query heads per KV head, Dk, Dv, rotated-dim choices, theta
SHAPES = [
    ("local", [1, 2, 8], [1, 2, 4, 8], 256, 256, [0, 64, 256], 1e4),
    ("global", [1, 2, 4], [1, 2, 4, 8], 512, 256, [0, 128, 512], 1e6),
    ("kv", [1, 2, 4], [1, 2, 4, 8], 512, 512, [0, 128, 512], 1e6),
    ("d128", [1, 2, 4], [1, 2, 4, 8], 128, 128, [0, 32, 128], 1e4),
]


def prefill_cases(seed=2026, n=24):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        name, hkvs, gs, Dk, Dv, Rs, th = SHAPES[i % len(SHAPES)]
        Hkv, G = int(rng.choice(hkvs)), int(rng.choice(gs))
        B, T = int(rng.integers(1, 3)), int(rng.integers(1, 260))
        W = int(rng.choice([0, 0, 1, int(rng.integers(2, 64)), int(rng.integers(64, 600))]))
        R = int(rng.choice(Rs))
        pos0 = int(rng.choice([0, int(rng.integers(1, 1 << 24))]))
        mask = 1 if name == "kv" else int(rng.choice([0, 1, 2, 3]))
        out.append((name, B, T, G * Hkv, Hkv, Dk, Dv, W, R, th, pos0, mask))
    return out


@pytest.mark.parametrize("case", prefill_cases(), ids=lambda c: "-".join(map(str, c)))
def test_prefill_sweep(gpu_lib, case):
    name, B, T, Hq, Hkv, Dk, Dv, W, R, th, pos0, mask = case
    c = inputs.PrefillCase(B, T, Hq, Hkv, Dk, Dv, window=W, rotary_dims=R, theta=th, dtype=BF,
                           pos0=pos0)
    q, k, v = inputs.prefill_inputs(c, 7, device=DEV)
    print(f"sweep {case}", flush=True)
    if name == "kv":  # keys turned once, passed as keys and values; RoPE on q only
        pos = (torch.arange(T, dtype=torch.int32, device=DEV) + pos0).repeat(B)
        kr = gpu_lib.prope(k.reshape(B * T, Hkv, Dk), pos, rotary_dims=R,
                           theta=th).reshape(B, T, Hkv, Dk)
        o = gpu_lib.prefill(q, kr, kr, window=W, scale=c.scale, rotary_dims=R, theta=th,
                            pos0=pos0, rope_mask=gpu_lib.ROPE_Q)
        torch.cuda.synchronize()
        ref = oracle.prefill_kv_shared(q.cpu(), k.cpu(), window=W, scale=c.scale,
                                       rotary_dims=R, theta=th, pos0=pos0)
    else:
        o = gpu_lib.prefill(q, k, v, window=W, scale=c.scale, rotary_dims=R, theta=th,
                            rope_mask=mask, pos0=pos0)
        torch.cuda.synchronize()
        ref = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), window=W, scale=c.scale,
                             rotary_dims=R, theta=th, rope_mask=mask, pos0=pos0)
    assert_close(o, ref, BF, f"sweep {name}")


def decode_cases(seed=2027, n=8):
    rng = np.random.default_rng(seed)
    shapes = [(32, 4, 512, 256, 128, 1e6), (16, 8, 256, 256, 256, 1e4),
              (8, 1, 256, 256, 256, 1e4), (8, 2, 128, 128, 32, 1e4)]
    out = []
    for i in range(n):
        Hq, Hkv, Dk, Dv, R, th = shapes[i % len(shapes)]
        W = int(rng.choice([0, int(rng.integers(1, 200)), 512, 1024]))
        lens = sorted(int(x) for x in rng.integers(1, 6000, size=int(rng.integers(1, 6))))
        out.append((Hq, Hkv, Dk, Dv, W, R, th, tuple(lens)))
    return out


@pytest.mark.parametrize("case", decode_cases(), ids=lambda c: "-".join(map(str, c[:7])))
def test_decode_sweep(gpu_lib, case):
    Hq, Hkv, Dk, Dv, W, R, th, lens = case
    run_decode(gpu_lib, Hq, Hkv, Dk, Dv, W, R, th, list(lens), seed=11)
