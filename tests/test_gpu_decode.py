"""attn_decode (HIP) vs the fp64 oracle on ragged caches."""
import numpy as np
import pytest
import torch

import inputs
import oracle
from parity import assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF = torch.bfloat16


def run(ar, Hq, Hkv, Dk, Dv, W, R, theta, lens, seed=3, poison=True, shared=False):
    """shared: one cache serves as keys and values (K = V), passed twice."""
    c = inputs.DecodeCase(len(lens), Hq, Hkv, Dk, Dv, window=W, rotary_dims=R, theta=theta,
                          len_lo=1, len_hi=1)
    kvl = torch.tensor(lens, dtype=torch.int32)
    print(f"decode Hq={Hq} Hkv={Hkv} Dk={Dk} Dv={Dv} W={W} shared={shared} lens={lens}",
          flush=True)
    q, kc, vc, off, kvl = inputs.decode_inputs(c, seed, device=DEV, kv_len=kvl,
                                              poison_outside_window=poison)
    if shared:
        assert Dk == Dv
        vc = kc
    o = ar.decode(q, kc, vc, off.to(DEV), kvl.to(DEV), window=W, scale=c.scale,
                  rotary_dims=R, theta=theta, max_kv_len=max(1, max(lens)))
    torch.cuda.synchronize()
    ref = oracle.decode(q.cpu(), kc.cpu(), vc.cpu(), off, kvl, window=W, scale=c.scale,
                        rotary_dims=R, theta=theta)
    assert_close(o, ref, BF, "decode")
    return o


LENS = [1, 2, 31, 32, 33, 127, 128, 129, 1023, 1024, 1025, 3000, 5000]


def test_decode_global(gpu_lib):
    run(gpu_lib, 32, 4, 512, 256, 0, 128, 1e6, LENS)


def test_decode_local_window(gpu_lib):
    # rows outside the window are NaN: reading any would poison the output
    run(gpu_lib, 16, 8, 256, 256, 1024, 256, 1e4, LENS)


def test_decode_local_g8(gpu_lib):
    # small-model local layer: window 512, 8 query heads per KV head
    run(gpu_lib, 8, 1, 256, 256, 512, 256, 1e4, LENS)
    run(gpu_lib, 16, 8, 256, 256, 100, 256, 1e4, [1, 50, 99, 100, 101, 700])


@pytest.mark.parametrize("Hq,Hkv,Dk,Dv,R", [(8, 1, 128, 128, 32), (4, 4, 256, 128, 0),
                                            (16, 1, 512, 256, 512), (6, 2, 128, 256, 128)])
def test_decode_shapes(gpu_lib, Hq, Hkv, Dk, Dv, R):
    run(gpu_lib, Hq, Hkv, Dk, Dv, 0, R, 1e4, [5, 64, 700, 2049])


@pytest.mark.parametrize("Hq,Hkv,D,W,R,th", [(32, 4, 512, 0, 128, 1e6),
                                             (16, 8, 256, 1024, 256, 1e4),
                                             (8, 1, 128, 0, 32, 1e4)])
def test_decode_keys_as_values(gpu_lib, Hq, Hkv, D, W, R, th):
    """K = V: the same cache pointer as keys and values (tiles hold K only)."""
    run(gpu_lib, Hq, Hkv, D, D, W, R, th, LENS, shared=True)


def test_decode_512_dim_values(gpu_lib):
    """Separate 512-dim values (one-wave ring) next to the shared form."""
    run(gpu_lib, 32, 4, 512, 512, 0, 128, 1e6, [1, 17, 33, 700, 2049])
    run(gpu_lib, 32, 4, 512, 512, 0, 128, 1e6, [1, 17, 33, 700, 2049], shared=True)


def test_decode_long_chunks(gpu_lib):
    """Enough sequences x KV heads that chunks stay 8192 rows long; lengths
    straddle chunk boundaries, mixed with short sequences."""
    lens = [8191, 8192, 8193, 16385] + [1 + 37 * i for i in range(28)]
    run(gpu_lib, 16, 8, 256, 256, 0, 64, 1e6, lens)
    run(gpu_lib, 16, 8, 256, 256, 0, 64, 1e6, lens, shared=True)


@pytest.mark.parametrize("R", [4, 12, 36])
def test_decode_rotary_dims_not_multiple_of_8(gpu_lib, R):
    run(gpu_lib, 8, 2, 128, 128, 0, R, 1e4, [3, 40, 300])


def test_decode_empty_sequence_is_zero(gpu_lib):
    o = run(gpu_lib, 32, 4, 512, 256, 0, 128, 1e6, [0, 10, 0, 300])
    assert torch.all(o[0] == 0) and torch.all(o[2] == 0)
    # one chunk per sequence (window 100): the streaming kernel writes o itself
    o = run(gpu_lib, 16, 8, 256, 256, 100, 256, 1e4, [0, 10, 0, 300])
    assert torch.all(o[0] == 0) and torch.all(o[2] == 0)


def test_decode_equals_last_prefill_row(gpu_lib):
    """Decode over a cache whose keys were rotated by prope_apply equals the
    last row of a prefill over the same tokens (both on the GPU)."""
    T, Hq, Hkv, Dk, Dv, R, th = 700, 32, 4, 512, 256, 128, 1e6
    c = inputs.PrefillCase(1, T, Hq, Hkv, Dk, Dv, window=0, rotary_dims=R, theta=th, dtype=BF)
    q, k, v = inputs.prefill_inputs(c, 12, device=DEV)
    o_pre = gpu_lib.prefill(q, k, v, window=0, scale=c.scale, rotary_dims=R, theta=th)
    pos = torch.arange(T, dtype=torch.int32, device=DEV)
    k_rot = gpu_lib.prope(k[0], pos, rotary_dims=R, theta=th)
    o_dec = gpu_lib.decode(q[:, T - 1].contiguous(), k_rot, v[0].contiguous(),
                           torch.zeros(1, dtype=torch.int64, device=DEV),
                           torch.full((1,), T, dtype=torch.int32, device=DEV),
                           window=0, scale=c.scale, rotary_dims=R, theta=th, max_kv_len=T)
    torch.cuda.synchronize()
    d = np.abs(to64(o_dec[0]) - to64(o_pre[0, T - 1]))
    assert d.max() < 2e-2


def test_decode_kv_len_over_max_is_poisoned(gpu_lib):
    c = inputs.DecodeCase(2, 8, 1, 128, 128, window=0, rotary_dims=0, theta=1e4,
                          len_lo=1, len_hi=1)
    q, kc, vc, off, kvl = inputs.decode_inputs(c, 1, device=DEV,
                                              kv_len=torch.tensor([10, 20], dtype=torch.int32))
    o = gpu_lib.decode(q, kc, vc, off.to(DEV), kvl.to(DEV), max_kv_len=15)
    torch.cuda.synchronize()
    assert torch.isfinite(o[0].float()).all()
    assert torch.isnan(o[1].float()).all()


def test_decode_deterministic(gpu_lib):
    a = run(gpu_lib, 32, 4, 512, 256, 0, 128, 1e6, [4000, 17], seed=9)
    b = run(gpu_lib, 32, 4, 512, 256, 0, 128, 1e6, [4000, 17], seed=9)
    assert torch.equal(a, b)


@pytest.mark.parametrize("shape", ["global", "local", "kv"])
def test_decode_running_max_rescales(gpu_lib, shape):
    """Cached keys whose dim D-2 climbs with the row (0.0005 t) and a query
    whose dim D-2 is 2048: the scores gain ~2 (log2 units) per 32 rows, so
    the streaming softmax moves its running max many times inside a chunk,
    and the chunks of one sequence end with maxima hundreds of units apart
    for the merge. Lengths up to 9000 rows take 3 chunks on the global
    shape; the local call sees its last 1024 rows (the rest NaN)."""
    Hq, Hkv, Dk, Dv, W, R, th = {"global": (32, 4, 512, 256, 0, 128, 1e6),
                                 "local": (16, 8, 256, 256, 1024, 256, 1e4),
                                 "kv": (32, 4, 512, 512, 0, 128, 1e6)}[shape]
    lens = [700, 3000, 5000, 9000]
    c = inputs.DecodeCase(len(lens), Hq, Hkv, Dk, Dv, window=W, rotary_dims=R, theta=th,
                          len_lo=1, len_hi=1)
    q, kc, vc, off, kvl = inputs.decode_inputs(c, 13, device=DEV,
                                              kv_len=torch.tensor(lens, dtype=torch.int32))
    q[..., Dk - 2] = 2048.0
    q[..., Dk - 1] = 0.0
    for b, n in enumerate(lens):
        o0, lo = int(off[b]), (max(0, n - W) if W else 0)
        t = torch.arange(lo, n, device=DEV, dtype=torch.float32)
        kc[o0 + lo:o0 + n, :, Dk - 2] = (0.0005 * t).to(BF)[:, None]
        kc[o0 + lo:o0 + n, :, Dk - 1] = 0.0
    if shape == "kv":
        vc = kc
    print(f"decode rescales {shape} lens={lens}", flush=True)
    o = gpu_lib.decode(q, kc, vc, off.to(DEV), kvl.to(DEV), window=W, scale=c.scale,
                       rotary_dims=R, theta=th, max_kv_len=max(lens))
    torch.cuda.synchronize()
    ref = oracle.decode(q.cpu(), kc.cpu(), vc.cpu(), off, kvl, window=W, scale=c.scale,
                        rotary_dims=R, theta=th)
    assert_close(o, ref, BF, f"decode rescales {shape}")
