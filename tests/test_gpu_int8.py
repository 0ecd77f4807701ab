"""int8 KV cache (HIP): the quantiser bit-exact against the oracle's codes and
scales, and attn_decode_int8 against the fp64 decode of the dequantised rows."""
import numpy as np
import pytest
import torch

import inputs
import oracle
from parity import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF = torch.bfloat16


@pytest.mark.parametrize("D", [128, 256, 512])
def test_kv_quantize_int8_bit_exact(gpu_lib, D):
    x = inputs.normal((333, 4, D), 3, 0, BF, DEV)
    x[5] *= 1e-3
    x[6] *= 300.0
    x[7, 2] = 0.0
    # values on the grid and exact half steps (scale 1 once 127 is the max)
    x[8, 0] = 0.0
    x[8, 0, 0] = 127.0
    x[8, 0, 1:6] = torch.tensor([0.5, 1.5, 2.5, -0.5, -2.5])
    print(f"quantise N=333 H=4 D={D}", flush=True)
    codes, scales = gpu_lib.kv_quantize_int8(x)
    torch.cuda.synchronize()
    rc, rs = oracle.kv_quantize_int8(x.cpu())
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy(), rs)


def _int8_caches(ar, c, seed, kvl, poison):
    q, kc, vc, off, kvl = inputs.decode_inputs(c, seed, device=DEV, kv_len=kvl,
                                              poison_outside_window=poison)
    # quantise with NaN rows (outside the window) as zeros, then give those
    # rows a NaN scale: a kernel that reads one returns NaN
    kz, vz = torch.nan_to_num(kc), torch.nan_to_num(vc)
    kq, ks = ar.kv_quantize_int8(kz)
    vq, vs = ar.kv_quantize_int8(vz)
    bad_k = torch.isnan(kc).any(-1)
    bad_v = torch.isnan(vc).any(-1)
    ks[bad_k] = float("nan")
    vs[bad_v] = float("nan")
    return q, kq, ks, vq, vs, off, kvl


def run(ar, Hq, Hkv, Dk, Dv, W, R, theta, lens, seed=4, poison=True):
    c = inputs.DecodeCase(len(lens), Hq, Hkv, Dk, Dv, window=W, rotary_dims=R, theta=theta,
                          len_lo=1, len_hi=1)
    print(f"int8 decode Hq={Hq} Hkv={Hkv} Dk={Dk} Dv={Dv} W={W} lens={lens}", flush=True)
    q, kq, ks, vq, vs, off, kvl = _int8_caches(ar, c, seed,
                                               torch.tensor(lens, dtype=torch.int32), poison)
    o = ar.decode_int8(q, kq, ks, vq, vs, off.to(DEV), kvl.to(DEV), window=W, scale=c.scale,
                       rotary_dims=R, theta=theta, max_kv_len=max(1, max(lens)))
    torch.cuda.synchronize()
    ksc, vsc = torch.nan_to_num(ks).cpu(), torch.nan_to_num(vs).cpu()
    ref = oracle.decode_int8(q.cpu(), kq.cpu(), ksc, vq.cpu(), vsc, off, kvl, window=W,
                             scale=c.scale, rotary_dims=R, theta=theta)
    assert_close(o, ref, BF, "int8 decode")
    return o


LENS = [0, 1, 2, 15, 16, 17, 127, 128, 129, 1023, 1025, 3000, 5000]


def test_decode_int8_global(gpu_lib):
    run(gpu_lib, 32, 4, 512, 256, 0, 128, 1e6, LENS)


def test_decode_int8_local_window(gpu_lib):
    run(gpu_lib, 16, 8, 256, 256, 1024, 256, 1e4, LENS)
    run(gpu_lib, 16, 8, 256, 256, 100, 256, 1e4, [1, 50, 99, 100, 101, 700])


def test_decode_int8_long_chunks(gpu_lib):
    """Enough sequences x KV heads for 4096-row chunks, lengths across them."""
    lens = [4095, 4096, 4097, 8193] + [1 + 37 * i for i in range(60)]
    run(gpu_lib, 16, 8, 256, 256, 0, 64, 1e6, lens, poison=False)


def test_decode_int8_close_to_bf16_decode(gpu_lib):
    """Quantisation error only: the int8 decode stays near the bf16 decode of
    the same cache (a loose bound, not a parity check)."""
    c = inputs.DecodeCase(3, 32, 4, 512, 256, window=0, rotary_dims=128, theta=1e6,
                          len_lo=1, len_hi=1)
    kvl = torch.tensor([10, 700, 4000], dtype=torch.int32)
    q, kc, vc, off, kvl = inputs.decode_inputs(c, 6, device=DEV, kv_len=kvl)
    kq, ks = gpu_lib.kv_quantize_int8(kc)
    vq, vs = gpu_lib.kv_quantize_int8(vc)
    a = gpu_lib.decode(q, kc, vc, off.to(DEV), kvl.to(DEV), rotary_dims=128, theta=1e6,
                       max_kv_len=4000)
    b = gpu_lib.decode_int8(q, kq, ks, vq, vs, off.to(DEV), kvl.to(DEV), rotary_dims=128,
                            theta=1e6, max_kv_len=4000)
    torch.cuda.synchronize()
    assert (a.float() - b.float()).abs().max().item() < 0.05


def test_decode_int8_empty_and_out_of_range(gpu_lib):
    """kv_len 0 gives zeros, kv_len past max_kv_len poisons the row (NaN), with
    one chunk (window 100) and with several (global, 4096-row chunks)."""
    for W, Hq, Hkv, D in [(100, 16, 8, 256), (0, 32, 4, 512)]:
        c = inputs.DecodeCase(3, Hq, Hkv, D, 256, window=W, rotary_dims=64, theta=1e4,
                              len_lo=1, len_hi=1)
        kvl = torch.tensor([0, 50, 9000], dtype=torch.int32)
        print(f"int8 edge W={W} D={D}", flush=True)
        q, kq, ks, vq, vs, off, kvl = _int8_caches(gpu_lib, c, 8, kvl, poison=False)
        o = gpu_lib.decode_int8(q, kq, ks, vq, vs, off.to(DEV), kvl.to(DEV), window=W,
                                rotary_dims=64, theta=1e4, max_kv_len=1000)
        torch.cuda.synchronize()
        assert torch.all(o[0] == 0)
        assert torch.isfinite(o[1].float()).all()
        assert torch.isnan(o[2].float()).all()
