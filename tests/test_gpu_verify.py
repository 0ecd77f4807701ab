"""attn_verify (HIP): several new tokens per sequence vs the fp64 oracle.

Token j of sequence b sits at position kv_len[b] - n_q + j and attends the
cache rows up to its own (within the window). Rows that no token may see are
NaN, so an out-of-range read shows up in the output.
"""
import numpy as np
import pytest
import torch

import inputs
import oracle
from parity import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run(ar, n_q, Hq, Hkv, Dk, Dv, W, R, theta, lens, seed=5, shared=False):
    # draw every row some token sees: a window widened by n_q - 1
    c = inputs.DecodeCase(len(lens), Hq, Hkv, Dk, Dv, window=(W + n_q - 1) if W else 0,
                          rotary_dims=R, theta=theta, len_lo=1, len_hi=1)
    print(f"verify n_q={n_q} Hq={Hq} Hkv={Hkv} Dk={Dk} Dv={Dv} W={W} shared={shared} "
          f"lens={lens}", flush=True)
    kvl = torch.tensor(lens, dtype=torch.int32)
    _, kc, vc, off, kvl = inputs.decode_inputs(c, seed, device=DEV, kv_len=kvl)
    q = inputs.normal((len(lens), n_q, Hq, Dk), seed, 77, torch.bfloat16, DEV)
    if shared:
        vc = kc
    o = ar.verify(q, kc, vc, off.to(DEV), kvl.to(DEV), window=W, scale=Dk ** -0.5,
                  rotary_dims=R, theta=theta, max_kv_len=max(1, max(lens)))
    torch.cuda.synchronize()
    ok = [b for b, n in enumerate(lens) if n == 0 or n >= n_q]
    ref = oracle.verify(q.cpu(), kc.cpu(), vc.cpu(), off, kvl, window=W, scale=Dk ** -0.5,
                        rotary_dims=R, theta=theta, seqs=ok)
    assert_close(o[ok], ref, torch.bfloat16, "verify")
    bad = [b for b, n in enumerate(lens) if 0 < n < n_q]
    for b in bad:
        assert torch.isnan(o[b].float()).all()
    return o


LENS = [0, 1, 2, 3, 8, 31, 33, 129, 1023, 1025, 3000, 5000]


def test_verify_global_two_tokens(gpu_lib):
    """8 heads per KV head x 2 tokens fill the 16 MFMA columns exactly."""
    run(gpu_lib, 2, 32, 4, 512, 256, 0, 128, 1e6, LENS)


def test_verify_global_four_tokens_keys_as_values(gpu_lib):
    """32 (token, head) pairs per KV head: two column groups; K = V."""
    run(gpu_lib, 4, 32, 4, 512, 512, 0, 128, 1e6, LENS, shared=True)


@pytest.mark.parametrize("W", [1024, 5, 1])
def test_verify_local_window(gpu_lib, W):
    """Each token's window starts at its own position - W + 1."""
    run(gpu_lib, 8, 16, 8, 256, 256, W, 256, 1e4, LENS)


def test_verify_many_tokens_small_heads(gpu_lib):
    run(gpu_lib, 20, 2, 2, 128, 128, 0, 32, 1e4, [20, 21, 64, 700, 2049])


def test_verify_one_token_is_decode(gpu_lib):
    c = inputs.DecodeCase(4, 32, 4, 512, 256, window=0, rotary_dims=128, theta=1e6,
                          len_lo=1, len_hi=1)
    kvl = torch.tensor([1, 100, 4000, 9000], dtype=torch.int32)
    q, kc, vc, off, kvl = inputs.decode_inputs(c, 8, device=DEV, kv_len=kvl)
    a = gpu_lib.decode(q, kc, vc, off.to(DEV), kvl.to(DEV), rotary_dims=128, theta=1e6,
                       max_kv_len=9000)
    b = gpu_lib.verify(q[:, None], kc, vc, off.to(DEV), kvl.to(DEV), rotary_dims=128,
                       theta=1e6, max_kv_len=9000)
    torch.cuda.synchronize()
    assert torch.equal(a, b[:, 0])


def test_verify_tokens_equal_separate_decodes(gpu_lib):
    """Token j equals a one-token decode at kv_len - n_q + j + 1 (GPU vs GPU)."""
    n_q, lens = 3, [50, 3000]
    c = inputs.DecodeCase(2, 32, 4, 512, 256, window=0, rotary_dims=128, theta=1e6,
                          len_lo=1, len_hi=1)
    kvl = torch.tensor(lens, dtype=torch.int32)
    _, kc, vc, off, kvl = inputs.decode_inputs(c, 9, device=DEV, kv_len=kvl)
    q = inputs.normal((2, n_q, 32, 512), 9, 78, torch.bfloat16, DEV)
    o = gpu_lib.verify(q, kc, vc, off.to(DEV), kvl.to(DEV), rotary_dims=128, theta=1e6,
                       max_kv_len=max(lens))
    for j in range(n_q):
        kj = (kvl - n_q + j + 1).to(torch.int32)
        d = gpu_lib.decode(q[:, j].contiguous(), kc, vc, off.to(DEV), kj.to(DEV),
                           rotary_dims=128, theta=1e6, max_kv_len=max(lens))
        torch.cuda.synchronize()
        assert (o[:, j].float() - d.float()).abs().max().item() < 2e-2


@pytest.mark.parametrize("shape", [
    (32, 4, 512, 256, 0, 128, 1e6),    # global layer, p-RoPE
    (16, 8, 256, 256, 512, 256, 1e4),  # local layer, window 512
    (8, 1, 256, 256, 512, 256, 1e4),   # small-model local layer: 8 query heads per KV head
], ids=["global", "local", "local-g8"])
def test_drafter_cross_attention(gpu_lib, shape):
    """An MTP drafter's queries attend the target model's cache, which holds
    no rows of theirs: drafting step j puts its query at position L_b + j past
    a cache of L_b rows. The entry points express it as prope_apply at L_b + j
    followed by attn_decode with no rotation, kv_len = L_b and the window
    narrowed by j + 1 (the rows a query at L_b + j may see). Rows outside the
    decode window are NaN."""
    Hq, Hkv, Dk, Dv, W, R, theta = shape
    lens = [1, 40, 511, 512, 513, 3000]
    c = inputs.DecodeCase(len(lens), Hq, Hkv, Dk, Dv, window=W, rotary_dims=R, theta=theta,
                          len_lo=1, len_hi=1)
    kvl = torch.tensor(lens, dtype=torch.int32)
    _, kc, vc, off, kvl = inputs.decode_inputs(c, 11, device=DEV, kv_len=kvl)
    q = inputs.normal((len(lens), Hq, Dk), 11, 79, torch.bfloat16, DEV)
    for j in range(3):
        print(f"drafter step {j} Hq={Hq} Hkv={Hkv} Dk={Dk} Dv={Dv} W={W}", flush=True)
        qpos = (kvl + j).to(torch.int32)
        qr = gpu_lib.prope(q, qpos.to(DEV), rotary_dims=R, theta=theta)
        o = gpu_lib.decode(qr, kc, vc, off.to(DEV), kvl.to(DEV),
                           window=(W - j - 1) if W else 0, scale=Dk ** -0.5, rotary_dims=0,
                           max_kv_len=max(lens))
        torch.cuda.synchronize()
        ref = oracle.cross_attend(q.cpu(), kc.cpu(), vc.cpu(), off, kvl, qpos, window=W,
                                  scale=Dk ** -0.5, rotary_dims=R, theta=theta)
        assert_close(o, ref, torch.bfloat16, f"drafter step {j}")
