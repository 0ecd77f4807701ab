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


@pytest.mark.parametrize("n_q", [3, 4, 5, 6, 8, 12])
def test_verify_global_column_groups(gpu_lib, n_q):
    """24 to 96 (token, head) pairs per KV head: 2 to 6 16-column groups,
    which one workgroup serves up to four at a time from the same cache rows
    (3 groups take a 4-group workgroup with one idle set of waves; 6 take two
    workgroups, the second half idle)."""
    run(gpu_lib, n_q, 32, 4, 512, 256, 0, 128, 1e6, LENS)


@pytest.mark.parametrize("n_q,W", [(9, 1024), (9, 5), (32, 1024), (27, 40)])
def test_verify_local_column_groups(gpu_lib, n_q, W):
    """9 tokens x 2 heads: 18 pairs per KV head, two groups in one workgroup;
    32 and 27 tokens: four groups (the last partly empty), each token with
    its own window start."""
    run(gpu_lib, n_q, 16, 8, 256, 256, W, 256, 1e4, LENS)


@pytest.mark.parametrize("n_q", [4, 8])
def test_verify_global_tokens_keys_as_values(gpu_lib, n_q):
    """32 and 64 (token, head) pairs per KV head: two and four column groups
    in one workgroup; K = V (one 512-wide cache)."""
    run(gpu_lib, n_q, 32, 4, 512, 512, 0, 128, 1e6, LENS, shared=True)


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


@pytest.mark.parametrize("shape", ["local", "global"])
def test_prefill_into_cache(gpu_lib, shape):
    """attn_prefill_into_cache fills the decode cache in its K/V pass:
    - o is attn_prefill's output bit for bit (the same kernels read keys
      turned by the same arithmetic);
    - each sequence's cache rows hold its keys turned at their positions (the
      oracle's rope, to bf16 rounding) and its values bit for bit;
    - rows outside the sequences' ranges keep their NaN poison;
    - decoding each sequence's last token over the filled cache gives the
      oracle's last prefill row, as a decode after a prompt should."""
    base, W = {"local": (inputs.LOCAL, 100), "global": (inputs.GLOBAL, 0)}[shape]
    c = inputs.PrefillCase(2, 300, window=W, dtype=torch.bfloat16, pos0=0, **base)
    print(f"prefill_into_cache {shape} B={c.B} T={c.T}", flush=True)
    q, k, v = inputs.prefill_inputs(c, 31, device=DEV)
    offsets = [17, 17 + c.T + 40]
    rows = offsets[-1] + c.T + 23
    kc = torch.full((rows, c.Hkv, c.Dk), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = torch.full((rows, c.Hkv, c.Dv), float("nan"), dtype=torch.bfloat16, device=DEV)
    off = torch.tensor(offsets, dtype=torch.int64, device=DEV)
    kw = dict(window=W, scale=c.scale, rotary_dims=c.rotary_dims, theta=c.theta)
    o = gpu_lib.prefill_into_cache(q, k, v, kc, vc, off, **kw)
    o_plain = gpu_lib.prefill(q, k, v, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain)

    pos = np.arange(c.T)
    pos_d = torch.arange(c.T, dtype=torch.int32, device=DEV)
    used = np.zeros(rows, dtype=bool)
    for b, r0 in enumerate(offsets):
        kr = oracle.rope(k[b].cpu(), pos, c.rotary_dims, c.theta)
        assert_close(kc[r0:r0 + c.T], kr, torch.bfloat16, f"cached keys b={b}")
        # the same bits as turning the keys with prope_apply
        kp = gpu_lib.prope(k[b].contiguous(), pos_d, rotary_dims=c.rotary_dims, theta=c.theta)
        assert torch.equal(kc[r0:r0 + c.T], kp)
        assert torch.equal(vc[r0:r0 + c.T], v[b])
        used[r0:r0 + c.T] = True
    assert torch.isnan(kc[torch.from_numpy(~used).to(DEV)].float()).all()
    assert torch.isnan(vc[torch.from_numpy(~used).to(DEV)].float()).all()

    # the prompt's last token decoded over its own cache rows
    kvl = torch.full((c.B,), c.T, dtype=torch.int32, device=DEV)
    od = gpu_lib.decode(q[:, -1].contiguous(), kc, vc, off, kvl, window=W, scale=c.scale,
                        rotary_dims=c.rotary_dims, theta=c.theta, max_kv_len=c.T)
    torch.cuda.synchronize()
    ref = oracle.prefill(q[:, -1:].cpu(), k.cpu(), v.cpu(), rows=[c.T - 1], **kw)
    assert_close(od, ref[:, 0], torch.bfloat16, "decode after prefill_into_cache")


def test_prefill_into_cache_fp32(gpu_lib):
    """The fp32 form (general attention kernel, 4-element chunks in the K/V
    pass): cache rows against the oracle's rope at fp32 tolerance, values bit
    for bit, o equal to attn_prefill's."""
    c = inputs.PrefillCase(2, 200, 8, 2, 64, 48, window=70, rotary_dims=32, theta=1e4,
                           dtype=torch.float32, pos0=0)
    print("prefill_into_cache fp32", flush=True)
    q, k, v = inputs.prefill_inputs(c, 32, device=DEV)
    offsets = [250, 5]
    rows = 500
    kc = torch.full((rows, c.Hkv, c.Dk), float("nan"), dtype=torch.float32, device=DEV)
    vc = torch.full((rows, c.Hkv, c.Dv), float("nan"), dtype=torch.float32, device=DEV)
    off = torch.tensor(offsets, dtype=torch.int64, device=DEV)
    kw = dict(window=c.window, scale=c.scale, rotary_dims=c.rotary_dims, theta=c.theta,
              pos0=7)
    o = gpu_lib.prefill_into_cache(q, k, v, kc, vc, off, **kw)
    o_plain = gpu_lib.prefill(q, k, v, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain)
    ref_o = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), **kw)
    assert_close(o, ref_o, torch.float32, "fp32 prefill_into_cache output")
    used = np.zeros(rows, dtype=bool)
    for b, r0 in enumerate(offsets):
        kr = oracle.rope(k[b].cpu(), np.arange(7, 7 + c.T), c.rotary_dims, c.theta)
        assert_close(kc[r0:r0 + c.T], kr, torch.float32, f"fp32 cached keys b={b}")
        assert torch.equal(vc[r0:r0 + c.T], v[b])
        used[r0:r0 + c.T] = True
    assert torch.isnan(kc[torch.from_numpy(~used).to(DEV)]).all()


def test_prefill_into_cache_out_of_range_rows_skipped(gpu_lib):
    """A batch row whose cache rows would leave [0, cache_rows) is not written
    to the cache (negative offset, or past the end); the others are, and o is
    attn_prefill's for every batch row."""
    c = inputs.PrefillCase(3, 96, window=0, dtype=torch.bfloat16, **inputs.SMALL_GLOBAL)
    print("prefill_into_cache out-of-range rows", flush=True)
    q, k, v = inputs.prefill_inputs(c, 33, device=DEV)
    rows = 300
    offsets = [-5, 100, rows - c.T + 1]
    kc = torch.full((rows, c.Hkv, c.Dk), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = torch.full((rows, c.Hkv, c.Dv), float("nan"), dtype=torch.bfloat16, device=DEV)
    off = torch.tensor(offsets, dtype=torch.int64, device=DEV)
    kw = dict(window=0, scale=c.scale, rotary_dims=c.rotary_dims, theta=c.theta)
    o = gpu_lib.prefill_into_cache(q, k, v, kc, vc, off, **kw)
    o_plain = gpu_lib.prefill(q, k, v, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain)
    assert torch.equal(vc[100:100 + c.T], v[1])
    written = torch.zeros(rows, dtype=torch.bool, device=DEV)
    written[100:100 + c.T] = True
    assert not torch.isnan(kc[written].float()).any()
    assert torch.isnan(kc[~written].float()).all()
    assert torch.isnan(vc[~written].float()).all()
