"""attn_prefill (HIP) vs the fp64 oracle on small and ragged shapes.

Sizes span several 32-key tiles and query tiles with ragged tails; they cover
the MFMA kernel (bf16, model head shapes) and the general kernel (fp32, other
shapes), every GQA ratio the MFMA kernel has, windows of 1, 2, odd, T-1, T and
> T, RoPE off / q only / k only / both, and nonzero pos0.
"""
import numpy as np
import pytest
import torch

import inputs
import oracle
from parity import assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF, F32 = torch.bfloat16, torch.float32


def run_case(ar, B, T, Hq, Hkv, Dk, Dv, W, R, theta, dtype, seed=1, rope_mask=3, pos0=0,
             v_dist="normal", rows=None):
    c = inputs.PrefillCase(B, T, Hq, Hkv, Dk, Dv, window=W, rotary_dims=R, theta=theta,
                           dtype=dtype, v_dist=v_dist, pos0=pos0)
    q, k, v = inputs.prefill_inputs(c, seed, device=DEV)
    print(f"case B={B} T={T} Hq={Hq} Hkv={Hkv} Dk={Dk} Dv={Dv} W={W} R={R} {dtype}",
          flush=True)
    o = ar.prefill(q, k, v, window=W, scale=c.scale, rotary_dims=R, theta=theta,
                   rope_mask=rope_mask, pos0=pos0)
    torch.cuda.synchronize()
    qc = q.cpu() if rows is None else q.cpu()[:, rows]
    ref = oracle.prefill(qc, k.cpu(), v.cpu(), window=W, scale=c.scale, rotary_dims=R,
                         theta=theta, rope_mask=rope_mask, pos0=pos0, rows=rows)
    got = o if rows is None else o[:, rows]
    return assert_close(got, ref, dtype, "prefill"), (q, k, v, o)


MFMA_CASES = [
    # local layer shape (2 q heads / KV head, D=256, full RoPE theta=1e4)
    (2, 200, 16, 8, 256, 256, 64, 256, 1e4),
    (1, 333, 4, 2, 256, 256, 512, 256, 1e4),
    (1, 97, 4, 2, 256, 256, 1, 256, 1e4),
    (1, 70, 2, 1, 256, 256, 2, 64, 1e4),
    # global layer shape (8 q heads / KV head, Dk=512, Dv=256, p-RoPE)
    (1, 300, 32, 4, 512, 256, 0, 128, 1e6),
    (2, 45, 16, 2, 512, 256, 0, 128, 1e6),
    (1, 129, 8, 1, 512, 256, 100, 512, 1e6),
    # 512-dim values: two passes over 256-dim halves of v and o
    (1, 300, 32, 4, 512, 512, 0, 128, 1e6),
    (2, 130, 16, 2, 512, 512, 100, 512, 1e6),
    # D=128 heads, every GQA ratio the kernel instantiates
    (1, 130, 8, 1, 128, 128, 0, 32, 1e6),
    (1, 65, 4, 4, 128, 128, 17, 0, 1e4),
    (3, 33, 8, 2, 128, 128, 31, 128, 1e4),
    (1, 1, 16, 8, 256, 256, 0, 256, 1e4),
    (1, 7, 32, 4, 512, 256, 3, 128, 1e6),
    (1, 64, 16, 8, 256, 256, 63, 256, 1e4),
    (1, 64, 16, 8, 256, 256, 64, 256, 1e4),
    (1, 64, 16, 8, 256, 256, 500, 256, 1e4),
    # small-model local layers: window 512 with 8 or 4 query heads per KV head
    (1, 300, 8, 1, 256, 256, 512, 256, 1e4),
    (2, 100, 8, 2, 256, 256, 33, 256, 1e4),
]


@pytest.mark.parametrize("case", MFMA_CASES, ids=lambda c: "-".join(map(str, c)))
def test_prefill_bf16(gpu_lib, case):
    run_case(gpu_lib, *case, BF)


GENERAL_CASES = [
    # fp32 general kernel (the fp32 config shape, and odd shapes)
    (1, 256, 8, 1, 128, 128, 0, 32, 1e6, F32),
    (2, 50, 6, 3, 64, 48, 5, 16, 1e4, F32),
    (1, 33, 2, 2, 510, 2, 0, 510, 1e4, F32),
    (1, 40, 3, 1, 32, 512, 7, 0, 1e4, F32),
    # bf16 shapes the MFMA kernel does not cover run the general kernel
    (1, 70, 6, 2, 96, 64, 9, 32, 1e4, BF),
    (1, 40, 16, 1, 128, 128, 0, 32, 1e6, BF),   # 16 q heads per KV head
    # 2 and 3 dim pairs per lane, and long rows over the four-wave key split
    (1, 100, 4, 2, 256, 256, 17, 64, 1e4, F32),
    (1, 90, 4, 1, 384, 192, 0, 96, 1e6, BF),
    (1, 1500, 4, 2, 64, 64, 0, 32, 1e4, F32),
    (2, 1200, 2, 1, 128, 64, 700, 128, 1e4, F32),
    # query heads per workgroup (4, 2 or 1 of a KV head's heads) against dim
    # pairs per lane: 4 heads x 2 pairs (windowed), 2 x 4, 2 x 3 with 6 heads
    # per KV head, 4 heads over long windowed bf16 rows
    (1, 150, 8, 2, 256, 192, 40, 64, 1e4, F32),
    (1, 77, 4, 2, 512, 512, 0, 128, 1e6, F32),
    (2, 60, 12, 2, 320, 160, 0, 80, 1e6, F32),
    (1, 700, 16, 2, 128, 128, 300, 32, 1e6, BF),
]


@pytest.mark.parametrize("case", GENERAL_CASES, ids=lambda c: "-".join(map(str, c[:-1])))
def test_prefill_general(gpu_lib, case):
    run_case(gpu_lib, *case)


@pytest.mark.parametrize("rope_mask", [0, 1, 2])
def test_prefill_rope_mask(gpu_lib, rope_mask):
    run_case(gpu_lib, 1, 90, 16, 2, 512, 256, 0, 128, 1e6, BF, rope_mask=rope_mask)
    run_case(gpu_lib, 1, 90, 4, 2, 256, 256, 40, 256, 1e4, BF, rope_mask=rope_mask)


@pytest.mark.parametrize("pos0", [1, 1000, 131000, 2 ** 31 - 78])
def test_prefill_pos0(gpu_lib, pos0):
    """Token t at position pos0 + t, up to the largest position the ABI takes
    (2^31 - 2): the 512-dim-key kernel, the 8-wave kernel (8 q heads per KV
    head, 128- and 256-dim heads), the K pre-pass, and the fp32 general kernel."""
    run_case(gpu_lib, 1, 77, 16, 2, 512, 256, 0, 128, 1e6, BF, pos0=pos0)
    run_case(gpu_lib, 1, 77, 8, 1, 128, 128, 0, 32, 1e6, BF, pos0=pos0)
    run_case(gpu_lib, 1, 77, 8, 1, 256, 256, 30, 256, 1e4, BF, pos0=pos0)
    run_case(gpu_lib, 1, 77, 8, 1, 128, 128, 0, 32, 1e6, F32, pos0=pos0)


@pytest.mark.parametrize("R", [64, 256])
@pytest.mark.parametrize("pos0", [1, 1000, 131000, 2 ** 31 - 301])
def test_prefill_local_pos0(gpu_lib, pos0, R):
    # Each kernel turns q by the (cos, sin) row of its wave's first position
    # (fp64) and then by the lane's offset from it; both must give what the
    # oracle's direct rotation at pos0 + t gives.
    run_case(gpu_lib, 1, 300, 16, 8, 256, 256, 128, R, 1e4, BF, rope_mask=1, pos0=pos0)
    run_case(gpu_lib, 2, 97, 4, 2, 256, 256, 0, R, 1e6, BF, rope_mask=3, pos0=pos0)


def test_prefill_uniform_values(gpu_lib):
    run_case(gpu_lib, 1, 200, 32, 4, 512, 256, 0, 128, 1e6, BF, v_dist="uniform")


@pytest.mark.parametrize("shape,W", [("local", 0), ("local", 250), ("global", 0), ("global", 300),
                                     ("kv", 0), ("kv", 300), ("small_local", 0), ("d128", 0),
                                     ("general_fp32", 0), ("general_bf16", 200)])
def test_prefill_running_max_rescales(gpu_lib, shape, W):
    """Scores that climb with the key's position: one dim of q is 128 and the
    same dim of every key is 0.01 j (dim D-2, which p-RoPE leaves unturned
    and full RoPE turns by at most ~0.04 rad here). A row's scores then gain
    2.6-5 (log2 units) per 32-key tile, so the online softmax must move its
    running max, and rescale O, two or more times inside each long row, not only
    at the first tile as with N(0,1) inputs. Every MFMA kernel, causal and
    windowed; "kv" passes the turned keys as values too. The general kernel
    (fp32, and a bf16 head size the MFMA kernels do not take) as well."""
    Hq, Hkv, D, Dv, R, th = {"local": (16, 8, 256, 256, 256, 1e4),
                             "global": (32, 4, 512, 256, 128, 1e6),
                             "kv": (32, 4, 512, 512, 128, 1e6),
                             "small_local": (8, 1, 256, 256, 256, 1e4),
                             "d128": (8, 1, 128, 128, 128, 1e4),
                             "general_fp32": (8, 1, 128, 128, 32, 1e6),
                             "general_bf16": (6, 2, 96, 64, 32, 1e4)}[shape]
    T = 400
    dt = F32 if shape == "general_fp32" else BF
    c = inputs.PrefillCase(1, T, Hq, Hkv, D, Dv, window=W, rotary_dims=R, theta=th, dtype=dt)
    q, k, v = inputs.prefill_inputs(c, 5, device=DEV)
    q[..., D - 2] = 128.0
    q[..., D - 1] = 0.0
    k[..., D - 2] = (0.01 * torch.arange(T, device=DEV, dtype=torch.float32)).to(dt)[None, :, None]
    k[..., D - 1] = 0.0
    # the climb over the longest visible range, in log2 units of the scores
    span = (min(W, T) if W else T) - 1
    assert 128 * 0.01 * span * c.scale * 1.4426950408889634 > 16  # >= 2 moves of 2^8
    print(f"rescales {shape} W={W}", flush=True)
    if shape == "kv":
        pos = torch.arange(T, dtype=torch.int32, device=DEV)
        kr = gpu_lib.prope(k[0], pos, rotary_dims=R, theta=th).unsqueeze(0)
        o = gpu_lib.prefill(q, kr, kr, window=W, scale=c.scale, rotary_dims=R, theta=th,
                            rope_mask=gpu_lib.ROPE_Q)
        torch.cuda.synchronize()
        ref = oracle.prefill_kv_shared(q.cpu(), k.cpu(), window=W, scale=c.scale,
                                       rotary_dims=R, theta=th)
    else:
        o = gpu_lib.prefill(q, k, v, window=W, scale=c.scale, rotary_dims=R, theta=th)
        torch.cuda.synchronize()
        ref = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), window=W, scale=c.scale,
                             rotary_dims=R, theta=th)
    assert_close(o, ref, dt, f"rescales {shape}")


@pytest.mark.parametrize("Dk,Dv,Hq,Hkv", [(256, 256, 4, 2), (512, 256, 16, 2), (128, 128, 8, 1)])
def test_mask_readout(gpu_lib, Dk, Dv, Hq, Hkv):
    """scale = 0 and one-hot values V = I (keys as value dims) make the output
    the kernel's effective attention row: visible keys get 1/|A(i)|, masked
    keys exactly 0. Compared with brute-force enumeration."""
    T = Dv  # one-hot needs T <= Dv
    for W in (0, 1, 3, 31, 32, 33, T - 1):
        q = inputs.normal((1, T, Hq, Dk), 3, 0, BF, DEV)
        k = inputs.normal((1, T, Hkv, Dk), 3, 1, BF, DEV)
        v = torch.zeros((1, T, Hkv, Dv), dtype=BF, device=DEV)
        for j in range(T):
            v[0, j, :, j] = 1.0
        o = gpu_lib.prefill(q, k, v, window=W, scale=0.0, rotary_dims=0)
        torch.cuda.synchronize()
        got = to64(o)[0]
        i = np.arange(T)[:, None]
        j = np.arange(T)[None, :]
        allowed = (j <= i) & ((W == 0) | (i - j < W))
        for h in range(Hq):
            assert np.array_equal(got[:, h, :T] != 0, allowed), (W, h)
            expect = allowed / allowed.sum(1, keepdims=True)
            np.testing.assert_allclose(got[:, h, :T], expect, atol=4e-3)


def test_window_one_is_identity(gpu_lib):
    """W = 1: every query sees only itself, so o == v bit for bit."""
    c = inputs.PrefillCase(2, 150, 16, 8, 256, 256, window=1, rotary_dims=256,
                           theta=1e4, dtype=BF)
    q, k, v = inputs.prefill_inputs(c, 4, device=DEV)
    o = gpu_lib.prefill(q, k, v, window=1, scale=c.scale, rotary_dims=256, theta=1e4)
    torch.cuda.synchronize()
    assert torch.equal(o, v.repeat_interleave(2, dim=2))


def test_constant_values(gpu_lib):
    c = inputs.PrefillCase(1, 230, 32, 4, 512, 256, window=0, rotary_dims=128,
                           theta=1e6, dtype=BF)
    q, k, _ = inputs.prefill_inputs(c, 5, device=DEV)
    v = torch.full((1, 230, 4, 256), 0.375, dtype=BF, device=DEV)
    o = gpu_lib.prefill(q, k, v, window=0, scale=c.scale, rotary_dims=128, theta=1e6)
    torch.cuda.synchronize()
    assert torch.all(o == 0.375)


def test_inputs_outside_tensors_never_read(gpu_lib):
    """q/k/v sit inside NaN-filled buffers; a read past a tensor would make
    the output non-finite."""
    B, T, Hq, Hkv, Dk, Dv = 1, 100, 32, 4, 512, 256
    def padded(shape):
        n = int(np.prod(shape))
        buf = torch.full((n + 8192,), float("nan"), dtype=BF, device=DEV)
        t = buf[4096:4096 + n].view(shape)
        t.copy_(inputs.normal(shape, 8, n % 97, BF, DEV))
        return t
    q, k, v = padded((B, T, Hq, Dk)), padded((B, T, Hkv, Dk)), padded((B, T, Hkv, Dv))
    o = gpu_lib.prefill(q, k, v, window=0, scale=Dk ** -0.5, rotary_dims=128, theta=1e6)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    ref = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), window=0, scale=Dk ** -0.5,
                         rotary_dims=128, theta=1e6)
    assert_close(o, ref, BF)


def test_deterministic(gpu_lib):
    c = inputs.PrefillCase(1, 400, 32, 4, 512, 256, window=0, rotary_dims=128,
                           theta=1e6, dtype=BF)
    q, k, v = inputs.prefill_inputs(c, 6, device=DEV)
    a = gpu_lib.prefill(q, k, v, window=0, scale=c.scale, rotary_dims=128, theta=1e6)
    b = gpu_lib.prefill(q, k, v, window=0, scale=c.scale, rotary_dims=128, theta=1e6)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_prefill_errors_raise(gpu_lib):
    q = torch.zeros((1, 8, 4, 64), dtype=BF, device=DEV)
    kv = torch.zeros((1, 8, 2, 64), dtype=BF, device=DEV)
    with pytest.raises(gpu_lib.AttnError):
        gpu_lib.prefill(q, kv, kv, rotary_dims=66)
    with pytest.raises(ValueError):
        gpu_lib.prefill(q, q[:, :, :2], q[:, :, :2])  # non-contiguous views


@pytest.mark.parametrize("B,T,Hq,Hkv,D,W,R,th,p0", [
    (1, 150, 16, 2, 512, 0, 128, 1e6, 0),
    (1, 300, 16, 8, 256, 100, 256, 1e4, 0),
    (1, 333, 8, 8, 512, 0, 0, 1e6, 0),        # 512-dim: one query head per KV head, no rotation
    (1, 517, 8, 4, 512, 130, 512, 1e4, 0),    # 2 heads per KV head, window, every dim turned
    (2, 260, 16, 4, 512, 0, 128, 1e6, 5000),  # 4 heads per KV head, two sequences, pos0
    (1, 97, 32, 4, 512, 33, 128, 1e6, 0),     # 8 heads per KV head, short window
    (1, 700, 32, 4, 512, 0, 128, 1e6, 0),     # 22 key tiles: the tile ring wraps many times
    (1, 1, 32, 4, 512, 0, 128, 1e6, 0),       # one token
])
def test_prefill_keys_as_values(gpu_lib, B, T, Hq, Hkv, D, W, R, th, p0):
    """K = V prefill: keys rotated once by prope_apply serve as keys (with
    RoPE on q only) and as values; the oracle rotates them itself. With
    512-dim heads this is the one-pass kernel whose key tile in LDS feeds
    both products."""
    c = inputs.PrefillCase(B, T, Hq, Hkv, D, D, window=W, rotary_dims=R, theta=th, dtype=BF)
    q, k, _ = inputs.prefill_inputs(c, 21, device=DEV)
    print(f"kv-shared prefill B={B} T={T} Hq={Hq} Hkv={Hkv} D={D} W={W} R={R} pos0={p0}",
          flush=True)
    pos = (torch.arange(T, dtype=torch.int32, device=DEV) + p0).repeat(B)
    kr = gpu_lib.prope(k.reshape(B * T, Hkv, D), pos, rotary_dims=R,
                       theta=th).reshape(B, T, Hkv, D)
    o = gpu_lib.prefill(q, kr, kr, window=W, scale=c.scale, rotary_dims=R, theta=th, pos0=p0,
                        rope_mask=gpu_lib.ROPE_Q)
    torch.cuda.synchronize()
    ref = oracle.prefill_kv_shared(q.cpu(), k.cpu(), window=W, scale=c.scale, rotary_dims=R,
                                   theta=th, pos0=p0)
    assert_close(o, ref, BF, "prefill K=V")


@pytest.mark.parametrize("shape", ["local", "global", "small_local"])
def test_grid_order_independent(gpu_lib, shape):
    """A sequence's output does not depend on where and when its workgroups
    run: computed alone (B=1) and as the second row of a batch (B=2, so the
    grid and the block-to-tile mapping change), its rows are the same bits."""
    kw = {"local": (inputs.LOCAL, 512), "global": (inputs.GLOBAL, 0),
          "small_local": (inputs.SMALL_LOCAL, 512)}[shape]
    c = inputs.PrefillCase(2, 1100, window=kw[1], dtype=BF, **kw[0])
    q, k, v = inputs.prefill_inputs(c, 13, device=DEV)
    both = gpu_lib.prefill(q, k, v, window=c.window, scale=c.scale, rotary_dims=c.rotary_dims,
                           theta=c.theta)
    alone = gpu_lib.prefill(q[1:].contiguous(), k[1:].contiguous(), v[1:].contiguous(),
                            window=c.window, scale=c.scale, rotary_dims=c.rotary_dims,
                            theta=c.theta)
    torch.cuda.synchronize()
    assert torch.equal(both[1:], alone)
