"""prope_apply (HIP) vs the oracle's rotation."""
import numpy as np
import pytest
import torch

import inputs
import oracle
from parity import assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D,R,theta", [(512, 128, 1e6), (256, 256, 1e4), (128, 32, 1e6),
                                       (64, 0, 1e4), (6, 2, 10.0)])
def test_prope_vs_oracle(gpu_lib, dtype, D, R, theta):
    N, H = 37, 3
    x = inputs.normal((N, H, D), 5, 0, dtype, DEV)
    pos = torch.tensor([0, 1, 2, 3, 255, 256, 1023, 4095, 32767, 65535, 131071, 131072,
                        131073, 2 ** 20, 2 ** 31 - 2] + list(range(100, 122)),
                       dtype=torch.int32, device=DEV)
    y = gpu_lib.prope(x, pos, rotary_dims=R, theta=theta)
    torch.cuda.synchronize()
    ref = oracle.rope(x.cpu(), pos.cpu().numpy(), R, theta)
    got = to64(y)
    # untouched dims are bit-identical
    assert torch.equal(y[:, :, R:], x[:, :, R:])
    if dtype == torch.float32:
        np.testing.assert_allclose(got, ref, rtol=0, atol=2e-6 * np.abs(ref).max())
    else:
        # within one bf16 rounding step of the exact rotation
        ulp = np.abs(ref) * 2.0 ** -7 + 1e-6 * np.abs(ref).max()
        assert np.all(np.abs(got - ref) <= ulp)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prope_in_place(gpu_lib, dtype):
    N, H, D, R = 50, 4, 512, 128
    x = inputs.normal((N, H, D), 9, 0, dtype, DEV)
    pos = torch.arange(N, dtype=torch.int32, device=DEV) * 977
    ref = gpu_lib.prope(x, pos, rotary_dims=R, theta=1e6)
    y = x.clone()
    gpu_lib.prope(y, pos, rotary_dims=R, theta=1e6, out=y)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    assert torch.equal(y[:, :, R:], x[:, :, R:])


def test_prope_errors(gpu_lib):
    x = torch.zeros((4, 2, 8), dtype=torch.bfloat16, device=DEV)
    pos = torch.zeros(4, dtype=torch.int32, device=DEV)
    with pytest.raises(gpu_lib.AttnError):
        gpu_lib.prope(x, pos, rotary_dims=10, theta=1e4)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("N,H,D,R", [(300, 4, 64, 32), (2520, 2, 128, 32), (7, 1, 4, 2)])
def test_prope_2d(gpu_lib, dtype, N, H, D, R):
    """2-D RoPE (each half turned by one patch coordinate) vs the oracle; 2520
    patches is the 280-token budget's patch count, coordinates on a 60 x 42 grid."""
    g = torch.Generator().manual_seed(N + D)
    x = torch.randn(N, H, D, generator=g).to(dtype)
    pxy = torch.stack([torch.arange(N) % 60, torch.arange(N) // 60], 1).to(torch.int32)
    print(f"prope_2d N={N} H={H} D={D} R={R} {dtype}", flush=True)
    y = gpu_lib.prope_2d(x.to(DEV), pxy.to(DEV), rotary_dims=R, theta=1e4)
    torch.cuda.synchronize()
    ref = oracle.rope_2d(x, pxy.numpy(), R, 1e4)
    assert_close(y, ref, dtype, "prope_2d")
    # in place gives the same values
    xi = x.to(DEV).clone()
    gpu_lib.prope_2d(xi, pxy.to(DEV), rotary_dims=R, theta=1e4, out=xi)
    torch.cuda.synchronize()
    assert torch.equal(xi, y)


def test_prope_2d_rejects_odd_halves(gpu_lib):
    x = torch.zeros(4, 1, 6, dtype=torch.bfloat16, device=DEV)
    pxy = torch.zeros(4, 2, dtype=torch.int32, device=DEV)
    with pytest.raises(gpu_lib.AttnError):
        gpu_lib.prope_2d(x, pxy, rotary_dims=2, theta=1e4)
