"""attn_decode_noalloc (split-K partials in the library's static device
scratch) against attn_decode (caller's workspace), through the C ABI, on two
calls in a row, the second smaller; each also against the fp64 oracle."""
import numpy as np
import pytest
import torch

import inputs
import oracle
from parity import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("kind", ["global", "local"])
def test_noalloc_matches_workspace_entry(gpu_lib, kind):
    ar = gpu_lib
    if kind == "global":
        d = inputs.DecodeCase(8, 32, 4, 512, 256, window=0, rotary_dims=128, theta=1e6,
                              len_lo=1, len_hi=1)
        lens = [[30000, 1, 4097, 9000, 0, 16385, 12345, 2], [700, 3, 4096, 1]]
    else:
        d = inputs.DecodeCase(8, 16, 8, 256, 256, window=1024, rotary_dims=256, theta=1e4,
                              len_lo=1, len_hi=1)
        lens = [[5000, 1, 1024, 1025, 0, 3000, 77, 2048], [600, 1500, 2]]
    for call, kl in enumerate(lens):
        dd = inputs.DecodeCase(len(kl), d.Hq, d.Hkv, d.Dk, d.Dv, d.window, d.rotary_dims,
                               d.theta, 1, 1)
        kvl = torch.tensor(kl, dtype=torch.int32)
        q, kc, vc, off, kvl = inputs.decode_inputs(dd, 60 + call, device=DEV, kv_len=kvl)
        offd, kvld = off.to(DEV), kvl.to(DEV)
        maxl = max(int(kvl.max()), 1)
        print(f"noalloc {kind} call {call}: B={len(kl)} max_kv_len={maxl}", flush=True)
        ref_o = ar.decode(q, kc, vc, offd, kvld, window=dd.window, scale=dd.scale,
                          rotary_dims=dd.rotary_dims, theta=dd.theta, max_kv_len=maxl)
        o = torch.full_like(ref_o, float("nan"))
        ar.decode_noalloc(q, kc, vc, offd, kvld, window=dd.window, scale=dd.scale,
                          rotary_dims=dd.rotary_dims, theta=dd.theta, max_kv_len=maxl, out=o)
        torch.cuda.synchronize()
        # same kernels, same split plan: the same bits
        assert torch.equal(o, ref_o), f"call {call}: outputs differ"
        for b in range(len(kl)):
            n = kl[b]
            lo = max(0, n - dd.window) if dd.window else 0
            a = int(off[b])
            ref = oracle.decode_one(q[b].cpu(), kc[a + lo:a + n].cpu(), vc[a + lo:a + n].cpu(),
                                    kv_len=n, row0=lo, window=dd.window, scale=dd.scale,
                                    rotary_dims=dd.rotary_dims, theta=dd.theta)
            assert_close(o[b], ref, torch.bfloat16, f"noalloc call {call} seq {b}")


def test_noalloc_rejects_beyond_scratch(gpu_lib):
    ar = gpu_lib
    d = inputs.DecodeCase(64, 32, 4, 512, 256, window=0, rotary_dims=128, theta=1e6,
                          len_lo=1, len_hi=1)
    kvl = torch.full((64,), 2, dtype=torch.int32)
    q, kc, vc, off, kvl = inputs.decode_inputs(d, 3, device=DEV, kv_len=kvl)
    o = torch.empty((64, 32, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ar.AttnError, match="scratch"):
        ar.decode_noalloc(q, kc, vc, off.to(DEV), kvl.to(DEV), scale=d.scale,
                          rotary_dims=128, theta=1e6, max_kv_len=131073, out=o)
