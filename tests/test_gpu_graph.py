"""The library's calls captured in a HIP graph (as the benchmark replays the
prefill step): every replay, with eager work and synchronisations between
replays, gives the eager results bit for bit."""
import pytest
import torch

import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF = torch.bfloat16


def test_graph_replays_match_eager(gpu_lib):
    ar = gpu_lib
    c = inputs.PrefillCase(1, 640, 16, 8, 256, 256, window=128, rotary_dims=256, theta=1e4,
                           dtype=BF)
    q, k, v = inputs.prefill_inputs(c, 31, device=DEV)
    o = torch.empty((1, 640, 16, 256), dtype=BF, device=DEV)
    ws = torch.empty(ar.prefill_workspace_bytes(1, 640, 8, 256, rotary_dims=256, theta=1e4),
                     dtype=torch.uint8, device=DEV)
    d = inputs.DecodeCase(3, 32, 4, 512, 256, window=0, rotary_dims=128, theta=1e6,
                          len_lo=1, len_hi=1)
    kvl = torch.tensor([5, 900, 3000], dtype=torch.int32)
    dq, kc, vc, off, kvl = inputs.decode_inputs(d, 32, device=DEV, kv_len=kvl)
    off, kvl = off.to(DEV), kvl.to(DEV)
    do = torch.empty((3, 32, 256), dtype=BF, device=DEV)
    dws = torch.empty(ar.decode_workspace_bytes(3, 32, 4, 256, 3000, 0), dtype=torch.uint8,
                      device=DEV)

    def step():
        ar.prefill(q, k, v, window=128, scale=c.scale, rotary_dims=256, theta=1e4, out=o,
                   pos0=17, workspace=ws)
        ar.decode(dq, kc, vc, off, kvl, rotary_dims=128, theta=1e6, max_kv_len=3000, out=do,
                  workspace=dws)

    step()
    torch.cuda.synchronize()
    ref_o, ref_do = o.clone(), do.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        o.zero_()
        do.zero_()
        ws.zero_()
        # unrelated eager work between replays
        ar.prefill(q[:, :64].contiguous(), k[:, :64].contiguous(), v[:, :64].contiguous(),
                   window=0, rotary_dims=256, theta=1e4)
        torch.cuda.synchronize()
        print(f"graph replay {r}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o), f"prefill output differs on replay {r}"
        assert torch.equal(do, ref_do), f"decode output differs on replay {r}"
