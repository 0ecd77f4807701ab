"""Key tiles the MFMA prefill kernels visit, against the mask.

The debug build (libattn_rope_dbg.so: the same sources compiled with
ATTN_DEBUG_TILES) counts, per call, the key tiles each workgroup stages and
the (wave, key tile) pairs whose scores a wave computes. The expected counts
come from the mask itself (key j is visible from position i iff j <= i and,
with a window W, i - j < W, "Gemma 4: End-to-End Architecture Walkthrough",
Phase 3 section 3a) over each workgroup's and each wave's query positions:
a tile counts iff it holds a key one of those positions may see. Equality
means no tile outside a band is ever visited and none inside it is skipped.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import attention_rope_amd as ar
import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BN = 32  # keys per tile
LIB_DBG = os.path.join(os.path.dirname(os.path.abspath(ar.__file__)), "libattn_rope_dbg.so")


@pytest.fixture(scope="module")
def dbg():
    if not os.path.exists(LIB_DBG):
        pytest.fail(f"{LIB_DBG} is missing: build with python -m attention_rope_amd._build")
    L = ctypes.CDLL(LIB_DBG)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.attn_prefill.argtypes = [vp] * 4 + [i32] * 7 + [ctypes.c_float, ar._Rope, i32, i32, vp,
                                                       sz, ctypes.c_int, vp]
    L.attn_prefill.restype = ctypes.c_int
    L.attn_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32, ar._Rope, i32, ctypes.c_int]
    L.attn_prefill_workspace_bytes.restype = sz
    L.attn_debug_tile_visits.argtypes = [ctypes.POINTER(ctypes.c_uint64), i32]
    L.attn_debug_tile_visits.restype = ctypes.c_int
    return L


def needed(lo, hi, W, T):
    """Key tiles holding a key some position in [lo, hi] (clipped to T) sees."""
    hi = min(hi, T - 1)
    if lo > hi:
        return 0
    k_lo = max(0, lo - W + 1) if W else 0
    return sum(1 for kb in range(k_lo // BN, hi // BN + 1)
               if any(j <= i and (not W or i - j < W)
                      for i in range(lo, hi + 1)
                      for j in range(kb * BN, min(kb * BN + BN, T))))


def expected(kernel, c, W):
    """(wave-tile pairs, staged tiles) for one call, from the mask."""
    G = c.Hq // c.Hkv
    if kernel in ("1w", "kv"):  # 4 waves of 32 rows; every wave runs every staged tile
        NW, PW = 4, 128 // G
        per_wave = None
    else:                # 32-row waves: head w % G, positions p0 + 32 (w // G)
        NW = 4 if kernel == "2g" else 8
        PW = NW * 32 // G
        per_wave = [(32 * (w // G), 32 * (w // G) + 31) for w in range(NW)]
    pairs = staged = 0
    for p0 in range(0, c.T, PW):
        s = needed(p0, p0 + PW - 1, W, c.T)
        staged += s
        pairs += NW * s if per_wave is None else sum(
            needed(p0 + a, p0 + b, W, c.T) for a, b in per_wave)
    n = c.B * c.Hkv
    return pairs * n, staged * n


CASES = [("2g", inputs.LOCAL, 1000, 512), ("2g", inputs.LOCAL, 333, 31),
         ("2g", inputs.LOCAL, 640, 1), ("2g", inputs.LOCAL, 257, 0),
         ("8w", inputs.SMALL_LOCAL, 700, 512), ("8w", inputs.SMALL_LOCAL, 300, 33),
         ("1w", inputs.GLOBAL, 500, 0), ("1w", inputs.SMALL_GLOBAL, 300, 100),
         ("kv", inputs.GLOBAL, 400, 0), ("kv", inputs.GLOBAL, 300, 70)]


@pytest.mark.parametrize("kernel,shape,T,W", CASES)
def test_tile_visits_match_the_mask(dbg, kernel, shape, T, W):
    if kernel == "kv":   # keys as values: the same keys as k and v, RoPE on q only
        shape = {**shape, "Dv": shape["Dk"]}
    c = inputs.PrefillCase(2, T, window=W, dtype=torch.bfloat16, **shape)
    print(f"tile visits {kernel} Hq={c.Hq} Hkv={c.Hkv} Dk={c.Dk} Dv={c.Dv} T={T} W={W}",
          flush=True)
    q, k, v = inputs.prefill_inputs(c, 41, device=DEV)
    mask = 3
    if kernel == "kv":
        v, mask = k, 1
    o = torch.empty((c.B, c.T, c.Hq, c.Dv), dtype=torch.bfloat16, device=DEV)
    rope = ar._Rope(c.rotary_dims, c.theta)
    nws = dbg.attn_prefill_workspace_bytes(c.B, c.T, c.Hkv, c.Dk, rope, mask, ar.ATTN_BF16)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=DEV)
    got = (ctypes.c_uint64 * 2)()
    assert dbg.attn_debug_tile_visits(got, 1) == 0          # zero the counters
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = dbg.attn_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), c.B, c.T,
                          c.Hq, c.Hkv, c.Dk, c.Dv, W, c.scale, rope, mask, 0, ws.data_ptr(), nws,
                          ar.ATTN_BF16, st)
    assert rc == 0
    assert dbg.attn_debug_tile_visits(got, 1) == 0
    want = expected(kernel, c, W)
    assert (got[0], got[1]) == want, f"(wave-tile pairs, staged tiles) {tuple(got)} != {want}"
