"""Comparison helpers for the GPU-vs-oracle parity tests."""
import numpy as np
import torch

# Tolerances: bf16 results within max-abs 2e-2 and rel-RMS 1e-2 of the fp64
# oracle; fp32 results within 1e-4 (both measures).
TOL = {torch.bfloat16: (2e-2, 1e-2), torch.float32: (1e-4, 1e-4)}


def to64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").double().numpy()
    return np.asarray(t, dtype=np.float64)


def errors(got, ref):
    g, r = to64(got), to64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    d = np.abs(g - r)
    rel = float(np.sqrt((d ** 2).sum() / max((r ** 2).sum(), 1e-300)))
    return float(d.max(initial=0.0)), rel


def assert_close(got, ref, dtype, what=""):
    atol, rtol = TOL[dtype]
    g = to64(got)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    mx, rel = errors(g, ref)
    assert mx <= atol and rel <= rtol, f"{what}: max_abs={mx:.3e} rel_rms={rel:.3e}"
    return mx, rel
