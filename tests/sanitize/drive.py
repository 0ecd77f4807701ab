"""Child process of tests/test_sanitize.py, run with AddressSanitizer preloaded:
drives a sanitizer build of the ABI layer (abi.cpp + plan.cpp, kernel
launchers stubbed) through its validation and dispatch paths, and the
sanitizer build of the fp64 oracle (ATTN_ORACLE_LIB) on small problems.
Any sanitizer report aborts the process with a non-zero status."""
import ctypes
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)


class Rope(ctypes.Structure):
    _fields_ = [("rotary_dims", ctypes.c_int32), ("theta", ctypes.c_double)]


def abi_paths(path):
    L = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.attn_prefill.argtypes = [vp] * 4 + [i32] * 7 + [ctypes.c_float, Rope, i32, i32, vp, sz,
                                                       ctypes.c_int, vp]
    L.attn_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32, Rope, i32, ctypes.c_int]
    L.attn_prefill_workspace_bytes.restype = sz
    L.attn_decode.argtypes = [vp] * 6 + [i32] * 6 + [ctypes.c_float, Rope, i32, vp, sz,
                                                      ctypes.c_int, vp]
    L.attn_decode_workspace_bytes.argtypes = [i32] * 6
    L.attn_decode_workspace_bytes.restype = sz
    L.attn_verify.argtypes = [vp] * 6 + [i32] * 7 + [ctypes.c_float, Rope, i32, vp, sz,
                                                      ctypes.c_int, vp]
    L.attn_verify_workspace_bytes.argtypes = [i32] * 8
    L.attn_verify_workspace_bytes.restype = sz
    L.attn_decode_noalloc.argtypes = [vp] * 6 + [i32] * 6 + [ctypes.c_float, Rope, i32,
                                                              ctypes.c_int, vp]
    L.attn_decode_int8.argtypes = [vp] * 8 + [i32] * 6 + [ctypes.c_float, Rope, i32, vp, sz, vp]
    L.attn_decode_int8_workspace_bytes.argtypes = [i32] * 6
    L.attn_decode_int8_workspace_bytes.restype = sz
    L.attn_kv_quantize_int8.argtypes = [vp, vp, vp, i32, i32, i32, ctypes.c_int, vp]
    L.prope_apply.argtypes = [vp, vp, vp, i32, i32, i32, Rope, ctypes.c_int, vp]
    L.prope_apply_2d.argtypes = [vp, vp, vp, i32, i32, i32, Rope, ctypes.c_int, vp]
    L.attn_last_error.restype = ctypes.c_char_p
    L.attn_status_string.restype = ctypes.c_char_p
    L.stub_launches.restype = ctypes.c_int
    P = vp
    A, B_, C, D, E, F, WS = (P(0x10000 * (i + 1)) for i in range(7))
    BIG = 1 << 40
    n = 0
    # prefill: every rejection path, then valid calls of each dispatch branch
    for kw in [dict(q=None), dict(Hq=3), dict(Dk=63), dict(Dk=1024), dict(scale=float("nan")),
               dict(rope=Rope(3, 1e4)), dict(rope=Rope(32, -1.0)), dict(rope_mask=4), dict(dtype=7),
               dict(o=A), dict(q=P(0x10001)), dict(pos0=-1), dict(pos0=2**31 - 4),
               dict(rope=Rope(32, 1e4))]:
        a = dict(q=A, k=B_, v=C, o=D, B=1, T=8, Hq=4, Hkv=2, Dk=64, Dv=64, window=0, scale=0.1,
                 rope=Rope(0, 1e4), rope_mask=3, pos0=0, ws=None, wsb=0, dtype=1)
        a.update(kw)
        rc = L.attn_prefill(a["q"], a["k"], a["v"], a["o"], a["B"], a["T"], a["Hq"], a["Hkv"],
                            a["Dk"], a["Dv"], a["window"], a["scale"], a["rope"], a["rope_mask"],
                            a["pos0"], a["ws"], a["wsb"], a["dtype"], None)
        assert rc != 0, kw
        L.attn_last_error()
    for (B, T, Hq, Hkv, Dk, Dv, W, R, dt) in [(2, 300, 32, 4, 512, 256, 0, 128, 1),
                                              (4, 4096, 16, 8, 256, 256, 512, 256, 1),
                                              (1, 333, 8, 1, 128, 128, 17, 32, 0),
                                              (1, 50, 6, 3, 96, 64, 9, 32, 1),
                                              (1, 64, 16, 2, 512, 512, 0, 512, 1)]:
        need = L.attn_prefill_workspace_bytes(B, T, Hkv, Dk, Rope(R, 1e6), 3, dt)
        rc = L.attn_prefill(A, B_, C, P(BIG), B, T, Hq, Hkv, Dk, Dv, W, Dk ** -0.5, Rope(R, 1e6), 3,
                            5, P(BIG * 2) if need else None, need, dt, None)
        assert rc == 0, (rc, L.attn_last_error())
        n += 1
    # decode / verify / no-alloc / int8: rejections and valid calls
    for maxl, W in [(131073, 0), (131073, 1024), (300, 0), (1, 0)]:
        need = L.attn_decode_workspace_bytes(64, 32, 4, 256, maxl, W)
        assert L.attn_decode(A, B_, C, E, F, P(BIG), 64, 32, 4, 512, 256, W, 0.05,
                             Rope(128, 1e6), maxl, P(BIG * 2), need, 1, None) == 0
        assert L.attn_decode(A, B_, C, E, F, P(BIG), 64, 32, 4, 512, 256, W, 0.05,
                             Rope(128, 1e6), maxl, P(BIG * 2), max(need - 1, 0), 1, None) == 4
        vneed = L.attn_verify_workspace_bytes(64, 3, 32, 4, 512, 256, maxl, W)
        assert L.attn_verify(A, B_, C, E, F, P(BIG), 64, 3, 32, 4, 512, 256, W, 0.05,
                             Rope(128, 1e6), maxl, P(BIG * 2), vneed, 1, None) == 0
        rc = L.attn_decode_noalloc(A, B_, C, E, F, P(BIG), 64, 32, 4, 512, 256, W, 0.05,
                                   Rope(128, 1e6), maxl, 1, None)
        assert rc in (0, 4), rc
        ineed = L.attn_decode_int8_workspace_bytes(64, 32, 4, 256, maxl, W)
        assert L.attn_decode_int8(A, B_, P(0x7000), C, P(0x8000), E, F, P(BIG), 64, 32, 4, 512,
                                  256, W, 0.05, Rope(128, 1e6), maxl, P(BIG * 2), ineed, None) == 0
        n += 4
    for kw in [dict(B=-1), dict(Hq=7, Hkv=2), dict(Dk=64), dict(maxl=0), dict(scale=-1.0)]:
        a = dict(B=2, Hq=8, Hkv=1, Dk=128, Dv=128, maxl=100, scale=0.1)
        a.update(kw)
        assert L.attn_decode(A, B_, C, E, F, P(BIG), a["B"], a["Hq"], a["Hkv"], a["Dk"], a["Dv"], 0,
                             a["scale"], Rope(32, 1e6), a["maxl"], P(BIG * 2), 1 << 30, 1, None) != 0
    assert L.attn_kv_quantize_int8(A, P(BIG), P(BIG * 2), 1000, 4, 512, 1, None) == 0
    assert L.prope_apply(A, P(BIG), E, 100, 4, 512, Rope(128, 1e6), 1, None) == 0
    assert L.prope_apply_2d(A, P(BIG), E, 100, 4, 512, Rope(64, 1e4), 0, None) == 0
    assert L.prope_apply(A, A, E, 100, 4, 512, Rope(0, 1e6), 1, None) == 0
    for s in range(-1, 9):
        L.attn_status_string(s)
    assert L.stub_launches() > n
    print("abi paths ok:", L.stub_launches(), "stub launches", flush=True)


def oracle_paths():
    import oracle
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 40, 8, 64))
    k = rng.standard_normal((2, 40, 2, 64))
    v = rng.standard_normal((2, 40, 2, 32))
    for W, R in [(0, 64), (7, 16), (1, 0)]:
        o = oracle.prefill(q, k, v, window=W, scale=0.125, rotary_dims=R, theta=1e4, pos0=3)
        assert np.isfinite(o).all()
    rows = np.array([0, 5, 39], dtype=np.int32)
    oracle.prefill(q[:, rows], k, v, window=0, scale=0.125, rotary_dims=64, theta=1e4, rows=rows)
    kc = rng.standard_normal((30, 2, 64))
    vc = rng.standard_normal((30, 2, 32))
    oracle.decode_one(q[0, 0], kc, vc, kv_len=30, window=0, scale=0.1, rotary_dims=32, theta=1e6)
    oracle.decode_one(q[0, 0], kc[20:], vc[20:], kv_len=30, row0=20, window=10, scale=0.1)
    oracle.rope(k[0], np.arange(40), 32, 1e4)
    print("oracle paths ok", flush=True)


if __name__ == "__main__":
    abi_paths(sys.argv[1])
    oracle_paths()
