"""Host-side checks of the C ABI (no GPU needed, no compute calls).

The library must load, export every symbol include/attn_rope.h declares, and
reject invalid arguments with the right status before any HIP call.
"""
import ctypes
import os
import re

import pytest

import attention_rope_amd as ar

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "attn_rope.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ar.LIB_PATH):
        from attention_rope_amd import _build
        _build.build()
    return ar.load()


def _declared():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    return sorted({n for n in names if n.startswith(("attn_", "prope_"))})


def test_header_symbols_exported(lib):
    names = _declared()
    assert set(names) == set(ar.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s, text in ar.STATUS.items():
        assert lib.attn_status_string(s).decode() == text
    assert lib.attn_status_string(99).decode() == "unknown status"


R = ar._Rope
P = ctypes.c_void_p
FAKE = P(0x10000)      # never dereferenced: every call below fails validation
FAKE2 = P(0x20000000)


def _prefill(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE2, B=1, T=8, Hq=4, Hkv=2, Dk=64, Dv=64,
             window=0, scale=0.125, rope=R(0, 1e4), rope_mask=3, pos0=0, ws=None,
             ws_bytes=0, dtype=ar.ATTN_BF16, stream=None)
    a.update(kw)
    return lib.attn_prefill(a["q"], a["k"], a["v"], a["o"], a["B"], a["T"], a["Hq"],
                            a["Hkv"], a["Dk"], a["Dv"], a["window"], a["scale"], a["rope"],
                            a["rope_mask"], a["pos0"], a["ws"], a["ws_bytes"], a["dtype"],
                            a["stream"])


def test_prefill_validation(lib):
    assert _prefill(lib, q=None) == 1
    assert _prefill(lib, Hq=3, Hkv=2) == 2
    assert _prefill(lib, Dk=63) == 2
    assert _prefill(lib, Dk=1024) == 2
    assert _prefill(lib, scale=float("nan")) == 2
    assert _prefill(lib, rope=R(3, 1e4)) == 2
    assert _prefill(lib, rope=R(66, 1e4)) == 2
    assert _prefill(lib, rope=R(32, -1.0)) == 2
    assert _prefill(lib, rope_mask=4) == 2
    assert _prefill(lib, dtype=7) == 3
    assert _prefill(lib, o=FAKE) == 6                 # o aliases q
    assert _prefill(lib, q=P(0x10001)) == 2          # misaligned
    # positions pos0 .. pos0+T-1 must stay in [0, 2^31 - 1)
    assert _prefill(lib, pos0=-1) == 2
    assert _prefill(lib, pos0=2**31 - 8, T=8) == 2
    assert b"pos0" in lib.attn_last_error()
    # empty problems are a no-op success, even with NULL pointers
    assert _prefill(lib, q=None, k=None, v=None, o=None, T=0) == 0
    assert lib.attn_last_error() == b""


def test_prefill_workspace(lib):
    """Whenever K turns, its rotary dims [B, T, Hkv, R] in the call's element
    type; nothing otherwise (every angle is formed in-kernel)."""
    ws = lib.attn_prefill_workspace_bytes
    assert ws(2, 8, 4, 128, R(32, 1e6), 3, ar.ATTN_BF16) == 2 * 8 * 4 * 32 * 2
    assert ws(2, 8, 4, 256, R(256, 1e4), 2, ar.ATTN_BF16) == 2 * 8 * 4 * 256 * 2
    assert ws(2, 8, 4, 128, R(32, 1e6), 3, ar.ATTN_F32) == 2 * 8 * 4 * 32 * 4
    assert ws(2, 8, 4, 128, R(6, 1e6), 2, ar.ATTN_BF16) == 2 * 8 * 4 * 6 * 2
    # nothing to turn ahead: q only, no rope, empty, bad dtype or width
    assert ws(2, 8, 4, 128, R(32, 1e6), 1, ar.ATTN_BF16) == 0
    assert ws(2, 8, 4, 128, R(0, 1e6), 3, ar.ATTN_BF16) == 0
    assert ws(0, 8, 4, 128, R(32, 1e6), 3, ar.ATTN_BF16) == 0
    assert ws(2, 8, 4, 128, R(32, 1e6), 3, 9) == 0
    assert ws(2, 8, 4, 128, R(130, 1e6), 3, ar.ATTN_BF16) == 0
    kw = dict(Dk=128, Dv=128, rope=R(32, 1e6))
    need = 1 * 8 * 2 * 32 * 2
    assert _prefill(lib, **kw) == 4                                   # missing
    assert _prefill(lib, ws=P(0x50000000), ws_bytes=need - 1, **kw) == 4  # too small
    assert b"workspace" in lib.attn_last_error()
    assert _prefill(lib, ws=P(0x50000008), ws_bytes=need, **kw) == 2    # misaligned
    assert _prefill(lib, ws=FAKE, ws_bytes=need, **kw) == 6             # overlaps q/k/v
    assert _prefill(lib, ws=FAKE2, ws_bytes=need, **kw) == 6            # overlaps o
    assert _prefill(lib, dtype=ar.ATTN_F32, **kw) == 4                  # fp32 turns K too
    # q-only rotation needs no workspace (the NULL q is what fails)
    assert _prefill(lib, rope=R(32, 1e4), rope_mask=1, q=None) == 1


def _into_cache(lib, **kw):
    a = dict(q=P(0x10000), k=P(0x20000), v=P(0x30000), o=P(0x40000), B=2, T=8, Hq=4, Hkv=2,
             Dk=64, Dv=64, window=0, scale=0.125, rope=R(16, 1e4), pos0=0,
             kc=P(0x1000000), vc=P(0x2000000), off=P(0x3000000), rows=100,
             ws=P(0x4000000), ws_bytes=1 << 20, dtype=ar.ATTN_BF16, stream=None)
    a.update(kw)
    return lib.attn_prefill_into_cache(a["q"], a["k"], a["v"], a["o"], a["B"], a["T"], a["Hq"],
                                       a["Hkv"], a["Dk"], a["Dv"], a["window"], a["scale"],
                                       a["rope"], a["pos0"], a["kc"], a["vc"], a["off"],
                                       a["rows"], a["ws"], a["ws_bytes"], a["dtype"],
                                       a["stream"])


def test_prefill_into_cache_validation(lib):
    """The cache-filling prefill checks everything attn_prefill checks, plus
    its caches (present, aligned, disjoint from every other buffer and from
    each other), row_offset and the 8-dim granularity of its K/V pass."""
    assert _into_cache(lib, kc=None) == 1
    assert _into_cache(lib, vc=None) == 1
    assert _into_cache(lib, off=None) == 1
    assert _into_cache(lib, q=None) == 1
    assert _into_cache(lib, Dk=60, Dv=60, rope=R(0, 1e4)) == 2      # not a multiple of 8
    assert _into_cache(lib, rope=R(12, 1e4)) == 2
    assert _into_cache(lib, rows=7) == 2                            # fewer rows than T
    assert _into_cache(lib, kc=P(0x1000008)) == 2                   # misaligned cache
    assert _into_cache(lib, off=P(0x3000004)) == 2                  # misaligned row_offset
    assert _into_cache(lib, kc=P(0x10000)) == 6                     # cache over q
    assert _into_cache(lib, vc=P(0x1000000 + 64)) == 6              # caches overlap
    assert _into_cache(lib, off=P(0x1000000 + 8)) == 6              # row_offset in the cache
    assert _into_cache(lib, ws=P(0x1000000)) == 6                   # workspace in the cache
    assert b"prefill_into_cache" in lib.attn_last_error()
    assert _into_cache(lib, ws=None, ws_bytes=0) == 4               # K turns: workspace
    assert _into_cache(lib, dtype=7) == 3
    assert _into_cache(lib, B=0, q=None, kc=None) == 0              # empty: no-op


def _decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, off=FAKE, kvl=FAKE, o=FAKE2, B=2, Hq=8, Hkv=1,
             Dk=128, Dv=128, window=0, scale=0.1, rope=R(32, 1e6), max_kv_len=100,
             ws=P(0x40000000), ws_bytes=1 << 30, dtype=ar.ATTN_BF16, stream=None)
    a.update(kw)
    return lib.attn_decode(a["q"], a["k"], a["v"], a["off"], a["kvl"], a["o"], a["B"],
                           a["Hq"], a["Hkv"], a["Dk"], a["Dv"], a["window"], a["scale"],
                           a["rope"], a["max_kv_len"], a["ws"], a["ws_bytes"], a["dtype"],
                           a["stream"])


def test_decode_validation(lib):
    assert _decode(lib, dtype=ar.ATTN_F32) == 3
    assert _decode(lib, kvl=None) == 1
    assert _decode(lib, Dk=64) == 3
    assert _decode(lib, Hq=34, Hkv=2) == 3          # 17 heads per KV head
    assert _decode(lib, Hq=7, Hkv=2) == 2
    assert _decode(lib, max_kv_len=0) == 2
    assert _decode(lib, scale=-1.0) == 3
    assert _decode(lib, ws_bytes=16) == 4
    assert _decode(lib, ws=None) == 4
    assert _decode(lib, o=FAKE) == 6
    assert _decode(lib, B=0, q=None) == 0
    assert _decode(lib, Dk=256, Dv=512) == 3        # 512-dim values need 512-dim keys
    assert _decode(lib, B=1, max_kv_len=2**31 - 1) == 2   # > 65535 chunks of 8192 rows
    assert b"too large" in lib.attn_last_error()


def test_decode_workspace_bytes(lib):
    """Chunks: up to 4096 rows (global) or the whole window (local), halved
    (down to 256) while B * Hkv * splits < 512."""
    ws = lib.attn_decode_workspace_bytes
    assert ws(64, 32, 4, 256, 131073, 0) == 64 * 32 * 33 * 258 * 4      # 4096-row chunks
    assert ws(64, 16, 8, 256, 131073, 1024) == 64 * 16 * 1 * 258 * 4    # one 1024-row window
    assert ws(1, 32, 4, 256, 131072, 0) == 1 * 32 * 128 * 258 * 4       # 1024-row chunks
    assert ws(8, 16, 8, 256, 131073, 1024) == 8 * 16 * 4 * 258 * 4      # 256-row chunks
    assert ws(1, 8, 1, 128, 300, 0) == 1 * 8 * 2 * 130 * 4              # floor of 256 rows
    assert ws(0, 16, 8, 256, 10, 0) == 0


def test_prope_validation(lib):
    f = lambda **kw: lib.prope_apply(kw.get("x", FAKE), kw.get("y", FAKE2),
                                     kw.get("pos", FAKE), kw.get("N", 4), kw.get("H", 2),
                                     kw.get("D", 64), kw.get("rope", R(16, 1e4)),
                                     kw.get("dtype", ar.ATTN_BF16), None)
    assert f(x=None) == 1
    assert f(D=63) == 2
    assert f(rope=R(80, 1e4)) == 2
    assert f(y=P(0x10000 + 64)) == 6                 # partial overlap
    assert f(dtype=5) == 3
    assert f(N=0) == 0


def test_verify_validation_and_workspace(lib):
    ws = lib.attn_verify_workspace_bytes
    q_region = 64 * 2 * 32 * 512 * 2
    assert ws(64, 2, 32, 4, 512, 256, 131073, 0) == q_region + 64 * 2 * 32 * 33 * 258 * 4
    # 20 tokens x 1 head: two 16-column groups; 256-row chunks over 300 rows
    assert ws(1, 20, 2, 2, 128, 128, 300, 0) == 10240 + 1 * 20 * 2 * 2 * 130 * 4
    assert ws(0, 2, 32, 4, 512, 256, 10, 0) == 0

    def verify(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, off=FAKE, kvl=FAKE, o=FAKE2, B=2, n_q=3, Hq=8, Hkv=1,
                 Dk=128, Dv=128, window=0, scale=0.1, rope=R(32, 1e6), max_kv_len=100,
                 ws=P(0x40000000), ws_bytes=1 << 30, dtype=ar.ATTN_BF16, stream=None)
        a.update(kw)
        return lib.attn_verify(a["q"], a["k"], a["v"], a["off"], a["kvl"], a["o"], a["B"],
                               a["n_q"], a["Hq"], a["Hkv"], a["Dk"], a["Dv"], a["window"],
                               a["scale"], a["rope"], a["max_kv_len"], a["ws"], a["ws_bytes"],
                               a["dtype"], a["stream"])
    assert verify(n_q=0) == 2
    assert verify(n_q=5000) == 2
    assert verify(Dk=64) == 3
    assert verify(kvl=None) == 1
    assert verify(ws_bytes=16) == 4
    assert verify(dtype=ar.ATTN_F32) == 3
    assert verify(B=0, q=None) == 0


def test_decode_noalloc_validation(lib):
    """The entry point that allocates nothing rejects, before touching the GPU,
    a call whose split-K partials exceed its static scratch, and validates the
    other arguments as attn_decode does."""
    assert lib.attn_decode_noalloc_max_bytes() == 32 << 20
    f = lambda **kw: lib.attn_decode_noalloc(
        kw.get("q", FAKE), FAKE, FAKE, FAKE, kw.get("kvl", FAKE), kw.get("o", FAKE2),
        kw.get("B", 64), 32, 4, 512, 256, 0, 0.05, R(128, 1e6), kw.get("max_kv_len", 131073),
        kw.get("dtype", ar.ATTN_BF16), None)
    # 64 sequences up to 131073 rows: 33 chunks of 4096 rows -> ~70 MB of partials
    assert f() == 4
    assert b"scratch" in lib.attn_last_error()
    assert lib.attn_decode_workspace_bytes(64, 32, 4, 256, 131073, 0) > 32 << 20
    assert f(B=1, kvl=None) == 1                      # fits; a NULL kv_len is caught first
    assert f(B=1, dtype=ar.ATTN_F32) == 3
    assert f(B=1, max_kv_len=0) == 2
    assert f(B=0, q=None) == 0                        # empty batch: no-op


def test_no_device_is_a_launch_error(lib):
    """With no GPU present, a call that passes validation reaches the HIP
    runtime, which refuses it: ATTN_ERR_LAUNCH with the runtime's message, no
    crash. (Skipped where a GPU is visible: the pointers here are fake.)"""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible")
    rc = _prefill(lib, q=P(0x10000), k=P(0x20000), v=P(0x30000), o=P(0x40000))
    assert rc == 5
    assert b"HIP error" in lib.attn_last_error()
    rc = lib.attn_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE2, 1, 8, 1, 128, 128, 0, 0.1,
                                 R(0, 1e4), 10, ar.ATTN_BF16, None)
    assert rc == 5
    assert lib.attn_status_string(rc) == b"kernel launch failed"
