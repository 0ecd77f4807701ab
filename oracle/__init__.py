"""fp64 CPU oracle for the hybrid attention path (thin ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path (the HIP library and
its binding) never does. The arithmetic lives in ``attn_oracle.c`` (plain fp64
loops); this module only converts arrays to contiguous fp64 and calls it.

Sources: "Gemma 4: End-to-End Architecture Walkthrough" (Phase 3, sections
3a-3c), "Gemma 4 Architecture Reference" ("Attention Architecture",
"Positional Encoding: Proportional RoPE (p-RoPE)"), "Gemma 4 Technical Report"
reader ("Core Model Architecture").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# Tests that plant a mistake in a copy of the oracle point this at that build.
_LIB_OVERRIDE = os.environ.get("ATTN_ORACLE_LIB")
_lib = None

ROPE_Q = 1
ROPE_K = 2


def build() -> str:
    """Compile the C oracle with gcc (OpenMP, fp64, no HIP)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
    dp = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.oracle_rope.argtypes = [dp, dp, i64p, ctypes.c_int64, ctypes.c_int,
                                ctypes.c_int, ctypes.c_int, ctypes.c_double]
    lib.oracle_rope.restype = None
    lib.oracle_prefill.argtypes = [dp, dp, dp, dp] + [ctypes.c_int] * 7 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_double, ctypes.c_int,
        ctypes.c_int64, i32p, ctypes.c_int, ctypes.c_int]
    lib.oracle_prefill.restype = ctypes.c_int
    lib.oracle_decode_one.argtypes = [dp, dp, dp, ctypes.c_int64,
                                      ctypes.c_int64, dp] + [ctypes.c_int] * 5 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_double, ctypes.c_int]
    lib.oracle_decode_one.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _f64(a) -> np.ndarray:
    """Exact conversion of a torch tensor / array to contiguous fp64 numpy."""
    if hasattr(a, "detach"):  # torch tensor (bf16 and fp32 widen exactly)
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray, ctype=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def rope(x, positions, rotary_dims: int, theta: float) -> np.ndarray:
    """x [N, H, D] -> rotated copy (fp64). positions [N] integers."""
    lib = _load()
    x = _f64(x)
    N, H, D = x.shape
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int64).reshape(N))
    y = np.empty_like(x)
    lib.oracle_rope(_ptr(x), _ptr(y), _ptr(pos, ctypes.c_int64), N, H, D,
                    int(rotary_dims), float(theta))
    return y


def rope_2d(x, positions_xy, rotary_dims: int, theta: float) -> np.ndarray:
    """2-D RoPE for image patches, fp64: each half of the D dims is a vector
    of its own, turned like D/2-dim RoPE by one patch coordinate -- the first
    half by the width (x) coordinate, the second by the height (y) coordinate
    ("Gemma 4: End-to-End Architecture Walkthrough", Phase 1 section 1b).
    rotary_dims applies within each half. x [N, H, D]; positions_xy [N, 2]."""
    x = _f64(x)
    N, H, D = x.shape
    assert D % 4 == 0
    pxy = np.asarray(positions_xy, dtype=np.int64).reshape(N, 2)
    h = D // 2
    first = rope(np.ascontiguousarray(x[:, :, :h]), pxy[:, 0], rotary_dims, theta)
    second = rope(np.ascontiguousarray(x[:, :, h:]), pxy[:, 1], rotary_dims, theta)
    return np.concatenate([first, second], axis=2)


def prefill(q, k, v, *, window: int, scale: float, rotary_dims: int = 0,
            theta: float = 10000.0, rope_mask: int = ROPE_Q | ROPE_K,
            pos0: int = 0, rows=None, nthreads: int | None = None) -> np.ndarray:
    """Causal (optionally windowed) GQA attention, fp64.

    q [B, n_rows, Hq, Dk] holds the query rows at positions ``rows`` (all T
    rows when ``rows`` is None); k [B, T, Hkv, Dk], v [B, T, Hkv, Dv].
    Returns o [B, n_rows, Hq, Dv].
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, Hkv, Dk = k.shape
    Dv = v.shape[3]
    Hq = q.shape[2]
    if rows is None:
        rows_arr = None
        n_rows = T
        assert q.shape == (B, T, Hq, Dk)
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        n_rows = rows_arr.size
        assert q.shape == (B, n_rows, Hq, Dk)
        assert rows_arr.min(initial=0) >= 0 and rows_arr.max(initial=0) < max(T, 1)
    o = np.zeros((B, n_rows, Hq, Dv), dtype=np.float64)
    nt = nthreads or max_threads()
    rc = lib.oracle_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), B, T, Hq, Hkv, Dk, Dv, int(window),
        float(scale), int(rotary_dims), float(theta), int(rope_mask), int(pos0),
        _ptr(rows_arr, ctypes.c_int32) if rows_arr is not None else None,
        int(n_rows), int(nt))
    if rc != 0:
        raise RuntimeError("oracle_prefill failed (bad arguments or out of memory)")
    return o


def prefill_kv_shared(q, k, *, window: int, scale: float, rotary_dims: int = 0,
                      theta: float = 10000.0, pos0: int = 0, rows=None,
                      nthreads: int | None = None) -> np.ndarray:
    """Attention with the keys reused as values (K = V), fp64.

    Global layers drop the value projection and weight the key matrix itself,
    so only keys are cached ("Gemma 4: End-to-End Architecture Walkthrough",
    Phase 3 section 3b; "Gemma 4 Technical Report" reader, "Core Model
    Architecture", worked example). The pages leave open whether the values
    are the keys before or after RoPE. Reading taken: after -- the values are
    the keys exactly as Q K^T uses them, which are the rows a decode cache
    holds. q [B, n_rows, Hq, Dk], k [B, T, Hkv, Dk] (unrotated); returns
    o [B, n_rows, Hq, Dk].
    """
    k = _f64(k)
    B, T, Hkv, Dk = k.shape
    pos = np.tile(np.arange(pos0, pos0 + T, dtype=np.int64), B)
    kr = rope(k.reshape(B * T, Hkv, Dk), pos, rotary_dims, theta).reshape(B, T, Hkv, Dk)
    return prefill(q, kr, kr, window=window, scale=scale, rotary_dims=rotary_dims,
                   theta=theta, rope_mask=ROPE_Q, pos0=pos0, rows=rows, nthreads=nthreads)


def decode_one(q, k_rows, v_rows, *, kv_len: int, row0: int = 0, window: int,
               scale: float, rotary_dims: int = 0, theta: float = 10000.0,
               nthreads: int | None = None) -> np.ndarray:
    """One sequence of kv_len cache rows: q [Hq, Dk] (unrotated, position
    kv_len-1); k_rows [kv_len-row0, Hkv, Dk] (already rotated) and v_rows
    [kv_len-row0, Hkv, Dv] are cache rows row0..kv_len-1; rows before row0 must
    be outside the window. Returns o [Hq, Dv]."""
    lib = _load()
    q, k_rows, v_rows = _f64(q), _f64(k_rows), _f64(v_rows)
    Hq, Dk = q.shape
    n, Hkv, _ = k_rows.shape
    assert n == kv_len - row0 and v_rows.shape[0] == n
    Dv = v_rows.shape[2]
    o = np.zeros((Hq, Dv), dtype=np.float64)
    nt = nthreads or max_threads()
    rc = lib.oracle_decode_one(_ptr(q), _ptr(k_rows), _ptr(v_rows), int(row0),
                               int(kv_len), _ptr(o), Hq, Hkv, Dk, Dv, int(window),
                               float(scale), int(rotary_dims), float(theta), int(nt))
    if rc != 0:
        raise RuntimeError("oracle_decode_one failed (bad arguments, a visible "
                           "row before row0, or out of memory)")
    return o


def decode(q, k_cache, v_cache, row_offset, kv_len, *, window: int, scale: float,
           rotary_dims: int = 0, theta: float = 10000.0, seqs=None,
           nthreads: int | None = None) -> np.ndarray:
    """Ragged-cache decode: q [B, Hq, Dk]; caches [rows, Hkv, D]; sequence b
    occupies cache rows row_offset[b] .. row_offset[b] + kv_len[b] - 1.
    Only the rows inside the window are handed over (the oracle checks that the
    rest are invisible), and only the sequences in ``seqs`` (default: all) are
    computed. Returns [len(seqs), Hq, Dv].
    """
    row_offset = [int(x) for x in (row_offset.tolist() if hasattr(row_offset, "tolist") else row_offset)]
    kv_len = [int(x) for x in (kv_len.tolist() if hasattr(kv_len, "tolist") else kv_len)]
    if seqs is None:
        seqs = range(len(kv_len))
    outs = []
    for b in seqs:
        n = kv_len[b]
        lo = max(0, n - window) if window > 0 else 0
        off = row_offset[b]
        outs.append(decode_one(q[b], k_cache[off + lo: off + n],
                               v_cache[off + lo: off + n], kv_len=n, row0=lo,
                               window=window, scale=scale, rotary_dims=rotary_dims,
                               theta=theta, nthreads=nthreads))
    Hq = q.shape[1]
    Dv = v_cache.shape[2]
    return np.stack(outs) if outs else np.zeros((0, Hq, Dv))


def verify(q, k_cache, v_cache, row_offset, kv_len, *, window: int, scale: float,
           rotary_dims: int = 0, theta: float = 10000.0, seqs=None,
           nthreads: int | None = None) -> np.ndarray:
    """Several new tokens per sequence checked in one pass (speculative
    decoding's verify step: "Gemma 4: End-to-End Architecture Walkthrough",
    Phase 4; "Gemma 4 Technical Report" reader, "Speculative Decoding and
    Infrastructure"). q [B, n_q, Hq, Dk]; sequence b's last n_q cache rows are
    the new tokens, token j at position kv_len[b] - n_q + j. By definition
    each token is a one-token decode over the cache prefix that ends at its
    own row (causal within the draft). Returns [len(seqs), n_q, Hq, Dv].
    """
    kv_len = [int(x) for x in (kv_len.tolist() if hasattr(kv_len, "tolist") else kv_len)]
    row_offset = [int(x) for x in (row_offset.tolist() if hasattr(row_offset, "tolist") else row_offset)]
    n_q, Hq = q.shape[1], q.shape[2]
    Dv = v_cache.shape[2]
    if seqs is None:
        seqs = range(len(kv_len))
    out = []
    for b in seqs:
        n = kv_len[b]
        if n == 0:
            out.append(np.zeros((n_q, Hq, Dv)))
            continue
        if n < n_q:
            raise RuntimeError("verify: kv_len smaller than the number of new tokens")
        rows = []
        for j in range(n_q):
            m = n - n_q + j + 1  # the prefix that token j sees ends at its own row
            lo = max(0, m - window) if window > 0 else 0
            off = row_offset[b]
            rows.append(decode_one(q[b, j], k_cache[off + lo: off + m],
                                   v_cache[off + lo: off + m], kv_len=m, row0=lo,
                                   window=window, scale=scale, rotary_dims=rotary_dims,
                                   theta=theta, nthreads=nthreads))
        out.append(np.stack(rows))
    return np.stack(out) if out else np.zeros((0, n_q, Hq, Dv))


def cross_attend(q, k_cache, v_cache, row_offset, kv_len, q_pos, *, window: int,
                 scale: float, rotary_dims: int = 0, theta: float = 10000.0) -> np.ndarray:
    """A drafter's attention into the target model's KV cache ("Gemma 4:
    End-to-End Architecture Walkthrough", Phase 4: the MTP drafter attends the
    target's already-computed cache instead of keeping one of its own), fp64.

    q [B, Hq, Dk] unrotated; sequence b's query sits at position q_pos[b]
    (>= kv_len[b] - 1: the drafted tokens lie past the cache) and is rotated
    there. Cache rows row_offset[b] .. row_offset[b] + kv_len[b] - 1 hold the
    target's keys (already rotated) and values for positions 0 .. kv_len[b]-1.
    Row r is visible when r < kv_len[b] and, for window > 0, q_pos[b] - r <
    window. KV head of query head h: h // (Hq / Hkv). With no visible row the
    output is 0. Softmax in two passes (max, then exp and sums), plain numpy.
    Returns [B, Hq, Dv].
    """
    q = _f64(q)
    B, Hq, Dk = q.shape
    Hkv, Dv = k_cache.shape[1], v_cache.shape[2]
    G = Hq // Hkv
    row_offset = [int(x) for x in (row_offset.tolist() if hasattr(row_offset, "tolist") else row_offset)]
    kv_len = [int(x) for x in (kv_len.tolist() if hasattr(kv_len, "tolist") else kv_len)]
    q_pos = [int(x) for x in (q_pos.tolist() if hasattr(q_pos, "tolist") else q_pos)]
    qr = rope(q, q_pos, rotary_dims, theta)
    out = np.zeros((B, Hq, Dv), dtype=np.float64)
    for b in range(B):
        n, off, p = kv_len[b], row_offset[b], q_pos[b]
        assert p >= n - 1, "the query lies past the cache"
        lo = max(0, p - window + 1) if window > 0 else 0
        if lo >= n:
            continue
        K = _f64(k_cache[off + lo: off + n])
        V = _f64(v_cache[off + lo: off + n])
        for h in range(Hq):
            g = h // G
            s = scale * (K[:, g, :] @ qr[b, h])
            e = np.exp(s - s.max())
            out[b, h] = (e @ V[:, g, :]) / e.sum()
    return out


# ---- int8 KV cache --------------------------------------------------------
# The pages name int8 KV caching ("Gemma 4 Technical Report" reader,
# "Quantization and Efficiency", Table 3 caption) but give no scheme. Reading
# taken: symmetric codes with one scale per (cache row, KV head),
# s = max|x| / 127 and code = round-half-even(x / s). The codes are integers
# that floating point decides, so this function takes those decisions in the
# kernel's precision (fp32, IEEE division) rather than fp64; everything after
# dequantisation is fp64.

def kv_quantize_int8(x):
    """x [N, H, D] (the stored values, e.g. bf16) -> (codes int8 [N, H, D],
    scales float32 [N, H]). A row of zeros gets scale 0 and codes 0."""
    x32 = np.asarray(x.float() if hasattr(x, "float") else x, dtype=np.float32)
    amax = np.abs(x32).max(axis=-1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    code = np.rint(x32 / safe[..., None]).astype(np.float32)
    code = np.where(s[..., None] > 0, code, np.float32(0.0))
    return code.astype(np.int8), s


def kv_dequantize_int8(codes, scales) -> np.ndarray:
    """codes [N, H, D] int8, scales [N, H] -> fp64 values code * scale."""
    c = np.asarray(codes.cpu() if hasattr(codes, "cpu") else codes).astype(np.float64)
    s = np.asarray(scales.cpu() if hasattr(scales, "cpu") else scales).astype(np.float64)
    return c * s[..., None]


def decode_int8(q, k_codes, k_scales, v_codes, v_scales, row_offset, kv_len, *,
                window: int, scale: float, rotary_dims: int = 0, theta: float = 10000.0,
                seqs=None, nthreads: int | None = None) -> np.ndarray:
    """Decode over an int8 cache: the plain decode of the dequantised rows."""
    return decode(q, kv_dequantize_int8(k_codes, k_scales),
                  kv_dequantize_int8(v_codes, v_scales), row_offset, kv_len, window=window,
                  scale=scale, rotary_dims=rotary_dims, theta=theta, seqs=seqs,
                  nthreads=nthreads)
