"""Python binding of the MI355X hybrid-attention library (libattn_rope.so).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. torch provides device memory and the current stream. The entry
points mirror the C ABI in include/attn_rope.h:

    prefill(q, k, v, *, window, scale, rotary_dims, theta, rope_mask, pos0)
    verify(q, k_cache, v_cache, row_offset, kv_len, *, ...)
    kv_quantize_int8(x), decode_int8(q, k_codes, k_scales, v_codes, v_scales, ...)
    prope_2d(x, positions_xy, *, rotary_dims, theta)
    decode(q, k_cache, v_cache, row_offset, kv_len, *, window, scale,
           rotary_dims, theta, max_kv_len)
    prope(x, positions, *, rotary_dims, theta, out=None)

There is no CPU fallback: if the shared library is missing or fails to load,
every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # imported first so the HIP runtime torch ships is the one in use

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn_rope.so")

ATTN_F32, ATTN_BF16 = 0, 1
ROPE_Q, ROPE_K = 1, 2
STATUS = {0: "ok", 1: "null pointer", 2: "invalid shape or argument",
          3: "unsupported configuration", 4: "workspace missing or too small",
          5: "kernel launch failed", 6: "output overlaps an input"}

# Every symbol the header declares (checked by the tests).
EXPORTS = ("attn_prefill", "attn_prefill_into_cache",
           "attn_prefill_workspace_bytes", "attn_decode",
           "attn_decode_workspace_bytes", "attn_decode_noalloc", "attn_decode_noalloc_max_bytes",
           "attn_verify", "attn_verify_workspace_bytes",
           "attn_kv_quantize_int8", "attn_decode_int8", "attn_decode_int8_workspace_bytes",
           "prope_apply", "prope_apply_2d", "attn_status_string", "attn_last_error")


class AttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class _Rope(ctypes.Structure):
    _fields_ = [("rotary_dims", ctypes.c_int32), ("theta", ctypes.c_double)]


_lib = None


def load(path: str = LIB_PATH):
    """Load the shared library (once). Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m attention_rope_amd._build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.attn_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32, _Rope, i32, ctypes.c_int]
    lib.attn_prefill_workspace_bytes.restype = sz
    lib.attn_prefill.argtypes = [vp, vp, vp, vp] + [i32] * 7 + [
        ctypes.c_float, _Rope, i32, i32, vp, sz, ctypes.c_int, vp]
    lib.attn_prefill.restype = ctypes.c_int
    lib.attn_prefill_into_cache.argtypes = [vp, vp, vp, vp] + [i32] * 7 + [
        ctypes.c_float, _Rope, i32, vp, vp, vp, ctypes.c_int64, vp, sz, ctypes.c_int, vp]
    lib.attn_prefill_into_cache.restype = ctypes.c_int
    lib.attn_decode_workspace_bytes.argtypes = [i32] * 6
    lib.attn_decode_workspace_bytes.restype = sz
    lib.attn_decode.argtypes = [vp] * 6 + [i32] * 6 + [
        ctypes.c_float, _Rope, i32, vp, sz, ctypes.c_int, vp]
    lib.attn_decode.restype = ctypes.c_int
    lib.attn_decode_noalloc_max_bytes.argtypes = []
    lib.attn_decode_noalloc_max_bytes.restype = sz
    lib.attn_decode_noalloc.argtypes = [vp] * 6 + [i32] * 6 + [
        ctypes.c_float, _Rope, i32, ctypes.c_int, vp]
    lib.attn_decode_noalloc.restype = ctypes.c_int
    lib.attn_verify_workspace_bytes.argtypes = [i32] * 8
    lib.attn_verify_workspace_bytes.restype = sz
    lib.attn_verify.argtypes = [vp] * 6 + [i32] * 7 + [
        ctypes.c_float, _Rope, i32, vp, sz, ctypes.c_int, vp]
    lib.attn_verify.restype = ctypes.c_int
    lib.prope_apply.argtypes = [vp, vp, vp, i32, i32, i32, _Rope, ctypes.c_int, vp]
    lib.prope_apply.restype = ctypes.c_int
    lib.attn_kv_quantize_int8.argtypes = [vp, vp, vp, i32, i32, i32, ctypes.c_int, vp]
    lib.attn_kv_quantize_int8.restype = ctypes.c_int
    lib.attn_decode_int8_workspace_bytes.argtypes = [i32] * 6
    lib.attn_decode_int8_workspace_bytes.restype = sz
    lib.attn_decode_int8.argtypes = [vp] * 8 + [i32] * 6 + [
        ctypes.c_float, _Rope, i32, vp, sz, vp]
    lib.attn_decode_int8.restype = ctypes.c_int
    lib.prope_apply_2d.argtypes = [vp, vp, vp, i32, i32, i32, _Rope, ctypes.c_int, vp]
    lib.prope_apply_2d.restype = ctypes.c_int
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise AttnError(rc, _lib.attn_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _need_dims(t: torch.Tensor, n: int, name: str):
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dims, got shape {tuple(t.shape)}")


def _need_shape(t: torch.Tensor, shape, name: str):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _same_device(ref: torch.Tensor, ref_name: str, **others):
    for name, t in others.items():
        if t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, {ref_name} on {ref.device}")


def _same(ref: torch.Tensor, ref_name: str, **others):
    """Same device, and for the float tensors the same dtype, as ``ref``."""
    _same_device(ref, ref_name, **others)
    for name, t in others.items():
        if t.is_floating_point() and t.dtype != ref.dtype:
            raise TypeError(f"{name} is {t.dtype}, {ref_name} is {ref.dtype}")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def prefill_workspace_bytes(B: int, T: int, Hkv: int, Dk: int, *, rotary_dims: int,
                            theta: float = 10000.0, rope_mask: int = 3,
                            dtype=torch.bfloat16) -> int:
    code = 0 if dtype == torch.float32 else 1
    return int(load().attn_prefill_workspace_bytes(B, T, Hkv, Dk, _Rope(rotary_dims, theta),
                                                   rope_mask, code))


def prefill(q, k, v, *, window: int = 0, scale: float | None = None,
            rotary_dims: int = 0, theta: float = 10000.0,
            rope_mask: int = ROPE_Q | ROPE_K, pos0: int = 0, out=None, workspace=None):
    """q [B,T,Hq,Dk], k [B,T,Hkv,Dk], v [B,T,Hkv,Dv] -> o [B,T,Hq,Dv].

    Token t sits at position pos0 + t. ``workspace`` is a device byte buffer
    of at least prefill_workspace_bytes() (K's turned rotary dims); allocated
    here when not given."""
    lib = load()
    _need_dims(q, 4, "q")
    _need_dims(k, 4, "k")
    _need_dims(v, 4, "v")
    B, T, Hq, Dk = q.shape
    Hkv, Dv = k.shape[2], v.shape[3]
    if tuple(k.shape) != (B, T, Hkv, Dk) or tuple(v.shape) != (B, T, Hkv, Dv):
        raise ValueError(f"q/k/v shapes disagree: {tuple(q.shape)} {tuple(k.shape)} "
                         f"{tuple(v.shape)}")
    _same(q, "q", k=k, v=v)
    if scale is None:
        scale = Dk ** -0.5
    o = out if out is not None else torch.empty((B, T, Hq, Dv), dtype=q.dtype, device=q.device)
    _need_shape(o, (B, T, Hq, Dv), "out")
    _same(q, "q", out=o)
    need = int(lib.attn_prefill_workspace_bytes(B, T, Hkv, Dk, _Rope(rotary_dims, theta),
                                                int(rope_mask), _dtype_code(q)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _same(q, "q", workspace=workspace)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = _nbytes(workspace) if workspace is not None else 0
    _check(lib.attn_prefill(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"),
                            B, T, Hq, Hkv, Dk, Dv, int(window), float(scale),
                            _Rope(rotary_dims, theta), int(rope_mask), int(pos0),
                            ws_ptr, ws_bytes, _dtype_code(q), _stream(q)))
    return o


def prefill_into_cache(q, k, v, k_cache, v_cache, row_offset, *, window: int = 0,
                       scale: float | None = None, rotary_dims: int = 0,
                       theta: float = 10000.0, pos0: int = 0, out=None, workspace=None):
    """prefill() with RoPE on q and k that also writes the decode cache:
    k_cache[row_offset[b] + t] = rope(k[b, t]) at position pos0 + t,
    v_cache[row_offset[b] + t] = v[b, t]. k_cache [rows, Hkv, Dk], v_cache
    [rows, Hkv, Dv], row_offset int64 [B] on the device. Returns o."""
    lib = load()
    _need_dims(q, 4, "q")
    _need_dims(k, 4, "k")
    _need_dims(v, 4, "v")
    B, T, Hq, Dk = q.shape
    Hkv, Dv = k.shape[2], v.shape[3]
    if tuple(k.shape) != (B, T, Hkv, Dk) or tuple(v.shape) != (B, T, Hkv, Dv):
        raise ValueError(f"q/k/v shapes disagree: {tuple(q.shape)} {tuple(k.shape)} "
                         f"{tuple(v.shape)}")
    _need_dims(k_cache, 3, "k_cache")
    _need_dims(v_cache, 3, "v_cache")
    rows = k_cache.shape[0]
    _need_shape(k_cache, (rows, Hkv, Dk), "k_cache")
    _need_shape(v_cache, (rows, Hkv, Dv), "v_cache")
    if row_offset.dtype != torch.int64 or row_offset.numel() != B:
        raise ValueError(f"row_offset must be int64 with {B} entries")
    _same(q, "q", k=k, v=v, k_cache=k_cache, v_cache=v_cache)
    _same_device(q, "q", row_offset=row_offset)
    if scale is None:
        scale = Dk ** -0.5
    o = out if out is not None else torch.empty((B, T, Hq, Dv), dtype=q.dtype, device=q.device)
    _need_shape(o, (B, T, Hq, Dv), "out")
    _same(q, "q", out=o)
    need = int(lib.attn_prefill_workspace_bytes(B, T, Hkv, Dk, _Rope(rotary_dims, theta),
                                                ROPE_Q | ROPE_K, _dtype_code(q)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _same(q, "q", workspace=workspace)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = _nbytes(workspace) if workspace is not None else 0
    _check(lib.attn_prefill_into_cache(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), B, T, Hq, Hkv, Dk, Dv,
        int(window), float(scale), _Rope(rotary_dims, theta), int(pos0),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(row_offset, "row_offset"),
        int(rows), ws_ptr, ws_bytes, _dtype_code(q), _stream(q)))
    return o


def _cache_args(q, k_cache, v_cache, row_offset, kv_len, n_q=None):
    """Shapes, dtypes and devices of a decode-style call, checked on the host
    (the kernels build buffer descriptors from these sizes)."""
    if n_q is None:
        _need_dims(q, 3, "q")
        B, Hq, Dk = q.shape
    else:
        _need_dims(q, 4, "q")
        B, _, Hq, Dk = q.shape
    _need_dims(k_cache, 3, "k_cache")
    _need_dims(v_cache, 3, "v_cache")
    rows, Hkv = k_cache.shape[0], k_cache.shape[1]
    Dv = v_cache.shape[2]
    if k_cache.shape[2] != Dk:
        raise ValueError(f"k_cache head dim {k_cache.shape[2]} != q head dim {Dk}")
    if tuple(v_cache.shape[:2]) != (rows, Hkv):
        raise ValueError(f"v_cache {tuple(v_cache.shape)} does not match k_cache "
                         f"{tuple(k_cache.shape)} in rows and KV heads")
    if row_offset.dtype != torch.int64 or kv_len.dtype != torch.int32:
        raise TypeError("row_offset must be int64 and kv_len int32")
    if row_offset.numel() != B or kv_len.numel() != B:
        raise ValueError(f"row_offset and kv_len need {B} entries "
                         f"(got {row_offset.numel()}, {kv_len.numel()})")
    _same(q, "q", row_offset=row_offset, kv_len=kv_len)
    return B, Hq, Hkv, Dk, Dv


def decode_workspace_bytes(B: int, Hq: int, Hkv: int, Dv: int, max_kv_len: int,
                           window: int) -> int:
    return int(load().attn_decode_workspace_bytes(B, Hq, Hkv, Dv, max_kv_len, window))


def decode(q, k_cache, v_cache, row_offset, kv_len, *, window: int = 0,
           scale: float | None = None, rotary_dims: int = 0, theta: float = 10000.0,
           max_kv_len: int, out=None, workspace=None):
    """q [B,Hq,Dk]; caches [rows,Hkv,Dk|Dv]; row_offset int64 [B]; kv_len int32 [B]."""
    lib = load()
    B, Hq, Hkv, Dk, Dv = _cache_args(q, k_cache, v_cache, row_offset, kv_len)
    _same(q, "q", k_cache=k_cache, v_cache=v_cache)
    if scale is None:
        scale = Dk ** -0.5
    o = out if out is not None else torch.empty((B, Hq, Dv), dtype=q.dtype, device=q.device)
    _need_shape(o, (B, Hq, Dv), "out")
    _same(q, "q", out=o)
    need = decode_workspace_bytes(B, Hq, Hkv, Dv, max_kv_len, window)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _same(q, "q", workspace=workspace)
    _check(lib.attn_decode(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                           _dev(row_offset, "row_offset"), _dev(kv_len, "kv_len"),
                           _dev(o, "o"), B, Hq, Hkv, Dk, Dv, int(window), float(scale),
                           _Rope(rotary_dims, theta), int(max_kv_len),
                           _dev(workspace, "workspace"), _nbytes(workspace),
                           _dtype_code(q), _stream(q)))
    return o


def decode_noalloc(q, k_cache, v_cache, row_offset, kv_len, *, window: int = 0,
                   scale: float | None = None, rotary_dims: int = 0, theta: float = 10000.0,
                   max_kv_len: int, out):
    """decode() through the entry point that allocates nothing: the split-K
    partials live in the library's static device scratch. ``out`` [B,Hq,Dv]
    is required (this call allocates no tensor either)."""
    lib = load()
    B, Hq, Hkv, Dk, Dv = _cache_args(q, k_cache, v_cache, row_offset, kv_len)
    _same(q, "q", k_cache=k_cache, v_cache=v_cache, out=out)
    _need_shape(out, (B, Hq, Dv), "out")
    if scale is None:
        scale = Dk ** -0.5
    _check(lib.attn_decode_noalloc(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                   _dev(row_offset, "row_offset"), _dev(kv_len, "kv_len"),
                                   _dev(out, "o"), B, Hq, Hkv, Dk, Dv, int(window), float(scale),
                                   _Rope(rotary_dims, theta), int(max_kv_len), _dtype_code(q),
                                   _stream(q)))
    return out


def decode_noalloc_max_bytes() -> int:
    return int(load().attn_decode_noalloc_max_bytes())


def verify_workspace_bytes(B: int, n_q: int, Hq: int, Hkv: int, Dk: int, Dv: int,
                           max_kv_len: int, window: int) -> int:
    return int(load().attn_verify_workspace_bytes(B, n_q, Hq, Hkv, Dk, Dv, max_kv_len, window))


def verify(q, k_cache, v_cache, row_offset, kv_len, *, window: int = 0,
           scale: float | None = None, rotary_dims: int = 0, theta: float = 10000.0,
           max_kv_len: int, out=None, workspace=None):
    """q [B,n_q,Hq,Dk] (token j of sequence b at position kv_len[b]-n_q+j);
    caches [rows,Hkv,Dk|Dv]; row_offset int64 [B]; kv_len int32 [B] ->
    o [B,n_q,Hq,Dv]."""
    lib = load()
    n_q = q.shape[1] if q.dim() == 4 else 0
    B, Hq, Hkv, Dk, Dv = _cache_args(q, k_cache, v_cache, row_offset, kv_len, n_q=n_q)
    _same(q, "q", k_cache=k_cache, v_cache=v_cache)
    if scale is None:
        scale = Dk ** -0.5
    o = out if out is not None else torch.empty((B, n_q, Hq, Dv), dtype=q.dtype,
                                                device=q.device)
    _need_shape(o, (B, n_q, Hq, Dv), "out")
    _same(q, "q", out=o)
    need = verify_workspace_bytes(B, n_q, Hq, Hkv, Dk, Dv, max_kv_len, window)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _same(q, "q", workspace=workspace)
    _check(lib.attn_verify(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                           _dev(row_offset, "row_offset"), _dev(kv_len, "kv_len"),
                           _dev(o, "o"), B, n_q, Hq, Hkv, Dk, Dv, int(window), float(scale),
                           _Rope(rotary_dims, theta), int(max_kv_len),
                           _dev(workspace, "workspace"), _nbytes(workspace),
                           _dtype_code(q), _stream(q)))
    return o


def prope(x, positions, *, rotary_dims: int, theta: float, out=None):
    """x [N,H,D] -> rotated copy (or in place when out is x); positions int32 [N]."""
    lib = load()
    N, H, D = x.shape
    if positions.dtype != torch.int32:
        raise TypeError("positions must be int32")
    y = out if out is not None else torch.empty_like(x)
    _check(lib.prope_apply(_dev(x, "x"), _dev(y, "y"), _dev(positions, "positions"),
                           N, H, D, _Rope(rotary_dims, theta), _dtype_code(x), _stream(x)))
    return y


def prope_2d(x, positions_xy, *, rotary_dims: int, theta: float, out=None):
    """x [N,H,D] -> 2-D RoPE copy (or in place when out is x); positions_xy
    int32 [N,2] = (width, height) coordinates; each half of D turns by one."""
    lib = load()
    N, H, D = x.shape
    if positions_xy.dtype != torch.int32 or tuple(positions_xy.shape) != (N, 2):
        raise TypeError("positions_xy must be int32 [N, 2]")
    y = out if out is not None else torch.empty_like(x)
    _check(lib.prope_apply_2d(_dev(x, "x"), _dev(y, "y"), _dev(positions_xy, "positions_xy"),
                              N, H, D, _Rope(rotary_dims, theta), _dtype_code(x), _stream(x)))
    return y


def kv_quantize_int8(x, *, codes=None, scales=None):
    """x [N,H,D] bf16 -> (codes int8 [N,H,D], scales float32 [N,H]); one
    symmetric scale per (row, head), s = max|x| / 127."""
    lib = load()
    N, H, D = x.shape
    c = codes if codes is not None else torch.empty((N, H, D), dtype=torch.int8, device=x.device)
    sc = scales if scales is not None else torch.empty((N, H), dtype=torch.float32,
                                                       device=x.device)
    _check(lib.attn_kv_quantize_int8(_dev(x, "x"), _dev(c, "codes"), _dev(sc, "scales"), N, H, D,
                                     _dtype_code(x), _stream(x)))
    return c, sc


def decode_int8_workspace_bytes(B: int, Hq: int, Hkv: int, Dv: int, max_kv_len: int,
                                window: int) -> int:
    return int(load().attn_decode_int8_workspace_bytes(B, Hq, Hkv, Dv, max_kv_len, window))


def decode_int8(q, k_codes, k_scales, v_codes, v_scales, row_offset, kv_len, *,
                window: int = 0, scale: float | None = None, rotary_dims: int = 0,
                theta: float = 10000.0, max_kv_len: int, out=None, workspace=None):
    """attn_decode over int8 caches: codes [rows,Hkv,D] int8, scales
    [rows,Hkv] float32; q [B,Hq,Dk] bf16 -> o [B,Hq,Dv] bf16."""
    lib = load()
    B, Hq, Hkv, Dk, Dv = _cache_args(q, k_codes, v_codes, row_offset, kv_len)
    if q.dtype != torch.bfloat16:
        raise TypeError("q must be bfloat16")
    if k_codes.dtype != torch.int8 or v_codes.dtype != torch.int8:
        raise TypeError("codes must be int8")
    if k_scales.dtype != torch.float32 or v_scales.dtype != torch.float32:
        raise TypeError("scales must be float32")
    rows = k_codes.shape[0]
    _need_shape(k_scales, (rows, Hkv), "k_scales")
    _need_shape(v_scales, (rows, Hkv), "v_scales")
    _same_device(q, "q", k_codes=k_codes, v_codes=v_codes, k_scales=k_scales,
                 v_scales=v_scales)
    if scale is None:
        scale = Dk ** -0.5
    o = out if out is not None else torch.empty((B, Hq, Dv), dtype=q.dtype, device=q.device)
    _need_shape(o, (B, Hq, Dv), "out")
    _same(q, "q", out=o)
    need = decode_int8_workspace_bytes(B, Hq, Hkv, Dv, max_kv_len, window)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _same_device(q, "q", workspace=workspace)
    _check(lib.attn_decode_int8(_dev(q, "q"), _dev(k_codes, "k_codes"), _dev(k_scales, "k_scales"),
                                _dev(v_codes, "v_codes"), _dev(v_scales, "v_scales"),
                                _dev(row_offset, "row_offset"), _dev(kv_len, "kv_len"),
                                _dev(o, "o"), B, Hq, Hkv, Dk, Dv, int(window), float(scale),
                                _Rope(rotary_dims, theta), int(max_kv_len),
                                _dev(workspace, "workspace"), _nbytes(workspace), _stream(q)))
    return o
