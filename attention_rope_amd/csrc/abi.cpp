// abi.cpp — the C ABI of the hybrid-attention library: argument validation,
// workspace accounting, kernel selection and error reporting. Every check runs
// on the host before any HIP call; a failed check launches nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/attn_rope.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

attn_status_t fail(attn_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

attn_status_t ok() {
  g_last_error.clear();
  return ATTN_OK;
}

attn_status_t launch_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(ATTN_ERR_LAUNCH, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x0 = reinterpret_cast<uintptr_t>(a), y0 = reinterpret_cast<uintptr_t>(b);
  return x0 < y0 + nb && y0 < x0 + na;
}

size_t elem_size(attn_dtype_t d) { return d == ATTN_F32 ? 4 : 2; }

attn_status_t check_rope(attn_rope_t rope, int32_t D) {
  if (rope.rotary_dims < 0 || rope.rotary_dims > D || rope.rotary_dims % 2 != 0)
    return fail(ATTN_ERR_SHAPE, "rotary_dims=%d must be even and in [0, %d]",
                rope.rotary_dims, D);
  if (rope.rotary_dims > 0 && !(std::isfinite(rope.theta) && rope.theta > 0.0))
    return fail(ATTN_ERR_SHAPE, "rope theta must be finite and > 0");
  return ATTN_OK;
}

bool prefill_rotates(attn_rope_t rope, int32_t rope_mask) {
  return rope.rotary_dims > 0 && (rope_mask & (ATTN_ROPE_Q | ATTN_ROPE_K)) != 0;
}

// Whenever K turns, its rotary dims turn once ahead of the attention kernel,
// into the workspace ([B, T, Hkv, rotary_dims] in the call's element type).
bool prefill_turns_k_ahead(attn_rope_t rope, int32_t rope_mask) {
  return (rope_mask & ATTN_ROPE_K) && rope.rotary_dims > 0;
}

// attn_decode (n_q = 1) and attn_verify (n_q new tokens per sequence).
attn_status_t decode_call(const char* what, const void* q, const void* k_cache,
                          const void* v_cache, const int64_t* row_offset, const int32_t* kv_len,
                          void* o, int32_t B, int32_t n_q, int32_t Hq, int32_t Hkv, int32_t Dk,
                          int32_t Dv, int32_t window, float scale, attn_rope_t rope,
                          int32_t max_kv_len, void* workspace, size_t workspace_bytes,
                          attn_dtype_t dtype, void* stream, bool dry = false) {
  if (dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "%s supports the ATTN_BF16 cache only", what);
  if (B < 0 || B > 65535) return fail(ATTN_ERR_SHAPE, "B=%d must be in [0, 65535]", B);
  if (n_q < 1 || n_q > 4096) return fail(ATTN_ERR_SHAPE, "n_q=%d must be in [1, 4096]", n_q);
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return fail(ATTN_ERR_SHAPE, "Hq=%d must be a positive multiple of Hkv=%d", Hq, Hkv);
  if (!attn::decode_supported(Dk, Dv, Hq / Hkv))
    return fail(ATTN_ERR_UNSUPPORTED,
                "%s supports Dk in {128,256,512}, Dv in {128,256} (or 512 with "
                "Dk=512), Hq/Hkv <= 16 (got Dk=%d Dv=%d G=%d)", what, Dk, Dv, Hq / Hkv);
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(ATTN_ERR_UNSUPPORTED, "%s needs a finite scale >= 0", what);
  attn_status_t rs = check_rope(rope, Dk);
  if (rs != ATTN_OK) return rs;
  if (B == 0) return ok();
  if (max_kv_len < 1) return fail(ATTN_ERR_SHAPE, "max_kv_len=%d must be >= 1", max_kv_len);
  if (!attn::decode_shape_fits(B, n_q, Hq, Hkv, Dk, Dv, max_kv_len, window))
    return fail(ATTN_ERR_SHAPE, "cache too large for one call (max_kv_len=%d, Hkv=%d)",
                max_kv_len, Hkv);
  if (!q || !k_cache || !v_cache || !row_offset || !kv_len || !o)
    return fail(ATTN_ERR_NULL, "q, caches, row_offset, kv_len and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(ATTN_ERR_SHAPE, "q, caches and o must be 16-byte aligned");
  if (dry) return ok();
  const size_t need =
      attn::decode_workspace_bytes(B, n_q, Hq, Hkv, Dk, Dv, max_kv_len, window);
  if (!workspace || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(ATTN_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  const size_t no = (size_t)B * n_q * Hq * Dv * 2, nq = (size_t)B * n_q * Hq * Dk * 2;
  if (overlap(o, no, q, nq) || overlap(workspace, need, o, no) || overlap(workspace, need, q, nq))
    return fail(ATTN_ERR_ALIAS, "o / workspace must not overlap q or each other");

  attn::DecodeArgs a{};
  a.q = q; a.k_cache = k_cache; a.v_cache = v_cache;
  a.row_offset = row_offset; a.kv_len = kv_len; a.o = o;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Dk = Dk; a.Dv = Dv;
  a.window = window > 0 ? window : 0;
  a.rot_pairs = rope.rotary_dims / 2;
  a.theta = rope.rotary_dims > 0 ? rope.theta : 1.0;
  a.scale = scale;
  a.max_kv_len = max_kv_len;
  a.workspace = workspace;
  a.n_q = n_q;
  return launch_status(attn::launch_decode(a, reinterpret_cast<hipStream_t>(stream)), what);
}


// prope_apply (NH = 1) and prope_apply_2d (NH = 2 halves, positions [N, 2]).
attn_status_t prope_call(const void* x, void* y, const int32_t* positions, int32_t N,
                         int32_t H, int32_t D, int NH, attn_rope_t rope, attn_dtype_t dtype,
                         void* stream) {
  if (dtype != ATTN_F32 && dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "dtype %d is not ATTN_F32 or ATTN_BF16", (int)dtype);
  if (N < 0 || H < 0) return fail(ATTN_ERR_SHAPE, "N=%d and H=%d must be >= 0", N, H);
  if (D < 2 || D > 1024 || D % 2) return fail(ATTN_ERR_SHAPE, "D=%d must be even, 2..1024", D);
  attn_status_t rs = check_rope(rope, D / NH);
  if (rs != ATTN_OK) return rs;
  if (N == 0 || H == 0) return ok();
  if (!x || !y || !positions) return fail(ATTN_ERR_NULL, "x, y and positions must be non-NULL");
  const size_t es = elem_size(dtype);
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & (2 * es - 1))
    return fail(ATTN_ERR_SHAPE, "x and y must be aligned to a pair of elements");
  const size_t n = (size_t)N * H * D * es;
  if (x != y && overlap(x, n, y, n)) return fail(ATTN_ERR_ALIAS, "y partially overlaps x");
  if ((int64_t)N * NH * (rope.rotary_dims / 2) > (int64_t)INT32_MAX * 256)
    return fail(ATTN_ERR_SHAPE, "N too large");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (rope.rotary_dims == 0) {
    if (x == y) return ok();
    return launch_status(hipMemcpyAsync(y, x, n, hipMemcpyDeviceToDevice, st), "prope copy");
  }
  return launch_status(attn::launch_prope(x, y, positions, N, H, D, rope.rotary_dims / 2, NH,
                                          rope.theta, dtype == ATTN_BF16, st),
                       "prope");
}


}  // namespace

extern "C" {

const char* attn_status_string(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer";
    case ATTN_ERR_SHAPE: return "invalid shape or argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_ALIAS: return "output overlaps an input";
  }
  return "unknown status";
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

size_t attn_prefill_workspace_bytes(int32_t B, int32_t T, int32_t Hkv, int32_t Dk,
                                    attn_rope_t rope, int32_t rope_mask, attn_dtype_t dtype) {
  if (B <= 0 || T <= 0 || Hkv <= 0 || (dtype != ATTN_BF16 && dtype != ATTN_F32)) return 0;
  if (rope.rotary_dims > Dk || !prefill_turns_k_ahead(rope, rope_mask)) return 0;
  return (size_t)B * T * Hkv * rope.rotary_dims * elem_size(dtype);
}

namespace {

// Decode-cache outputs of attn_prefill_into_cache (k_cache == nullptr: none).
struct CacheOut {
  void* k_cache = nullptr;
  void* v_cache = nullptr;
  const int64_t* row_offset = nullptr;
  int64_t cache_rows = 0;
};

attn_status_t prefill_call(const char* what, const void* q, const void* k, const void* v,
                           void* o, int32_t B, int32_t T, int32_t Hq, int32_t Hkv, int32_t Dk,
                           int32_t Dv, int32_t window, float scale, attn_rope_t rope,
                           int32_t rope_mask, int32_t pos0, void* workspace,
                           size_t workspace_bytes, attn_dtype_t dtype, void* stream,
                           const CacheOut& cache) {
  if (dtype != ATTN_F32 && dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "dtype %d is not ATTN_F32 or ATTN_BF16", (int)dtype);
  if (B < 0 || T < 0) return fail(ATTN_ERR_SHAPE, "B=%d and T=%d must be >= 0", B, T);
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return fail(ATTN_ERR_SHAPE, "Hq=%d must be a positive multiple of Hkv=%d", Hq, Hkv);
  if (Dk < 2 || Dv < 2 || Dk > 512 || Dv > 512 || Dk % 2 || Dv % 2)
    return fail(ATTN_ERR_SHAPE, "head dims Dk=%d Dv=%d must be even and in [2, 512]", Dk, Dv);
  if (!std::isfinite(scale)) return fail(ATTN_ERR_SHAPE, "scale must be finite");
  if (rope_mask & ~(ATTN_ROPE_Q | ATTN_ROPE_K))
    return fail(ATTN_ERR_SHAPE, "rope_mask=%d has unknown bits", rope_mask);
  attn_status_t rs = check_rope(rope, Dk);
  if (rs != ATTN_OK) return rs;
  if (pos0 < 0 || (int64_t)pos0 + T > INT32_MAX)
    return fail(ATTN_ERR_SHAPE, "positions pos0=%d .. pos0+T-1 must lie in [0, 2^31-1)", pos0);
  if (B == 0 || T == 0) return ok();
  if (!q || !k || !v || !o)
    return fail(ATTN_ERR_NULL, "%s: q, k, v and o must be non-NULL", what);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_ERR_SHAPE, "q, k, v and o must be 16-byte aligned");
  const size_t es = elem_size(dtype);
  const size_t nq = (size_t)B * T * Hq * Dk * es, nk = (size_t)B * T * Hkv * Dk * es;
  const size_t nv = (size_t)B * T * Hkv * Dv * es, no = (size_t)B * T * Hq * Dv * es;
  if (overlap(o, no, q, nq) || overlap(o, no, k, nk) || overlap(o, no, v, nv))
    return fail(ATTN_ERR_ALIAS, "o must not overlap q, k or v");
  if ((int64_t)B * T * Hq / 4 + 1 > INT32_MAX)
    return fail(ATTN_ERR_SHAPE, "B*T*Hq too large");
  const bool rot = prefill_rotates(rope, rope_mask);
  const size_t nws = attn_prefill_workspace_bytes(B, T, Hkv, Dk, rope, rope_mask, dtype);
  if (nws > 0) {
    if (!workspace || workspace_bytes < nws)
      return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu at %p)", nws,
                  workspace_bytes, workspace);
    if (!aligned16(workspace)) return fail(ATTN_ERR_SHAPE, "workspace must be 16-byte aligned");
    if (overlap(workspace, nws, q, nq) || overlap(workspace, nws, k, nk) ||
        overlap(workspace, nws, v, nv) || overlap(workspace, nws, o, no))
      return fail(ATTN_ERR_ALIAS, "workspace must not overlap q, k, v or o");
  }

  const bool fill = cache.k_cache != nullptr;
  if (fill) {
    if (!cache.v_cache || !cache.row_offset)
      return fail(ATTN_ERR_NULL, "%s: k_cache, v_cache and row_offset must be non-NULL", what);
    if (Dk % 8 || Dv % 8 || rope.rotary_dims % 8)
      return fail(ATTN_ERR_SHAPE, "%s: Dk=%d, Dv=%d and rotary_dims=%d must be multiples of 8",
                  what, Dk, Dv, rope.rotary_dims);
    if (cache.cache_rows < T || cache.cache_rows > ((int64_t)1 << 40))
      return fail(ATTN_ERR_SHAPE, "%s: cache_rows=%lld must be in [T, 2^40]", what,
                  (long long)cache.cache_rows);
    if (!aligned16(cache.k_cache) || !aligned16(cache.v_cache) ||
        (reinterpret_cast<uintptr_t>(cache.row_offset) & 7u))
      return fail(ATTN_ERR_SHAPE, "%s: caches must be 16-byte and row_offset 8-byte aligned",
                  what);
    const size_t nkc = (size_t)cache.cache_rows * Hkv * Dk * es;
    const size_t nvc = (size_t)cache.cache_rows * Hkv * Dv * es;
    const size_t nro = (size_t)B * sizeof(int64_t);
    const void* ins[] = {q, k, v, o, workspace, cache.row_offset};
    const size_t ns[] = {nq, nk, nv, no, nws, nro};
    for (int i = 0; i < 6; ++i)
      if (overlap(cache.k_cache, nkc, ins[i], ns[i]) || overlap(cache.v_cache, nvc, ins[i], ns[i]))
        return fail(ATTN_ERR_ALIAS,
                    "%s: the caches must not overlap q, k, v, o, the workspace or row_offset",
                    what);
    if (overlap(cache.k_cache, nkc, cache.v_cache, nvc))
      return fail(ATTN_ERR_ALIAS, "%s: k_cache and v_cache must not overlap", what);
  }

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  attn::PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.B = B; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.Dk = Dk; a.Dv = Dv;
  a.window = (window > 0 && window < T) ? window : 0;
  a.rot_pairs = rot ? rope.rotary_dims / 2 : 0;
  a.rope_q = rot && (rope_mask & ATTN_ROPE_Q);
  a.rope_k = rot && (rope_mask & ATTN_ROPE_K);
  a.scale = scale;
  // Every kernel forms its angles from these (fp64), so all of them rotate
  // token t by position pos0 + t with this call's rope settings.
  a.pos0 = pos0;
  a.log2_theta = rot ? std::log2(rope.theta) : 0.0;
  a.rope_rho = rot ? std::pow(rope.theta, -2.0 / (double)Dk) : 1.0;
#ifdef ATTN_DEBUG_TILES
  if (attn::debug_visits_ptr(&a.dbg_visits) != hipSuccess) a.dbg_visits = nullptr;
#endif
  if (fill) {
    // One pass over K and V: K's rotary dims turn once into the workspace
    // (as below) and whole turned key rows and value rows go to the cache.
    attn_status_t r = launch_status(
        attn::launch_prefill_cache_fill(k, v, cache.k_cache, cache.v_cache,
                                        nws > 0 ? workspace : nullptr, cache.row_offset,
                                        cache.cache_rows, B, T, Hkv, Dk, Dv,
                                        a.rope_k ? rope.rotary_dims : 0, pos0, rope.theta,
                                        dtype == ATTN_BF16, st),
        "prefill (cache fill)");
    if (r != ATTN_OK) return r;
    if (a.rope_k && nws > 0) a.k_rot = workspace;
  } else if (a.rope_k && nws > 0) {
    // K's rotary dims turn once here, not once per query tile in the kernel.
    attn_status_t r = launch_status(
        attn::launch_rope_k_lead(k, workspace, B, T, Hkv, Dk, rope.rotary_dims, pos0,
                                 rope.theta, dtype == ATTN_BF16, st),
        "prefill (K rotation)");
    if (r != ATTN_OK) return r;
    a.k_rot = workspace;
  }
  if (dtype == ATTN_BF16 &&
      attn::prefill_mfma_supported(Dk, Dv, Hq / Hkv, scale, rot ? rope.rotary_dims : 0)) {
    hipError_t e = attn::launch_prefill_mfma(a, st);
    if (e != hipErrorNotSupported) return launch_status(e, "prefill (mfma)");
  }
  return launch_status(attn::launch_prefill_general(a, dtype == ATTN_BF16, st),
                       "prefill (general)");
}

}  // namespace

attn_status_t attn_prefill(const void* q, const void* k, const void* v, void* o,
                           int32_t B, int32_t T, int32_t Hq, int32_t Hkv, int32_t Dk,
                           int32_t Dv, int32_t window, float scale, attn_rope_t rope,
                           int32_t rope_mask, int32_t pos0, void* workspace,
                           size_t workspace_bytes, attn_dtype_t dtype, void* stream) {
  return prefill_call("prefill", q, k, v, o, B, T, Hq, Hkv, Dk, Dv, window, scale, rope,
                      rope_mask, pos0, workspace, workspace_bytes, dtype, stream, CacheOut{});
}

#ifdef ATTN_DEBUG_TILES
// Debug builds only (libattn_rope_dbg.so): the two prefill tile counters
// (see PrefillArgs::dbg_visits), copied to out[0..1] after the device is idle;
// reset != 0 zeroes them afterwards.
extern "C" attn_status_t attn_debug_tile_visits(uint64_t* out, int32_t reset) {
  unsigned long long* p = nullptr;
  hipError_t e = attn::debug_visits_ptr(&p);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess && out) e = hipMemcpy(out, p, 2 * sizeof(uint64_t), hipMemcpyDeviceToHost);
  if (e == hipSuccess && reset) e = hipMemset(p, 0, 2 * sizeof(uint64_t));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  return launch_status(e, "debug tile counters");
}
#endif

attn_status_t attn_prefill_into_cache(const void* q, const void* k, const void* v, void* o,
                                      int32_t B, int32_t T, int32_t Hq, int32_t Hkv,
                                      int32_t Dk, int32_t Dv, int32_t window, float scale,
                                      attn_rope_t rope, int32_t pos0, void* k_cache,
                                      void* v_cache, const int64_t* row_offset,
                                      int64_t cache_rows, void* workspace,
                                      size_t workspace_bytes, attn_dtype_t dtype,
                                      void* stream) {
  CacheOut c;
  c.k_cache = k_cache;
  c.v_cache = v_cache;
  c.row_offset = row_offset;
  c.cache_rows = cache_rows;
  if (B > 0 && T > 0 && !k_cache)
    return fail(ATTN_ERR_NULL, "prefill_into_cache: k_cache must be non-NULL");
  return prefill_call("prefill_into_cache", q, k, v, o, B, T, Hq, Hkv, Dk, Dv, window, scale,
                      rope, ATTN_ROPE_Q | ATTN_ROPE_K, pos0, workspace, workspace_bytes, dtype,
                      stream, c);
}

size_t attn_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t Dv,
                                   int32_t max_kv_len, int32_t window) {
  return attn::decode_workspace_bytes(B, 1, Hq, Hkv, 0, Dv, max_kv_len, window);
}

size_t attn_verify_workspace_bytes(int32_t B, int32_t n_q, int32_t Hq, int32_t Hkv, int32_t Dk,
                                   int32_t Dv, int32_t max_kv_len, int32_t window) {
  return attn::decode_workspace_bytes(B, n_q, Hq, Hkv, Dk, Dv, max_kv_len, window);
}

attn_status_t attn_decode(const void* q, const void* k_cache, const void* v_cache,
                          const int64_t* row_offset, const int32_t* kv_len, void* o,
                          int32_t B, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv,
                          int32_t window, float scale, attn_rope_t rope,
                          int32_t max_kv_len, void* workspace, size_t workspace_bytes,
                          attn_dtype_t dtype, void* stream) {
  return decode_call("decode", q, k_cache, v_cache, row_offset, kv_len, o, B, 1, Hq, Hkv, Dk,
                     Dv, window, scale, rope, max_kv_len, workspace, workspace_bytes, dtype,
                     stream);
}

size_t attn_decode_noalloc_max_bytes(void) { return attn::kDecodeScratchBytes; }

attn_status_t attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int64_t* row_offset, const int32_t* kv_len, void* o,
                                  int32_t B, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv,
                                  int32_t window, float scale, attn_rope_t rope,
                                  int32_t max_kv_len, attn_dtype_t dtype, void* stream) {
  // The same partials attn_decode keeps in its workspace; checked against the
  // static scratch before anything touches the GPU.
  if (B > 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0 && max_kv_len >= 1) {
    const size_t need = attn::decode_workspace_bytes(B, 1, Hq, Hkv, Dk, Dv, max_kv_len, window);
    if (need > attn::kDecodeScratchBytes)
      return fail(ATTN_ERR_WORKSPACE,
                  "decode_noalloc: this call needs %zu bytes of split-K scratch, the static "
                  "scratch holds %zu (use attn_decode with a workspace)",
                  need, attn::kDecodeScratchBytes);
  }
  // Everything but the scratch is validated by the shared path; an empty
  // batch or an invalid argument returns before the scratch is looked up.
  const size_t zero_ws = 0;
  attn_status_t pre = decode_call("decode_noalloc", q, k_cache, v_cache, row_offset, kv_len, o,
                                  B, 1, Hq, Hkv, Dk, Dv, window, scale, rope, max_kv_len,
                                  nullptr, zero_ws, dtype, nullptr, /*dry=*/true);
  if (pre != ATTN_OK || B == 0) return pre;
  void* ws = nullptr;
  attn_status_t r = launch_status(attn::decode_scratch(&ws), "decode_noalloc (scratch)");
  if (r != ATTN_OK) return r;
  return decode_call("decode_noalloc", q, k_cache, v_cache, row_offset, kv_len, o, B, 1, Hq, Hkv,
                     Dk, Dv, window, scale, rope, max_kv_len, ws, attn::kDecodeScratchBytes,
                     dtype, stream);
}

attn_status_t attn_verify(const void* q, const void* k_cache, const void* v_cache,
                          const int64_t* row_offset, const int32_t* kv_len, void* o,
                          int32_t B, int32_t n_q, int32_t Hq, int32_t Hkv, int32_t Dk,
                          int32_t Dv, int32_t window, float scale, attn_rope_t rope,
                          int32_t max_kv_len, void* workspace, size_t workspace_bytes,
                          attn_dtype_t dtype, void* stream) {
  return decode_call("verify", q, k_cache, v_cache, row_offset, kv_len, o, B, n_q, Hq, Hkv,
                     Dk, Dv, window, scale, rope, max_kv_len, workspace, workspace_bytes,
                     dtype, stream);
}

attn_status_t attn_kv_quantize_int8(const void* x, int8_t* codes, float* scales, int32_t N,
                                    int32_t H, int32_t D, attn_dtype_t dtype, void* stream) {
  if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "int8 quantiser reads ATTN_BF16");
  if (N < 0 || H < 0) return fail(ATTN_ERR_SHAPE, "N=%d and H=%d must be >= 0", N, H);
  if (D != 128 && D != 256 && D != 512)
    return fail(ATTN_ERR_UNSUPPORTED, "int8 quantiser supports D in {128,256,512}, got %d", D);
  if (N == 0 || H == 0) return ok();
  if (!x || !codes || !scales) return fail(ATTN_ERR_NULL, "x, codes and scales must be non-NULL");
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(scales) & 3))
    return fail(ATTN_ERR_SHAPE, "x must be 16-byte aligned, scales 4-byte aligned");
  const size_t rows = (size_t)N * H;
  if (overlap(x, rows * D * 2, codes, rows * D) || overlap(x, rows * D * 2, scales, rows * 4) ||
      overlap(codes, rows * D, scales, rows * 4))
    return fail(ATTN_ERR_ALIAS, "x, codes and scales must not overlap");
  return launch_status(attn::launch_kv_quantize_int8(x, codes, scales, N, H, D,
                                                     reinterpret_cast<hipStream_t>(stream)),
                       "int8 quantiser");
}

size_t attn_decode_int8_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t Dv,
                                        int32_t max_kv_len, int32_t window) {
  return attn::decode_workspace_bytes(B, 1, Hq, Hkv, 0, Dv, max_kv_len, window);
}

attn_status_t attn_decode_int8(const void* q, const int8_t* k_codes, const float* k_scales,
                               const int8_t* v_codes, const float* v_scales,
                               const int64_t* row_offset, const int32_t* kv_len, void* o,
                               int32_t B, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv,
                               int32_t window, float scale, attn_rope_t rope,
                               int32_t max_kv_len, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (B < 0 || B > 65535) return fail(ATTN_ERR_SHAPE, "B=%d must be in [0, 65535]", B);
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return fail(ATTN_ERR_SHAPE, "Hq=%d must be a positive multiple of Hkv=%d", Hq, Hkv);
  if (!attn::decode_int8_supported(Dk, Dv, Hq / Hkv))
    return fail(ATTN_ERR_UNSUPPORTED,
                "int8 decode supports (Dk, Dv) in {(512,256), (256,256)}, Hq/Hkv <= 16 "
                "(got Dk=%d Dv=%d G=%d)", Dk, Dv, Hq / Hkv);
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(ATTN_ERR_UNSUPPORTED, "int8 decode needs a finite scale >= 0");
  attn_status_t rs = check_rope(rope, Dk);
  if (rs != ATTN_OK) return rs;
  if (B == 0) return ok();
  if (max_kv_len < 1) return fail(ATTN_ERR_SHAPE, "max_kv_len=%d must be >= 1", max_kv_len);
  if (!attn::decode_shape_fits(B, 1, Hq, Hkv, Dk, Dv, max_kv_len, window))
    return fail(ATTN_ERR_SHAPE, "cache too large for one call (max_kv_len=%d, Hkv=%d)",
                max_kv_len, Hkv);
  if (!q || !k_codes || !k_scales || !v_codes || !v_scales || !row_offset || !kv_len || !o)
    return fail(ATTN_ERR_NULL, "q, codes, scales, row_offset, kv_len and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(o) ||
      ((reinterpret_cast<uintptr_t>(k_scales) | reinterpret_cast<uintptr_t>(v_scales)) & 3))
    return fail(ATTN_ERR_SHAPE, "q, codes and o must be 16-byte aligned, scales 4-byte");
  const size_t need = attn::decode_workspace_bytes(B, 1, Hq, Hkv, Dk, Dv, max_kv_len, window);
  if (!workspace || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(ATTN_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  const size_t no = (size_t)B * Hq * Dv * 2, nq = (size_t)B * Hq * Dk * 2;
  if (overlap(o, no, q, nq) || overlap(workspace, need, o, no) || overlap(workspace, need, q, nq))
    return fail(ATTN_ERR_ALIAS, "o / workspace must not overlap q or each other");
  attn::DecodeArgs a{};
  a.q = q; a.k_cache = k_codes; a.v_cache = v_codes; a.k_scale = k_scales;
  a.v_scale = v_scales; a.row_offset = row_offset; a.kv_len = kv_len; a.o = o;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Dk = Dk; a.Dv = Dv;
  a.window = window > 0 ? window : 0;
  a.rot_pairs = rope.rotary_dims / 2;
  a.theta = rope.rotary_dims > 0 ? rope.theta : 1.0;
  a.scale = scale;
  a.max_kv_len = max_kv_len;
  a.workspace = workspace;
  return launch_status(attn::launch_decode_int8(a, reinterpret_cast<hipStream_t>(stream)),
                       "int8 decode");
}

attn_status_t prope_apply(const void* x, void* y, const int32_t* positions, int32_t N,
                          int32_t H, int32_t D, attn_rope_t rope, attn_dtype_t dtype,
                          void* stream) {
  return prope_call(x, y, positions, N, H, D, 1, rope, dtype, stream);
}

attn_status_t prope_apply_2d(const void* x, void* y, const int32_t* positions_xy, int32_t N,
                             int32_t H, int32_t D, attn_rope_t rope, attn_dtype_t dtype,
                             void* stream) {
  if (D % 4) return fail(ATTN_ERR_SHAPE, "D=%d must be a multiple of 4 (two even halves)", D);
  return prope_call(x, y, positions_xy, N, H, D, 2, rope, dtype, stream);
}

}  // extern "C"
