/*
 * attn_rope.h — C ABI of the MI355X (gfx950) hybrid-attention library.
 *
 * The library computes the decoder attention of the Gemma 4 family as its
 * pages describe it: causal grouped-query attention in a sliding-window
 * (local) form and a full-context (global) form, with proportional RoPE on the
 * queries and keys.
 *   - "Gemma 4: End-to-End Architecture Walkthrough", Phase 3: section 3a
 *     (local layers see a fixed recent window — 512 or 1024 tokens — global
 *     layers the whole preceding context), section 3b (8 query heads per KV
 *     head in global layers, 2 in local ones, wider global keys) and section
 *     3c (p-RoPE: only the first quarter of the rotary pairs turn).
 *   - "Gemma 4 Architecture Reference": "Attention Architecture",
 *     "Positional Encoding: Proportional RoPE (p-RoPE)" (p = 0.25, theta = 1e6)
 *     and "Shared KV Cache" (later layers reuse an earlier layer's K/V: pass
 *     the same k/v pointers again; no separate entry point is needed).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller. The library
 *     never allocates or frees device memory, keeps no state between calls,
 *     never synchronises, and enqueues its kernels on `stream` (a hipStream_t;
 *     NULL = the default stream). Calls return as soon as the work is queued.
 *   - Layouts are dense row-major with the last dimension contiguous.
 *   - Element type: ATTN_BF16 (bfloat16 in and out, fp32 accumulation) or
 *     ATTN_F32 (fp32 throughout). All tensors of one call share it.
 *   - Every argument is validated on the host before any HIP call; on error
 *     nothing is launched and a status != ATTN_OK is returned, with detail in
 *     attn_last_error(). No call prints, throws or aborts.
 *   - Thread-safe: calls may come from several host threads at once.
 *
 * RoPE reading (the pages leave pairing and frequency base open): dims
 * (2p, 2p+1) form pair p, which turns by angle pos * theta^(-2p/D), D the full
 * head dim; only pairs p < rotary_dims/2 turn, the rest pass through
 * unchanged. rotary_dims = D is textbook RoPE, rotary_dims = D/4 is p-RoPE
 * with p = 0.25, rotary_dims = 0 disables rotation.
 */
#ifndef ATTN_ROPE_H
#define ATTN_ROPE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,       /* sizes inconsistent or out of range */
  ATTN_ERR_UNSUPPORTED = 3, /* valid but not implemented (e.g. head dim) */
  ATTN_ERR_WORKSPACE = 4,   /* workspace missing or too small */
  ATTN_ERR_LAUNCH = 5,      /* the HIP runtime refused a launch */
  ATTN_ERR_ALIAS = 6        /* an output overlaps an input it must not */
} attn_status_t;

/* Rotary settings: rotary_dims even, 0 <= rotary_dims <= head dim; theta > 0. */
typedef struct {
  int32_t rotary_dims;
  double theta;
} attn_rope_t;

enum { ATTN_ROPE_Q = 1, ATTN_ROPE_K = 2 };

/*
 * Prefill: o = softmax(scale * rope(q) rope(k)^T + mask) v for every query
 * row, per batch b and query head h, with KV head h / (Hq / Hkv).
 * Source: "Gemma 4: End-to-End Architecture Walkthrough", Phase 3 section 3a
 * (a local layer's query sees a fixed window of recent keys, a global layer's
 * every earlier key), section 3b (grouped-query attention: 2 query heads per
 * KV head on local layers, 8 on global ones, with wider global keys) and
 * section 3c (p-RoPE turns only the leading rotary pairs; the angle is the
 * token position times the pair's frequency).
 *   q [B, T, Hq, Dk], k [B, T, Hkv, Dk], v [B, T, Hkv, Dv]: unrotated inputs;
 *   o [B, T, Hq, Dv] output; must not overlap q, k or v.
 *   Token t of every batch row sits at position pos0 + t (pos0 >= 0,
 *   pos0 + T <= 2^31 - 1); rope_mask: ATTN_ROPE_Q | ATTN_ROPE_K selects which
 *   of q and k are rotated there. rope.rotary_dims == 0 or rope_mask == 0:
 *   nothing turns.
 *   window: <= 0 or >= T gives full causal attention; otherwise query i sees
 *   keys j with i - window < j <= i (the window includes the query itself).
 *   scale: finite (1/sqrt(Dk) in the usual model).
 * Supported: B, T >= 0 (an empty problem is a no-op), Hq % Hkv == 0,
 *   Dk, Dv even and <= 512. bf16 with (Dk, Dv) in {(128,128), (256,256),
 *   (512,256), (512,512)}, Hq/Hkv in {1, 2, 4, 8}, scale >= 0 and
 *   rotary_dims a multiple of 8 in {0, Dk/4, Dk} runs the MFMA flash kernel
 *   ((512,512) in one pass when k == v and K does not turn in the call,
 *   the keys-as-values form below; with separate values as two passes over
 *   256-dim halves of v and o); every other
 *   supported case runs a slower general kernel with the same results.
 *   Keys as values (K = V on a global layer): turn k once with prope_apply,
 *   pass it as both k and v with rope_mask = ATTN_ROPE_Q; the values are
 *   then the rotated keys, as a decode over that cache sees them.
 *   Every rotation angle is (pos0 + t) * theta^(-2p/Dk), formed from this
 *   call's own pos0 and rope arguments in fp64 inside the kernels.
 * Workspace: attn_prefill_workspace_bytes() bytes of device memory, 16-byte
 *   aligned (0 when nothing needs it: workspace may then be NULL). When K
 *   turns (ATTN_ROPE_K with rotary_dims > 0), the call first turns K's rotary
 *   dims once into it, [B, T, Hkv, rotary_dims] in the element type, and the
 *   attention kernel reads them from there.
 *   Contents are scratch, owned by the caller; the workspace must not overlap
 *   any tensor argument.
 * Errors (nothing is launched): NULL tensors -> ATTN_ERR_NULL; bad sizes,
 *   rope settings, pos0 or alignment -> ATTN_ERR_SHAPE; an unknown dtype ->
 *   ATTN_ERR_UNSUPPORTED; workspace missing or too small ->
 *   ATTN_ERR_WORKSPACE; overlaps -> ATTN_ERR_ALIAS; a refused launch ->
 *   ATTN_ERR_LAUNCH.
 * All tensor pointers must be 16-byte aligned.
 */
size_t attn_prefill_workspace_bytes(int32_t B, int32_t T, int32_t Hkv, int32_t Dk,
                                    attn_rope_t rope, int32_t rope_mask,
                                    attn_dtype_t dtype);

attn_status_t attn_prefill(const void *q, const void *k, const void *v, void *o,
                           int32_t B, int32_t T, int32_t Hq, int32_t Hkv,
                           int32_t Dk, int32_t Dv, int32_t window, float scale,
                           attn_rope_t rope, int32_t rope_mask, int32_t pos0,
                           void *workspace, size_t workspace_bytes,
                           attn_dtype_t dtype, void *stream);

/*
 * Prefill that also fills the decode cache: attn_prefill with rope_mask =
 * ATTN_ROPE_Q | ATTN_ROPE_K, whose K/V pass additionally writes every key,
 * turned at its position, and every value into the caches a later
 * attn_decode / attn_verify reads.
 * Source: "Gemma 4: End-to-End Architecture Walkthrough", Phase 3 section 3b
 * (the keys and values of the context are kept for the layers that attend
 * them) and Phase 4 (the draft model attends the cache the target model has
 * filled); the cached keys carry their rotation, as attn_decode expects.
 *   q, k, v, o, B, T, Hq, Hkv, Dk, Dv, window, scale, rope, pos0: as for
 *     attn_prefill (o is the same output).
 *   k_cache [cache_rows, Hkv, Dk], v_cache [cache_rows, Hkv, Dv]: written at
 *     rows row_offset[b] + t for t < T: k_cache gets rope(k[b, t]) at position
 *     pos0 + t (all Dk dims, the leading rotary_dims turned), v_cache gets
 *     v[b, t]. Other rows are not touched. Caller-owned device buffers.
 *   row_offset: device int64 [B], 8-byte aligned. A batch row with
 *     row_offset[b] < 0 or row_offset[b] + T > cache_rows is not written to
 *     the cache (its o still is).
 * Supported: Dk, Dv and rotary_dims multiples of 8; otherwise as attn_prefill.
 *   Keys-as-values layers fill their one cache with prope_apply instead.
 * Workspace: attn_prefill_workspace_bytes(B, T, Hkv, Dk, rope,
 *   ATTN_ROPE_Q | ATTN_ROPE_K, dtype) bytes.
 * Errors: as attn_prefill; NULL caches or row_offset -> ATTN_ERR_NULL;
 *   caches overlapping each other, q, k, v, o, the workspace or row_offset ->
 *   ATTN_ERR_ALIAS; cache_rows < T -> ATTN_ERR_SHAPE.
 */
attn_status_t attn_prefill_into_cache(const void *q, const void *k, const void *v, void *o,
                                      int32_t B, int32_t T, int32_t Hq, int32_t Hkv,
                                      int32_t Dk, int32_t Dv, int32_t window, float scale,
                                      attn_rope_t rope, int32_t pos0, void *k_cache,
                                      void *v_cache, const int64_t *row_offset,
                                      int64_t cache_rows, void *workspace,
                                      size_t workspace_bytes, attn_dtype_t dtype,
                                      void *stream);

/*
 * Decode: one new token per sequence over a ragged KV cache (bf16 only).
 * Source: "Gemma 4: End-to-End Architecture Walkthrough", Phase 3 section 3b
 * (global layers must keep the keys and values of the whole context; local
 * layers only their window) and "Gemma 4 Architecture Reference", "Shared KV
 * Cache"; the new token attends the cache exactly as its row of a prefill
 * over the whole sequence would.
 *   q [B, Hq, Dk]: the new tokens' queries, unrotated; sequence b's query sits
 *     at position kv_len[b] - 1 and is rotated there (rope applies to q only).
 *   k_cache [rows, Hkv, Dk], v_cache [rows, Hkv, Dv]: cached keys (stored
 *     already rotated; attn_prefill_into_cache writes a prompt's rows) and
 *     values; sequence b owns rows
 *     row_offset[b] .. row_offset[b] + kv_len[b] - 1, the last one being the
 *     new token's own row (the caller appends it before the call).
 *   Keys as values (K = V, the global-layer form of "Gemma 4: End-to-End
 *     Architecture Walkthrough", Phase 3 section 3b, and of the "Gemma 4
 *     Technical Report" reader, "Core Model Architecture"): pass the same
 *     pointer as k_cache and v_cache with Dv == Dk. The attention weights then
 *     multiply the cached (rotated) keys, and each cache row is read once for
 *     both products.
 *   row_offset: device int64 [B]; kv_len: device int32 [B], 0 <= kv_len[b] <=
 *     max_kv_len. kv_len[b] == 0 gives o[b] = 0. The caches carry no row
 *     count, and these two arrays live on the device, so the library cannot
 *     check them against the caches' size: the caller guarantees that every
 *     row a sequence owns lies inside both caches (a kv_len[b] above
 *     max_kv_len is caught in-kernel: o[b] becomes NaN and no row is read).
 *   window: <= 0: all rows; otherwise only the last `window` rows
 *     [kv_len - window, kv_len) are read (rows before are never touched, so
 *     they may hold anything).
 *   o [B, Hq, Dv] output.
 *   Drafter cross-attention (an MTP drafter attends the target model's cache,
 *     "Gemma 4: End-to-End Architecture Walkthrough", Phase 4): for the
 *     drafter's k-th proposal at position L + k over a target cache of L
 *     rows, turn q there with prope_apply, then call attn_decode with
 *     rope.rotary_dims = 0, kv_len = L and window = W - k - 1 (0 for global
 *     layers). On a local layer this holds for k < W - 1; from k = W - 1 on
 *     no target row lies inside the proposal's window, so there is nothing to
 *     attend (the result is the empty-row 0) and no call is made.
 * Supported: Hq % Hkv == 0 with Hq / Hkv <= 16, Dk in {128, 256, 512},
 *   Dv in {128, 256} (or 512 with Dk = 512); max_kv_len >= 1, and a cache
 *   that fits one call (ATTN_ERR_SHAPE past about 5 * 10^8 rows per sequence,
 *   or past 2 GB per 8192 rows of all KV heads).
 * Workspace: attn_decode_workspace_bytes() bytes of device memory for the
 *   split-K partial results (the split depends on B, Hkv, max_kv_len and
 *   window, so pass the same values to both calls); contents are scratch.
 */
size_t attn_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t Dv,
                                   int32_t max_kv_len, int32_t window);

attn_status_t attn_decode(const void *q, const void *k_cache, const void *v_cache,
                          const int64_t *row_offset, const int32_t *kv_len,
                          void *o, int32_t B, int32_t Hq, int32_t Hkv,
                          int32_t Dk, int32_t Dv, int32_t window, float scale,
                          attn_rope_t rope, int32_t max_kv_len, void *workspace,
                          size_t workspace_bytes, attn_dtype_t dtype,
                          void *stream);

/*
 * Decode that allocates nothing, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): attn_decode's arguments and results without the
 * workspace. The split-K partials live in a static device array of
 * attn_decode_noalloc_max_bytes() bytes (32 MiB) inside the library, one
 * copy per GPU, held until the process ends. A call whose partials need more
 * (attn_decode_workspace_bytes() of the same arguments above that size)
 * returns ATTN_ERR_WORKSPACE and launches nothing. Every call on a GPU uses
 * that GPU's one array: calls that overlap on one GPU (other streams, or host
 * threads without ordering) race on it. Nothing in it needs clearing between
 * calls: a call reads only partials it wrote itself.
 */
size_t attn_decode_noalloc_max_bytes(void);

attn_status_t attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                  const int64_t *row_offset, const int32_t *kv_len,
                                  void *o, int32_t B, int32_t Hq, int32_t Hkv,
                                  int32_t Dk, int32_t Dv, int32_t window, float scale,
                                  attn_rope_t rope, int32_t max_kv_len, attn_dtype_t dtype,
                                  void *stream);

/*
 * Verify (speculative decoding) / append attention: n_q new tokens per
 * sequence at once, as when a target model checks a drafter's proposals in one
 * pass ("Gemma 4: End-to-End Architecture Walkthrough", Phase 4; "Gemma 4
 * Technical Report" reader, "Speculative Decoding and Infrastructure").
 *   Sequence b's last n_q cache rows are the new tokens (the caller appends
 *   them, rotated keys, before the call). Token j sits at position
 *   p_j = kv_len[b] - n_q + j and attends exactly what a one-token decode at
 *   kv_len = p_j + 1 would: cache rows up to its own (causal within the
 *   draft), or the last `window` of those.
 *   q [B, n_q, Hq, Dk] unrotated (token j is turned at p_j);
 *   o [B, n_q, Hq, Dv]. Caches, row_offset, window, rope, scale, K = V and
 *   the supported shapes as for attn_decode; n_q in [1, 4096].
 *   kv_len[b] == 0 gives o[b] = 0; 0 < kv_len[b] < n_q (tokens without
 *   their rows) or kv_len[b] > max_kv_len poison o[b] with NaN.
 *   n_q * (Hq / Hkv) <= 64 reads each cache row once per KV head (pairs
 *   in groups of 16, up to four groups per workgroup); more (token, head)
 *   pairs re-read it once per 64.
 * Workspace: attn_verify_workspace_bytes() bytes (the turned queries and the
 *   split-K partials); contents are scratch.
 */
size_t attn_verify_workspace_bytes(int32_t B, int32_t n_q, int32_t Hq, int32_t Hkv,
                                   int32_t Dk, int32_t Dv, int32_t max_kv_len,
                                   int32_t window);

attn_status_t attn_verify(const void *q, const void *k_cache, const void *v_cache,
                          const int64_t *row_offset, const int32_t *kv_len,
                          void *o, int32_t B, int32_t n_q, int32_t Hq, int32_t Hkv,
                          int32_t Dk, int32_t Dv, int32_t window, float scale,
                          attn_rope_t rope, int32_t max_kv_len, void *workspace,
                          size_t workspace_bytes, attn_dtype_t dtype, void *stream);

/*
 * (p-)RoPE on its own: y[n, h, :] = rope(x[n, h, :], positions[n]).
 * Source: "Gemma 4: End-to-End Architecture Walkthrough", Phase 3 section 3c
 * (pair p of a head vector turns by position * theta^(-2p/D); p-RoPE keeps
 * only the leading quarter of the pairs turning) and "Gemma 4 Architecture
 * Reference", "Positional Encoding: Proportional RoPE (p-RoPE)" (p = 0.25,
 * theta = 1e6 on global layers).
 *   x, y [N, H, D]; positions: device int32 [N], each >= 0.
 *   y may equal x (in place: dims >= rotary_dims are then not touched);
 *   partial overlap is rejected (ATTN_ERR_ALIAS). D even, 2 <= D <= 1024;
 *   bad sizes or rope settings -> ATTN_ERR_SHAPE; NULL -> ATTN_ERR_NULL.
 */
attn_status_t prope_apply(const void *x, void *y, const int32_t *positions,
                          int32_t N, int32_t H, int32_t D, attn_rope_t rope,
                          attn_dtype_t dtype, void *stream);

/*
 * int8 KV cache ("Gemma 4 Technical Report" reader, "Quantization and
 * Efficiency": int8 KV caching). The pages give no scheme; this library's:
 * symmetric codes, one fp32 scale per (cache row, KV head):
 *   s = max_d |x[n, h, d]| / 127, codes[n, h, d] = round-half-even(x / s)
 *   (fp32, IEEE division; a row of zeros gets s = 0 and codes 0).
 * attn_kv_quantize_int8: x [N, H, D] bf16 (16-byte aligned) -> codes int8
 *   [N, H, D], scales float [N, H]; D in {128, 256, 512}; no overlaps.
 * attn_decode_int8: attn_decode over such caches, attending the dequantised
 *   rows code * s. k_codes [rows, Hkv, Dk] / k_scales [rows, Hkv] hold the
 *   keys (already rotated before quantising), v_codes / v_scales the values;
 *   other arguments as for attn_decode. (Dk, Dv) in {(512, 256), (256, 256)};
 *   bf16 q and o. Reads half the bytes of the bf16 cache.
 * Workspace: attn_decode_int8_workspace_bytes() bytes (split-K partials).
 */
attn_status_t attn_kv_quantize_int8(const void *x, int8_t *codes, float *scales,
                                    int32_t N, int32_t H, int32_t D,
                                    attn_dtype_t dtype, void *stream);

size_t attn_decode_int8_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t Dv,
                                        int32_t max_kv_len, int32_t window);

attn_status_t attn_decode_int8(const void *q, const int8_t *k_codes, const float *k_scales,
                               const int8_t *v_codes, const float *v_scales,
                               const int64_t *row_offset, const int32_t *kv_len, void *o,
                               int32_t B, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv,
                               int32_t window, float scale, attn_rope_t rope,
                               int32_t max_kv_len, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * 2-D RoPE for image patches ("Gemma 4: End-to-End Architecture Walkthrough",
 * Phase 1 section 1b; "Gemma 4 Architecture Reference", "Vision Encoder"):
 * each patch vector is split in half and each half is turned like a
 * D/2-dim RoPE vector, the first half by the patch's width (x) coordinate,
 * the second by its height (y) coordinate.
 *   y[n, h, 0:D/2] = rope(x[n, h, 0:D/2], positions_xy[n][0]),
 *   y[n, h, D/2:D] = rope(x[n, h, D/2:D], positions_xy[n][1]),
 *   with pair p of a half turned by coordinate * theta^(-2p/(D/2)) for the
 *   first rope.rotary_dims dims of each half.
 *   x, y [N, H, D], D a multiple of 4, 4 <= D <= 1024; positions_xy: device
 *   int32 [N, 2], each >= 0; rope.rotary_dims even, <= D/2. In place and
 *   overlap rules as for prope_apply.
 */
attn_status_t prope_apply_2d(const void *x, void *y, const int32_t *positions_xy,
                             int32_t N, int32_t H, int32_t D, attn_rope_t rope,
                             attn_dtype_t dtype, void *stream);

/* Static text for a status code. */
const char *attn_status_string(attn_status_t s);

/* Detail of the last non-OK status returned on this host thread ("" if none). */
const char *attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_ROPE_H */
