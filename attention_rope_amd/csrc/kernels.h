// kernels.h — host-side launch functions of the gfx950 kernels. All launches
// go onto the given stream and return the launch status; nothing synchronises.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// ---- RoPE -----------------------------------------------------------------
// NH = 1: pos [N]; NH = 2 (2-D RoPE): pos [N, 2], each half of D turned by
// its own coordinate. P = rotary pairs per half.
hipError_t launch_prope(const void* x, void* y, const int32_t* pos, int N, int H,
                        int D, int P, int NH, double theta, bool bf16, hipStream_t st);
// out[b, t, h, 0:R] = rotation of the first R dims of k[b, t, h, :] at
// position pos0 + t (bf16 or fp32 elements, R even).
hipError_t launch_rope_k_lead(const void* k, void* out, int B, int T, int H, int D, int R,
                              int pos0, double theta, bool bf16, hipStream_t st);
// K turned into the workspace (as launch_rope_k_lead) and into k_cache rows
// row_offset[b] + t, V copied into v_cache rows, in one pass (rope.hip).
hipError_t launch_prefill_cache_fill(const void* k, const void* v, void* k_cache, void* v_cache,
                                     void* k_rot, const int64_t* row_offset, int64_t cache_rows,
                                     int B, int T, int H, int Dk, int Dv, int R, int pos0,
                                     double theta, bool bf16, hipStream_t st);

// ---- prefill ----------------------------------------------------------------
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const void* k_rot;       // [B][T][Hkv][2*rot_pairs] K's rotary dims, turned (when K turns)
  int B, T, Hq, Hkv, Dk, Dv;
  int window;              // 0: full causal
  int rot_pairs;           // rotary pairs (0: none)
  int rope_q, rope_k;      // apply rotation to q / k
  float scale;
  // Element strides of v and o per token and per head (0: dense, Hkv * Dv
  // and Dv for v, Hq * Dv and Dv for o); the 512-dim value path runs as two
  // 256-dim halves over strided views.
  int64_t v_tok = 0, v_head = 0, o_tok = 0, o_head = 0;
  // Token t sits at position pos0 + t; pair p turns by (pos0 + t) *
  // theta^(-2p/Dk). log2_theta = log2(theta); rope_rho = theta^(-2/Dk), the
  // ratio of successive pair frequencies (kernels that turn a base row further
  // by a small position offset use it).
  int pos0 = 0;
  double log2_theta = 0.0;
  double rope_rho = 1.0;
  // Debug builds (ATTN_DEBUG_TILES) only: [0] += the (wave, key tile) pairs
  // whose scores a wave computes and softmaxes, [1] += the key tiles each
  // workgroup stages. Release kernels never read it.
  unsigned long long* dbg_visits = nullptr;
};
#ifdef ATTN_DEBUG_TILES
// Device address of the debug builds' two tile counters (prefill_general.hip).
hipError_t debug_visits_ptr(unsigned long long** p);
#endif

// MFMA flash kernel (bf16). Returns hipErrorNotSupported for shapes it has no
// instantiation for; the caller then uses the general kernel. When K turns,
// k_rot must hold K's rotary dims already turned (launch_rope_k_lead).
hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t st);
bool prefill_mfma_supported(int Dk, int Dv, int G, float scale, int rotary_dims);
// The variant for 512-dim keys (called by launch_prefill_mfma): 32-row
// waves, one per SIMD, accumulators in AGPRs (prefill_mfma1w.hip).
hipError_t launch_prefill_mfma1w(const PrefillArgs& a, hipStream_t st);
// Keys as values (k == v, Dk = Dv = 512, K not turned in the call) in one pass:
// O^T for 512 value dims in AGPRs, one key tile in LDS serving both products
// (prefill_kv1w.hip); called by launch_prefill_mfma.
bool prefill_kv1w_applies(const PrefillArgs& a);
hipError_t launch_prefill_kv1w(const PrefillArgs& a, hipStream_t st);
// The local-layer shape (256-dim heads, G = 2) with 4-wave workgroups, two
// per CU (prefill_mfma2g.hip); called by launch_prefill_mfma.
hipError_t launch_prefill_mfma2g(const PrefillArgs& a, hipStream_t st);

// General kernel: any supported shape, fp32 or bf16.
hipError_t launch_prefill_general(const PrefillArgs& a, bool bf16, hipStream_t st);

// ---- decode -----------------------------------------------------------------
struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int64_t* row_offset;
  const int32_t* kv_len;
  void* o;
  int B, Hq, Hkv, Dk, Dv;
  int window;              // 0: all rows
  int rot_pairs;
  double theta;
  float scale;
  int max_kv_len;
  void* workspace;
  // New tokens per sequence (1: decode). Token j of sequence b sits at
  // position kv_len[b] - n_q + j and attends the rows up to its own; q and o
  // are [B, n_q, Hq, D]. With q_rotated the queries are already turned.
  int n_q = 1;
  int q_rotated = 0;
  // int8 caches (attn_decode_int8): per (row, KV head) scales, fp32 [rows, Hkv].
  const float* k_scale = nullptr;
  const float* v_scale = nullptr;
};

// Split-K plan shared by the decode kernels: ch rows per chunk, ns chunks per
// sequence. groups = workgroups per (sequence, chunk).
struct SplitPlan {
  int ch, ns;
};
SplitPlan decode_plan(int B, int groups, int max_kv_len, int window, int n_q = 1);
// 16-column MFMA groups of (token, head) pairs per KV head, and the bytes of
// the turned queries a verify call keeps ahead of its partials.
int decode_column_groups(int n_q, int G);
int decode_groups_per_block(int n_q, int G);
int decode_column_blocks(int n_q, int G);
size_t decode_rotated_q_bytes(int B, int n_q, int Hq, int Dk);
// Merge of the chunk partials into o (any supported Dv).
hipError_t launch_decode_merge(const DecodeArgs& a, const SplitPlan& pl, hipStream_t st);

// Workspace of a decode (n_q = 1) or verify (n_q > 1) call: the split-K
// partials, and for n_q > 1 the turned queries ahead of them.
size_t decode_workspace_bytes(int B, int n_q, int Hq, int Hkv, int Dk, int Dv, int max_kv_len,
                              int window);
bool decode_supported(int Dk, int Dv, int G);
// Device scratch of attn_decode_noalloc: a file-scope array of this many
// bytes in decode.hip, one per GPU; decode_scratch returns the current
// device's copy (its address taken once per device, nothing allocated).
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
hipError_t decode_scratch(void** ptr);
bool decode_shape_fits(int B, int n_q, int Hq, int Hkv, int Dk, int Dv, int max_kv_len,
                       int window);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);

// ---- int8 KV cache -------------------------------------------------------------
// codes[n, h, :] = round-half-even(x / s), s = max|x[n, h, :]| / 127 (fp32).
hipError_t launch_kv_quantize_int8(const void* x, int8_t* codes, float* scales, int N, int H,
                                   int D, hipStream_t st);
// Decode over int8 caches (k_cache / v_cache hold the codes, k_scale / v_scale
// the scales); (Dk, Dv) in {(512, 256), (256, 256)}.
bool decode_int8_supported(int Dk, int Dv, int G);
hipError_t launch_decode_int8(const DecodeArgs& a, hipStream_t st);

}  // namespace attn
