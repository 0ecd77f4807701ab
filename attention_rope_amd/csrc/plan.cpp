// plan.cpp — host-side planning of the kernels: which shapes each path
// supports, the decode split-K plan and the workspace sizes that follow from
// it. Plain host C++ with no device code, so a sanitizer build of the ABI
// layer (abi.cpp) can include it as it is.
#include "kernels.h"

namespace attn {

// Split-K plan: each workgroup streams `ch` consecutive visible rows of one
// sequence for one KV head. A workgroup's start (locating its rows, turning
// the query, filling the DMA ring) and end (draining, writing its partial)
// leave its CU's memory pipe idle, so chunks are made as long as possible:
// up to kMaxChunk rows (global layers) or the whole window (local layers),
// halved while the grid would hold fewer than kMinGroups workgroups.
constexpr int kMaxChunk = 4096, kMinChunk = 256, kMinGroups = 512;

// groups: workgroups per (sequence, chunk); n_q new tokens per sequence widen
// a window's range by n_q - 1 rows.
SplitPlan decode_plan(int B, int groups, int max_kv_len, int window, int n_q) {
  const int64_t wr = (int64_t)window + n_q - 1;
  const int range = (window > 0 && wr < max_kv_len) ? (int)wr : max_kv_len;
  int ch = (window > 0) ? range : kMaxChunk;
  ch = ch > kMaxChunk ? kMaxChunk : (ch < 1 ? 1 : ch);
  auto splits = [&](int c) { return (int)(((int64_t)range + c - 1) / c); };
  while (ch > kMinChunk && (int64_t)B * groups * splits(ch) < kMinGroups) ch = (ch + 1) / 2;
  return {ch, splits(ch)};
}

// 16-column groups of (token, head) pairs per KV head.
int decode_column_groups(int n_q, int G) { return (n_q * G + 15) / 16; }

// Column groups one decode workgroup serves from the same cache rows (one set
// of waves each): 1, 2 or 4 (a verify call with more than 16 (token, head)
// pairs per KV head; 3 groups take 4 with one idle set rather than a second
// pass over the rows).
int decode_groups_per_block(int n_q, int G) {
  const int n = decode_column_groups(n_q, G);
  return n >= 3 ? 4 : n;
}

// Workgroups per (sequence, chunk, KV head).
int decode_column_blocks(int n_q, int G) {
  const int n = decode_groups_per_block(n_q, G);
  return (decode_column_groups(n_q, G) + n - 1) / n;
}

// Turned queries of a verify call (n_q > 1) ahead of the partials.
size_t decode_rotated_q_bytes(int B, int n_q, int Hq, int Dk) {
  if (n_q <= 1) return 0;
  return ((size_t)B * n_q * Hq * Dk * 2 + 255) & ~(size_t)255;
}

size_t decode_workspace_bytes(int B, int n_q, int Hq, int Hkv, int Dk, int Dv, int max_kv_len,
                              int window) {
  if (B <= 0 || n_q <= 0 || Hq <= 0 || Hkv <= 0 || Dv <= 0 || max_kv_len <= 0) return 0;
  const int ncb = decode_column_blocks(n_q, Hq / Hkv);
  const int ns = decode_plan(B, Hkv * ncb, max_kv_len, window, n_q).ns;
  return decode_rotated_q_bytes(B, n_q, Hq, Dk) + (size_t)B * n_q * Hq * ns * (Dv + 2) * sizeof(float);
}

bool decode_shape_fits(int B, int n_q, int Hq, int Hkv, int Dk, int Dv, int max_kv_len,
                       int window) {
  const int ncb = decode_column_blocks(n_q, Hq / Hkv);
  const SplitPlan pl = decode_plan(B, Hkv * ncb, max_kv_len, window, n_q);
  // 32-bit chunk-relative offsets (chunk plus the deepest read-ahead) and the
  // grid's x and y extents.
  const int64_t row = (int64_t)Hkv * (Dk > Dv ? Dk : Dv) * 2;
  return pl.ns <= 65535 && (int64_t)Hkv * ncb < ((int64_t)1 << 31) &&
         ((int64_t)pl.ch + 192) * row < ((int64_t)1 << 31);
}

bool decode_supported(int Dk, int Dv, int G) {
  const bool kdim = Dk == 128 || Dk == 256 || Dk == 512;
  const bool vdim = Dv == 128 || Dv == 256 || (Dv == 512 && Dk == 512);
  return kdim && vdim && G >= 1 && G <= 16;
}

bool decode_int8_supported(int Dk, int Dv, int G) {
  return (Dk == 512 || Dk == 256) && Dv == 256 && G >= 1 && G <= 16;
}

bool prefill_mfma_supported(int Dk, int Dv, int G, float scale, int rotary_dims) {
  const bool shape = (Dk == 128 && Dv == 128) || (Dk == 256 && Dv == 256) ||
                     (Dk == 512 && (Dv == 256 || Dv == 512));
  const bool rot = rotary_dims == 0 || rotary_dims == Dk / 4 || rotary_dims == Dk;
  return shape && rot && (G == 1 || G == 2 || G == 4 || G == 8) && scale >= 0.f;
}

}  // namespace attn
