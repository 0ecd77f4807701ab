// prefill_common.h — LDS layout and RoPE helpers shared by the MFMA prefill
// kernels (prefill_mfma.hip, prefill_mfma2g.hip, prefill_mfma1w.hip).
#pragma once
#include "attn_common.h"

namespace attn {
namespace prefill {

// XOR swizzle of 16-byte chunks inside a region row of `width` chunks. The
// mask P-1 uses the largest power of two P <= 16 dividing the width, so the
// swizzled index stays inside the row.
template <int width>
struct Swz {
  static constexpr int P = (width & 15) == 0 ? 16 : (width & 7) == 0 ? 8 : (width & 3) == 0 ? 4
                           : (width & 1) == 0 ? 2 : 1;
  static constexpr int M = P - 1;
};
template <int width>
__device__ __forceinline__ int kswz(int r, int c) {
  return c ^ (r & Swz<width>::M);
}
// V rows: chunk c of key row r sits at c ^ 4(r & 3). A transposing read of
// the V^T operand takes 4 consecutive keys x 4 consecutive chunks (one
// 32-dim tile) per 32 lanes; this swizzle puts the 16 pieces in 16 distinct
// bank groups (an XOR by r & 15 would keep them in 4).
__device__ __forceinline__ int vswz(int r, int c) { return c ^ ((r & 3) << 2); }

// One rotary pair (two bf16 in a dword) turned by (c, s) in fp32.
__device__ __forceinline__ uint32_t rot_pair(uint32_t w, float c, float s) {
  const float x0 = bf16_lo(w), x1 = bf16_hi(w);
  return pack_bf16x2(x0 * c - x1 * s, x0 * s + x1 * c);
}
// Rotate 8 bf16 (4 pairs) with (c0 s0 c1 s1) (c2 s2 c3 s3).
__device__ __forceinline__ u32x4 rotate4(u32x4 w, f32x4 t0, f32x4 t1) {
  u32x4 r;
  r[0] = rot_pair(w[0], t0[0], t0[1]);
  r[1] = rot_pair(w[1], t0[2], t0[3]);
  r[2] = rot_pair(w[2], t1[0], t1[1]);
  r[3] = rot_pair(w[3], t1[2], t1[3]);
  return r;
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace prefill
}  // namespace attn
