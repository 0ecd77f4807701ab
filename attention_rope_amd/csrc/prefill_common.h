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

typedef __attribute__((address_space(3))) f32x2 lds_float2;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

// Base row of a wave's Q rotation: slot[p] = (cos, sin) of pair p at position
// pos (p < P), the angle pos * theta^(-2p/D) formed and evaluated in fp64.
// Lanes take pairs lane, lane + 64, ...; the caller reads the slot only after
// the wave's LDS writes landed (rotate_q_chunks waits for them).
__device__ __forceinline__ void rope_base_row(lds_float2* slot, int64_t pos, int P, int D,
                                              double log2_theta, int lane) {
  for (int p = lane; p < P; p += 64) {
    float c, s;
    rope_cos_sin(pos, rope_freq(p, D, log2_theta), &c, &s);
    slot[p] = f32x2{c, s};
  }
}

// The (cos, sin) of d * rho^i for the pairs i = 8u + 4h + j (u < NU, j < 4)
// of this lane's rotated Q^T chunks 2u + h: the small angle that turns the
// base row's pair i from the wave's base position to the lane's own (d
// positions further). rho = theta^(-2/D), so rho^i is pair i's frequency;
// the powers come from an fp64 product chain, d * rho^i / (2 pi) is formed in
// fp64 and its fraction goes through the sine and cosine units (which take
// revolutions). Issued before the wait for Q, so it runs under Q's latency.
template <int NU>
__device__ __forceinline__ void rope_offsets(float (&dcs)[NU > 0 ? NU : 1][8], int d,
                                             double rho, int h) {
  const double rho2 = rho * rho, rho4 = rho2 * rho2, rho5 = rho4 * rho;
  const double turns = (double)d * 0.15915494309189535;  // d / (2 pi)
  double w = h ? rho4 : 1.0;
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = __builtin_amdgcn_fractf((float)(turns * w));
      dcs[u][2 * j] = __builtin_amdgcn_cosf(x);
      dcs[u][2 * j + 1] = __builtin_amdgcn_sinf(x);
      w *= (j == 3) ? rho5 : rho;
    }
}

// Turn this lane's first NU Q^T chunks (qw[u] = dims 16u + 8h .. +7) by the
// base row in `slot` combined with the offsets from rope_offsets: (c, s) of
// base + offset by angle addition, then rotate4. Waits for the slot's LDS
// writes first, and for the slot's reads before returning (the memory clobber
// keeps later DMAs into the slot's region behind them).
template <int NU>
__device__ __forceinline__ void rotate_q_chunks(u32x4* qw, const lds_float2* slot,
                                                const float (&dcs)[NU > 0 ? NU : 1][8], int h) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const lds_f32x4* trow = (const lds_f32x4*)slot;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const f32x4 t0 = trow[4 * u + 2 * h], t1 = trow[4 * u + 2 * h + 1];
    float cs[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float cb = (j < 2 ? t0 : t1)[2 * (j % 2)], sb = (j < 2 ? t0 : t1)[2 * (j % 2) + 1];
      const float cd = dcs[u][2 * j], sd = dcs[u][2 * j + 1];
      cs[2 * j] = cb * cd - sb * sd;
      cs[2 * j + 1] = sb * cd + cb * sd;
    }
    qw[u] = rotate4(qw[u], f32x4{cs[0], cs[1], cs[2], cs[3]}, f32x4{cs[4], cs[5], cs[6], cs[7]});
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

}  // namespace prefill
}  // namespace attn
