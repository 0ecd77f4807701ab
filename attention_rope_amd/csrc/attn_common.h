// attn_common.h — device-side helpers shared by the gfx950 kernels of the
// hybrid-attention library (types, bf16 conversion, launch-parameter structs).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two fp32 -> packed bf16x2 bits, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu);
}

// Rotary frequency of pair p for head dim D: theta^(-2p/D), in fp64.
__device__ __forceinline__ double rope_freq(int p, int D, double log2_theta) {
  return exp2(-2.0 * (double)p / (double)D * log2_theta);
}

// Angle pos * w reduced and evaluated in fp64, returned as fp32 cos/sin.
__device__ __forceinline__ void rope_cos_sin(int64_t pos, double w, float* c, float* s) {
  double sd, cd;
  sincos((double)pos * w, &sd, &cd);
  *c = (float)cd;
  *s = (float)sd;
}

// Reductions over the 4 lanes {l, l^16, l^32, l^48} with the gfx950 row-swap
// instructions (no LDS traffic): v_permlane32_swap exchanges lane halves and
// v_permlane16_swap exchanges neighbouring 16-lane rows, so each step leaves
// {x[l], x[l^32]} (then {y[l], y[l^16]}) in the two results of every lane.
__device__ __forceinline__ float xor32_16_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xor32_16_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Blocks are dispatched round-robin over the 8 XCDs (block x runs on XCD x%8).
// Return the logical index such that each XCD receives one contiguous range of
// logical indices, keeping neighbouring tiles on the same L2.
__device__ __forceinline__ int xcd_contiguous(int x, int n) {
  const int q = n / 8, r = n % 8;
  const int xcd = x % 8, j = x / 8;
  return (xcd < r) ? xcd * (q + 1) + j : r * (q + 1) + (xcd - r) * q + j;
}

}  // namespace attn
