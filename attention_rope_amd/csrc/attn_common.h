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
typedef short s16x4 __attribute__((ext_vector_type(4)));

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

// ---- LDS DMA streaming (buffer loads with the lds flag) --------------------

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Raw buffer descriptor (stride 0, 32-bit format): reads at byte offsets
// >= bytes return 0. Word 3 = 0x00020000 selects that format on gfx9.
__device__ __forceinline__ u32x4 buffer_desc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(p >> 32) & 0xffffu)),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), 0x00020000u};
}

// One DMA: lane l copies 16 bytes at byte offset voff of the buffer into LDS
// at lds + 16 l. M0 carries the LDS base and is restored afterwards. Issued
// from inline asm, so the compiler sees no LDS DMA and adds none of its
// conservative "wait for every LDS DMA" stalls before LDS reads: the caller
// waits explicitly (the instruction counts in vmcnt like any buffer load).
// STREAM marks data read once (the nt cache policy), such as a KV cache during
// decode; tiles that neighbouring workgroups re-read keep the default policy.
template <bool STREAM = false>
__device__ __forceinline__ void dma16(u32x4 desc, uint32_t lds, uint32_t voff) {
  uint32_t saved;
  if constexpr (STREAM)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(voff), "s"(desc));
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(voff), "s"(desc));
}

// Synchronise the workgroup after this wave's LDS reads have returned. Unlike
// __syncthreads this carries no memory fence, which would also wait for the
// DMAs still in flight; the memory clobber keeps LDS accesses on their side.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most n vector-memory operations of this wave are in flight
// (vmcnt = n in bits 3:0 and 15:14; expcnt and lgkmcnt left alone), and keep
// the scheduler from hoisting LDS reads of what landed above the wait.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace attn
