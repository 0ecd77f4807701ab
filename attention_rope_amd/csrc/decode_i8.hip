// decode_i8.hip — single-token decode over an int8 KV cache on gfx950, and
// the quantiser that writes such a cache.
//
// The pages name int8 KV caching as a deployment option ("Gemma 4 Technical
// Report" reader, "Quantization and Efficiency", Table 3 caption) without a
// scheme. This library's scheme: symmetric codes with one fp32 scale per
// (cache row, KV head), s = max|x| / 127 and code = round-half-even(x / s).
// The attention itself is the decode of "Gemma 4: End-to-End Architecture
// Walkthrough", Phase 3 sections 3a-3c, over the dequantised rows code * s.
//
// Design for CDNA4: the cache bytes halve, so the kernel must turn twice as
// many rows per second into MFMA operands without adding HBM traffic.
//  * Same split-K plan, DMA ring, MFMA layout and output path as the bf16
//    streaming kernel; one wave per workgroup (16-row tiles, a 2-stage ring
//    of 25 KB) and at most 256 registers per wave, so six workgroups share
//    a CU. The bytes a CU keeps in flight grow with the workgroups resident,
//    and with one tile ahead per wave those bytes set the read rate.
//  * Scales never touch the codes: the K scale multiplies the 16 scores of a
//    tile after Q.K^T, the V scale multiplies the probabilities before P.V.
//  * Q.K^T on v_mfma_i32_16x16x64_i8 straight from the K codes in LDS: the
//    query is split into two int8 parts (a code and the code of its
//    residual), so two exact int32 products replace any conversion of K.
//  * V codes are converted once per tile into a bf16 tile in LDS, written
//    over the stage's own codes once Q.K^T has read them, from which the
//    transposing reads of the bf16 kernel build the P.V operand. They are
//    converted with a +128 bias: code ^ 0x80 is code + 128 as an
//    unsigned byte, which v_cvt_f32_ubyte turns into fp32 in one instruction
//    and which bf16 holds exactly; 128 * sum(bf16 P') per head is removed
//    from the P.V accumulator afterwards.
#include <algorithm>

#include "attn_common.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// One wave per (row, head): scale from the row's max magnitude (wave max),
// then codes by IEEE fp32 division and round-half-even.
template <int D>
__global__ __launch_bounds__(256) void kv_quantize_kernel(const uint16_t* __restrict__ x,
                                                          int8_t* __restrict__ codes,
                                                          float* __restrict__ scales,
                                                          int64_t rows) {
  constexpr int E = D / 64;  // elements per lane
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  float v[E];
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    v[e] = bf16_to_f32(x[r * D + lane * E + e]);
    amax = fmaxf(amax, fabsf(v[e]));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  const float s = __fdiv_rn(amax, 127.0f);
  int8_t c[E];
#pragma unroll
  for (int e = 0; e < E; ++e) c[e] = s > 0.f ? (int8_t)(int)rintf(__fdiv_rn(v[e], s)) : 0;
#pragma unroll
  for (int e = 0; e < E; ++e) codes[r * D + lane * E + e] = c[e];
  if (lane == 0) scales[r] = s;
}

// One DMA of 4 bytes per lane into LDS at lds + 4 lane (buffer_load_dword
// ... lds); counts in vmcnt like dma16.
__device__ __forceinline__ void dma4(u32x4 desc, uint32_t lds, uint32_t voff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dword %2, %3, 0 offen nt lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(desc));
}

// 4 biased codes (one dword) -> 4 fp32 values code + 128.
__device__ __forceinline__ f32x4 ubytes(uint32_t w) {
  w ^= 0x80808080u;
  return f32x4{(float)(w & 0xffu), (float)((w >> 8) & 0xffu), (float)((w >> 16) & 0xffu),
               (float)(w >> 24)};
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Stage layout (bytes): K codes [16][DK] (16-byte chunks swizzled by row),
// V codes [16][DV], then two 256-byte blocks of scales (lanes 0-15 of each
// scale DMA hold rows 0-15; the other lanes read zeros). Once Q.K^T has read
// the K codes and the V codes are in registers, the tile's V as bf16 (+128),
// [16][DV] rows of 2 DV bytes, is written over the stage's codes.
template <int DK, int DV, int STAGES_>
struct I8Cfg {
  static constexpr int STAGES = STAGES_, AHEAD = STAGES - 1;
  static constexpr int KC = DK / 16, VC = DV / 16;  // 16-byte chunks per row
  static constexpr int KT = 16 * DK, VT = 16 * DV, SC = 512;
  static constexpr int ST = KT + VT + SC;
  static constexpr int K_DMA = KT / 1024, V_DMA = VT / 1024;
  static constexpr int N_DMA = K_DMA + V_DMA + 2;
  static constexpr int VB = 16 * DV * 2;  // the tile's V as bf16 (+128)
  static constexpr int RING = STAGES * ST, RED = 16 * (DV + 2) * 4;
  static constexpr int LDS = RING > RED ? RING : RED;
  static_assert(KC >= 16 && VC >= 16, "row swizzle uses 16 chunk groups");
  static_assert(KT % 1024 == 0 && VT % 1024 == 0, "whole DMA blocks");
  static_assert(VB <= KT + VT, "the bf16 V tile fits over the codes");
  static_assert(DK / 2 * 8 <= ST, "the query's cos/sin rows fit a stage");
  static_assert((AHEAD - 1) * N_DMA < 64 && LDS <= 160 * 1024, "vmcnt / LDS limits");
};

template <class C, int DK, int DV>
__global__ __launch_bounds__(64, 2) void decode_i8_kernel(DecodeArgs a, int ch, int n_split) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS];
  // The query's (cos, sin) rows live in stage AHEAD, which the prologue's
  // DMAs leave free and the loop first refills after the query is turned.
  float2* cs_tab = reinterpret_cast<float2*>(lds + C::AHEAD * C::ST);

  const int kvh = blockIdx.x, split = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int col = lane & 15, g = lane >> 4;
  const int G = a.Hq / a.Hkv;

  const int kv_len = a.kv_len[b];
  if (kv_len <= 0 || kv_len > a.max_kv_len) {
    if (n_split == 1) {
      uint16_t* o = (uint16_t*)a.o + ((int64_t)b * a.Hq + kvh * G) * DV;
      for (int idx = lane; idx < G * DV; idx += 64) o[idx] = kv_len == 0 ? 0 : 0x7fc0;
    }
    return;
  }
  const int lo = (a.window > 0) ? max(0, kv_len - a.window) : 0;
  const int c0 = lo + split * ch;
  if (c0 >= kv_len) return;
  const int c1 = min(kv_len, c0 + ch);
  const int n_tiles = (c1 - c0 + 15) / 16;
  const int64_t row0 = a.row_offset[b] + c0;

  // Descriptors over the chunk's rows of KV head kvh (codes and scales);
  // rows at or past c1 read zeros.
  const int krow = a.Hkv * DK, vrow = a.Hkv * DV, srow = a.Hkv * 4;
  const int nr = c1 - c0;
  const u32x4 kdesc = buffer_desc((const char*)a.k_cache + (row0 * a.Hkv + kvh) * DK,
                                  (uint32_t)((nr - 1) * krow + DK));
  const u32x4 vdesc = buffer_desc((const char*)a.v_cache + (row0 * a.Hkv + kvh) * DV,
                                  (uint32_t)((nr - 1) * vrow + DV));
  const u32x4 ksdesc = buffer_desc((const char*)a.k_scale + (row0 * a.Hkv + kvh) * 4,
                                   (uint32_t)((nr - 1) * srow + 4));
  const u32x4 vsdesc = buffer_desc((const char*)a.v_scale + (row0 * a.Hkv + kvh) * 4,
                                   (uint32_t)((nr - 1) * srow + 4));
  uint32_t koff[C::K_DMA], voff[C::V_DMA];
#pragma unroll
  for (int i = 0; i < C::K_DMA; ++i) {
    const int q = i * 64 + lane, r = q / C::KC;
    koff[i] = r * krow + ((q % C::KC) ^ (r & 15)) * 16;
  }
#pragma unroll
  for (int i = 0; i < C::V_DMA; ++i) {
    const int q = i * 64 + lane, r = q / C::VC;
    voff[i] = r * vrow + ((q % C::VC) ^ (r & 15)) * 16;
  }
  const uint32_t soff = lane < 16 ? lane * srow : 0x80000000u;
  auto dma_tile = [&](int t, int stage) {
    const uint32_t st = lds_addr(lds) + stage * C::ST;
    const uint32_t far = t < n_tiles ? 0u : 0x80000000u;
    const uint32_t j0 = t * 16;
#pragma unroll
    for (int i = 0; i < C::K_DMA; ++i) dma16<true>(kdesc, st + i * 1024, (koff[i] + j0 * krow) | far);
#pragma unroll
    for (int i = 0; i < C::V_DMA; ++i)
      dma16<true>(vdesc, st + C::KT + i * 1024, (voff[i] + j0 * vrow) | far);
    dma4(ksdesc, st + C::KT + C::VT, (soff + j0 * srow) | far);
    dma4(vsdesc, st + C::KT + C::VT + 256, (soff + j0 * srow) | far);
  };
#pragma unroll
  for (int i = 0; i < C::AHEAD; ++i) dma_tile(i, i);

  // ---- rotated queries as two int8 B operands -----------------------------
  // Q.K^T runs on v_mfma_i32_16x16x64_i8 straight from the K codes. The bf16
  // query of head `col` (lane holds dims 64s + 16g .. +15) is split as
  // q = s1 q1 + s2 q2 + e: q1 = rint(q / s1) with s1 = max|q| / 127, q2 the
  // same for the residual, so |e| <= max|q| / (4 * 127^2) -- far below the
  // bf16 rounding the query already carries. Both int32 dot products are
  // exact; the score is ks * (s1 S1 + s2 S2).
  i32x4 q1[DK / 64], q2[DK / 64];
  float qs1, qs2;
  {
    const int qpos = kv_len - 1;
    const double l2t = log2(a.theta);
    for (int p = lane; p < a.rot_pairs; p += 64) {
      float c, sn;
      rope_cos_sin(qpos, rope_freq(p, DK, l2t), &c, &sn);
      cs_tab[p] = make_float2(c, sn);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const bool hv = col < G;
    const uint16_t* qrow =
        (const uint16_t*)a.q + ((int64_t)b * a.Hq + kvh * G + (hv ? col : 0)) * DK;
    // This lane's 16 dims per 64-dim step, turned and kept as packed bf16
    // (the query's own precision); the split below reads them three times
    // rather than holding them as fp32.
    uint32_t qw[DK / 8];
    float amax = 0.f;
#pragma unroll
    for (int s = 0; s < DK / 64; ++s) {
      const int d0 = 64 * s + 16 * g;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 w = *(const u32x4*)(qrow + d0 + 8 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int pr = d0 / 2 + 4 * h + e;
          if (pr < a.rot_pairs) {
            const float2 t = cs_tab[pr];
            const float x0 = bf16_lo(w[e]), x1 = bf16_hi(w[e]);
            w[e] = pack_bf16x2(x0 * t.x - x1 * t.y, x0 * t.y + x1 * t.x);
          }
          qw[8 * s + 4 * h + e] = hv ? w[e] : 0u;
          amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(qw[8 * s + 4 * h + e])),
                                   fabsf(bf16_hi(qw[8 * s + 4 * h + e]))));
        }
      }
    }
    amax = xor32_16_max(amax);
    qs1 = amax / 127.f;
    const float r1 = amax > 0.f ? 127.f / amax : 0.f;
    // element i (i < DK/4) of this lane: dim pair i/2 of the packed words
    auto elem = [&](int i) {
      const uint32_t w = qw[i / 2];
      return (i & 1) ? bf16_hi(w) : bf16_lo(w);
    };
    auto residual = [&](int i, float* c) {
      const float x = elem(i);
      *c = rintf(x * r1);
      return x - qs1 * *c;
    };
    float rmax = 0.f;
#pragma unroll
    for (int i = 0; i < DK / 4; ++i) {
      float c;
      const float r = residual(i, &c);
      rmax = fmaxf(rmax, fabsf(r));
      const int s = i / 16, e = i % 16;
      const uint32_t byte = (uint32_t)(int)c & 0xffu;
      if (e % 4 == 0) q1[s][e / 4] = (int)byte;
      else q1[s][e / 4] |= (int)(byte << (8 * (e % 4)));
    }
    rmax = xor32_16_max(rmax);
    qs2 = rmax / 127.f;
    const float r2 = rmax > 0.f ? 127.f / rmax : 0.f;
#pragma unroll
    for (int i = 0; i < DK / 4; ++i) {
      float c;
      const float r = residual(i, &c);
      const int s = i / 16, e = i % 16;
      const uint32_t byte = (uint32_t)(int)rintf(r * r2) & 0xffu;
      if (e % 4 == 0) q2[s][e / 4] = (int)byte;
      else q2[s][e / 4] |= (int)(byte << (8 * (e % 4)));
    }
  }
  wait_vm<(C::AHEAD - 1) * C::N_DMA>();
  lds_barrier();

  const float c2 = fmaxf(a.scale * kLog2e, 1e-30f);
  float m_run = -INFINITY, l_run = 0.f, sp_run = 0.f;  // per head `col`
  f32x4 oacc[DV / 16];
#pragma unroll
  for (int d = 0; d < DV / 16; ++d) oacc[d] = f32x4{};

  // K codes: row col, dims 64s + 16g .. +15 = chunk 4s + g.
  const int krd = col * DK;
  // V^T from the bf16 tile (layout of the bf16 kernel's V rows, one wave).
  int vo[8];
  {
    const int x = 4 * g + (col >> 2), c4 = col & 3;
    const int vrow_l = x * (DV / 8) * 16 + ((((c4 >> 1) ^ (x & 1))) << 4) + ((c4 & 1) << 3);
#pragma unroll
    for (int B = 0; B < 8; ++B) vo[B] = vrow_l + ((B ^ (x >> 1)) << 5);
  }

  int cur = 0;
  for (int t = 0; t < n_tiles; ++t) {
    dma_tile(t + C::AHEAD, cur == 0 ? C::AHEAD : cur - 1);
    const lds_u8* st = (const lds_u8*)lds + __builtin_amdgcn_readfirstlane(cur * C::ST);
    // S^T[16 keys][16 heads] = ks * (s1 K.q1 + s2 K.q2), int32 dot products.
    i32x4 S1 = i32x4{}, S2 = i32x4{};
#pragma unroll
    for (int k = 0; k < DK / 64; ++k) {
      const i32x4 kc = *(const __attribute__((address_space(3))) i32x4*)(
          st + krd + (((4 * k + g) ^ col) << 4));
      S1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(kc, q1[k], S1, 0, 0, 0);
      S2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(kc, q2[k], S2, 0, 0, 0);
    }
    // V codes of this tile -> bf16 (+128) rows written over the stage's codes
    // from its base: 4 chunks of 16 codes per lane, each into two 8-element
    // bf16 chunks (same row swizzle). Every code and K operand is read before
    // the first write (one wave: its LDS operations complete in order).
    u32x4 vw[16 * C::VC / 64];
#pragma unroll
    for (int i = 0; i < 16 * C::VC / 64; ++i) {
      const int q = i * 64 + lane, r = q / C::VC, c = q % C::VC;
      vw[i] = *(const __attribute__((address_space(3))) u32x4*)(st + C::KT + r * DV +
                                                                ((c ^ (r & 15)) << 4));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    unsigned char* vb = (unsigned char*)lds + __builtin_amdgcn_readfirstlane(cur * C::ST);
#pragma unroll
    for (int i = 0; i < 16 * C::VC / 64; ++i) {
      const int q = i * 64 + lane, r = q / C::VC, c = q % C::VC;
      const u32x4 w = vw[i];
      const f32x4 f0 = ubytes(w[0]), f1 = ubytes(w[1]), f2 = ubytes(w[2]), f3 = ubytes(w[3]);
      const u32x4 lo4 = {pack_bf16x2(f0[0], f0[1]), pack_bf16x2(f0[2], f0[3]),
                         pack_bf16x2(f1[0], f1[1]), pack_bf16x2(f1[2], f1[3])};
      const u32x4 hi4 = {pack_bf16x2(f2[0], f2[1]), pack_bf16x2(f2[2], f2[3]),
                         pack_bf16x2(f3[0], f3[1]), pack_bf16x2(f3[2], f3[3])};
      unsigned char* rowp = vb + r * DV * 2;
      *(u32x4*)(rowp + (((2 * c) ^ (r & 15)) << 4)) = lo4;
      *(u32x4*)(rowp + (((2 * c + 1) ^ (r & 15)) << 4)) = hi4;
    }
    const f32x4 ks = *(const __attribute__((address_space(3))) f32x4*)(st + C::KT + C::VT + 16 * g);
    const f32x4 vs = *(const __attribute__((address_space(3))) f32x4*)(st + C::KT + C::VT + 256 + 16 * g);
    f32x4 s;
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = (qs1 * (float)S1[i] + qs2 * (float)S2[i]) * ks[i];
    const int key0 = c0 + t * 16 + 4 * g;
    if (c0 + (t + 1) * 16 > c1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = (key0 + i < c1) ? s[i] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = xor32_16_max(mx);
    const float mc = (mx == -INFINITY) ? -INFINITY : mx * c2;
    if (__any(mc > m_run + 8.f)) {
      const float m_new = fmaxf(m_run, mc);
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      sp_run *= alpha;
#pragma unroll
      for (int d = 0; d < DV / 16; ++d) oacc[d] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    f32x4 p, pv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -m_use));
      pv[i] = p[i] * vs[i];
    }
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    const bf16x4 pvb = __builtin_convertvector(pv, bf16x4);
    const f32x4 pvr = __builtin_convertvector(pvb, f32x4);
    sp_run += (pvr[0] + pvr[1]) + (pvr[2] + pvr[3]);  // the P' the MFMA sees
    const s16x4 pb = __builtin_bit_cast(s16x4, pvb);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int d = 0; d < DV / 16; ++d) {
      const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4*)(st + vo[d % 8] + (d / 8) * 256));
      oacc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, v), pb,
                                                          oacc[d], 0, 0, 0);
    }
    wait_vm<(C::AHEAD - 1) * C::N_DMA>();  // tile t+1 landed
    lds_barrier();                         // (one wave: also orders vb reuse)
    cur = cur == C::AHEAD ? 0 : cur + 1;
  }
  wait_vm<0>();
  lds_barrier();

  l_run = xor32_16_sum(l_run);
  sp_run = xor32_16_sum(sp_run);
  const float vbias = 128.f * sp_run;

  float* red = reinterpret_cast<float*>(lds);  // [16][DV + 2]
  const int RS = DV + 2;
  {
    float* wr = red + col * RS;
    if (g == 0) {
      wr[DV] = m_run;
      wr[DV + 1] = l_run;
    }
#pragma unroll
    for (int d = 0; d < DV / 16; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) wr[16 * d + 4 * g + i] = oacc[d][i] - vbias;
  }
  __syncthreads();
  if (n_split == 1) {
    uint16_t* o = (uint16_t*)a.o + ((int64_t)b * a.Hq + kvh * G) * DV;
    for (int idx = lane; idx < G * DV; idx += 64) {
      const int h = idx / DV, d = idx % DV;
      o[idx] = f32_to_bf16(red[h * RS + d] / red[h * RS + DV + 1]);
    }
    return;
  }
  float* part = reinterpret_cast<float*>(a.workspace);
  for (int idx = lane; idx < G * (DV + 2); idx += 64) {
    const int h = idx / (DV + 2), d = idx % (DV + 2);
    const int64_t slot = ((int64_t)b * a.Hq + kvh * G + h) * n_split + split;
    const float m = red[h * RS + DV];
    part[slot * (DV + 2) + d] = (d == DV || m != -INFINITY) ? red[h * RS + d] : 0.f;
  }
}

template <int DK, int DV>
hipError_t launch_i8(const DecodeArgs& a, hipStream_t st) {
  using C = I8Cfg<DK, DV, 2>;
  const SplitPlan pl = decode_plan(a.B, a.Hkv, a.max_kv_len, a.window, 1);
  if (pl.ns > 65535) return hipErrorInvalidValue;
  const int64_t row = (int64_t)a.Hkv * DK;
  if (((int64_t)pl.ch + 64) * row >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_i8_kernel<C, DK, DV>), dim3(a.Hkv, pl.ns, a.B), dim3(64), 0, st,
                     a, pl.ch, pl.ns);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.ns == 1) return e;
  return launch_decode_merge(a, pl, st);
}

}  // namespace

hipError_t launch_kv_quantize_int8(const void* x, int8_t* codes, float* scales, int N, int H,
                                   int D, hipStream_t st) {
  const int64_t rows = (int64_t)N * H;
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  switch (D) {
    case 128:
      hipLaunchKernelGGL(kv_quantize_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, st, xs,
                         codes, scales, rows);
      break;
    case 256:
      hipLaunchKernelGGL(kv_quantize_kernel<256>, dim3((unsigned)blocks), dim3(256), 0, st, xs,
                         codes, scales, rows);
      break;
    case 512:
      hipLaunchKernelGGL(kv_quantize_kernel<512>, dim3((unsigned)blocks), dim3(256), 0, st, xs,
                         codes, scales, rows);
      break;
    default:
      return hipErrorNotSupported;
  }
  return hipGetLastError();
}

hipError_t launch_decode_int8(const DecodeArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  if (a.Dk == 512 && a.Dv == 256) return launch_i8<512, 256>(a, st);
  if (a.Dk == 256 && a.Dv == 256) return launch_i8<256, 256>(a, st);
  return hipErrorNotSupported;
}

}  // namespace attn
