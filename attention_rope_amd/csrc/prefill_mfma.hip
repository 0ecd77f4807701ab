// prefill_mfma.hip — flash-style causal / sliding-window GQA prefill on gfx950
// bf16 matrix cores (v_mfma_f32_16x16x32_bf16), with RoPE fused into the Q and
// K loads.
//
// What it computes (Gemma 4 pages): "Gemma 4: End-to-End Architecture
// Walkthrough", Phase 3 — section 3a (local layers: query i sees the window of
// keys i-W+1..i; global layers: keys 0..i), section 3b (grouped-query
// attention, 2 or 8 query heads per KV head, widened global keys) and section
// 3c (p-RoPE: only the leading quarter of the rotary pairs turn); "Gemma 4
// Architecture Reference", "Positional Encoding: Proportional RoPE (p-RoPE)".
// The result equals softmax(scale * rope(q) rope(k)^T + mask) v exactly in
// exact arithmetic; here q/k are rounded to bf16 after rotation, P to bf16
// before the P.V product, and everything accumulates in fp32.
//
// Design for CDNA4:
//  * A workgroup of 8 waves (2 per SIMD) owns one (batch, KV head) and PW
//    consecutive query positions for all G query heads sharing that KV head:
//    128 (head, position) rows, so each K/V tile staged in LDS serves G heads.
//    Two waves per SIMD let one wave's softmax overlap the other's MFMAs.
//  * Each wave owns 16 rows and computes S^T = K Q^T with 16x16x32 MFMAs
//    (M = 16 keys, N = 16 rows): every lane holds 8 scores of one query row,
//    so the softmax max/sum need two cross-lane swaps. Q^T (DK/32 x 16 bytes
//    per lane) and the O^T accumulator (DV/4 fp32 per lane) stay in registers;
//    at 16 rows a wave fits in half the register file.
//  * O^T = V^T P^T (K = 32 keys per MFMA): the P^T operand is the lane's own
//    scores when the key order inside the MFMA matches the score layout; V
//    tiles are written to LDS transposed, in exactly that key order.
//  * K tiles (32 keys) move HBM -> LDS by direct DMA (buffer loads with the
//    lds flag): no staging registers, out-of-range rows read as zero. The
//    rotated chunks of each K row sit in their own LDS region, so every thread
//    turns exactly the chunks its own DMA wrote (one barrier per tile, all
//    lanes busy), with cos/sin from the per-position table prefetched one tile
//    ahead. Tiles are double-buffered; the next tile's loads overlap the
//    current tile's matrix work.
//  * K rows are XOR-swizzled in 16-byte chunks so the MFMA operand reads are
//    bank-conflict free without the padding the 1 KB DMA blocks cannot have.
//  * Only key tiles intersecting the causal band / sliding window are visited
//    (window-aware skipping); masking runs only on tiles that cross the
//    diagonal or the window edge.
//  * The running max is updated lazily: O is rescaled only when a row's block
//    max exceeds the max in use by more than 2^8 (probabilities stay <= 256,
//    exact after the final division).
//  * Causal tiles are issued longest-first; sliding-window launches map
//    neighbouring query tiles onto the same XCD so their K/V windows share L2.
#include "attn_common.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;  // log2 headroom before the running max moves
constexpr int NW = 8;          // waves per workgroup
constexpr int NT = NW * 64;
constexpr int RW = 16;         // query rows per wave
constexpr int BN = 32;         // keys per tile
// Buffer descriptor word 3 for raw (stride 0) 32-bit-format buffers on gfx9.
constexpr int kBufFlags = 0x00020000;

typedef __attribute__((address_space(3))) void lds_void;

template <int DK, int DV, int G, int RCH>
struct Cfg {
  static constexpr int ROWS = NW * RW;        // (head, position) rows per WG
  static constexpr int PW = ROWS / G;         // query positions per WG
  static constexpr int NC = DK / 8;           // 16-byte chunks per K row
  static constexpr int NP = NC - RCH;         // plain (unrotated) chunks per K row
  // K tile: rotated region [32][RCH] chunks, then plain region [32][NP].
  static constexpr int KR_BYTES = BN * RCH * 16;
  static constexpr int KT_BYTES = BN * NC * 16;
  static constexpr int KR_DMA = KR_BYTES / 1024;   // 1 KB DMA blocks per region
  static constexpr int KP_DMA = (KT_BYTES - KR_BYTES) / 1024;
  // V^T tile: [DV][VS] bf16, keys in the permuted order of the score layout.
  static constexpr int VS = BN + 8;           // padded row (80 bytes)
  static constexpr int VT_BYTES = DV * VS * 2;
  static constexpr int KSTAGES = 3;           // K tiles in flight: t, t+1, t+2
  static constexpr int LDS_BYTES = KSTAGES * KT_BYTES + 2 * VT_BYTES;
  static constexpr int VU = (BN / 2) * (DV / 8);   // V units: 2 keys x 8 dims
  static constexpr int VUT = (VU + NT - 1) / NT;
  static constexpr int KROT = (KR_DMA + NW - 1) / NW;  // rotated blocks per wave
  static constexpr int KDMA_W = KROT + (KP_DMA + NW - 1) / NW;  // K DMA issues per wave (max)
  // Every wave issues the same number of K DMAs per tile, so "everything but
  // the newest K tile has landed" is one vmcnt value.
  static constexpr bool UNIFORM = KR_DMA % NW == 0 && KP_DMA % NW == 0;
  static_assert(ROWS % G == 0 && PW % RW == 0, "rows must split evenly over the heads");
  static_assert(KR_BYTES % 1024 == 0 && KT_BYTES % 1024 == 0, "DMA blocks");
  static_assert(DK % 32 == 0 && DV % 16 == 0, "MFMA tiling");
};

// XOR swizzle of 16-byte chunks inside a K region row of `width` chunks. The
// mask P-1 uses the largest power of two P <= 16 dividing the width, so the
// swizzled index stays inside the row; with P = 16, 16 consecutive rows
// reading the same chunk hit 16 distinct bank groups.
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

// Per-lane addressing of the K operand reads (row r, chunk 4s + g for
// s = 0, 1, ...) inside a region of `width` chunks starting at byte `base`:
// chunk (4s + g) ^ x = 4((s ^ x2)) + ((g ^ x) & 3) with x2 = x >> 2, so the
// offset is row_base + (((s & H) << 6) ^ x2s) + ((s & ~H) << 6).
template <int width>
struct KAddr {
  int row_base, x2s;
  __device__ __forceinline__ KAddr(int base, int r, int g) {
    const int x = r & Swz<width>::M;
    row_base = base + r * width * 16 + (((g ^ x) & 3) << 4);
    x2s = (x >> 2) << 6;
  }
  __device__ __forceinline__ int operator()(int s) const {
    constexpr int H = (Swz<width>::P >= 4 ? Swz<width>::P / 4 : 1) - 1;
    return row_base + (((s & H) << 6) ^ x2s) + ((s & ~H) << 6);
  }
};

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

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// LDS stores issued as plain instructions. The compiler treats every LDS
// access that may alias an in-flight LDS DMA as needing that DMA to finish
// first, which would drain the tile loaded two steps ahead. These stores never
// touch a DMA target, so they are issued directly with no memory clobber: they
// keep their order with the other volatile asm (the barrier below) and their
// register dependences, and lds_barrier waits for them before publishing.
__device__ __forceinline__ void lds_store_b128(uint32_t addr, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v));
}
__device__ __forceinline__ void lds_store_b32(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v));
}
// Publish this wave's LDS stores to the workgroup and synchronise, without the
// workgroup-scope fence of __syncthreads (which would also wait for the
// in-flight DMA); the memory clobber keeps compiler-visible LDS accesses on
// their side of the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int DK, int DV, int G, int RCH>
__global__ __launch_bounds__(NT, 1) void prefill_mfma_kernel(PrefillArgs a, int n_qt,
                                                             int contig) {
  using C = Cfg<DK, DV, G, RCH>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS_BYTES];
  unsigned char* const vt_base = lds + C::KSTAGES * C::KT_BYTES;  // 2 V^T buffers

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int T = a.T, W = a.window;
  const int n_wg = n_qt * a.Hkv * a.B;
  const int L = contig ? xcd_contiguous((int)blockIdx.x, n_wg) : (int)blockIdx.x;
  const int grp = L / n_qt;
  const int qt = n_qt - 1 - (L % n_qt);  // longest causal tiles first
  const int kvh = grp % a.Hkv, b = grp / a.Hkv;
  const int p0 = qt * C::PW;

  // This lane's query row; the wave's 16 rows are 16 positions of one head.
  const int R = wave * RW + r16;
  const int head = kvh * G + R / C::PW;
  const int pos = p0 + R % C::PW;
  const bool valid = pos < T;
  const int wlo = p0 + (wave * RW) % C::PW;
  const int whi = wlo + RW - 1;

  const int kv_lo = (W > 0) ? max(0, p0 - W + 1) : 0;
  const int kv_hi = min(T, p0 + C::PW);
  const int kb_lo = kv_lo / BN;
  const int kb_hi = (kv_hi + BN - 1) / BN;

  // Buffer descriptors: K and V of this (batch, KV head); rows past T read 0.
  const int krow = a.Hkv * DK * 2, vrow = a.Hkv * DV * 2;  // bytes per token
  const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)a.k + ((int64_t)b * T * a.Hkv + kvh) * DK * 2), (short)0,
      (T - 1) * krow + DK * 2, kBufFlags);
  const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)a.v + ((int64_t)b * T * a.Hkv + kvh) * DV * 2), (short)0,
      (T - 1) * vrow + DV * 2, kBufFlags);
  const bool rot_k = RCH > 0 && a.rope_k;
  const bool rot_q = RCH > 0 && a.rope_q;
  const int tab_row = a.rot_pairs * 8;  // bytes per table row
  const __amdgpu_buffer_rsrc_t tres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.rope_tab, (short)0, (RCH > 0 && (rot_k || rot_q)) ? T * tab_row : 0, kBufFlags);

  // ---- K: DMA into LDS; this thread turns the rotated chunks it loaded -----
  f32x4 ktab[C::KROT > 0 ? C::KROT : 1][2];
  auto rot_chunk = [&](int i, int& r, int& c) {
    const int q = (i * NW + wave) * 64 + lane;
    r = q / (RCH > 0 ? RCH : 1);
    c = kswz<RCH>(r, q % (RCH > 0 ? RCH : 1));  // swizzle is an involution
  };
  auto load_ktab = [&](int kb) {
    const int j0 = kb * BN;
#pragma unroll
    for (int i = 0; i < C::KROT; ++i) {
      if (C::KR_DMA % NW == 0 || i * NW + wave < C::KR_DMA) {
        int r, c;
        rot_chunk(i, r, c);
        const int off = min(j0 + r, T - 1) * tab_row + c * 32;
        ktab[i][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(tres, off, 0, 0));
        ktab[i][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(tres, off + 16, 0, 0));
      }
    }
  };
  auto dma_k = [&](int kb, unsigned char* st) {
    const int j0 = kb * BN;
#pragma unroll
    for (int i = 0; i < C::KROT; ++i) {
      if (C::KR_DMA % NW == 0 || i * NW + wave < C::KR_DMA) {
        int r, c;
        rot_chunk(i, r, c);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kres, (lds_void*)(st + (i * NW + wave) * 1024),
                                                 16, (j0 + r) * krow + c * 16, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < (C::KP_DMA + NW - 1) / NW; ++i) {
      const int n = i * NW + wave;
      if (C::KP_DMA % NW == 0 || n < C::KP_DMA) {
        const int q = n * 64 + lane;
        constexpr int NPd = C::NP > 0 ? C::NP : 1;  // loop is empty when NP == 0
        const int r = q / NPd;
        const int c = RCH + kswz<NPd>(r, q % NPd);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            kres, (lds_void*)(st + C::KR_BYTES + n * 1024), 16, (j0 + r) * krow + c * 16, 0, 0,
            0);
      }
    }
  };
  auto rotate_k = [&](unsigned char* st) {
#pragma unroll
    for (int i = 0; i < C::KROT; ++i) {
      if (C::KR_DMA % NW == 0 || i * NW + wave < C::KR_DMA) {
        const unsigned char* p = st + ((i * NW + wave) * 64 + lane) * 16;
        lds_store_b128(lds_addr(p), rotate4(*(const u32x4*)p, ktab[i][0], ktab[i][1]));
      }
    }
  };

  // ---- V: registers, then LDS transposed in the score-matched key order ----
  // Slot 8g + i of a V^T row holds key 16(i/4) + 4g + (i%4): key 16a + 4g + r
  // sits in slot 8g + 4a + r, so an even/odd key pair fills 2 adjacent slots.
  // Unit u = key pair kp (keys 2kp, 2kp+1) x 8 dims d8; a step loads the next
  // tile's units and writes them transposed at its end.
  u32x4 vreg[C::VUT][2];
  auto load_v = [&](int kb, u32x4 (&vr)[C::VUT][2]) {
    const int j0 = kb * BN;
#pragma unroll
    for (int ut = 0; ut < C::VUT; ++ut) {
      const int u = tid + NT * ut;
      const int kp = u % 16, d8 = u / 16;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        vr[ut][e] = (C::VU % NT == 0 || u < C::VU)
                        ? __builtin_amdgcn_raw_buffer_load_b128(vres, (j0 + 2 * kp + e) * vrow + d8 * 16, 0, 0)
                        : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_v = [&](const u32x4 (&vr)[C::VUT][2], unsigned char* vt) {
    uint16_t* Vt = (uint16_t*)vt;
#pragma unroll
    for (int ut = 0; ut < C::VUT; ++ut) {
      const int u = tid + NT * ut;
      if (C::VU % NT == 0 || u < C::VU) {
        const int kp = u % 16, d8 = u / 16;
        const int k = 2 * kp;  // = 16a + 4g' + r with r even
        const int slot = 8 * ((k % 16) / 4) + 4 * (k / 16) + (k % 4);
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          const int wi = dd / 2;
          const uint32_t w = (dd % 2 == 0) ? ((vr[ut][0][wi] & 0xffffu) | (vr[ut][1][wi] << 16))
                                           : ((vr[ut][0][wi] >> 16) | (vr[ut][1][wi] & 0xffff0000u));
          lds_store_b32(lds_addr(Vt + (8 * d8 + dd) * C::VS + slot), w);
        }
      }
    }
  };

  // Wait until every load issued before the newest K tile's DMAs has
  // completed (loads complete in issue order and those DMAs are always the
  // last loads issued), then keep the scheduler from hoisting LDS reads of the
  // landed tile above the wait.
  auto wait_all_but_newest_k = [&]() {
    if constexpr (C::UNIFORM) {
      constexpr int n = C::KDMA_W;  // K DMAs per wave per tile
      static_assert(n < 16, "vmcnt field");
      // s_waitcnt: vmcnt[3:0] = n, expcnt = 7 (no wait), lgkmcnt = 15 (no wait)
      __builtin_amdgcn_s_waitcnt(0x0F70 | n);
    } else {
      __builtin_amdgcn_s_waitcnt(0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto wait_all = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: tile 0 (K, V, table), the Q rows, then tile 1's K DMA ----
  const int n_tiles = kb_hi - kb_lo;
  if (n_tiles > 0) {
    dma_k(kb_lo, lds);
    if (rot_k) load_ktab(kb_lo);
    load_v(kb_lo, vreg);
  }
  // Q^T operand: step s covers dims 32s + 8g .. 32s + 8g + 7 of this row.
  bf16x8 qf[DK / 32];
  {
    const int prow = valid ? pos : T - 1;
    const uint16_t* qrow =
        (const uint16_t*)a.q + (((int64_t)b * T + prow) * a.Hq + head) * DK + 8 * g;
    u32x4 qw[DK / 32];
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) qw[s] = *(const u32x4*)(qrow + 32 * s);
    if (rot_q) {
      // rotated chunks: 32s + 8g < 8*RCH  <=>  s < RCH/4 for every g
#pragma unroll
      for (int s0 = 0; s0 < RCH / 4; s0 += 4) {
        f32x4 t[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int off = prow * tab_row + (32 * (s0 + u) + 8 * g) * 4;
          t[u][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(tres, off, 0, 0));
          t[u][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(tres, off + 16, 0, 0));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (s0 + u < RCH / 4) qw[s0 + u] = rotate4(qw[s0 + u], t[u][0], t[u][1]);
      }
    }
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
      u32x4 w = valid ? qw[s] : u32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }
  if (n_tiles > 0) {
    dma_k(kb_lo + 1, lds + C::KT_BYTES);  // may lie past the range: never read
    wait_all_but_newest_k();  // tile 0 landed; tile 1's K may still be in flight
    if (rot_k) rotate_k(lds);
    store_v(vreg, vt_base);
    lds_barrier();
  }


  // ---- online softmax state (one row per lane; 4 lanes share a row) --------
  // scores to log2 units; kept > 0 so a masked -inf score never meets a zero
  // factor (scale 0 then acts as 1e-30: every visible key weighs the same)
  const float c2 = fmaxf(a.scale * kLog2e, 1e-30f);
  const unsigned wcap = (W > 0) ? (unsigned)W : 0x80000000u;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[DV / 16];
#pragma unroll
  for (int d = 0; d < DV / 16; ++d) oacc[d] = f32x4{};

  // K operand: key 16mb + r16, chunk 4s + g.
  const KAddr<(RCH > 0 ? RCH : 16)> kaddr_r0(0, r16, g), kaddr_r1(0, r16 + 16, g);
  const KAddr<(C::NP > 0 ? C::NP : 16)> kaddr_p0(C::KR_BYTES, r16, g),
      kaddr_p1(C::KR_BYTES, r16 + 16, g);
  const int vt_off = (r16 * C::VS + 8 * g) * 2;  // + 16*db*VS*2

  auto compute = [&](const unsigned char* st, const unsigned char* vt, int kb) {
    const int j0 = kb * BN;
    if (j0 > whi) return;                            // beyond every row (causal)
    if (W > 0 && j0 + BN - 1 <= wlo - W) return;     // before every row's window
    f32x4 s0 = f32x4{}, s1 = f32x4{};
    // dims 32s + 8g..: s < RCH/4 in the rotated region, the rest in the plain one
#pragma unroll
    for (int s = 0; s < RCH / 4; ++s) {
      const bf16x8 k0 = *(const bf16x8*)(st + kaddr_r0(s));
      const bf16x8 k1 = *(const bf16x8*)(st + kaddr_r1(s));
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[s], s1, 0, 0, 0);
    }
#pragma unroll
    for (int s = RCH / 4; s < DK / 32; ++s) {
      const bf16x8 k0 = *(const bf16x8*)(st + kaddr_p0(s - RCH / 4));
      const bf16x8 k1 = *(const bf16x8*)(st + kaddr_p1(s - RCH / 4));
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[s], s1, 0, 0, 0);
    }
    // lane holds keys j0 + 4g + i (s0) and j0 + 16 + 4g + i (s1) of its row
    float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    const bool need_mask = (j0 + BN - 1 > wlo) || (W > 0 && j0 <= whi - W);
    if (need_mask) {
      const int d0 = pos - j0 - 4 * g;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const unsigned d = (unsigned)(d0 - (16 * (i / 4) + (i % 4)));  // pos - key
        sv[i] = (d < wcap) ? sv[i] : -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    mx = xor32_16_max(mx);
    const float mc = (mx == -INFINITY) ? -INFINITY : mx * c2;
    if (__any(mc > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mc);
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < DV / 16; ++d) oacc[d] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float pv[8];  // masked scores are -inf and c2 > 0, so they give exactly 0
#pragma unroll
    for (int i = 0; i < 8; ++i) pv[i] = fast_exp2(fmaf(sv[i], c2, -m_use));
    l_run += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
    const f32x4 plo = {pv[0], pv[1], pv[2], pv[3]}, phi = {pv[4], pv[5], pv[6], pv[7]};
    const bf16x4 pa = __builtin_convertvector(plo, bf16x4);
    const bf16x4 pb = __builtin_convertvector(phi, bf16x4);
    const bf16x8 pop = __builtin_shufflevector(pa, pb, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int d = 0; d < DV / 16; ++d) {
      const bf16x8 va = *(const bf16x8*)(vt + vt_off + d * 16 * C::VS * 2);
      oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pop, oacc[d], 0, 0, 0);
    }
  };

  // ---- main loop: K tiles in 3 LDS stages, V^T in 2 buffers ---------------
  // Step t computes tile t while K(t+1) (issued a step ago) and K(t+2)
  // (issued now, last) load, with V(t+1) and the cos/sin of K(t+1); it then
  // turns K(t+1) and writes V^T(t+1). Every step issues the same loads, also
  // the last two (their tiles may lie past the range or past T, where the
  // buffer descriptors return zeros, and are never read), so one vmcnt value
  // separates the newest K tile from everything older on every path.
  for (int t = 0; t < n_tiles; ++t) {
    const int kb = kb_lo + t;
    unsigned char* ks = lds + (t % 3) * C::KT_BYTES;
    unsigned char* k1 = lds + ((t + 1) % 3) * C::KT_BYTES;
    unsigned char* k2 = lds + ((t + 2) % 3) * C::KT_BYTES;
    unsigned char* vt = vt_base + (t & 1) * C::VT_BYTES;
    unsigned char* vt1 = vt_base + ((t + 1) & 1) * C::VT_BYTES;
    if (rot_k) load_ktab(kb + 1);
    load_v(kb + 1, vreg);
    dma_k(kb + 2, k2);
    compute(ks, vt, kb);
    wait_all_but_newest_k();  // K(t+1), V(t+1) and its table landed
    if (t + 1 < n_tiles) {
      if (rot_k) rotate_k(k1);
      store_v(vreg, vt1);
    }
    lds_barrier();  // tile t+1 complete everywhere; tile t buffers free
  }
  wait_all();  // no DMA may still target LDS when the block ends

  // ---- epilogue: O = O^T / l, bf16, 4 consecutive dims per store ----------
  l_run = xor32_16_sum(l_run);
  if (valid) {
    const float inv = 1.f / l_run;
    uint16_t* orow = (uint16_t*)a.o + (((int64_t)b * T + pos) * a.Hq + head) * DV + 4 * g;
#pragma unroll
    for (int d = 0; d < DV / 16; ++d) {
      const uint32_t w0 = pack_bf16x2(oacc[d][0] * inv, oacc[d][1] * inv);
      const uint32_t w1 = pack_bf16x2(oacc[d][2] * inv, oacc[d][3] * inv);
      *(u32x2*)(orow + 16 * d) = u32x2{w0, w1};
    }
  }
}

template <int DK, int DV, int G, int RCH>
hipError_t launch_one(const PrefillArgs& a, hipStream_t st) {
  using C = Cfg<DK, DV, G, RCH>;
  const int n_qt = (a.T + C::PW - 1) / C::PW;
  const int64_t n = (int64_t)n_qt * a.Hkv * a.B;
  if (n == 0) return hipSuccess;
  if (n > 0x7fffffff) return hipErrorInvalidValue;
  // Sliding-window tiles reuse their neighbours' K/V: keep neighbours on one
  // XCD. Causal tiles share the prefix of every key stream: interleave.
  const int contig = (a.window > 0 && a.window < a.T) ? 1 : 0;
  hipLaunchKernelGGL((prefill_mfma_kernel<DK, DV, G, RCH>), dim3((unsigned)n), dim3(NT), 0,
                     st, a, n_qt, contig);
  return hipGetLastError();
}

template <int DK, int DV, int G>
hipError_t dispatch_rot(const PrefillArgs& a, hipStream_t st) {
  const int rch = (a.rope_q || a.rope_k) ? (2 * a.rot_pairs) / 8 : 0;
  if (rch == 0) return launch_one<DK, DV, G, 0>(a, st);
  if (rch == DK / 32) return launch_one<DK, DV, G, DK / 32>(a, st);
  if (rch == DK / 8) return launch_one<DK, DV, G, DK / 8>(a, st);
  return hipErrorNotSupported;
}

template <int DK, int DV>
hipError_t dispatch_g(const PrefillArgs& a, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return dispatch_rot<DK, DV, 1>(a, st);
    case 2: return dispatch_rot<DK, DV, 2>(a, st);
    case 4: return dispatch_rot<DK, DV, 4>(a, st);
    case 8: return dispatch_rot<DK, DV, 8>(a, st);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

bool prefill_mfma_supported(int Dk, int Dv, int G, float scale) {
  const bool shape = (Dk == 128 && Dv == 128) || (Dk == 256 && Dv == 256) ||
                     (Dk == 512 && Dv == 256);
  return shape && (G == 1 || G == 2 || G == 4 || G == 8) && scale >= 0.f;
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t st) {
  if ((a.rope_q || a.rope_k) && (2 * a.rot_pairs) % 8 != 0) return hipErrorNotSupported;
  // 32-bit buffer offsets: one batch's K or V, and the cos/sin table, < 2 GiB.
  const int64_t per_b = (int64_t)a.T * a.Hkv * (a.Dk > a.Dv ? a.Dk : a.Dv) * 2;
  if (per_b >= (int64_t)1 << 31 || (int64_t)a.T * a.rot_pairs * 8 >= (int64_t)1 << 31)
    return hipErrorNotSupported;
  if (a.Dk == 512 && a.Dv == 256) return dispatch_g<512, 256>(a, st);
  if (a.Dk == 256 && a.Dv == 256) return dispatch_g<256, 256>(a, st);
  if (a.Dk == 128 && a.Dv == 128) return dispatch_g<128, 128>(a, st);
  return hipErrorNotSupported;
}

}  // namespace attn
