// prefill_mfma16.hip — flash-style causal GQA prefill on gfx950 bf16 matrix
// cores (v_mfma_f32_16x16x32_bf16) with 16-row waves, with RoPE applied on the
// way in. It serves the 512-dim keys of the global layers, where a 32-row
// wave's Q^T and O^T would not fit two waves per SIMD; prefill_mfma.hip holds
// the 32-row kernel used for smaller heads.
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
//    per lane) and the O^T accumulator (DV/4 fp32 per lane) stay in registers.
//  * O^T = V^T P^T (K = 32 keys per MFMA): the P^T operand is the lane's own
//    scores when the key order inside the MFMA matches the score layout. V
//    tiles sit in LDS in their natural [key][dim] layout and the V^T operand
//    is read with the transposing LDS read (ds_read_b64_tr_b16), two reads
//    of 4 keys each per operand, in that key order.
//  * K and V tiles (32 keys) move HBM -> LDS by direct DMA (buffer loads with
//    the lds flag): no staging registers, no VALU work, rows past T read as
//    zero. The rotated leading dims of K come already turned from a rotation
//    pass that runs once per key (not once per query tile) into a workspace;
//    each K tile keeps them in a region of its own, so every DMA block has
//    one source. Tiles run in a 3-stage ring, loaded two tiles ahead, with one
//    barrier per tile. The DMAs are issued from inline asm: the compiler then
//    sees no LDS DMA and adds none of its conservative "wait for every LDS
//    DMA" stalls before LDS reads; the kernel waits explicitly instead.
//  * K and V rows are XOR-swizzled in 16-byte chunks so the MFMA operand reads
//    (plain and transposing) are bank-conflict free without the padding that
//    1 KB DMA blocks cannot have.
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

template <int DK, int DV, int G, int RCH>
struct Cfg {
  static constexpr int ROWS = NW * RW;        // (head, position) rows per WG
  static constexpr int PW = ROWS / G;         // query positions per WG
  static constexpr int NC = DK / 8;           // 16-byte chunks per K row
  static constexpr int NP = NC - RCH;         // plain (unrotated) chunks per K row
  // K tile: rotated region [32][RCH] chunks, then plain region [32][NP].
  static constexpr int KR_BYTES = BN * RCH * 16;
  static constexpr int KT_BYTES = BN * NC * 16;
  static constexpr int VC = DV / 8;           // 16-byte chunks per V row
  static constexpr int VT_BYTES = BN * VC * 16;
  static constexpr int ST_BYTES = KT_BYTES + VT_BYTES;  // one ring stage
  // Ring depth: as many stages as LDS holds, at most 4 (tiles loaded up to
  // three ahead): 3 for the 512-dim keys, 4 for 256- and 128-dim heads.
  static constexpr int STAGES = (4 * ST_BYTES <= 160 * 1024) ? 4 : 3;
  static constexpr int AHEAD = STAGES - 1;    // tiles in flight after a step's issue
  static constexpr int LDS_BYTES = STAGES * ST_BYTES;
  // 1 KB DMA blocks per tile: rotated K, plain K, V.
  static constexpr int KR_DMA = KR_BYTES / 1024;
  static constexpr int KP_DMA = (KT_BYTES - KR_BYTES) / 1024;
  static constexpr int V_DMA = VT_BYTES / 1024;
  static constexpr int N_DMA = KR_DMA + KP_DMA + V_DMA;
  static constexpr int DMA_W = N_DMA / NW;    // DMA issues per wave per tile
  // Region boundaries fall on whole issue slots: slot i's region is the same
  // for every wave and known at compile time.
  static constexpr bool ALIGNED = KR_DMA % NW == 0 && KP_DMA % NW == 0;
  __host__ __device__ static constexpr int region(int n) {
    return n < KR_DMA ? 0 : n < KR_DMA + KP_DMA ? 1 : 2;
  }
  static_assert(ROWS % G == 0 && PW % RW == 0, "rows must split evenly over the heads");
  static_assert(KR_BYTES % 1024 == 0 && KT_BYTES % 1024 == 0 && VT_BYTES % 1024 == 0,
                "DMA blocks");
  static_assert(N_DMA % NW == 0, "every wave issues the same number of DMAs per tile");
  static_assert((AHEAD - 1) * DMA_W < 64, "vmcnt field");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(DK % 32 == 0 && DV % 16 == 0, "MFMA tiling");
};

// XOR swizzle of 16-byte chunks inside a region row of `width` chunks. The
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

template <int DK, int DV, int G, int RCH>
__global__ __launch_bounds__(NT, 1) void prefill_mfma_kernel(PrefillArgs a, int n_qt,
                                                             int contig) {
  using C = Cfg<DK, DV, G, RCH>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS_BYTES];

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

  // ---- DMA sources: K (plain dims), K's rotated dims, V of this (b, head) --
  const int krow = a.Hkv * DK * 2, vrow = a.Hkv * DV * 2;  // bytes per token
  const bool rot_q = RCH > 0 && a.rope_q;
  const bool krot_ws = RCH > 0 && a.rope_k;  // rotated dims from the workspace
  const int rrow = krot_ws ? a.Hkv * RCH * 16 : krow;
  const u32x4 kdesc = buffer_desc((const char*)a.k + ((int64_t)b * T * a.Hkv + kvh) * DK * 2,
                                  (T - 1) * krow + DK * 2);
  const u32x4 vdesc = buffer_desc((const char*)a.v + ((int64_t)b * T * a.Hkv + kvh) * DV * 2,
                                  (T - 1) * vrow + DV * 2);
  const u32x4 rdesc =
      krot_ws ? buffer_desc((const char*)a.k_rot + ((int64_t)b * T * a.Hkv + kvh) * RCH * 16,
                            (T - 1) * rrow + RCH * 16)
              : kdesc;

  // Block n of a tile (n = i*NW + wave) covers 64 chunks; this lane's chunk's
  // byte offset inside tile row 0 and row stride are fixed, so a tile adds
  // j0 * stride. Region by block: rotated K, plain K, V.
  uint32_t dma_off[C::DMA_W];
#pragma unroll
  for (int i = 0; i < C::DMA_W; ++i) {
    const int n = i * NW + wave;
    if (n < C::KR_DMA) {
      constexpr int RCHd = RCH > 0 ? RCH : 1;  // branch is dead when RCH == 0
      const int q = n * 64 + lane, r = q / RCHd;
      dma_off[i] = r * rrow + kswz<RCHd>(r, q % RCHd) * 16;
    } else if (n < C::KR_DMA + C::KP_DMA) {
      constexpr int NPd = C::NP > 0 ? C::NP : 1;
      const int q = (n - C::KR_DMA) * 64 + lane, r = q / NPd;
      dma_off[i] = r * krow + (RCH + kswz<NPd>(r, q % NPd)) * 16;
    } else {
      const int q = (n - C::KR_DMA - C::KP_DMA) * 64 + lane, r = q / C::VC;
      dma_off[i] = r * vrow + kswz<C::VC>(r, q % C::VC) * 16;
    }
  }
  // Tiles past the range are issued too (one vmcnt value then covers every
  // step), but at an offset past the descriptors' end: they return zeros
  // without touching memory.
  auto dma_tile = [&](int kb, int stage) {
    const int j0 = kb * BN;
    const uint32_t st = lds_addr(lds) + stage * C::ST_BYTES;
    const uint32_t far = kb < kb_hi ? 0u : 0x80000000u;
    // Blocks are laid out back to back (rotated K, plain K, V), so block n
    // lands at st + 1024 n whatever its region.
#pragma unroll
    for (int i = 0; i < C::DMA_W; ++i) {
      const int n = i * NW + wave;
      const int reg = C::ALIGNED ? C::region(i * NW) : C::region(n);
      if (reg == 0)
        dma16(rdesc, st + n * 1024, (dma_off[i] + j0 * rrow) | far);
      else if (reg == 1)
        dma16(kdesc, st + n * 1024, (dma_off[i] + j0 * krow) | far);
      else
        dma16(vdesc, st + n * 1024, (dma_off[i] + j0 * vrow) | far);
    }
  };

  // ---- prologue: tiles 0 and 1 in flight around the Q load ----------------
  const int n_tiles = kb_hi - kb_lo;
  if (n_tiles > 0) dma_tile(kb_lo, 0);

  // Q^T operand: step s covers dims 32s + 8g .. 32s + 8g + 7 of this row.
  bf16x8 qf[DK / 32];
  {
    const int tab_row = a.rot_pairs * 8;  // bytes per table row
    const __amdgpu_buffer_rsrc_t tres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.rope_tab, (short)0, rot_q ? T * tab_row : 0, 0x00020000);
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
    // tiles 1 .. AHEAD-1 (they may lie past the range: never read)
#pragma unroll
    for (int u = 1; u < C::AHEAD; ++u) dma_tile(kb_lo + u, u);
    wait_vm<(C::AHEAD - 1) * C::DMA_W>();  // tile 0 landed; the rest may be in flight
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

  // K operand: key 16mb + r16, chunk 4s + g. Keys r16 and r16 + 16 share the
  // swizzle, so the second is the first plus a constant; the lane-dependent
  // part of the offset takes H+1 values (s & H), the rest is an immediate.
  using KR = KAddr<(RCH > 0 ? RCH : 16)>;
  using KP = KAddr<(C::NP > 0 ? C::NP : 16)>;
  constexpr int HR = (Swz<(RCH > 0 ? RCH : 16)>::P >= 4 ? Swz<(RCH > 0 ? RCH : 16)>::P / 4 : 1);
  constexpr int HP = (Swz<(C::NP > 0 ? C::NP : 16)>::P >= 4 ? Swz<(C::NP > 0 ? C::NP : 16)>::P / 4 : 1);
  constexpr int KR_ROW16 = 16 * (RCH > 0 ? RCH : 16) * 16;   // 16 rows of the rotated region
  constexpr int KP_ROW16 = 16 * (C::NP > 0 ? C::NP : 16) * 16;
  int kro[HR], kpo[HP];
  {
    const KR kr(0, r16, g);
    const KP kp(C::KR_BYTES, r16, g);
#pragma unroll
    for (int h = 0; h < HR; ++h) kro[h] = kr(h);
#pragma unroll
    for (int h = 0; h < HP; ++h) kpo[h] = kp(h);
  }
  // V^T operand, transposing reads: in each 16-lane group, lane 4r + c reads
  // dims 16d + 4c .. 16d + 4c + 3 of key 16h + 4g + r; the row's swizzle is
  // x = 4g + r (both halves), so chunk 2d + (c >> 1) sits at
  // 2(d ^ (x >> 1)) + ((c >> 1) ^ (x & 1)). With d = 8A + B, d ^ (x >> 1) =
  // 8A + (B ^ (x >> 1)): 8 lane-dependent offsets, A and h immediates.
  int vto[8];
  {
    const int vx = 4 * g + (r16 >> 2), vc = r16 & 3;
    const int v_lane =
        C::KT_BYTES + vx * C::VC * 16 + (((vc >> 1) ^ (vx & 1)) << 4) + ((vc & 1) << 3);
#pragma unroll
    for (int B = 0; B < 8; ++B) vto[B] = v_lane + ((B ^ (vx >> 1)) << 5);
  }

  auto live = [&](int kb) {
    const int j0 = kb * BN;
    return j0 <= whi && !(W > 0 && j0 + BN - 1 <= wlo - W);
  };

  // One tile, read from the ring stage at LDS pointer st.
  auto compute = [&](const lds_u8* st, int kb) {
    const int j0 = kb * BN;
    const lds_u8* krb[HR];
    const lds_u8* kpb[HP];
#pragma unroll
    for (int h = 0; h < HR; ++h) krb[h] = st + kro[h];
#pragma unroll
    for (int h = 0; h < HP; ++h) kpb[h] = st + kpo[h];
    f32x4 s0 = f32x4{}, s1 = f32x4{};
    // dims 32s + 8g..: s < RCH/4 in the rotated region, the rest in the plain one
#pragma unroll
    for (int s = 0; s < RCH / 4; ++s) {
      const lds_u8* p = krb[s % HR] + (s / HR) * HR * 64;
      const bf16x8 k0 = *(const lds_bf16x8*)p;
      const bf16x8 k1 = *(const lds_bf16x8*)(p + KR_ROW16);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[s], s1, 0, 0, 0);
    }
#pragma unroll
    for (int s = RCH / 4; s < DK / 32; ++s) {
      const int sp = s - RCH / 4;
      const lds_u8* p = kpb[sp % HP] + (sp / HP) * HP * 64;
      const bf16x8 k0 = *(const lds_bf16x8*)p;
      const bf16x8 k1 = *(const lds_bf16x8*)(p + KP_ROW16);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[s], s1, 0, 0, 0);
    }
    // lane holds keys j0 + 4g + i (s0) and j0 + 16 + 4g + i (s1) of its row
    float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    // Only tiles crossing the diagonal or a window edge of this wave's rows
    // pay for the per-score test; the empty asm keeps this a branch (the
    // compiler would otherwise run the selects on every tile).
    if ((j0 + BN - 1 > wlo) || (W > 0 && j0 <= whi - W)) {
      asm volatile("");
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
    const lds_u8* vb[8];
#pragma unroll
    for (int B = 0; B < 8; ++B) vb[B] = st + vto[B];
#pragma unroll
    for (int d = 0; d < DV / 16; ++d) {
      const lds_u8* p = vb[d % 8] + (d / 8) * 256;
      const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
      const bf16x4 v1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 16 * C::VC * 16));
      const bf16x8 va = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pop, oacc[d], 0, 0, 0);
    }
  };
  // ---- main loop: a ring of STAGES tiles, loaded AHEAD tiles ahead --------
  // Step t issues tile t+AHEAD into the stage tile t-1 used, computes tile t,
  // then waits for tile t+1 (everything but the AHEAD-1 newest groups of DMAs,
  // which are always the last loads issued) and synchronises. Every step
  // issues the same DMAs, also the last ones (their tiles may lie past the
  // range or past T, where the descriptors return zeros, and are never read).
  int cur = 0;  // stage of tile t
  for (int t = 0; t < n_tiles; ++t) {
    const int kb = kb_lo + t;
    const int prev = cur == 0 ? C::STAGES - 1 : cur - 1;  // stage of t-1 = of t+AHEAD
    dma_tile(kb + C::AHEAD, prev);
    // The stage offset goes through readfirstlane so the compiler treats it as
    // an opaque scalar: every LDS read is then base register + immediate,
    // instead of strength-reduced per-read induction registers.
    const int so = __builtin_amdgcn_readfirstlane(cur * C::ST_BYTES);
    if (live(kb)) compute((const lds_u8*)lds + so, kb);
    cur = cur == C::STAGES - 1 ? 0 : cur + 1;
    wait_vm<(C::AHEAD - 1) * C::DMA_W>();  // tile t+1 landed
    lds_barrier();  // ... for every wave; stage of tile t free
  }
  wait_vm<0>();  // no DMA may still target LDS when the block ends

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

// 512-dim keys with 256-dim values; the caller checked the rest.
hipError_t launch_prefill_mfma16(const PrefillArgs& a, hipStream_t st) {
  if (a.Dk == 512 && a.Dv == 256) return dispatch_g<512, 256>(a, st);
  return hipErrorNotSupported;
}

}  // namespace attn
