// prefill_mfma.hip — flash-style causal / sliding-window GQA prefill on gfx950
// bf16 matrix cores (v_mfma_f32_32x32x16_bf16), with RoPE applied on the way
// in.
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
// Used for heads up to 256 dims; the 512-dim keys of the global layers go to
// the one-wave-per-SIMD kernel in prefill_mfma1w.hip, and the local layers'
// shape (256-dim heads, 2 query heads per KV head) to the two-workgroups-per-
// CU variant of this kernel in prefill_mfma2g.hip.
//
// Design for CDNA4:
//  * A workgroup of 8 waves (two per SIMD) owns one (batch, KV head) and PW
//    consecutive query positions for all G query heads sharing that KV head:
//    256 (head, position) rows, so each K/V tile staged in LDS serves G heads.
//  * Each wave owns 32 rows and computes S^T = K Q^T with 32x32x16 MFMAs
//    (M = 32 keys, N = 32 rows): every 1 KB K operand read from LDS feeds a
//    32-row MFMA, which halves the LDS read traffic per FLOP against 16-row
//    waves (LDS bandwidth, not the matrix cores, bounded those). Every lane
//    holds 16 scores of one query row and its partner lane (l ^ 32) the other
//    16, so the row max and sum need one cross-lane swap. Q^T (DK/16 x 16
//    bytes per lane) and the O^T accumulator (DV/2 fp32 per lane) stay in
//    registers, which fits two waves per SIMD for heads up to 256 dims.
//  * O^T = V^T P^T (K = 16 keys per MFMA): the P^T operand is the lane's own
//    scores (first or last 8) when the key order inside the MFMA matches the
//    score layout. V tiles sit in LDS in their natural [key][dim] layout and
//    the V^T operand is read with the transposing LDS read (ds_read_b64_tr_b16),
//    two reads of 4 keys each per operand, in that key order.
//  * K and V tiles (32 keys) move HBM -> LDS by direct DMA (buffer loads with
//    the lds flag): no staging registers, no VALU work, rows past T read as
//    zero. The rotated leading dims of K come already turned from a rotation
//    pass that runs once per key (not once per query tile) into a workspace;
//    each K tile keeps them in a region of its own, so every DMA block has
//    one source. Tiles run in a ring of 3 or 4 stages, loaded 2 or 3 tiles
//    ahead, with one barrier per tile.
//  * K and V rows are XOR-swizzled in 16-byte chunks so the MFMA operand reads
//    (plain and transposing) spread over the LDS banks without the padding
//    that 1 KB DMA blocks cannot have.
//  * Only key tiles intersecting the causal band / sliding window are visited
//    (window-aware skipping); masking runs only on tiles that cross the
//    diagonal or the window edge.
//  * The running max is updated lazily: O is rescaled only when a row's block
//    max exceeds the max in use by more than 2^8 (probabilities stay <= 256,
//    exact after the final division).
//  * Causal tiles are issued longest-first; sliding-window launches map
//    neighbouring query tiles onto the same XCD so their K/V windows share L2.
#include <type_traits>

#include "attn_common.h"
#include "kernels.h"
#include "prefill_common.h"

namespace attn {
namespace {

constexpr int RW = 32;         // query rows per wave
constexpr int BN = 32;         // keys per tile

template <int DK, int DV, int G, int RCH>
struct Cfg {
  // Waves per workgroup: two per SIMD (a wave's registers fit in half the
  // file for heads up to 256 dims).
  static constexpr int NW = 8;
  static_assert(DK <= 256 && DV <= 256, "larger heads use prefill_mfma1w.hip");
  static constexpr int NT = NW * 64;
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
  // Ring of 4 stages; the prologue puts tiles 0-2 in flight and step t
  // issues tile t+3 (the phase schedule below).
  static constexpr int STAGES = 4;
  static constexpr int AHEAD = STAGES - 1;
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
  static_assert(ROWS % G == 0, "rows split evenly over the heads");
  static_assert(KR_BYTES % 1024 == 0 && KT_BYTES % 1024 == 0 && VT_BYTES % 1024 == 0,
                "DMA blocks");
  static_assert(N_DMA % NW == 0, "every wave issues the same number of DMAs per tile");
  static_assert((AHEAD - 1) * DMA_W < 64, "vmcnt field");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(DK % 16 == 0 && DV % 32 == 0 && RCH % 2 == 0, "MFMA tiling");
  static_assert(VC >= 16, "V rows swizzle over 16 chunk groups");
};

using namespace prefill;

template <int DK, int DV, int G, int RCH>
__global__ __launch_bounds__((Cfg<DK, DV, G, RCH>::NT), 1) void prefill_mfma_kernel(
    PrefillArgs a, int n_qt, int contig) {
  using C = Cfg<DK, DV, G, RCH>;
  constexpr int NW = C::NW;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, h = lane >> 5;  // this lane's row; half of the k range
  const int T = a.T, W = a.window;
  const int n_wg = n_qt * a.Hkv * a.B;
  const int L = contig ? xcd_contiguous((int)blockIdx.x, n_wg) : (int)blockIdx.x;
  const int grp = L / n_qt;
  const int qt = n_qt - 1 - (L % n_qt);  // longest causal tiles first
  const int kvh = grp % a.Hkv, b = grp / a.Hkv;
  const int p0 = qt * C::PW;

  // This lane's query row: wave w takes head w % G and the 32 positions of
  // block w / G. Waves w and w + 4 share a SIMD; for G < 8 they get position
  // blocks 4 / G apart, so the tiles one of them skips (past its diagonal,
  // before its window) are not the tiles the other skips and the SIMD's
  // matrix pipe keeps one wave's work.
  static_assert(C::NW % G == 0 && C::PW == RW * (C::NW / G), "wave -> (head, block) map");
  const int head = kvh * G + wave % G;
  const int wlo = p0 + RW * (wave / G);
  const int pos = wlo + r32;
  const bool valid = pos < T;
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
    if (n < C::KR_DMA)
      dma_off[i] = k_rot_dma_off<RCH>(n, lane, rrow);
    else if (n < C::KR_DMA + C::KP_DMA)
      dma_off[i] = k_plain_dma_off<RCH, C::NP>(n - C::KR_DMA, lane, krow);
    else
      dma_off[i] = v_dma_off<C::VC>(n - C::KR_DMA - C::KP_DMA, lane, vrow);
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

  // ---- prologue: tiles 0 .. AHEAD-1 in flight around the Q load ------------
  const int n_tiles = kb_hi - kb_lo;
  if (n_tiles > 0) dma_tile(kb_lo, 0);

  // Q^T operand: step s covers dims 16s + 8h .. 16s + 8h + 7 of this row.
  bf16x8 qf[DK / 16];
  {
    const int prow = valid ? pos : T - 1;
    // Q's rotation by angle addition: the wave builds the (cos, sin) row of
    // its first position in fp64 in block `wave` of ring stage 1 (which only
    // this wave's own DMA of tile 1 overwrites, after the rotation), and each
    // lane turns that row further by its offset d = prow - wlo (0..31).
    const int base = min(wlo, T - 1);
    lds_float2* slot = (lds_float2*)((lds_u8*)lds + C::ST_BYTES + wave * 1024);
    const uint16_t* qrow =
        (const uint16_t*)a.q + (((int64_t)b * T + prow) * a.Hq + head) * DK + 8 * h;
    u32x4 qw[DK / 16];
#pragma unroll
    for (int s = 0; s < DK / 16; ++s) qw[s] = *(const u32x4*)(qrow + 16 * s);
    if (rot_q) {
      rope_base_row(slot, (int64_t)a.pos0 + base, a.rot_pairs, DK, a.log2_theta, lane);
      float dcs[RCH / 2 > 0 ? RCH / 2 : 1][8];
      rope_offsets<RCH / 2>(dcs, prow - base, a.rope_rho, h);
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<0>();  // Q landed (and tile 0 before it)
      rotate_q_chunks<RCH / 2>(qw, slot, dcs, h);
    }
#pragma unroll
    for (int s = 0; s < DK / 16; ++s) {
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

  // ---- online softmax state (one row per lane; lanes l and l^32 share it) --
  // scores to log2 units; kept > 0 so a masked -inf score never meets a zero
  // factor (scale 0 then acts as 1e-30: every visible key weighs the same)
  const float c2 = fmaxf(a.scale * kLog2e, 1e-30f);
  const unsigned wcap = (W > 0) ? (unsigned)W : 0x80000000u;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) oacc[d] = f32x16{};

  // K operand of step s: key r32, chunk 2s + h of its region row, stored at
  // chunk (2s + h) ^ x with x = r32 & M, i.e. at byte 16((2s + h) ^ x) =
  // 32s ^ 16(h ^ x) of the row: one XOR-add per read from a per-lane row
  // offset and mask (precomputed addresses would hold 8 registers).
  constexpr int RW_ = RCH > 0 ? RCH : 16, PW_ = C::NP > 0 ? C::NP : 16;
  const int kr_row = r32 * RW_ * 16, kp_row = C::KR_BYTES + r32 * PW_ * 16;
  const int kxr = 16 * (h ^ (r32 & Swz<RW_>::M)), kxp = 16 * (h ^ (r32 & Swz<PW_>::M));
  // V^T operand, transposing reads. In 16-lane group gi (h = gi >> 1, dim
  // block db = gi & 1), lane 4r + c reads dims 32dt + 16db + 4c .. +3 of key
  // 16j + 8hs + 4h + r. That key row's swizzle is 4r, so chunk 4dt + y
  // (y = 2db + (c >> 1)) sits at 4(dt ^ r) + y: byte 64((dt & 3) ^ r) plus
  // 256(dt >> 2), 16y, 8(c & 1) and the row offsets of j and hs.
  int v_row, vx;
  {
    const int li = lane & 15, gi = lane >> 4, r = li >> 2, c = li & 3;
    const int y = 2 * (gi & 1) + (c >> 1);
    v_row = C::KT_BYTES + (4 * h + r) * C::VC * 16 + (y << 4) + ((c & 1) << 3);
    vx = r << 6;
  }

  // A wave computes a tile only if it holds a key one of its rows may see
  // (a wave whose rows all lie past T, the padding of the last query tile,
  // computes none).
  auto live = [&](int kb) {
    const int j0 = kb * BN;
    return wlo < T && j0 <= whi && !(W > 0 && j0 + BN - 1 <= wlo - W);
  };

  // Operand reads run OD-1 MFMAs ahead of their use, in a ring of OD
  // registers; the scheduling barriers keep the compiler from sinking each
  // read next to its MFMA (it would then wait out the full LDS latency
  // before every MFMA). Read i+OD-1 reuses the registers of MFMA i-1.
  constexpr int OD = 4;
  constexpr int NS = DK / 16;                 // QK MFMAs per tile
  constexpr int NDT = DV / 32, NPV = 2 * NDT;  // P.V MFMAs per tile
  // Per-stage operand addressing: row bases for the stage and the lane masks,
  // passed through an empty asm so the compiler neither hoists the per-read
  // XORs out of the tile loop nor folds them into long-lived registers.
  struct Addr {
    const lds_u8 *kr, *kp, *v;
    int kxr, kxp, vx;
  };
  auto addr = [&](const lds_u8* st) {
    Addr ad{st + kr_row, st + kp_row, st + v_row, kxr, kxp, vx};
    asm volatile("" : "+v"(ad.kxr), "+v"(ad.kxp), "+v"(ad.vx));
    return ad;
  };
  // K operand of QK step s (one 16-byte read per lane).
  auto kread = [&](const Addr& ad, int s) {
    return k_operand<RCH>(ad.kr, ad.kp, ad.kxr, ad.kxp, s);
  };
  // V^T operand of P.V step i (key half j = i / NDT, dim tile dt = i % NDT):
  // two transposing reads of 4 keys each, 8 key rows apart.
  auto vread = [&](const Addr& ad, int i) { return vt_operand<NDT, C::VC>(ad.v, ad.vx, i); };

  // S^T[32 keys][32 rows] of the tile in flight: element e holds key
  // 8(e/4) + 4h + (e%4). P^T operands of the tile whose softmax ran last.
  f32x16 sc = f32x16{};
  bf16x8 pop[2];
  bf16x8 ob[OD];  // operand ring

  // One matrix phase as a single stream of MFMAs: P.V of one tile (ops
  // 0 .. NPV-1, V from stage sv) then QK of the next (ops NPV .. NPV+NS-1, K
  // from stage sk); either part may be absent (PV_, QK_ are compile-time
  // flags). The first OD-1 operands were read into the ring by stream_head.
  // `side` runs once, after the stream's second MFMA: work placed there
  // (the next tile's DMA issue) fills issue slots while the matrix pipe is
  // busy instead of delaying the first MFMA.
  auto mfma_stream = [&](auto PV_, auto QK_, const Addr& av, const Addr& ak, auto&& side) {
    constexpr bool do_pv = decltype(PV_)::value, do_qk = decltype(QK_)::value;
    constexpr int lo = do_pv ? 0 : NPV, hi = do_qk ? NPV + NS : NPV;
    auto rd = [&](int i) { return i < NPV ? vread(av, i) : kread(ak, i - NPV); };
#pragma unroll
    for (int i = lo; i < hi; ++i) {
      if (i == lo + 2) {
        side();
        __builtin_amdgcn_sched_barrier(0);
      }
      // ring slot of op i counts from the stream's first op
      if (i + OD - 1 < hi) ob[(i - lo + OD - 1) % OD] = rd(i + OD - 1);
      const bf16x8 op = ob[(i - lo) % OD];
      if (i < NPV)
        oacc[i % NDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, pop[i / NDT], oacc[i % NDT], 0, 0, 0);
      else
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, qf[i - NPV], i == NPV ? f32x16{} : sc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto stream_head = [&](auto PV_, const Addr& av, const Addr& ak) {
#pragma unroll
    for (int i = 0; i < OD - 1; ++i) ob[i] = decltype(PV_)::value ? vread(av, i) : kread(ak, i);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

  // Softmax of the scores in sc (tile kb) into pop.
  auto softmax = [&](int kb) {
    const int j0 = kb * BN;
    mask_edge_tile(sc, j0, wlo, whi, W, pos, h, wcap);
    float sv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) sv[e] = sc[e];
    float mx = sv[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sv[e]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float mc = (mx == -INFINITY) ? -INFINITY : mx * c2;
    if (__any(mc > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mc);
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < DV / 32; ++d) oacc[d] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float pv[16];  // masked scores are -inf and c2 > 0, so they give exactly 0
#pragma unroll
    for (int e = 0; e < 16; ++e) pv[e] = fast_exp2(fmaf(sv[e], c2, -m_use));
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ps += pv[e];
    l_run += ps;
    // P^T operand of key step j: this lane's elements 8j .. 8j+7.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f32x4 lo = {pv[8 * j], pv[8 * j + 1], pv[8 * j + 2], pv[8 * j + 3]};
      const f32x4 hi = {pv[8 * j + 4], pv[8 * j + 5], pv[8 * j + 6], pv[8 * j + 7]};
      pop[j] = __builtin_shufflevector(__builtin_convertvector(lo, bf16x4),
                                       __builtin_convertvector(hi, bf16x4), 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };

  // ---- main loop: softmax phases against matrix phases ----------------------
  // Every wave runs, per tile t: softmax(t) | barrier | P.V(t) then QK(t+1) |
  // barrier. Waves w and w + 4 share a SIMD; group 1 (waves 4-7) passes one
  // extra barrier before the loop and group 0 one after it, so between any
  // two barriers one wave of each SIMD does its softmax (vector ALU) while
  // the other streams MFMAs, and the two alternate.
  //
  // Ring (4 stages): K(t) is read by QK(t) and V(t) by P.V(t), the latter in
  // the phase that starts at barrier 2t+1 (group 0) or 2t+2 (group 1); the
  // stage of tile t-1 is therefore free in the phase after barrier 2t+1,
  // where each wave issues its share of tile t+3. A wave may leave its share
  // of one tile in flight at a barrier (two for group 0 after a matrix
  // phase): each tile then has landed one barrier before the QK that reads
  // it, two steps after its issue.
  static_assert(C::STAGES == 4, "phase schedule assumes a 4-stage ring");
  auto stage = [&](int t) {
    return (const lds_u8*)lds + __builtin_amdgcn_readfirstlane((t & 3) * C::ST_BYTES);
  };
  const int lag = wave >> 2;
  if (n_tiles > 0) {
    if (live(kb_lo)) {
      const Addr a0 = addr(stage(0));
      stream_head(F_{}, a0, a0);
      mfma_stream(F_{}, T_{}, a0, a0, [] {});
    }
    if (lag) {
      wait_vm<C::DMA_W>();
      lds_barrier();
    }
  }
#ifdef ATTN_DEBUG_TILES
  int dbg_live = 0;
#endif
  for (int t = 0; t + 1 < n_tiles; ++t) {
    const int kb = kb_lo + t;
    const bool lv = live(kb), lv_next = live(kb + 1);
#ifdef ATTN_DEBUG_TILES
    dbg_live += lv;
#endif
    // The stage offset goes through readfirstlane so the compiler treats it
    // as an opaque scalar: every LDS read is then base register + immediate,
    // instead of strength-reduced per-read induction registers.
    const Addr at = addr(stage(t)), an = addr(stage(t + 1));
    if (lv)
      softmax(kb);
    else
      pop[0] = pop[1] = bf16x8{};
    // The first operands of the matrix phase read landed stages: they
    // overlap the barrier wait.
    // A tile dead for this wave next to a live one still runs through the
    // stream: its P^T is zero (P.V adds nothing) or its scores are never
    // used (the softmax skips it).
    const bool any = lv || lv_next;
    if (any) stream_head(T_{}, at, an);
    wait_vm<C::DMA_W>();
    lds_barrier();
    auto issue = [&] { dma_tile(kb + 3, (t + 3) & 3); };
    if (any)
      mfma_stream(T_{}, T_{}, at, an, issue);
    else
      issue();
    if (lag)
      wait_vm<C::DMA_W>();
    else
      wait_vm<2 * C::DMA_W>();
    lds_barrier();
  }
  // The last tile has no next one: its matrix phase is P.V alone (its DMA
  // issue, all past the range, keeps the waits above uniform).
  if (n_tiles > 0) {
    const int t = n_tiles - 1, kb = kb_lo + t;
    const bool lv = live(kb);
#ifdef ATTN_DEBUG_TILES
    dbg_live += lv;
#endif
    const Addr at = addr(stage(t)), an = addr(stage(t + 1));
    if (lv)
      softmax(kb);
    else
      pop[0] = pop[1] = bf16x8{};
    if (lv) stream_head(T_{}, at, an);
    wait_vm<C::DMA_W>();
    lds_barrier();
    auto issue = [&] { dma_tile(kb + 3, (t + 3) & 3); };
    if (lv)
      mfma_stream(T_{}, F_{}, at, an, issue);
    else
      issue();
    if (lag)
      wait_vm<C::DMA_W>();
    else
      wait_vm<2 * C::DMA_W>();
    lds_barrier();
  }
  if (n_tiles > 0 && !lag) lds_barrier();
#ifdef ATTN_DEBUG_TILES
  if (a.dbg_visits && lane == 0) {
    atomicAdd(a.dbg_visits, (unsigned long long)dbg_live);
    if (wave == 0) atomicAdd(a.dbg_visits + 1, (unsigned long long)n_tiles);
  }
#endif
  // ---- epilogue: O = O^T / l, bf16, through LDS ------------------------------
  // Once every wave's DMAs have landed and its reads returned, the ring is
  // free: each wave stages its 32 x DV output tile there, then writes whole
  // rows with 16-byte stores (a lane's registers hold 4-dim pieces of one row,
  // and storing those directly splits every output row over 32 partial-line
  // writes).
  wait_vm<0>();
  lds_barrier();
  // The partner lane (l ^ 32) summed the row's other 16 keys per tile under
  // the same running max.
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                     __float_as_uint(l_run), false, false);
    l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  static_assert(C::ROWS * DV * 2 <= C::LDS_BYTES, "output staging fits the ring");
  __attribute__((address_space(3))) unsigned char* ost =
      (__attribute__((address_space(3))) unsigned char*)lds + wave * (RW * DV * 2);
  stage_o<DV / 32>(ost, oacc, valid ? 1.f / l_run : 0.f, r32, h);
  store_o<DV, RW>(ost, lane, [&](int row) -> uint16_t* {
    const int p = wlo + row;
    return p < T ? (uint16_t*)a.o + (((int64_t)b * T + p) * a.Hq + head) * DV : nullptr;
  });
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
  hipLaunchKernelGGL((prefill_mfma_kernel<DK, DV, G, RCH>), dim3((unsigned)n), dim3(C::NT), 0,
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

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t st) {
  const int rdims = (a.rope_q || a.rope_k) ? 2 * a.rot_pairs : 0;
  if (!prefill_mfma_supported(a.Dk, a.Dv, a.Hq / a.Hkv, a.scale, rdims))
    return hipErrorNotSupported;
  if (a.rope_k && rdims > 0 && !a.k_rot) return hipErrorInvalidValue;
  // 32-bit buffer offsets: one batch's K, V (or turned K dims, at most Dk
  // wide) must stay under 2 GiB.
  const int64_t per_b = (int64_t)a.T * a.Hkv * (a.Dk > a.Dv ? a.Dk : a.Dv) * 2;
  if (per_b >= (int64_t)1 << 31) return hipErrorNotSupported;
  if (a.Dk == 512 && a.Dv == 256) return launch_prefill_mfma1w(a, st);
  if (a.Dk == 512 && a.Dv == 512) {
    // Keys as values (the same rotated keys as k and v): one pass, the key
    // tile in LDS serving both products.
    if (prefill_kv1w_applies(a)) return launch_prefill_kv1w(a, st);
    // Separate 512-dim values as two passes over 256-dim halves of v and o:
    // a second operand tile beside the 512-dim O accumulators would not fit.
    // Each pass recomputes Q.K^T (3/2 of the useful FLOPs in all).
    PrefillArgs h = a;
    h.Dv = 256;
    h.v_tok = (int64_t)a.Hkv * 512;
    h.v_head = 512;
    h.o_tok = (int64_t)a.Hq * 512;
    h.o_head = 512;
    for (int half = 0; half < 2; ++half) {
      h.v = static_cast<const uint16_t*>(a.v) + 256 * half;
      h.o = static_cast<uint16_t*>(a.o) + 256 * half;
      const hipError_t e = launch_prefill_mfma1w(h, st);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (a.Dk == 256 && a.Dv == 256 && a.Hq / a.Hkv == 2) return launch_prefill_mfma2g(a, st);
  if (a.Dk == 256 && a.Dv == 256) return dispatch_g<256, 256>(a, st);
  if (a.Dk == 128 && a.Dv == 128) return dispatch_g<128, 128>(a, st);
  return hipErrorNotSupported;
}

}  // namespace attn
