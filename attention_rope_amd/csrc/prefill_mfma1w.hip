// prefill_mfma1w.hip — flash-style causal / sliding-window GQA prefill on
// gfx950 bf16 matrix cores (v_mfma_f32_32x32x16_bf16) with one wave per SIMD,
// RoPE applied on the way in.
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
//  * A workgroup of 4 waves, one per SIMD, owns one (batch, KV head) and PW
//    consecutive query positions for all G query heads of that KV head: 128
//    (head, position) rows. A wave holds 32 rows (two heads x 16 positions
//    for G = 8, else one head x 32 positions) and so the whole register file
//    of its SIMD: the O^T accumulator in AGPRs, which only MFMAs touch, and
//    Q^T (DK/16 x 16 bytes per lane, 128 registers for the 512-dim global
//    keys) in the AGPRs left over and the rest in VGPRs. 32-row waves use v_mfma_f32_32x32x16_bf16 for the widened
//    keys too, where two waves per SIMD would not fit.
//  * S^T = K Q^T (M = 32 keys, N = 32 rows) and O^T = V^T P^T as in the
//    two-wave kernel: every lane holds 16 scores of one row, its partner lane
//    (l ^ 32) the other 16, and the P^T operand is the lane's own scores.
//  * Software pipeline: iteration t runs one stream of MFMAs, P.V of tile t-1
//    and QK of tile t+1, and cuts the softmax of tile t into slices placed
//    between those MFMAs, so the vector ALU works while the matrix pipe is
//    busy. A dependent chain of these MFMAs issues every 32 cycles, so one
//    wave keeps its SIMD's matrix pipe full.
//  * K and V tiles (32 keys) move HBM -> LDS by direct DMA into two rings of
//    3 stages each: iteration t issues K(t+3) and V(t+1), two iterations
//    ahead of their use, with one barrier per iteration.
//  * K and V rows are XOR-swizzled in 16-byte chunks (conflict-free operand
//    reads); the output tile is staged in LDS and written as whole rows.
//  * Only key tiles intersecting the workgroup's causal band / window are
//    visited; a tile outside one wave's band is masked to -inf (no branch in
//    the stream).
//  * The running max is updated lazily: O is rescaled only when a row's block
//    max exceeds the max in use by more than 2^8.
#include <type_traits>

#include "attn_common.h"
#include "kernels.h"
#include "prefill_common.h"

namespace attn {
namespace {

constexpr int RW = 32;         // query rows per wave
constexpr int BN = 32;         // keys per tile
constexpr int NW = 4;          // waves per workgroup (one per SIMD)
constexpr int NT = NW * 64;

template <int DK, int DV, int G, int RCH>
struct Cfg1 : prefill::WaveRows<G> {
  using R = prefill::WaveRows<G>;
  static_assert(RW == 32 && NW == 4, "the row map is for 4 waves of 32 rows");
  static constexpr int NC = DK / 8;              // 16-byte chunks per K row
  static constexpr int NP = NC - RCH;            // plain (unrotated) chunks per K row
  static constexpr int KR_BYTES = BN * RCH * 16;  // K tile: rotated region, then plain
  static constexpr int KT_BYTES = BN * NC * 16;
  static constexpr int VC = DV / 8;
  static constexpr int VT_BYTES = BN * VC * 16;
  static constexpr int KS = 3, VS = 3;           // ring stages
  static constexpr int V_OFF = KS * KT_BYTES;
  static constexpr int LDS_BYTES = KS * KT_BYTES + VS * VT_BYTES;
  static constexpr int KR_DMA = KR_BYTES / 1024;
  static constexpr int KP_DMA = (KT_BYTES - KR_BYTES) / 1024;
  static constexpr int K_DMA = KR_DMA + KP_DMA;
  static constexpr int V_DMA = VT_BYTES / 1024;
  static constexpr int KW = K_DMA / NW, VW = V_DMA / NW;  // DMAs per wave per tile
  static constexpr bool ALIGNED = KR_DMA % NW == 0;
  __host__ __device__ static constexpr int kregion(int n) { return n < KR_DMA ? 0 : 1; }
  static_assert(KR_BYTES % 1024 == 0 && KT_BYTES % 1024 == 0 && VT_BYTES % 1024 == 0, "DMA blocks");
  static_assert(K_DMA % NW == 0 && V_DMA % NW == 0, "even DMA split");
  static_assert(KW + VW < 64, "vmcnt field");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(NW * RW * DV * 2 <= LDS_BYTES, "output staging fits");
  static_assert(NW * DK * 4 <= VT_BYTES, "Q rotation rows fit the third V stage");
  static_assert(DK % 16 == 0 && DV % 32 == 0 && RCH % 2 == 0 && VC >= 16, "tiling");
};

using namespace prefill;

template <int DK, int DV, int G, int RCH>
__global__ __launch_bounds__(NT, 1) void prefill_mfma1w_kernel(PrefillArgs a, int n_qt,
                                                               int contig) {
  using C = Cfg1<DK, DV, G, RCH>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS_BYTES];
  // Only MFMAs read or write the accumulators: this asm operand lets the
  // compiler place them in AGPRs (the other half of the register file).
  {
    int z = 0;
    asm volatile("; accumulators in AGPRs %0" : "+a"(z));
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, h = lane >> 5;  // this lane's row; half of the k range
  const int T = a.T, W = a.window;
  const int n_wg = n_qt * a.Hkv * a.B;
  int grp, qt;
  block_tile((int)blockIdx.x, n_wg, n_qt, contig, grp, qt);
  const int kvh = grp % a.Hkv, b = grp / a.Hkv;
  const int p0 = qt * C::PW;

  // This lane's row: wave w takes head group w % NHG (HW heads) and position
  // block w / NHG (PPW positions); row r32 is head r32 / PPW of the group at
  // position r32 % PPW of the block.
  const int hg = wave % C::NHG, pb = wave / C::NHG;
  const int head = kvh * G + hg * C::HW + r32 / C::PPW;
  const int wlo = p0 + pb * C::PPW;
  const int pos = wlo + r32 % C::PPW;
  const bool valid = pos < T;
  const int whi = wlo + C::PPW - 1;

  const int kv_lo = (W > 0) ? max(0, p0 - W + 1) : 0;
  const int kv_hi = min(T, p0 + C::PW);
  const int kb_lo = kv_lo / BN;
  const int kb_hi = (kv_hi + BN - 1) / BN;
  const int n_tiles = kb_hi - kb_lo;

  // ---- DMA sources -------------------------------------------------------------
  const int64_t v_tok = a.v_tok ? a.v_tok : (int64_t)a.Hkv * DV;
  const int64_t v_head = a.v_head ? a.v_head : DV;
  const int krow = a.Hkv * DK * 2, vrow = (int)(v_tok * 2);  // bytes per token
  const bool rot_q = RCH > 0 && a.rope_q;
  const bool krot_ws = RCH > 0 && a.rope_k;  // rotated dims from the workspace
  const int rrow = krot_ws ? a.Hkv * RCH * 16 : krow;
  const u32x4 kdesc = buffer_desc((const char*)a.k + ((int64_t)b * T * a.Hkv + kvh) * DK * 2,
                                  (T - 1) * krow + DK * 2);
  const u32x4 vdesc = buffer_desc((const char*)a.v + ((int64_t)b * T * v_tok + kvh * v_head) * 2,
                                  (T - 1) * vrow + DV * 2);
  const u32x4 rdesc =
      krot_ws ? buffer_desc((const char*)a.k_rot + ((int64_t)b * T * a.Hkv + kvh) * RCH * 16,
                            (T - 1) * rrow + RCH * 16)
              : kdesc;

  // Block n (n = i*NW + wave) of a tile covers 64 chunks; this lane's chunk
  // offset inside tile row 0 is fixed, a tile adds j0 * row stride.
  uint32_t koff[C::KW], voff[C::VW];
#pragma unroll
  for (int i = 0; i < C::KW; ++i) {
    const int n = i * NW + wave;
    koff[i] = n < C::KR_DMA ? k_rot_dma_off<RCH>(n, lane, rrow)
                            : k_plain_dma_off<RCH, C::NP>(n - C::KR_DMA, lane, krow);
  }
#pragma unroll
  for (int i = 0; i < C::VW; ++i) voff[i] = v_dma_off<C::VC>(i * NW + wave, lane, vrow);
  // Tiles past the range go out with a descriptor of 0 records: they return
  // zeros without touching memory, so every iteration issues the same number
  // of DMAs and one vmcnt value covers every wait.
  // Per-tile descriptors: the tile's first row becomes the base, so each DMA
  // takes the lane's fixed offset; a tile past the range gets 0 records.
  const uint32_t ktot = (T - 1) * krow + DK * 2, rtot = (T - 1) * rrow + RCH * 16;
  const uint32_t vtot = (T - 1) * vrow + DV * 2;
  auto tdesc = [&](u32x4 d, uint32_t off, uint32_t total, bool in) -> u32x4 {
    const uint64_t base = (((uint64_t)(d[1] & 0xffffu) << 32) | d[0]) + off;
    return u32x4{(uint32_t)base, (uint32_t)(base >> 32) & 0xffffu, in ? total - off : 0u, d[3]};
  };
  auto dma_k1 = [&](int kb, int stage, int i) {
    const int j0 = kb * BN;
    const uint32_t st = lds_addr(lds) + stage * C::KT_BYTES;
    const bool in = kb < kb_hi;
    const int n = i * NW + wave;
    const int reg = C::ALIGNED ? C::kregion(i * NW) : C::kregion(n);
    if (reg == 0)
      dma16(tdesc(rdesc, in ? j0 * rrow : 0u, rtot, in), st + n * 1024, koff[i]);
    else
      dma16(tdesc(kdesc, in ? j0 * krow : 0u, ktot, in), st + n * 1024, koff[i]);
  };
  auto dma_v1 = [&](int kb, int stage, int i) {
    const int j0 = kb * BN;
    const uint32_t st = lds_addr(lds) + C::V_OFF + stage * C::VT_BYTES;
    const bool in = kb < kb_hi;
    dma16(tdesc(vdesc, in ? j0 * vrow : 0u, vtot, in), st + (i * NW + wave) * 1024, voff[i]);
  };
  auto dma_k = [&](int kb, int stage) {
#pragma unroll
    for (int i = 0; i < C::KW; ++i) dma_k1(kb, stage, i);
  };
  auto dma_v = [&](int kb, int stage) {
#pragma unroll
    for (int i = 0; i < C::VW; ++i) dma_v1(kb, stage, i);
  };

  // ---- prologue: K(0), V(0) around the Q load, then K(1), K(2) ---------------
  if (n_tiles > 0) {
    dma_k(kb_lo, 0);
    dma_v(kb_lo, 0);
  }
  bf16x8 qf[DK / 16];  // Q^T operand: step s covers dims 16s + 8h .. +7 of the row
  {
    const int prow = valid ? pos : T - 1;
    // Q's rotation by angle addition: the wave builds the (cos, sin) row of
    // its first position in fp64 in its slot of the third V stage (first
    // refilled in iteration 1, after barriers), and each lane turns that row
    // further by its offset d = prow - base (< 32) from it.
    const int base = min(wlo, T - 1);
    lds_float2* slot =
        (lds_float2*)((lds_u8*)lds + C::V_OFF + 2 * C::VT_BYTES + wave * 2048);
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
      wait_vm<0>();  // Q landed (and K(0), V(0) before it)
      rotate_q_chunks<RCH / 2>(qw, slot, dcs, h);
    }
    // Q^T is only ever an MFMA operand, so it lives in the AGPRs the O
    // accumulator (DV/2) and the QK result (16) leave free; the rest stays in
    // VGPRs. Left to itself the allocator spreads Q over both files and copies
    // each step's operand into place before its MFMA (~130 extra moves per
    // tile on the 512-dim keys, in the wave's one issue stream). With every
    // key dim rotated the extra K addressing leaves no VGPRs for that split:
    // there Q stays in VGPRs.
    constexpr int QA0 = (256 - DV / 2 - 16) / 4 < DK / 16 ? (256 - DV / 2 - 16) / 4 : DK / 16;
    constexpr int QA = RCH == DK / 8 ? 0 : QA0;
#pragma unroll
    for (int s = 0; s < DK / 16; ++s) {
      qf[s] = __builtin_bit_cast(bf16x8, valid ? qw[s] : u32x4{});
      // rotated before the next DMAs go out
      if (s < QA)
        asm volatile("" : "+a"(qf[s]));
      else
        asm volatile("" : "+v"(qf[s]));
    }
  }
  if (n_tiles > 0) {
    dma_k(kb_lo + 1, 1);
    dma_k(kb_lo + 2, 2);
    wait_vm<C::KW>();  // K(0), V(0), K(1) landed; K(2) may be in flight
    lds_barrier();
  }

  // ---- operand addressing ----------------------------------------------------
  // K operand of step s: key r32, chunk 2s + h of its region row, stored at
  // chunk (2s + h) ^ x (x = r32 & M): byte 32s ^ 16(h ^ x) of the row.
  constexpr int RW_ = RCH > 0 ? RCH : 16, PW_ = C::NP > 0 ? C::NP : 16;
  const int kr_row = r32 * RW_ * 16, kp_row = C::KR_BYTES + r32 * PW_ * 16;
  const int kxr = 16 * (h ^ (r32 & Swz<RW_>::M)), kxp = 16 * (h ^ (r32 & Swz<PW_>::M));
  // V^T operand, transposing reads: in 16-lane group gi (h = gi >> 1, dim
  // block db = gi & 1), lane 4r + c reads dims 32dt + 16db + 4c .. +3 of key
  // 16j + 8hs + 4h + r, whose chunk 4dt + y (y = 2db + (c >> 1)) sits at
  // 4(dt ^ r) + y: byte 64((dt & 3) ^ r) + 256(dt >> 2) + 16y + 8(c & 1).
  int v_row, vx;
  {
    const int li = lane & 15, gi = lane >> 4, r = li >> 2, c = li & 3;
    const int y = 2 * (gi & 1) + (c >> 1);
    v_row = (4 * h + r) * C::VC * 16 + (y << 4) + ((c & 1) << 3);
    vx = r << 6;
  }
  struct Addr {
    const lds_u8 *kr, *kp, *v;
    int kxr, kxp, vx;
  };
  // Row bases of K stage sk and V stage sv; the masks pass through an empty
  // asm so the per-read XORs are neither hoisted nor folded into registers.
  auto addr = [&](int sk, int sv) {
    const lds_u8* kst =
        (const lds_u8*)lds + __builtin_amdgcn_readfirstlane(sk * C::KT_BYTES);
    const lds_u8* vst =
        (const lds_u8*)lds + __builtin_amdgcn_readfirstlane(C::V_OFF + sv * C::VT_BYTES);
    Addr ad{kst + kr_row, kst + kp_row, vst + v_row, kxr, kxp, vx};
    asm volatile("" : "+v"(ad.kxr), "+v"(ad.kxp), "+v"(ad.vx));
    return ad;
  };
  constexpr int NS = DK / 16;                 // QK MFMAs per tile
  constexpr int NDT = DV / 32, NPV = 2 * NDT;  // P.V MFMAs per tile
  auto kread = [&](const Addr& ad, int s) {
    return k_operand<RCH>(ad.kr, ad.kp, ad.kxr, ad.kxp, s);
  };
  auto vread = [&](const Addr& ad, int i) { return vt_operand<NDT, C::VC>(ad.v, ad.vx, i); };

  // ---- state -------------------------------------------------------------------
  const unsigned wcap = (W > 0) ? (unsigned)W : 0x80000000u;
  f32x16 oacc[NDT];
#pragma unroll
  for (int d = 0; d < NDT; ++d) oacc[d] = f32x16{};
  // S^T of the tile whose softmax runs next (sc; element e holds key
  // 8(e/4) + 4h + (e%4)) and of the tile whose QK runs in the current stream
  // (sn). P^T operands of the tile whose P.V is in the stream (pop) and of the
  // tile whose softmax is in the stream (pn). The softmax of sc runs in
  // SliceSoftmax::NSL slices with its scaled scores in stt and probabilities
  // in sp.
  f32x16 sc = f32x16{}, sn = f32x16{};
  bf16x8 pop[2] = {bf16x8{}, bf16x8{}}, pn[2];
  SliceSoftmax sm(a.scale);
  float sp[16], stt[16];
  constexpr int NSL = SliceSoftmax::NSL;
  auto sm_slice = [&](auto K_) { sm.slice<decltype(K_)::value>(sc, stt, sp, pn); };

  // One stream: P.V of the tile in pop (V at av) and QK of the next tile (K
  // at ak, into sn), MFMAs interleaved (P.V first for PV_ ops, then QK), with
  // the softmax slices of sc spread between them when SM_. Operand reads run
  // OD-1 MFMAs ahead in a ring of OD registers; `side` runs after the second
  // MFMA (the next tiles' DMA issue).
  constexpr int OD = 4;
  bf16x8 ob[OD];
  // `side(j)` runs after MFMA j + 2 for j < NSIDE: the tile DMAs, one DMA
  // group per MFMA so their issue never holds up the matrix pipe for long.
  constexpr int NSIDE = C::KW + C::VW;
  auto phase = [&](auto PV_, auto QK_, auto SM_, const Addr& av, const Addr& ak, auto&& side) {
    constexpr bool do_pv = decltype(PV_)::value, do_qk = decltype(QK_)::value;
    constexpr bool do_sm = decltype(SM_)::value;
    constexpr int lo = do_pv ? 0 : NPV, hi = do_qk ? NPV + NS : NPV;
    constexpr int nops = hi - lo;
    auto rd = [&](int i) { return i < NPV ? vread(av, i) : kread(ak, i - NPV); };
    if constexpr (nops == 0) {
      static_for<0, NSIDE>([&](auto J_) { side(J_); });
      if constexpr (do_sm) static_for<0, NSL>([&](auto K_) { sm_slice(K_); });
    } else {
#pragma unroll
      for (int i = 0; i < OD - 1 && i < nops; ++i) ob[i] = rd(lo + i);
      static_for<0, nops>([&](auto I_) {
        constexpr int i = lo + decltype(I_)::value, n = decltype(I_)::value;
        if constexpr (n >= 2 && n < 2 + NSIDE) side(IC<n - 2>{});
        if constexpr (n + OD - 1 < nops) ob[(n + OD - 1) % OD] = rd(i + OD - 1);
        const bf16x8 op = ob[n % OD];
        if constexpr (i < NPV)
          oacc[i % NDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, pop[i / NDT], oacc[i % NDT], 0, 0, 0);
        else
          sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, qf[i - NPV], i == NPV ? f32x16{} : sn, 0, 0, 0);
        if constexpr (do_sm) {
          // softmax slices k with k * nops / NSL landing on this MFMA
          static_for<0, NSL>([&](auto K_) {
            constexpr int k = decltype(K_)::value;
            if constexpr ((k * nops) / NSL == n) sm_slice(K_);
          });
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      static_for<(nops > 2 ? (nops - 2 < NSIDE ? nops - 2 : NSIDE) : 0), NSIDE>(
          [&](auto J_) { side(J_); });
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  auto nothing = [](auto) {};

  // Before the softmax of tile kb: tiles crossing this wave's diagonal or
  // window edge (or outside its band) get the per-score mask.
  auto mask = [&](int kb) { mask_edge_tile(sc, kb * BN, wlo, whi, W, pos, h, wcap); };
  // After a stream with a softmax: fold it into l and O, hand its P^T on.
  auto settle = [&] {
    sm.fold();
    if (sm.rescale) {
#pragma unroll
      for (int d = 0; d < NDT; ++d) oacc[d] *= sm.alpha;
    }
    pop[0] = pn[0];
    pop[1] = pn[1];
  };

  // ---- main loop ---------------------------------------------------------------
  // Iteration t: mask S(t) | stream: P.V(t-1), QK(t+1), softmax(t) in slices |
  // settle | wait, barrier. It issues K(t+3) and V(t+1): their stages held
  // K(t) (read by QK(t) in iteration t-1) and V(t-2) (read in iteration t-1).
  // Before its barrier a wave waits until all but its newest DMA group
  // landed, so K(t+2) and V(t) are ready for iteration t+1.
  // j-th DMA of iteration t's issue (K blocks first, then V).
  auto issue = [&](int t, auto J_) {
    constexpr int j = decltype(J_)::value;
    if constexpr (j < C::KW)
      dma_k1(kb_lo + t + 3, (t + 3) % 3, j);
    else
      dma_v1(kb_lo + t + 1, (t + 1) % 3, j - C::KW);
  };
  if (n_tiles > 0) {
    {  // QK(0); iteration 0 refills its stage with K(3): all reads end first
      const Addr a0 = addr(0, 0);
      phase(F_{}, T_{}, F_{}, a0, a0, nothing);
      sc = sn;
      lds_barrier();
    }
    int t = 0;
    // iteration 0: QK(1) and softmax(0), no P.V yet
    mask(kb_lo);
    if (n_tiles > 1)
      phase(F_{}, T_{}, T_{}, addr(1, 0), addr(1, 0), [&](auto J_) { issue(0, J_); });
    else
      phase(F_{}, F_{}, T_{}, addr(0, 0), addr(0, 0), [&](auto J_) { issue(0, J_); });
    settle();
    sc = sn;
    wait_vm<C::KW + C::VW>();
    lds_barrier();
    for (t = 1; t + 1 < n_tiles; ++t) {
      mask(kb_lo + t);
      phase(T_{}, T_{}, T_{}, addr((t + 1) % 3, (t - 1) % 3), addr((t + 1) % 3, (t - 1) % 3),
            [&](auto J_) { issue(t, J_); });
      settle();
      sc = sn;
      wait_vm<C::KW + C::VW>();
      lds_barrier();
    }
    if (n_tiles > 1) {  // iteration n-1: P.V(n-2) and softmax(n-1)
      t = n_tiles - 1;
      mask(kb_lo + t);
      phase(T_{}, F_{}, T_{}, addr(0, (t - 1) % 3), addr(0, (t - 1) % 3), [&](auto J_) { issue(t, J_); });
      settle();
      wait_vm<C::KW + C::VW>();
      lds_barrier();
    }
    {  // P.V(n-1)
      const Addr an = addr(0, (n_tiles - 1) % 3);
      phase(T_{}, F_{}, F_{}, an, an, nothing);
    }
  }

#ifdef ATTN_DEBUG_TILES
  if (a.dbg_visits && lane == 0) {  // every wave computes every staged tile
    atomicAdd(a.dbg_visits, (unsigned long long)(n_tiles > 0 ? n_tiles : 0));
    if (wave == 0) atomicAdd(a.dbg_visits + 1, (unsigned long long)(n_tiles > 0 ? n_tiles : 0));
  }
#endif
  // ---- epilogue: O = O^T / l, bf16, staged through LDS ---------------------------
  wait_vm<0>();
  lds_barrier();
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sm.l_run),
                                                     __float_as_uint(sm.l_run), false, false);
    sm.l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  __attribute__((address_space(3))) unsigned char* ost =
      (__attribute__((address_space(3))) unsigned char*)lds + wave * (RW * DV * 2);
  stage_o<NDT>(ost, oacc, valid ? 1.f / sm.l_run : 0.f, r32, h);
  const int64_t o_tok = a.o_tok ? a.o_tok : (int64_t)a.Hq * DV;
  const int64_t o_head = a.o_head ? a.o_head : DV;
  // row r of a wave: head group hg's head r / PPW at position wlo + r % PPW
  store_o<DV, RW>(ost, lane, [&](int row) -> uint16_t* {
    const int p = wlo + row % C::PPW;
    const int hd = kvh * G + hg * C::HW + row / C::PPW;
    return p < T ? (uint16_t*)a.o + ((int64_t)b * T + p) * o_tok + hd * o_head : nullptr;
  });
}

template <int DK, int DV, int G, int RCH>
hipError_t launch_one(const PrefillArgs& a, hipStream_t st) {
  using C = Cfg1<DK, DV, G, RCH>;
  const int n_qt = (a.T + C::PW - 1) / C::PW;
  const int64_t n = (int64_t)n_qt * a.Hkv * a.B;
  if (n == 0) return hipSuccess;
  if (n > 0x7fffffff) return hipErrorInvalidValue;
  // Sliding-window tiles reuse their neighbours' K/V: keep neighbours on one
  // XCD. Causal tiles are grouped per XCD by (batch, KV head) in the kernel.
  const int contig = (a.window > 0 && a.window < a.T) ? 1 : 0;
  hipLaunchKernelGGL((prefill_mfma1w_kernel<DK, DV, G, RCH>), dim3((unsigned)n), dim3(NT), 0, st,
                     a, n_qt, contig);
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

hipError_t launch_prefill_mfma1w(const PrefillArgs& a, hipStream_t st) {
  if (a.Dk == 512 && a.Dv == 256) return dispatch_g<512, 256>(a, st);
  return hipErrorNotSupported;
}

}  // namespace attn
