// prefill_mfma2g.hip — the sliding-window / causal GQA prefill of the local
// layers (256-dim heads, 2 query heads per KV head) on gfx950 bf16 matrix
// cores, two workgroups per CU.
//
// What it computes is what prefill_mfma.hip computes ("Gemma 4: End-to-End
// Architecture Walkthrough", Phase 3 sections 3a-3c; "Gemma 4 Architecture
// Reference", "Attention Architecture" and "Positional Encoding"):
// softmax(scale * rope(q) rope(k)^T + mask) v with the local window, q/k
// rounded to bf16 after rotation, P to bf16 before P.V, fp32 accumulation.
// The wave-level tiling is the same (32 query rows per wave, S^T = K Q^T and
// O^T = V^T P^T on 32x32x16 MFMAs, DMA-fed XOR-swizzled K/V tiles, lazy
// rescaling, window-aware tile skipping, output staged through LDS).
//
// What differs, for CDNA4: a workgroup is 4 waves (128 rows, 64 positions),
// its K and V rings have 2 stages each (64 KB), and each wave keeps 256
// registers, so two workgroups share a CU. With one 8-wave workgroup per CU
// every CU loads Q, turns it and stores O at the same moment, and nothing
// hides those phases (about a third of the kernel's time on the local
// workload). Two independent workgroups per CU drift apart, so one's
// prologue and epilogue run under the other's tile loop: 630-645 TFLOP/s
// against 575-590 for the 8-wave kernel on the local prefill workload.
//  * Split rings: K(t) is read by the QK of matrix phase t-1, V(t) by the
//    P.V of phase t, so iteration m issues K(m+2) and V(m+1) into the stages
//    freed by phase m-1; each tile then has two phases of flight, as with a
//    4-stage joint ring, in half the LDS.
//  * Two barriers per tile: softmax | barrier | P.V(m), QK(m+1) | barrier.
//    The wave that shares a SIMD belongs to the other workgroup, which
//    fills this one's softmax phase with its MFMAs and vice versa.
#include <type_traits>

#include "attn_common.h"
#include "kernels.h"
#include "prefill_common.h"

namespace attn {
namespace {

constexpr int RW = 32;  // query rows per wave
constexpr int BN = 32;  // keys per tile

template <int DK, int DV, int G, int RCH>
struct Cfg2 {
  static constexpr int NW = 4;
  static_assert(DK <= 256 && DV <= 256, "heads up to 256 dims");
  static constexpr int NT = NW * 64;
  static constexpr int ROWS = NW * RW;
  static constexpr int PW = ROWS / G;
  static constexpr int NC = DK / 8;
  static constexpr int NP = NC - RCH;
  static constexpr int KR_BYTES = BN * RCH * 16;
  static constexpr int KT_BYTES = BN * NC * 16;
  static constexpr int VC = DV / 8;
  static constexpr int VT_BYTES = BN * VC * 16;
  static constexpr int KS = 2, VS = 2;  // ring stages
  static constexpr int V_BASE = KS * KT_BYTES;
  static constexpr int LDS_BYTES = KS * KT_BYTES + VS * VT_BYTES;
  static constexpr int KR_DMA = KR_BYTES / 1024;
  static constexpr int KP_DMA = (KT_BYTES - KR_BYTES) / 1024;
  static constexpr int K_DMA = KR_DMA + KP_DMA, V_DMA = VT_BYTES / 1024;
  static constexpr int KW = K_DMA / NW, VW = V_DMA / NW;  // DMAs per wave per tile
  static_assert(KR_DMA % NW == 0 && KP_DMA % NW == 0 && V_DMA % NW == 0, "uniform DMAs");
  static_assert(KW + VW < 64, "vmcnt field");
  static_assert(LDS_BYTES <= 80 * 1024, "two workgroups per CU");
  static_assert(ROWS * DV * 2 <= LDS_BYTES, "output staging fits");
  static_assert(ROWS % G == 0 && NW % G == 0, "rows split evenly over the heads");
  static_assert(VC >= 16, "V rows swizzle over 16 chunk groups");
};

using namespace prefill;

template <int DK, int DV, int G, int RCH>
__global__ __launch_bounds__((Cfg2<DK, DV, G, RCH>::NT), 2) void prefill_mfma2g_kernel(
    PrefillArgs a, int n_qt, int contig) {
  using C = Cfg2<DK, DV, G, RCH>;
  constexpr int NW = C::NW;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, h = lane >> 5;
  const int T = a.T, W = a.window;
  const int n_wg = n_qt * a.Hkv * a.B;
  const int L = contig ? xcd_contiguous((int)blockIdx.x, n_wg) : (int)blockIdx.x;
  const int grp = L / n_qt;
  const int qt = n_qt - 1 - (L % n_qt);
  const int kvh = grp % a.Hkv, b = grp / a.Hkv;
  const int p0 = qt * C::PW;

  const int head = kvh * G + wave % G;
  const int wlo = p0 + RW * (wave / G);
  const int pos = wlo + r32;
  const bool valid = pos < T;
  const int whi = wlo + RW - 1;

  const int kv_lo = (W > 0) ? max(0, p0 - W + 1) : 0;
  const int kv_hi = min(T, p0 + C::PW);
  const int kb_lo = kv_lo / BN;
  const int kb_hi = (kv_hi + BN - 1) / BN;

  const int krow = a.Hkv * DK * 2, vrow = a.Hkv * DV * 2;
  const bool rot_q = RCH > 0 && a.rope_q;
  const bool krot_ws = RCH > 0 && a.rope_k;
  const int rrow = krot_ws ? a.Hkv * RCH * 16 : krow;
  const u32x4 kdesc = buffer_desc((const char*)a.k + ((int64_t)b * T * a.Hkv + kvh) * DK * 2,
                                  (T - 1) * krow + DK * 2);
  const u32x4 vdesc = buffer_desc((const char*)a.v + ((int64_t)b * T * a.Hkv + kvh) * DV * 2,
                                  (T - 1) * vrow + DV * 2);
  const u32x4 rdesc =
      krot_ws ? buffer_desc((const char*)a.k_rot + ((int64_t)b * T * a.Hkv + kvh) * RCH * 16,
                            (T - 1) * rrow + RCH * 16)
              : kdesc;

  // K blocks n = i*NW + wave: rotated region then plain region; V blocks alike.
  uint32_t koff[C::KW], voff[C::VW];
#pragma unroll
  for (int i = 0; i < C::KW; ++i) {
    const int n = i * NW + wave;
    koff[i] = n < C::KR_DMA ? k_rot_dma_off<RCH>(n, lane, rrow)
                            : k_plain_dma_off<RCH, C::NP>(n - C::KR_DMA, lane, krow);
  }
#pragma unroll
  for (int i = 0; i < C::VW; ++i) voff[i] = v_dma_off<C::VC>(i * NW + wave, lane, vrow);
  auto dma_k = [&](int kb, int stage) {
    const int j0 = kb * BN;
    const uint32_t st = lds_addr(lds) + stage * C::KT_BYTES;
    const uint32_t far = kb < kb_hi ? 0u : 0x80000000u;
#pragma unroll
    for (int i = 0; i < C::KW; ++i) {
      const int n = i * NW + wave;
      if (i * NW < C::KR_DMA)  // same region for every wave (KR_DMA % NW == 0)
        dma16(rdesc, st + n * 1024, (koff[i] + j0 * rrow) | far);
      else
        dma16(kdesc, st + n * 1024, (koff[i] + j0 * krow) | far);
    }
  };
  auto dma_v = [&](int kb, int stage) {
    const int j0 = kb * BN;
    const uint32_t st = lds_addr(lds) + C::V_BASE + stage * C::VT_BYTES;
    const uint32_t far = kb < kb_hi ? 0u : 0x80000000u;
#pragma unroll
    for (int i = 0; i < C::VW; ++i)
      dma16(vdesc, st + (i * NW + wave) * 1024, (voff[i] + j0 * vrow) | far);
  };

  // ---- prologue: K(0), K(1), V(0) in flight around the Q load --------------
  const int n_tiles = kb_hi - kb_lo;
  if (n_tiles > 0) {
    dma_k(kb_lo, 0);
    dma_k(kb_lo + 1, 1);
    dma_v(kb_lo, 0);
  }

  bf16x8 qf[DK / 16];
  {
    const int prow = valid ? pos : T - 1;
    // Q's rotation by angle addition: the wave builds the (cos, sin) row of
    // its first position in fp64 in its slot of the second V stage (which
    // iteration 0 refills from this same wave), and each lane turns that row
    // further by its offset d = prow - base (0..31) from it.
    const int base = min(wlo, T - 1);
    lds_float2* slot =
        (lds_float2*)((lds_u8*)lds + C::V_BASE + C::VT_BYTES + wave * 1024);
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
      wait_vm<0>();  // Q landed (and the K/V DMAs before it)
      rotate_q_chunks<RCH / 2>(qw, slot, dcs, h);
    }
#pragma unroll
    for (int s = 0; s < DK / 16; ++s) {
      u32x4 w = valid ? qw[s] : u32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }
  if (n_tiles > 0) {
    wait_vm<C::KW + C::VW>();  // K(0) landed (K(1), V(0) may be in flight)
    lds_barrier();
  }

  const float c2 = fmaxf(a.scale * kLog2e, 1e-30f);
  const unsigned wcap = (W > 0) ? (unsigned)W : 0x80000000u;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) oacc[d] = f32x16{};

  constexpr int RW_ = RCH > 0 ? RCH : 16, PW_ = C::NP > 0 ? C::NP : 16;
  const int kr_row = r32 * RW_ * 16, kp_row = C::KR_BYTES + r32 * PW_ * 16;
  const int kxr = 16 * (h ^ (r32 & Swz<RW_>::M)), kxp = 16 * (h ^ (r32 & Swz<PW_>::M));
  int v_row, vx;
  {
    const int li = lane & 15, gi = lane >> 4, r = li >> 2, c = li & 3;
    const int y = 2 * (gi & 1) + (c >> 1);
    v_row = (4 * h + r) * C::VC * 16 + (y << 4) + ((c & 1) << 3);
    vx = r << 6;
  }

  // A wave computes a tile only if it holds a key one of its rows may see
  // (a wave whose rows all lie past T, the padding of the last query tile,
  // computes none).
  auto live = [&](int kb) {
    const int j0 = kb * BN;
    return wlo < T && j0 <= whi && !(W > 0 && j0 + BN - 1 <= wlo - W);
  };

  constexpr int OD = 4;
  constexpr int NS = DK / 16;
  constexpr int NDT = DV / 32, NPV = 2 * NDT;
  struct Addr {
    const lds_u8 *kr, *kp, *v;
    int kxr, kxp, vx;
  };
  // K stage of tile t and V stage of tile t.
  auto kst = [&](int t) {
    return (const lds_u8*)lds + __builtin_amdgcn_readfirstlane((t & 1) * C::KT_BYTES);
  };
  auto vst = [&](int t) {
    return (const lds_u8*)lds + __builtin_amdgcn_readfirstlane(C::V_BASE + (t & 1) * C::VT_BYTES);
  };
  auto addr = [&](const lds_u8* ks, const lds_u8* vs) {
    Addr ad{ks + kr_row, ks + kp_row, vs + v_row, kxr, kxp, vx};
    asm volatile("" : "+v"(ad.kxr), "+v"(ad.kxp), "+v"(ad.vx));
    return ad;
  };
  auto kread = [&](const Addr& ad, int s) {
    return k_operand<RCH>(ad.kr, ad.kp, ad.kxr, ad.kxp, s);
  };
  auto vread = [&](const Addr& ad, int i) { return vt_operand<NDT, C::VC>(ad.v, ad.vx, i); };

  f32x16 sc = f32x16{};
  bf16x8 pop[2];
  bf16x8 ob[OD];

  // P.V of one tile (V from av) then QK of the next (K from ak).
  auto mfma_stream = [&](auto PV_, auto QK_, const Addr& av, const Addr& ak) {
    constexpr bool do_pv = decltype(PV_)::value, do_qk = decltype(QK_)::value;
    constexpr int lo = do_pv ? 0 : NPV, hi = do_qk ? NPV + NS : NPV;
    auto rd = [&](int i) { return i < NPV ? vread(av, i) : kread(ak, i - NPV); };
#pragma unroll
    for (int i = 0; i < OD - 1; ++i)
      if (lo + i < hi) ob[i] = rd(lo + i);
#pragma unroll
    for (int i = lo; i < hi; ++i) {
      if (i + OD - 1 < hi) ob[(i - lo + OD - 1) % OD] = rd(i + OD - 1);
      const bf16x8 op = ob[(i - lo) % OD];
      if (i < NPV)
        oacc[i % NDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, pop[i / NDT], oacc[i % NDT], 0, 0, 0);
      else
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, qf[i - NPV], i == NPV ? f32x16{} : sc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

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
    float pv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) pv[e] = fast_exp2(fmaf(sv[e], c2, -m_use));
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ps += pv[e];
    l_run += ps;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f32x4 lo = {pv[8 * j], pv[8 * j + 1], pv[8 * j + 2], pv[8 * j + 3]};
      const f32x4 hi = {pv[8 * j + 4], pv[8 * j + 5], pv[8 * j + 6], pv[8 * j + 7]};
      pop[j] = __builtin_shufflevector(__builtin_convertvector(lo, bf16x4),
                                       __builtin_convertvector(hi, bf16x4), 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };

  // ---- main loop -------------------------------------------------------------
  // Iteration m: issue K(m+2) and V(m+1) into the stages whose readers (the
  // matrix phase m-1) passed the last barrier | softmax(m) | barrier (V(m),
  // K(m+1) landed) | P.V(m) then QK(m+1) | barrier. Each tile has two
  // phases of flight. The other workgroup on the CU fills this one's gaps.
  if (n_tiles > 0) {
    if (live(kb_lo)) {
      const Addr a0 = addr(kst(0), vst(0));
      mfma_stream(F_{}, T_{}, a0, a0);
    }
    lds_barrier();  // every wave is done with K(0) before K(2) overwrites it
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
    dma_k(kb + 2, t & 1);
    dma_v(kb + 1, (t + 1) & 1);
    if (lv)
      softmax(kb);
    else
      pop[0] = pop[1] = bf16x8{};
    wait_vm<C::KW + C::VW>();
    lds_barrier();
    if (lv || lv_next) mfma_stream(T_{}, T_{}, addr(kst(t + 1), vst(t)), addr(kst(t + 1), vst(t)));
    lds_barrier();
  }
  // The last tile has no next one: no DMAs (every later tile is past the
  // range), and its matrix phase is P.V alone.
  if (n_tiles > 0) {
    const int t = n_tiles - 1, kb = kb_lo + t;
    const bool lv = live(kb);
#ifdef ATTN_DEBUG_TILES
    dbg_live += lv;
#endif
    if (lv)
      softmax(kb);
    else
      pop[0] = pop[1] = bf16x8{};
    wait_vm<0>();
    lds_barrier();
    if (lv) mfma_stream(T_{}, F_{}, addr(kst(t + 1), vst(t)), addr(kst(t + 1), vst(t)));
    lds_barrier();
  }

#ifdef ATTN_DEBUG_TILES
  if (a.dbg_visits && lane == 0) {
    atomicAdd(a.dbg_visits, (unsigned long long)dbg_live);
    if (wave == 0) atomicAdd(a.dbg_visits + 1, (unsigned long long)n_tiles);
  }
#endif
  // ---- epilogue: O = O^T / l, bf16, through LDS ------------------------------
  wait_vm<0>();
  lds_barrier();
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                     __float_as_uint(l_run), false, false);
    l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  __attribute__((address_space(3))) unsigned char* ost =
      (__attribute__((address_space(3))) unsigned char*)lds + wave * (RW * DV * 2);
  stage_o<DV / 32>(ost, oacc, valid ? 1.f / l_run : 0.f, r32, h);
  store_o<DV, RW>(ost, lane, [&](int row) -> uint16_t* {
    const int p = wlo + row;
    return p < T ? (uint16_t*)a.o + (((int64_t)b * T + p) * a.Hq + head) * DV : nullptr;
  });
}

template <int DK, int DV, int G, int RCH>
hipError_t launch_2g(const PrefillArgs& a, hipStream_t st) {
  using C = Cfg2<DK, DV, G, RCH>;
  const int n_qt = (a.T + C::PW - 1) / C::PW;
  const int64_t n = (int64_t)n_qt * a.Hkv * a.B;
  if (n == 0) return hipSuccess;
  if (n > 0x7fffffff) return hipErrorInvalidValue;
  const int contig = (a.window > 0 && a.window < a.T) ? 1 : 0;
  hipLaunchKernelGGL((prefill_mfma2g_kernel<DK, DV, G, RCH>), dim3((unsigned)n), dim3(C::NT), 0,
                     st, a, n_qt, contig);
  return hipGetLastError();
}

}  // namespace

// Local-layer shape: 256-dim heads, 2 query heads per KV head; rotation of
// none, a quarter or all of the dims.
hipError_t launch_prefill_mfma2g(const PrefillArgs& a, hipStream_t st) {
  if (a.Dk != 256 || a.Dv != 256 || a.Hq / a.Hkv != 2) return hipErrorNotSupported;
  const int rch = (a.rope_q || a.rope_k) ? (2 * a.rot_pairs) / 8 : 0;
  if (rch == 0) return launch_2g<256, 256, 2, 0>(a, st);
  if (rch == 8) return launch_2g<256, 256, 2, 8>(a, st);
  if (rch == 32) return launch_2g<256, 256, 2, 32>(a, st);
  return hipErrorNotSupported;
}

}  // namespace attn
