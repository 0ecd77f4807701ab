// prefill_kv1w.hip — flash-style causal / sliding-window GQA prefill for
// keys that are also the values (K = V, 512 dims), in one pass over the keys,
// on gfx950 bf16 matrix cores (v_mfma_f32_32x32x16_bf16) with one wave per
// SIMD.
//
// What it computes (Gemma 4 pages): "Gemma 4: End-to-End Architecture
// Walkthrough", Phase 3 — section 3b (global layers without a value
// projection: the attention weights multiply the keys themselves; grouped
// query heads, 512-dim keys), section 3a (causal or windowed visibility) and
// section 3c (p-RoPE on q); "Gemma 4 Technical Report" reader, "Core Model
// Architecture". The caller passes the rotated keys as both k and v and turns
// only q here, so o = softmax(scale * rope(q) k^T + mask) k. q is rounded to
// bf16 after rotation, P to bf16 before P.V; sums are fp32.
//
// Design for CDNA4:
//  * The workgroup and wave layout of the one-wave kernel for 512-dim keys: 4
//    waves, one per SIMD, 32 (head, position) rows each. O^T now spans 512
//    value dims, 256 fp32 registers per lane: the whole AGPR file. Q^T (128
//    registers), the scores and the operand ring share the VGPRs.
//  * One 32-key tile in LDS (32 KB) is the K operand of Q.K^T and, read through
//    ds_read_b64_tr_b16, the V^T operand of P.V. Its 16-byte chunks are
//    XOR-swizzled by f(r) = 4(r & 3) | ((r >> 2) & 3): any 16 consecutive rows
//    land in 16 bank groups (the K operand reads one chunk column of 32 rows),
//    and so do the 4 keys x 2 chunks of each transposing read.
//  * Iteration t runs Q.K^T of tile t (32 MFMAs into the score registers),
//    then P.V of tile t-1 (32 MFMAs) with the softmax of tile t cut into
//    slices between them. Only one score tile is live at a time, which is what
//    leaves room for the 512-dim accumulator.
//  * A 4-stage ring (128 KB): iteration t loads tile t+2 by DMA into the stage
//    that held tile t-2, behind one barrier per iteration; tiles past the
//    range read zeros without memory traffic. The output is staged in the ring
//    and written as whole rows.
//  * Tiles outside the workgroup's band are not visited; a tile crossing one
//    wave's diagonal or window edge is masked per score. O is rescaled only
//    when a row's block max exceeds the max in use by more than 2^8.
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
constexpr int D = 512;                // key and value dims
constexpr int ROW = D * 2;            // bytes per key row in LDS
constexpr int TILE = BN * ROW;        // 32 KB
constexpr int KS = 4;                 // ring stages
constexpr int LDS_BYTES = KS * TILE;  // 128 KB
constexpr int KW = TILE / 1024 / NW;  // 1 KB DMAs (one key row each) per wave per tile
constexpr int NS = D / 16;            // Q.K^T MFMAs per tile
constexpr int NDT = D / 32;           // O^T dim tiles
constexpr int NPV = 2 * NDT;          // P.V MFMAs per tile
static_assert(ROW == 1024 && (TILE / 1024) % NW == 0, "one key row per DMA");
static_assert(NW * RW * D * 2 <= LDS_BYTES, "output staging fits the ring");
static_assert(LDS_BYTES <= 160 * 1024, "LDS");
static_assert(KW < 64, "vmcnt field");

// LDS chunk of key row r that holds the row's chunk c is c ^ kvswz(r).
__device__ __forceinline__ int kvswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

using namespace prefill;
static_assert(RW == 32 && NW == 4, "the row map is for 4 waves of 32 rows");

template <int G>
using Rows = WaveRows<G>;

template <int G, int RCH>
__global__ __launch_bounds__(NT, 1) void prefill_kv1w_kernel(PrefillArgs a, int n_qt,
                                                             int contig) {
  using R = Rows<G>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[LDS_BYTES];
  // Only MFMAs read or write the O accumulators: this asm operand lets the
  // compiler place them in AGPRs.
  {
    int z = 0;
    asm volatile("; accumulators in AGPRs %0" : "+a"(z));
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, h = lane >> 5;  // this lane's row; half of the k range
  const int T = a.T, W = a.window;
  const int n_wg = (int)gridDim.x;
  int grp, qt;
  block_tile((int)blockIdx.x, n_wg, n_qt, contig, grp, qt);
  const int kvh = grp % a.Hkv, b = grp / a.Hkv;
  const int p0 = qt * R::PW;

  // This lane's row: wave w takes head group w % NHG and position block
  // w / NHG; row r32 is head r32 / PPW of the group at position r32 % PPW.
  const int hg = wave % R::NHG, pb = wave / R::NHG;
  const int head = kvh * G + hg * R::HW + r32 / R::PPW;
  const int wlo = p0 + pb * R::PPW;
  const int pos = wlo + r32 % R::PPW;
  const bool valid = pos < T;
  const int whi = wlo + R::PPW - 1;

  const int kv_lo = (W > 0) ? max(0, p0 - W + 1) : 0;
  const int kv_hi = min(T, p0 + R::PW);
  const int kb_lo = kv_lo / BN;
  const int kb_hi = (kv_hi + BN - 1) / BN;
  const int n_tiles = kb_hi - kb_lo;

  // ---- DMA: block n of a tile is its key row n; lane l fetches the row's
  // chunk l ^ kvswz(n), which lands at LDS chunk l of that row.
  const int krow = a.Hkv * D * 2;  // bytes per token
  const u32x4 kdesc =
      buffer_desc((const char*)a.k + ((int64_t)b * T * a.Hkv + kvh) * D * 2, (T - 1) * krow + ROW);
  const uint32_t ktot = (T - 1) * krow + ROW;
  uint32_t koff[KW];
#pragma unroll
  for (int i = 0; i < KW; ++i) {
    const int n = i * NW + wave;
    koff[i] = (uint32_t)(n * krow + 16 * (lane ^ kvswz(n)));
  }
  // Per-tile descriptors: the tile's first row becomes the base; a tile past
  // the range gets 0 records (zeros, no memory traffic), so every iteration
  // issues the same number of DMAs and one vmcnt value covers every wait.
  auto tdesc = [&](uint32_t off, bool in) -> u32x4 {
    const uint64_t base = (((uint64_t)(kdesc[1] & 0xffffu) << 32) | kdesc[0]) + off;
    return u32x4{(uint32_t)base, (uint32_t)(base >> 32) & 0xffffu, in ? ktot - off : 0u, kdesc[3]};
  };
  auto dma_k1 = [&](int kb, int stage, int i) {
    const bool in = kb < kb_hi;
    const uint32_t st = lds_addr(lds) + stage * TILE;
    dma16(tdesc(in ? (uint32_t)(kb * BN) * krow : 0u, in), st + (i * NW + wave) * 1024, koff[i]);
  };
  auto dma_k = [&](int kb, int stage) {
#pragma unroll
    for (int i = 0; i < KW; ++i) dma_k1(kb, stage, i);
  };

  // ---- prologue: K(0) around the Q load, then K(1) -----------------------------
  if (n_tiles > 0) dma_k(kb_lo, 0);
  bf16x8 qf[D / 16];  // Q^T operand: step s covers dims 16s + 8h .. +7 of the row
  {
    const int prow = valid ? pos : T - 1;
    // Q's rotation by angle addition (as in the one-wave kernel): the wave's
    // base row goes to its slot in stage 3, which no DMA touches before
    // iteration 1, two barriers later.
    const int base = min(wlo, T - 1);
    lds_float2* slot = (lds_float2*)((lds_u8*)lds + 3 * TILE + wave * 2048);
    const uint16_t* qrow =
        (const uint16_t*)a.q + (((int64_t)b * T + prow) * a.Hq + head) * D + 8 * h;
    u32x4 qw[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qw[s] = *(const u32x4*)(qrow + 16 * s);
    if (RCH > 0 && a.rope_q) {
      rope_base_row(slot, (int64_t)a.pos0 + base, a.rot_pairs, D, a.log2_theta, lane);
      float dcs[RCH / 2 > 0 ? RCH / 2 : 1][8];
      rope_offsets<RCH / 2>(dcs, prow - base, a.rope_rho, h);
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<0>();  // Q landed (and K(0) before it)
      rotate_q_chunks<RCH / 2>(qw, slot, dcs, h);
    }
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qf[s] = __builtin_bit_cast(bf16x8, valid ? qw[s] : u32x4{});
      asm volatile("" : "+v"(qf[s]));
    }
  }
  if (n_tiles > 0) {
    dma_k(kb_lo + 1, 1);
    wait_vm<KW>();  // K(0) landed; K(1) may be in flight
    lds_barrier();
  }

  // ---- operand addressing ----------------------------------------------------
  // K operand of step s: key r32, chunk 2s + h, stored at (2s + h) ^ f(r32):
  // byte (32 s) ^ kx of the row, kx = 16 (h ^ f(r32)).
  const int k_row = r32 * ROW;
  const int kx = 16 * (h ^ kvswz(r32));
  // V^T operand of P.V step i (key half j = i / NDT, dim tile dt = i % NDT):
  // in 16-lane group gi (h = gi >> 1, db = gi & 1), lane 4r + c reads dims
  // 32dt + 16db + 4c .. +3 of keys R = 16j + 8hs + 4h + r (hs = 0, 1; two
  // transposing reads). That is chunk 4dt + y (y = 2db + (c >> 1)) of row R,
  // stored at (4dt + y) ^ (4r + 2hs + h): byte 64 (dt ^ r) + 16 (y ^ (2hs + h))
  // + 8 (c & 1) of the row, i.e. vrow[hs] + ((64 dt) ^ vx) + 16 KB j.
  int vrow0, vrow1, vx;
  {
    const int li = lane & 15, gi = lane >> 4, r = li >> 2, c = li & 3;
    const int y = 2 * (gi & 1) + (c >> 1);
    vrow0 = (4 * h + r) * ROW + 16 * (y ^ h) + 8 * (c & 1);
    vrow1 = (8 + 4 * h + r) * ROW + 16 * (y ^ (2 + h)) + 8 * (c & 1);
    vx = r << 6;
  }
  struct Addr {
    const lds_u8 *k, *v0, *v1;
    int kx, vx;
  };
  // Bases of the K stage sk and the V stage sv; the masks pass through an
  // empty asm so the per-read XORs are neither hoisted nor folded.
  auto addr = [&](int sk, int sv) {
    const lds_u8* kst = (const lds_u8*)lds + __builtin_amdgcn_readfirstlane(sk * TILE);
    const lds_u8* vst = (const lds_u8*)lds + __builtin_amdgcn_readfirstlane(sv * TILE);
    Addr ad{kst + k_row, vst + vrow0, vst + vrow1, kx, vx};
    asm volatile("" : "+v"(ad.kx), "+v"(ad.vx));
    return ad;
  };
  auto kread = [&](const Addr& ad, int s) -> bf16x8 {
    return *(const lds_bf16x8*)(ad.k + ((32 * s) ^ ad.kx));
  };
  auto vread = [&](const Addr& ad, int i) -> bf16x8 {
    const int j = i / NDT, dt = i % NDT;
    const int off = ((64 * dt) ^ ad.vx) + j * 16 * ROW;
    const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(ad.v0 + off));
    const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(ad.v1 + off));
    return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  // ---- state -------------------------------------------------------------------
  const unsigned wcap = (W > 0) ? (unsigned)W : 0x80000000u;
  f32x16 oacc[NDT];
#pragma unroll
  for (int d = 0; d < NDT; ++d) oacc[d] = f32x16{};
  // S^T of the current tile (element e holds key 8(e/4) + 4h + (e%4)); its
  // softmax runs in SliceSoftmax::NSL slices, in place. P^T operands of the
  // tile whose P.V is in the stream (pop) and of the tile being softmaxed (pn).
  f32x16 sc = f32x16{};
  bf16x8 pop[2] = {bf16x8{}, bf16x8{}}, pn[2] = {bf16x8{}, bf16x8{}};
  SliceSoftmax sm(a.scale);
  constexpr int NSL = SliceSoftmax::NSL;
  auto sm_slice = [&](auto K_) { sm.slice<decltype(K_)::value>(sc, sc, sc, pn); };

  // Before the softmax of tile kb: a tile crossing this wave's diagonal or
  // window edge gets the per-score mask.
  auto mask = [&](int kb) { mask_edge_tile(sc, kb * BN, wlo, whi, W, pos, h, wcap); };

  // One stream: Q.K^T of a tile (K at ak, into sc) when QK_, then P.V of the
  // previous tile (V at av, P^T in pop) when PV_. With SM_ the tile's mask
  // and softmax follow its Q.K^T: between the P.V MFMAs when there are any,
  // after the stream otherwise. Operand reads run OD-1 MFMAs ahead in a ring
  // of OD registers; side(j) (the next tile's DMAs) follows MFMA j + 2.
  constexpr int OD = 4;
  bf16x8 ob[OD];
  auto phase = [&](auto QK_, auto PV_, auto SM_, const Addr& ak, const Addr& av, int kb,
                   auto&& side) {
    constexpr bool do_qk = decltype(QK_)::value, do_pv = decltype(PV_)::value;
    constexpr bool do_sm = decltype(SM_)::value;
    constexpr int lo = do_qk ? 0 : NS, hi = do_pv ? NS + NPV : NS;
    constexpr int nops = hi - lo;
    constexpr int NSIDE = KW;
    constexpr bool sm_in = do_sm && do_qk && do_pv;
    auto rd = [&](int i) { return i < NS ? kread(ak, i) : vread(av, i - NS); };
#pragma unroll
    for (int i = 0; i < OD - 1 && i < nops; ++i) ob[i] = rd(lo + i);
    static_for<0, nops>([&](auto I_) {
      constexpr int n = decltype(I_)::value, i = lo + n;
      if constexpr (n >= 2 && n < 2 + NSIDE) side(IC<n - 2>{});
      if constexpr (n + OD - 1 < nops) ob[(n + OD - 1) % OD] = rd(i + OD - 1);
      const bf16x8 op = ob[n % OD];
      if constexpr (i < NS)
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, qf[i], i == 0 ? f32x16{} : sc, 0, 0, 0);
      else
        oacc[(i - NS) % NDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            op, pop[(i - NS) / NDT], oacc[(i - NS) % NDT], 0, 0, 0);
      if constexpr (sm_in) {
        // the mask after the first two P.V MFMAs (the scores are ready by
        // then), then slice k on P.V MFMA 2 + k (NPV - 2) / NSL
        if constexpr (i == NS + 1) mask(kb);
        static_for<0, NSL>([&](auto K_) {
          constexpr int k = decltype(K_)::value;
          if constexpr (i == NS + 2 + (k * (NPV - 2)) / NSL) sm_slice(K_);
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    static_for<(nops > 2 ? (nops - 2 < NSIDE ? nops - 2 : NSIDE) : 0), NSIDE>(
        [&](auto J_) { side(J_); });
    if constexpr (do_sm && !sm_in) {
      mask(kb);
      static_for<0, NSL>([&](auto K_) { sm_slice(K_); });
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  auto nothing = [](auto) {};

  // After a stream with a softmax: fold it into l and O, hand its P^T on.
  auto settle = [&] {
    sm.fold();
    if (sm.rescale) {
      // One dim tile at a time, pinned to AGPRs before and after: otherwise
      // the allocator stages all 256 accumulators through VGPRs and spills
      // in the main loop.
#pragma unroll
      for (int d = 0; d < NDT; ++d) {
        asm volatile("" : "+a"(oacc[d]));
        f32x16 x = oacc[d];
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] *= sm.alpha;
        asm volatile("" : "+a"(x));
        oacc[d] = x;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    pop[0] = pn[0];
    pop[1] = pn[1];
  };

  // ---- main loop ---------------------------------------------------------------
  // Iteration t: stream Q.K^T(t) | P.V(t-1) with mask and softmax(t) | settle |
  // wait, barrier. It issues K(t+2) into the stage of K(t-2), whose last reads
  // (P.V(t-2)) were in iteration t-1. Before the barrier a wave waits until
  // only its newest DMA group may be in flight, so K(t+1) is ready.
  auto issue = [&](int t, auto J_) { dma_k1(kb_lo + t + 2, (t + 2) % KS, decltype(J_)::value); };
  if (n_tiles > 0) {
    {
      const Addr a0 = addr(0, 0);
      phase(T_{}, F_{}, T_{}, a0, a0, kb_lo, [&](auto J_) { issue(0, J_); });
      settle();
      wait_vm<KW>();
      lds_barrier();
    }
    for (int t = 1; t < n_tiles; ++t) {
      const Addr at = addr(t % KS, (t - 1) % KS);
      phase(T_{}, T_{}, T_{}, at, at, kb_lo + t, [&](auto J_) { issue(t, J_); });
      settle();
      wait_vm<KW>();
      lds_barrier();
    }
    {  // P.V of the last tile
      const Addr an = addr(0, (n_tiles - 1) % KS);
      phase(F_{}, T_{}, F_{}, an, an, 0, nothing);
    }
  }

#ifdef ATTN_DEBUG_TILES
  if (a.dbg_visits && lane == 0) {  // every wave computes every staged tile
    atomicAdd(a.dbg_visits, (unsigned long long)(n_tiles > 0 ? n_tiles : 0));
    if (wave == 0) atomicAdd(a.dbg_visits + 1, (unsigned long long)(n_tiles > 0 ? n_tiles : 0));
  }
#endif
  // ---- epilogue: O = O^T / l, bf16, staged through LDS ---------------------------
  wait_vm<0>();  // the last DMAs (zeros past the range) land before staging
  lds_barrier();
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sm.l_run),
                                                     __float_as_uint(sm.l_run), false, false);
    sm.l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  __attribute__((address_space(3))) unsigned char* ost =
      (__attribute__((address_space(3))) unsigned char*)lds + wave * (RW * D * 2);
  stage_o<NDT>(ost, oacc, valid ? 1.f / sm.l_run : 0.f, r32, h);
  const int64_t o_tok = a.o_tok ? a.o_tok : (int64_t)a.Hq * D;
  const int64_t o_head = a.o_head ? a.o_head : D;
  store_o<D, RW>(ost, lane, [&](int row) -> uint16_t* {
    const int p = wlo + row % R::PPW;
    const int hd = kvh * G + hg * R::HW + row / R::PPW;
    return p < T ? (uint16_t*)a.o + ((int64_t)b * T + p) * o_tok + hd * o_head : nullptr;
  });
}

template <int G, int RCH>
hipError_t launch_one(const PrefillArgs& a, hipStream_t st) {
  using R = Rows<G>;
  const int n_qt = (a.T + R::PW - 1) / R::PW;
  const int64_t n = (int64_t)n_qt * a.Hkv * a.B;
  if (n == 0) return hipSuccess;
  if (n > 0x7fffffff) return hipErrorInvalidValue;
  // Sliding-window tiles reuse their neighbours' keys: keep neighbours on one
  // XCD. Causal tiles are grouped per XCD by (batch, KV head) in the kernel.
  const int contig = (a.window > 0 && a.window < a.T) ? 1 : 0;
  hipLaunchKernelGGL((prefill_kv1w_kernel<G, RCH>), dim3((unsigned)n), dim3(NT), 0, st, a, n_qt,
                     contig);
  return hipGetLastError();
}

template <int G>
hipError_t dispatch_rot(const PrefillArgs& a, hipStream_t st) {
  const int rch = a.rope_q ? (2 * a.rot_pairs) / 8 : 0;
  if (rch == 0) return launch_one<G, 0>(a, st);
  if (rch == D / 32) return launch_one<G, D / 32>(a, st);
  if (rch == D / 8) return launch_one<G, D / 8>(a, st);
  return hipErrorNotSupported;
}

}  // namespace

bool prefill_kv1w_applies(const PrefillArgs& a) {
  const bool dense_v = (a.v_tok == 0 || a.v_tok == (int64_t)a.Hkv * D) &&
                       (a.v_head == 0 || a.v_head == D);
  return a.Dk == D && a.Dv == D && a.k == a.v && dense_v && !(a.rope_k && a.rot_pairs > 0);
}

hipError_t launch_prefill_kv1w(const PrefillArgs& a, hipStream_t st) {
  if (!prefill_kv1w_applies(a)) return hipErrorNotSupported;
  switch (a.Hq / a.Hkv) {
    case 1: return dispatch_rot<1>(a, st);
    case 2: return dispatch_rot<2>(a, st);
    case 4: return dispatch_rot<4>(a, st);
    case 8: return dispatch_rot<8>(a, st);
    default: return hipErrorNotSupported;
  }
}

}  // namespace attn
