// prefill_mfma.hip — flash-style causal / sliding-window GQA prefill on gfx950
// bf16 matrix cores (v_mfma_f32_32x32x16_bf16), with RoPE fused into the Q and
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
//  * A workgroup owns one (batch, KV head) and PW consecutive query positions
//    for all G query heads that share the KV head: NW*32 (head, position)
//    rows, so each K/V tile staged in LDS serves G heads (GQA packing).
//  * Each wavefront owns 32 rows and computes S^T = K Q^T (M = 32 keys,
//    N = 32 rows): in the MFMA output layout every lane then holds 16 scores
//    of a single query row, so the softmax max/sum need one cross-lane swap
//    (lane ^ 32) instead of a 32-lane reduction. Q^T lives in registers for
//    the whole kernel; K tiles stream through LDS.
//  * O^T = V^T P^T accumulates in registers (every lane again owns one row).
//    The P^T operand is the lane's own scores — no data movement — provided
//    the key order inside each 16-key MFMA step matches the score layout; V^T
//    is staged in LDS in exactly that permuted key order.
//  * Key tiles of 32 are double-buffered in LDS; the next tile's global loads
//    are issued before the current tile's matrix work.
//  * Only key tiles intersecting the causal band / sliding window are visited
//    (window-aware skipping), and masking runs only on tiles that cross the
//    diagonal or the window edge.
//  * The O accumulator is rescaled only when some row's running max changed.
//  * Causal tiles are issued longest-first; sliding-window launches map
//    neighbouring query tiles onto the same XCD so their K/V windows share L2.
#include "attn_common.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int DK, int DV, int G, int NW, int RK>
struct Cfg {
  static constexpr int NT = NW * 64;        // threads
  static constexpr int ROWS = NW * 32;      // (head, position) rows per WG
  static constexpr int PW = ROWS / G;       // query positions per WG
  static constexpr int BN = 32;             // keys per tile
  static constexpr int KS = DK + 8;         // K row stride in LDS (elements)
  static constexpr int VS = BN + 8;         // V^T row stride in LDS (elements)
  static constexpr int KT = BN * KS;
  static constexpr int VT = DV * VS;
  static constexpr int STAGE = KT + VT;     // elements per LDS stage
  static constexpr int NC = DK / 8;         // 16-byte chunks per K row
  static constexpr int KCH = BN * NC / NT;  // K chunks per thread per tile
  static constexpr int NRC = BN * RK;       // rotated K chunks per tile
  static constexpr int KR = (NRC + NT - 1) / NT;  // iterations holding rotated chunks
  static constexpr int VU = (BN / 4) * (DV / 8);  // V units: 4 keys x 8 dims
  static constexpr int VUT = (VU + NT - 1) / NT;
  static_assert(ROWS % G == 0, "rows must split evenly over the heads");
  static_assert(PW >= 32 ? PW % 32 == 0 : 32 % PW == 0, "wave/row layout");
  static_assert((BN * NC) % NT == 0, "K tile must split evenly");
  static_assert(DK % 16 == 0 && DV % 32 == 0, "MFMA tiling");
  static_assert(RK >= 0 && RK <= NC, "rotary chunks");
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

template <int DK, int DV, int G, int NW, int RK>
__global__ __launch_bounds__(NW * 64) void prefill_mfma_kernel(PrefillArgs a, int n_qt,
                                                               int contig) {
  using C = Cfg<DK, DV, G, NW, RK>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * C::STAGE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 31, hh = lane >> 5;
  const int T = a.T, W = a.window;
  const int n_wg = n_qt * a.Hkv * a.B;
  const int L = contig ? xcd_contiguous((int)blockIdx.x, n_wg) : (int)blockIdx.x;
  const int grp = L / n_qt;
  const int qt = n_qt - 1 - (L % n_qt);  // longest causal tiles first
  const int kvh = grp % a.Hkv, b = grp / a.Hkv;
  const int p0 = qt * C::PW;

  // This lane's query row and the wave's position range.
  const int R = wave * 32 + lr;
  const int head = kvh * G + R / C::PW;
  const int pos = p0 + R % C::PW;
  const bool valid = pos < T;
  const int wlo = p0 + (wave * 32) % C::PW;
  const int whi = wlo + (C::PW < 32 ? C::PW : 32) - 1;

  // ---- Q^T operands in registers, rotated at the row's position ----------
  bf16x8 qf[DK / 16];
  {
    const int prow = valid ? pos : T - 1;
    const uint16_t* qrow =
        (const uint16_t*)a.q + (((int64_t)b * T + prow) * a.Hq + head) * DK;
    const float2* tab = a.rope_tab + (int64_t)prow * a.rot_pairs;
#pragma unroll
    for (int s = 0; s < DK / 16; ++s) {
      const int d0 = 16 * s + 8 * hh;
      u32x4 w = *(const u32x4*)(qrow + d0);
      if (a.rope_q && d0 < 2 * a.rot_pairs) {
        const f32x4 t0 = *(const f32x4*)(tab + d0 / 2);
        const f32x4 t1 = *(const f32x4*)(tab + d0 / 2 + 2);
        w = rotate4(w, t0, t1);
      }
      if (!valid) w = u32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int kv_lo = (W > 0) ? max(0, p0 - W + 1) : 0;
  const int kv_hi = min(T, p0 + C::PW);
  const int kb_lo = kv_lo / C::BN;
  const int kb_hi = (kv_hi + C::BN - 1) / C::BN;

  const uint16_t* kbase = (const uint16_t*)a.k + ((int64_t)b * T * a.Hkv + kvh) * DK;
  const uint16_t* vbase = (const uint16_t*)a.v + ((int64_t)b * T * a.Hkv + kvh) * DV;
  const int64_t krs = (int64_t)a.Hkv * DK, vrs = (int64_t)a.Hkv * DV;

  // ---- staging registers --------------------------------------------------
  u32x4 kreg[C::KCH];
  f32x4 ktab[C::KR > 0 ? C::KR : 1][2];
  u32x4 vreg[C::VUT][4];

  auto chunk_of = [&](int it, int& row, int& col8) {
    const int c = tid + C::NT * it;
    if (RK > 0 && c < C::NRC) {
      row = c / (RK > 0 ? RK : 1);
      col8 = c % (RK > 0 ? RK : 1);
    } else {
      constexpr int NP = (C::NC - RK > 0) ? C::NC - RK : 1;  // plain chunks per row
      const int c2 = c - C::NRC;
      row = c2 / NP;
      col8 = RK + c2 % NP;
    }
  };

  auto load_tile = [&](int kb) {
    const int j0 = kb * C::BN;
#pragma unroll
    for (int it = 0; it < C::KCH; ++it) {
      int row, col8;
      chunk_of(it, row, col8);
      const int j = j0 + row;
      kreg[it] = (j < T) ? *(const u32x4*)(kbase + j * krs + col8 * 8) : u32x4{0, 0, 0, 0};
      if (it < C::KR) {
        const int c = tid + C::NT * it;
        if (c < C::NRC && j < T) {
          const float2* t = a.rope_tab + (int64_t)j * a.rot_pairs + 4 * col8;
          ktab[it][0] = *(const f32x4*)t;
          ktab[it][1] = *(const f32x4*)(t + 2);
        } else {
          ktab[it][0] = f32x4{1.f, 0.f, 1.f, 0.f};
          ktab[it][1] = f32x4{1.f, 0.f, 1.f, 0.f};
        }
      }
    }
#pragma unroll
    for (int ut = 0; ut < C::VUT; ++ut) {
      const int u = tid + C::NT * ut;
      const int kg = u % 8, d8 = u / 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + 4 * kg + e;
        vreg[ut][e] = (u < C::VU && j < T) ? *(const u32x4*)(vbase + j * vrs + d8 * 8)
                                          : u32x4{0, 0, 0, 0};
      }
    }
  };

  auto store_tile = [&](uint16_t* Ks, uint16_t* Vt) {
#pragma unroll
    for (int it = 0; it < C::KCH; ++it) {
      int row, col8;
      chunk_of(it, row, col8);
      u32x4 w = kreg[it];
      if (it < C::KR) {
        const int c = tid + C::NT * it;
        if (c < C::NRC) w = rotate4(w, ktab[it][0], ktab[it][1]);
      }
      *(u32x4*)(Ks + row * C::KS + col8 * 8) = w;
    }
#pragma unroll
    for (int ut = 0; ut < C::VUT; ++ut) {
      const int u = tid + C::NT * ut;
      if (u < C::VU) {
        const int kg = u % 8, d8 = u / 8;
        // keys 4kg..4kg+3 occupy 4 consecutive slots of the permuted key order
        const int slot = 16 * (kg / 4) + 8 * (kg % 2) + 4 * ((kg % 4) / 2);
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          const int wi = dd / 2;
          uint32_t lo, hi;
          if (dd % 2 == 0) {
            lo = (vreg[ut][0][wi] & 0xffffu) | (vreg[ut][1][wi] << 16);
            hi = (vreg[ut][2][wi] & 0xffffu) | (vreg[ut][3][wi] << 16);
          } else {
            lo = (vreg[ut][0][wi] >> 16) | (vreg[ut][1][wi] & 0xffff0000u);
            hi = (vreg[ut][2][wi] >> 16) | (vreg[ut][3][wi] & 0xffff0000u);
          }
          *(u32x2*)(Vt + (8 * d8 + dd) * C::VS + slot) = u32x2{lo, hi};
        }
      }
    }
  };

  // ---- online softmax state (one row per lane; halves share the row) -------
  const float c2 = a.scale * kLog2e;  // scores to log2 units (>= 0)
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) oacc[d] = f32x16{};

  auto compute = [&](const uint16_t* Ks, const uint16_t* Vt, int kb) {
    const int j0 = kb * C::BN;
    if (j0 > whi) return;                          // beyond every row (causal)
    if (W > 0 && j0 + C::BN - 1 <= wlo - W) return;  // before every row's window
    f32x16 s = f32x16{};
#pragma unroll
    for (int st = 0; st < DK / 16; ++st) {
      const bf16x8 ka = *(const bf16x8*)(Ks + lr * C::KS + 16 * st + 8 * hh);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[st], s, 0, 0, 0);
    }
    // lane holds keys j0 + 8(i/4) + 4hh + (i%4) of its row, i = 0..15
    const bool need_mask = (j0 + C::BN - 1 > wlo) || (W > 0 && j0 <= whi - W);
    uint32_t okbits = 0xffffu;
    float mx = -INFINITY;
    if (need_mask) {
      okbits = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = j0 + 8 * (i / 4) + 4 * hh + (i % 4);
        const bool ok = (j <= pos) && (W <= 0 || pos - j < W);
        okbits |= (ok ? 1u : 0u) << i;
        mx = fmaxf(mx, ok ? s[i] : -INFINITY);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mb = (mx == -INFINITY) ? -INFINITY : mx * c2;
    const float m_new = fmaxf(m_run, mb);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float pv[16];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p = exp2f(fmaf(s[i], c2, -m_use));
      if (need_mask) p = ((okbits >> i) & 1u) ? p : 0.f;
      pv[i] = p;
      psum += p;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int d = 0; d < DV / 32; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
    }
    f32x4 lo0 = {pv[0], pv[1], pv[2], pv[3]}, lo1 = {pv[4], pv[5], pv[6], pv[7]};
    f32x4 hi0 = {pv[8], pv[9], pv[10], pv[11]}, hi1 = {pv[12], pv[13], pv[14], pv[15]};
    bf16x4 a0 = __builtin_convertvector(lo0, bf16x4), a1 = __builtin_convertvector(lo1, bf16x4);
    bf16x4 b0 = __builtin_convertvector(hi0, bf16x4), b1 = __builtin_convertvector(hi1, bf16x4);
    const bf16x8 pb0 = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    const bf16x8 pb1 = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) {
      const uint16_t* vrow = Vt + (32 * d + lr) * C::VS + 8 * hh;
      const bf16x8 v0 = *(const bf16x8*)(vrow);
      const bf16x8 v1 = *(const bf16x8*)(vrow + 16);
      oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, pb0, oacc[d], 0, 0, 0);
      oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, pb1, oacc[d], 0, 0, 0);
    }
  };

  // ---- main loop: double-buffered key tiles -------------------------------
  if (kb_lo < kb_hi) {
    load_tile(kb_lo);
    store_tile(lds, lds + C::KT);
    __syncthreads();
  }
  for (int kb = kb_lo; kb < kb_hi; ++kb) {
    const int cur = (kb - kb_lo) & 1;
    uint16_t* cs = lds + cur * C::STAGE;
    uint16_t* ns = lds + (cur ^ 1) * C::STAGE;
    const bool more = kb + 1 < kb_hi;
    if (more) load_tile(kb + 1);
    compute(cs, cs + C::KT, kb);
    if (more) store_tile(ns, ns + C::KT);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, bf16, 4 consecutive dims per store ----------
  const float lt = l_run + __shfl_xor(l_run, 32);
  if (valid) {
    const float inv = 1.f / lt;
    uint16_t* orow = (uint16_t*)a.o + (((int64_t)b * T + pos) * a.Hq + head) * DV;
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int bq = 0; bq < 4; ++bq) {
        const uint32_t w0 = pack_bf16x2(oacc[d][4 * bq] * inv, oacc[d][4 * bq + 1] * inv);
        const uint32_t w1 = pack_bf16x2(oacc[d][4 * bq + 2] * inv, oacc[d][4 * bq + 3] * inv);
        *(u32x2*)(orow + 32 * d + 8 * bq + 4 * hh) = u32x2{w0, w1};
      }
  }
}

template <int DK, int DV, int G, int NW, int RK>
hipError_t launch_one(const PrefillArgs& a, hipStream_t st) {
  using C = Cfg<DK, DV, G, NW, RK>;
  const int n_qt = (a.T + C::PW - 1) / C::PW;
  const int64_t n = (int64_t)n_qt * a.Hkv * a.B;
  if (n == 0) return hipSuccess;
  if (n > 0x7fffffff) return hipErrorInvalidValue;
  // Sliding-window tiles reuse their neighbours' K/V: keep neighbours on one
  // XCD. Causal tiles share the prefix of every key stream: interleave.
  const int contig = (a.window > 0 && a.window < a.T) ? 1 : 0;
  hipLaunchKernelGGL((prefill_mfma_kernel<DK, DV, G, NW, RK>), dim3((unsigned)n),
                     dim3(C::NT), 0, st, a, n_qt, contig);
  return hipGetLastError();
}

template <int DK, int DV, int G>
hipError_t dispatch_rk(const PrefillArgs& a, hipStream_t st) {
  const int rk = a.rope_k ? (2 * a.rot_pairs) / 8 : 0;
  if (rk == 0) return launch_one<DK, DV, G, 4, 0>(a, st);
  if (rk == DK / 32) return launch_one<DK, DV, G, 4, DK / 32>(a, st);
  if (rk == DK / 8) return launch_one<DK, DV, G, 4, DK / 8>(a, st);
  return hipErrorNotSupported;
}

template <int DK, int DV>
hipError_t dispatch_g(const PrefillArgs& a, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return dispatch_rk<DK, DV, 1>(a, st);
    case 2: return dispatch_rk<DK, DV, 2>(a, st);
    case 4: return dispatch_rk<DK, DV, 4>(a, st);
    case 8: return dispatch_rk<DK, DV, 8>(a, st);
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
  if (a.rope_q || a.rope_k) {
    if ((2 * a.rot_pairs) % 8 != 0) return hipErrorNotSupported;
  }
  if (a.Dk == 512 && a.Dv == 256) return dispatch_g<512, 256>(a, st);
  if (a.Dk == 256 && a.Dv == 256) return dispatch_g<256, 256>(a, st);
  if (a.Dk == 128 && a.Dv == 128) return dispatch_g<128, 128>(a, st);
  return hipErrorNotSupported;
}

}  // namespace attn
