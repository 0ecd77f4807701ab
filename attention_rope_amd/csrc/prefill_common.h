// prefill_common.h — LDS layout, operand reads, masking, output staging,
// RoPE helpers, the one-wave kernels' row map and block mapping, and the
// sliced online softmax, shared by the MFMA prefill kernels (prefill_mfma.hip,
// prefill_mfma2g.hip, prefill_mfma1w.hip, prefill_kv1w.hip).
#pragma once
#include <type_traits>

#include "attn_common.h"

namespace attn {
namespace prefill {

// log2(e); and the log2 headroom the online softmax keeps before it moves its
// running max (and with it rescales O).
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;

template <int N>
using IC = std::integral_constant<int, N>;

// Calls f(IC<I>{}) for I = 0 .. N-1 at compile time.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(IC<I>{});
    static_for<I + 1, N>(f);
  }
}

// XOR swizzle of 16-byte chunks inside a region row of `width` chunks. The
// mask P-1 uses the largest power of two P <= 16 dividing the width, so the
// swizzled index stays inside the row.
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
// V rows: chunk c of key row r sits at c ^ 4(r & 3). A transposing read of
// the V^T operand takes 4 consecutive keys x 4 consecutive chunks (one
// 32-dim tile) per 32 lanes; this swizzle puts the 16 pieces in 16 distinct
// bank groups (an XOR by r & 15 would keep them in 4).
__device__ __forceinline__ int vswz(int r, int c) { return c ^ ((r & 3) << 2); }

// One rotary pair (two bf16 in a dword) turned by (c, s) in fp32.
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

typedef __attribute__((address_space(3))) f32x2 lds_float2;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

// Base row of a wave's Q rotation: slot[p] = (cos, sin) of pair p at position
// pos (p < P), the angle pos * theta^(-2p/D) formed and evaluated in fp64.
// Lanes take pairs lane, lane + 64, ...; the caller reads the slot only after
// the wave's LDS writes landed (rotate_q_chunks waits for them).
__device__ __forceinline__ void rope_base_row(lds_float2* slot, int64_t pos, int P, int D,
                                              double log2_theta, int lane) {
  for (int p = lane; p < P; p += 64) {
    float c, s;
    rope_cos_sin(pos, rope_freq(p, D, log2_theta), &c, &s);
    slot[p] = f32x2{c, s};
  }
}

// The (cos, sin) of d * rho^i for the pairs i = 8u + 4h + j (u < NU, j < 4)
// of this lane's rotated Q^T chunks 2u + h: the small angle that turns the
// base row's pair i from the wave's base position to the lane's own (d
// positions further). rho = theta^(-2/D), so rho^i is pair i's frequency;
// the powers come from an fp64 product chain, d * rho^i / (2 pi) is formed in
// fp64 and its fraction goes through the sine and cosine units (which take
// revolutions). Issued before the wait for Q, so it runs under Q's latency.
template <int NU>
__device__ __forceinline__ void rope_offsets(float (&dcs)[NU > 0 ? NU : 1][8], int d,
                                             double rho, int h) {
  const double rho2 = rho * rho, rho4 = rho2 * rho2, rho5 = rho4 * rho;
  const double turns = (double)d * 0.15915494309189535;  // d / (2 pi)
  double w = h ? rho4 : 1.0;
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = __builtin_amdgcn_fractf((float)(turns * w));
      dcs[u][2 * j] = __builtin_amdgcn_cosf(x);
      dcs[u][2 * j + 1] = __builtin_amdgcn_sinf(x);
      w *= (j == 3) ? rho5 : rho;
    }
}

// Turn this lane's first NU Q^T chunks (qw[u] = dims 16u + 8h .. +7) by the
// base row in `slot` combined with the offsets from rope_offsets: (c, s) of
// base + offset by angle addition, then rotate4. Waits for the slot's LDS
// writes first, and for the slot's reads before returning (the memory clobber
// keeps later DMAs into the slot's region behind them).
template <int NU>
__device__ __forceinline__ void rotate_q_chunks(u32x4* qw, const lds_float2* slot,
                                                const float (&dcs)[NU > 0 ? NU : 1][8], int h) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const lds_f32x4* trow = (const lds_f32x4*)slot;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const f32x4 t0 = trow[4 * u + 2 * h], t1 = trow[4 * u + 2 * h + 1];
    float cs[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float cb = (j < 2 ? t0 : t1)[2 * (j % 2)], sb = (j < 2 ? t0 : t1)[2 * (j % 2) + 1];
      const float cd = dcs[u][2 * j], sd = dcs[u][2 * j + 1];
      cs[2 * j] = cb * cd - sb * sd;
      cs[2 * j + 1] = sb * cd + cb * sd;
    }
    qw[u] = rotate4(qw[u], f32x4{cs[0], cs[1], cs[2], cs[3]}, f32x4{cs[4], cs[5], cs[6], cs[7]});
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Per-lane DMA offsets. Block m of a tile region (64 lanes x 16 bytes) moves
// chunks 64m .. 64m + 63 of the region, row by row; each returns the byte
// offset of this lane's chunk inside the tile's first row (HBM side), where
// the chunk that lands at LDS chunk index c of row r is stored chunk
// swizzle(r, c). A tile then adds j0 times the region's row stride.
// K's turned region: rows of RCH chunks (the workspace rows, stride rrow).
template <int RCH>
__device__ __forceinline__ uint32_t k_rot_dma_off(int m, int lane, int rrow) {
  constexpr int W = RCH > 0 ? RCH : 1;  // unused when RCH == 0
  const int q = m * 64 + lane, r = q / W;
  return r * rrow + kswz<W>(r, q % W) * 16;
}
// K's plain region: rows of NP chunks starting at chunk RCH of k's rows.
template <int RCH, int NP>
__device__ __forceinline__ uint32_t k_plain_dma_off(int m, int lane, int krow) {
  constexpr int W = NP > 0 ? NP : 1;
  const int q = m * 64 + lane, r = q / W;
  return r * krow + (RCH + kswz<W>(r, q % W)) * 16;
}
// V rows of VC chunks.
template <int VC>
__device__ __forceinline__ uint32_t v_dma_off(int m, int lane, int vrow) {
  const int q = m * 64 + lane, r = q / VC;
  return r * vrow + vswz(r, q % VC) * 16;
}

// K operand of QK step s for key row r32 of a tile: dims 16s + 8h .. +7, the
// rotated region's chunk 2s + h while s < RCH / 2, else the plain region's;
// stored at chunk (2s + h) ^ mask, i.e. byte (32 s) ^ kx of the region row.
template <int RCH>
__device__ __forceinline__ bf16x8 k_operand(const lds_u8* kr, const lds_u8* kp, int kxr,
                                            int kxp, int s) {
  if (s < RCH / 2) return *(const lds_bf16x8*)(kr + ((32 * s) ^ kxr));
  return *(const lds_bf16x8*)(kp + ((32 * (s - RCH / 2)) ^ kxp));
}

// V^T operand of P.V step i (key half j = i / NDT, dim tile dt = i % NDT) of
// a tile whose rows hold VC 16-byte chunks swizzled by vswz: two transposing
// reads of 4 keys each, 8 key rows apart, from this lane's row offset v and
// row mask vx.
template <int NDT, int VC>
__device__ __forceinline__ bf16x8 vt_operand(const lds_u8* v, int vx, int i) {
  const int j = i / NDT, dt = i % NDT;
  const lds_u8* p = v + (((dt & 3) << 6) ^ vx) + (dt >> 2) * 256 + j * 16 * VC * 16;
  const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
  const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 8 * VC * 16));
  return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Scores of a 32-key tile starting at key j0, for a wave whose row
// positions run wlo .. whi: a tile crossing the diagonal or the window edge
// gets the per-score test (key j visible from position pos iff
// 0 <= pos - j < wcap; wcap is W, or 2^31 for causal), any other tile is
// left as it is. Element e of sc holds key j0 + 8(e/4) + 4h + (e%4). The
// empty asm keeps the test a branch (the selects would otherwise run on
// every tile); scores are masked in place.
__device__ __forceinline__ void mask_edge_tile(f32x16& sc, int j0, int wlo, int whi, int W,
                                               int pos, int h, unsigned wcap) {
  if ((j0 + 31 > wlo) || (W > 0 && j0 <= whi - W)) {
    asm volatile("");
    const int d0 = pos - j0 - 4 * h;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const unsigned d = (unsigned)(d0 - (8 * (e / 4) + (e % 4)));  // pos - key
      sc[e] = (d < wcap) ? sc[e] : -INFINITY;
    }
  }
}

// The output tile of one wave through LDS: stage_o writes O^T / l (NDT dim
// tiles of 32) as bf16 rows of this wave's staging area, where element e of
// dim tile dt is dim 32dt + 8(e/4) + 4h + (e%4), half h of 16-byte chunk
// 4dt + e/4 of row r32, chunks XOR-swizzled by the row; store_o reads whole
// 16-byte chunks back (64 / (DV/8) rows per instruction) and writes row r to
// dst(r), skipping rows for which dst returns nullptr. A wave reads back only
// what it wrote, and its LDS operations complete in order, so one
// lgkmcnt wait between the two suffices.
template <int NDT>
__device__ __forceinline__ void stage_o(__attribute__((address_space(3))) unsigned char* ost,
                                        const f32x16* oacc, float inv, int r32, int h) {
  constexpr int ORB = NDT * 64, VCM = NDT * 4 - 1;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t w0 = pack_bf16x2(oacc[dt][4 * jj] * inv, oacc[dt][4 * jj + 1] * inv);
      const uint32_t w1 = pack_bf16x2(oacc[dt][4 * jj + 2] * inv, oacc[dt][4 * jj + 3] * inv);
      const int c = 4 * dt + jj;
      *(__attribute__((address_space(3))) u32x2*)(ost + r32 * ORB + ((c ^ (r32 & VCM)) << 4) +
                                                  8 * h) = u32x2{w0, w1};
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

template <int DV, int RW, typename Dst>
__device__ __forceinline__ void store_o(const lds_u8* ost, int lane, Dst&& dst) {
  constexpr int VC = DV / 8, VCM = VC - 1, ORB = DV * 2;
  constexpr int RPI = 64 / VC;  // rows per store instruction
  const int c = lane % VC;
#pragma unroll
  for (int i = 0; i < RW / RPI; ++i) {
    const int row = i * RPI + lane / VC;
    const u32x4 val = *(const __attribute__((address_space(3))) u32x4*)(
        ost + row * ORB + ((c ^ (row & VCM)) << 4));
    uint16_t* d = dst(row);
    if (d) *(u32x4*)(d + 8 * c) = val;
  }
}

// Rows of the one-wave kernels (prefill_mfma1w.hip, prefill_kv1w.hip): 4
// waves, one per SIMD, of 32 (head, position) rows each. Wave w takes head
// group w % NHG (HW heads) and position block w / NHG (PPW positions); its
// row r is head r / PPW of the group at position r % PPW of the block. A
// workgroup covers PW positions of all G query heads of one KV head.
template <int G>
struct WaveRows {
  static constexpr int HW = G >= 8 ? G / 4 : 1;  // heads per wave
  static constexpr int PPW = 32 / HW;            // positions per wave
  static constexpr int NHG = G / HW;             // head groups across waves
  static constexpr int NPB = 4 / NHG;            // position blocks per workgroup
  static constexpr int PW = NPB * PPW;           // positions per workgroup
  static_assert(HW * NHG == G && 4 % NHG == 0 && NPB * NHG == 4, "wave -> rows map");
};

// Block -> (group = (batch, KV head), query tile) of the one-wave kernels.
// Blocks go round-robin over the 8 XCDs (block i to XCD i % 8, slot i / 8
// there). Causal tiles of one group share their key prefix, so they run on
// the same XCDs, whose L2 then streams that prefix once: with a multiple of 8
// groups each XCD takes whole groups, with 8 / k groups each group takes k
// XCDs, which alternate its tiles (equal work per XCD either way), longest
// tiles first. Sliding windows (contig) keep neighbouring tiles on one XCD
// instead.
__device__ __forceinline__ void block_tile(int block, int n_wg, int n_qt, int contig, int& grp,
                                           int& qt) {
  const int n_grp = n_wg / n_qt, x = block % 8, slot = block / 8;
  if (!contig && n_grp % 8 == 0) {
    const int gpx = n_grp / 8;  // groups per XCD
    grp = x * gpx + slot % gpx;
    qt = n_qt - 1 - slot / gpx;
  } else if (!contig && 8 % n_grp == 0 && n_qt % (8 / n_grp) == 0) {
    const int xpg = 8 / n_grp;  // XCDs per group
    grp = x / xpg;
    qt = n_qt - 1 - (slot * xpg + x % xpg);
  } else {
    const int L = contig ? xcd_contiguous(block, n_wg) : block;
    grp = L / n_qt;
    qt = n_qt - 1 - (L % n_qt);  // longest causal tiles first
  }
}

// Online softmax of one 32-key tile of S^T (each lane holds 16 scores of its
// row, element e for key 8(e/4) + 4h + (e%4); the partner lane l ^ 32 holds
// the other 16), cut into NSL slices that a kernel spreads between the MFMAs
// of its stream. The slices form a pipeline: every value a slice needs comes
// from an earlier slice, so none stalls the wave's in-order issue (and with
// it the next MFMA) on its own dependency chain.
//  0-3   partial maxima of 4 scores each
//  4     max of the partials; 5 the partner lane's half (row max)
//  6     scaled row max; 7 lazy-rescale vote; 8 new max, rescale factor
//  9     factor select, max in use
//  10-27 slice 10+j scales score j, exponentiates score j-1 and adds
//        probability j-2 to the row sum
//  28-29 the two bf16 P^T operands
// The running max moves, and O must be multiplied by alpha, only when a row's
// tile max exceeds the max in use by more than 2^kLazy (the first tile always
// does: alpha is then 0). The vote goes through a vector register, so the
// updates are selects, not a branch that would split the stream.
struct SliceSoftmax {
  static constexpr int NSL = 30;
  // scores to log2 units; kept > 0 so a masked -inf score never meets a zero
  // factor (scale 0 then acts as 1e-30: every visible key weighs the same)
  float c2;
  float m_run = -INFINITY;  // max in use (log2 units)
  float l_run = 0.f;        // this lane's half of the row sum
  float alpha = 1.f;        // factor for O and l of the tile just softmaxed
  bool rescale = false;     // wave-uniform: alpha != 1 for some row
  float smx[4] = {}, sst = 1.f, ssum = 0.f, muse = 0.f, smc = 0.f, smn = 0.f;
  int srv = 0;

  __device__ explicit SliceSoftmax(float scale) : c2(fmaxf(scale * kLog2e, 1e-30f)) {}

  // Slice k of the softmax of the scores in s: the scaled scores go to t and
  // the probabilities to p, either of which may be s itself (in place); slices
  // 28-29 write the P^T operands to pn. Plain register arrays for t and p are
  // pinned per element so the pipeline stays in the order the slices give.
  template <int k, class S, class Tt, class Pp>
  __device__ __forceinline__ void slice(S& s, Tt& t, Pp& p, bf16x8 (&pn)[2]) {
    if constexpr (k < 4) {
      smx[k] = fmaxf(fmaxf(s[4 * k], s[4 * k + 1]), fmaxf(s[4 * k + 2], s[4 * k + 3]));
      asm volatile("" : "+v"(smx[k]));
    } else if constexpr (k == 4) {
      smx[0] = fmaxf(fmaxf(smx[0], smx[1]), fmaxf(smx[2], smx[3]));
      asm volatile("" : "+v"(smx[0]));
    } else if constexpr (k == 5) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(smx[0]),
                                                       __float_as_uint(smx[0]), false, false);
      smx[1] = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      asm volatile("" : "+v"(smx[1]));
    } else if constexpr (k == 6) {
      smc = (smx[1] == -INFINITY) ? -INFINITY : smx[1] * c2;
      asm volatile("" : "+v"(smc));
    } else if constexpr (k == 7) {
      rescale = __any(smc > m_run + kLazy);  // wave-uniform
      srv = rescale;
      asm volatile("" : "+v"(srv));
    } else if constexpr (k == 8) {
      smn = srv ? fmaxf(m_run, smc) : m_run;
      sst = fast_exp2(m_run - smn);
      asm volatile("" : "+v"(smn), "+v"(sst));
    } else if constexpr (k == 9) {
      const float keep = (m_run == -INFINITY) ? 0.f : sst;
      alpha = srv ? keep : 1.f;
      m_run = smn;
      muse = (m_run == -INFINITY) ? 0.f : m_run;
      ssum = 0.f;
      asm volatile("" : "+v"(alpha), "+v"(muse), "+v"(ssum));
    } else if constexpr (k < 28) {
      constexpr int j = k - 10;
      if constexpr (j < 16) {  // masked scores are -inf: exactly 0 after exp2
        t[j] = fmaf(s[j], c2, -muse);
        if constexpr (std::is_array_v<Tt>) asm volatile("" : "+v"(t[j]));
      }
      if constexpr (j >= 1 && j <= 16) {
        p[j - 1] = fast_exp2(t[j - 1]);
        if constexpr (std::is_array_v<Pp>) asm volatile("" : "+v"(p[j - 1]));
      }
      if constexpr (j >= 2) {
        ssum += p[j - 2];
        asm volatile("" : "+v"(ssum));
      }
    } else {
      constexpr int jj = k - 28;  // P^T operand of key step jj: elements 8jj .. 8jj+7
      const f32x4 lo = {p[8 * jj], p[8 * jj + 1], p[8 * jj + 2], p[8 * jj + 3]};
      const f32x4 hi = {p[8 * jj + 4], p[8 * jj + 5], p[8 * jj + 6], p[8 * jj + 7]};
      pn[jj] = __builtin_shufflevector(__builtin_convertvector(lo, bf16x4),
                                       __builtin_convertvector(hi, bf16x4), 0, 1, 2, 3, 4, 5, 6, 7);
      asm volatile("" : "+v"(pn[jj]));
    }
  }

  // After the tile's last slice: fold its probabilities into the row sum (the
  // caller multiplies O by alpha when `rescale`).
  __device__ __forceinline__ void fold() { l_run = l_run * alpha + ssum; }
};

}  // namespace prefill
}  // namespace attn
