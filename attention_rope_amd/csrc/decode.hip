// decode.hip — single-token GQA decode over a ragged bf16 KV cache on gfx950:
// a split-K streaming kernel and a log-sum-exp merge of the chunks.
//
// What it computes (Gemma 4 pages): the new token attends every cached row of
// a global layer or the last W rows of a local one ("Gemma 4: End-to-End
// Architecture Walkthrough", Phase 3 sections 3a-3b: global layers must keep
// K/V for the whole context, which is why decode is bound by reading that
// cache); 8 (global) or 2 (local) query heads share each KV head; the query is
// rotated with (p-)RoPE at its own position (section 3c), cached keys are
// stored already rotated. On a K = V layer (section 3b; "Gemma 4 Technical
// Report" reader, "Core Model Architecture") one cache serves as keys and
// values, and each row is read once for both products.
//
// Design for CDNA4 (HBM-bound: ~8 FLOP per cache byte with 8 heads/KV head):
//  * Grid = (KV heads, chunks, sequences), KV heads fastest. A workgroup
//    streams one chunk of one sequence's rows for one KV head through an LDS
//    ring filled by DMA (buffer_load ... lds) and serves all G query heads of
//    that KV head from the same bytes, on MFMA.
//  * Chunks are long (up to 4096 rows, or a whole local window): each
//    workgroup start and end idles its CU's memory pipe for a few
//    microseconds, which short chunks pay many times over.
//  * With several chunks per sequence each writes an online-softmax partial
//    (max, sum, acc) and a second kernel merges them; with one chunk the
//    streaming kernel normalises and writes o itself.
#include <algorithm>
#include <type_traits>

#include "attn_common.h"
#include "kernels.h"

#include <mutex>

namespace attn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ---- streaming kernel: K/V tiles through an LDS DMA ring -------------------
// Decode is bound by the bytes of the cache, and there is little arithmetic
// per byte, so this kernel is built around keeping bytes in flight: 2 waves
// stream 32-row tiles (K and V) into a 3-stage LDS ring by DMA, two tiles
// ahead, with no staging registers; each wave takes 16 of a tile's rows.
// S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (16 keys x 16 head columns), then
// O^T += V^T P^T on v_mfma_f32_16x16x16_bf16: the P^T operand (keys 4g..4g+3
// of head col) is exactly what the score MFMA left in the lane, and V^T comes
// from one transposing LDS read (ds_read_b64_tr_b16) per MFMA.
// RW waves per workgroup, 16 rows per wave and tile, a STAGES-deep ring
// filled STAGES - 1 tiles ahead. A verify call with more than 16 (token,
// head) pairs per KV head adds sets of RW waves (up to 4 sets) that take the
// same rows for the next 16 pairs each, so the tiles serve all of them. SHARED: the values are the cached keys
// (one cache serves as both), so a tile holds K rows only and P.V reads its
// transposed operand from them.
template <int DK, int DV, int RW_, int STAGES_, bool SHARED_ = false>
struct RCfg {
  static constexpr int RW = RW_, STAGES = STAGES_, AHEAD = STAGES - 1;
  static constexpr bool SHARED = SHARED_;
  static constexpr int RBN = 16 * RW;  // rows per tile
  static constexpr int KC = DK / 8, VC = DV / 8;  // 16-byte chunks per row
  static constexpr int KT = RBN * DK * 2, VT = SHARED ? 0 : RBN * DV * 2;
  static constexpr int V_OFF = SHARED ? 0 : KT;  // V rows' offset in a stage
  static constexpr int ST = KT + VT;
  static constexpr int RING = STAGES * ST;
  static constexpr int RED = RW * 16 * (DV + 2) * 4;  // the wave merge reuses the ring
  static constexpr int LDS = RING > RED ? RING : RED;
  static constexpr int K_DMA = KT / 1024, N_DMA = ST / 1024;
  static constexpr int DMA_W = N_DMA / RW;  // DMAs per wave per tile
  static_assert(KC >= 16 && VC >= 16, "row swizzle uses 16 chunk groups");
  static_assert(K_DMA % RW == 0 && N_DMA % RW == 0, "uniform DMA counts");
  static_assert(STAGES >= 2 && (AHEAD - 1) * DMA_W < 64 && LDS <= 160 * 1024,
                "vmcnt / LDS limits");
  static_assert(!SHARED || DK == DV, "shared K/V rows have one width");
};

template <class C, int DK, int DV, int NGW>
__global__ __launch_bounds__(C::RW * NGW * 64, 1) void decode_ring_kernel(DecodeArgs a, int ch, int n_split) {
  // kRW row waves split each tile's rows; NGW column groups each have their
  // own kRW waves over the same rows, so a workgroup has kW waves.
  constexpr int kRW = C::RW, kRBN = C::RBN, kW = kRW * NGW;
  constexpr int DMA_W = C::N_DMA / kW;  // DMAs per wave per tile
  static_assert(C::N_DMA % kW == 0 && C::K_DMA % kW == 0, "uniform DMA counts");
  static_assert((C::AHEAD - 1) * DMA_W < 64, "vmcnt field");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS];

  // KV heads vary fastest in the grid, so the workgroups that share a chunk's
  // cache rows run side by side. The MFMA's 16 columns are (token, head)
  // pairs: column c of group cg is q = 16 cg + c, token q / G, head q % G. A
  // workgroup serves NGW consecutive groups (many new tokens of a verify
  // call) from the same cache bytes: wave w takes rows 16 (w % kRW) of each
  // tile for group NGW cgb + w / kRW.
  const int cgb = blockIdx.x / a.Hkv, kvh = blockIdx.x - cgb * a.Hkv;
  const int split = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave % kRW, wg = wave / kRW;  // row wave, column group
  const int col = lane & 15, g = lane >> 4;
  const int G = a.Hq / a.Hkv, n_q = a.n_q, ncol = n_q * G;
  auto col_ok_g = [&](int i, int c) { return 16 * (NGW * cgb + i) + c < ncol; };
  auto col_row_g = [&](int i, int c) -> int64_t {  // row of q and o: [B, n_q, Hq]
    const int q = 16 * (NGW * cgb + i) + c, j = q / G;
    return ((int64_t)b * n_q + j) * a.Hq + kvh * G + (q - j * G);
  };
  auto col_ok = [&](int c) { return col_ok_g(wg, c); };
  auto col_tok = [&](int c) { return (16 * (NGW * cgb + wg) + c) / G; };
  auto col_row = [&](int c) { return col_row_g(wg, c); };

  const int kv_len = a.kv_len[b];
  if (kv_len <= 0 || kv_len > a.max_kv_len || kv_len < n_q) {
    // No rows: o = 0; kv_len past max_kv_len or short of the new tokens:
    // poisoned (NaN). With several chunks the merge writes these rows.
    if (n_split == 1) {
      for (int idx = tid; idx < NGW * 16 * DV; idx += kW * 64) {
        const int i = idx / (16 * DV), c = (idx / DV) % 16;
        if (col_ok_g(i, c))
          ((uint16_t*)a.o)[col_row_g(i, c) * DV + idx % DV] = kv_len == 0 ? 0 : 0x7fc0;
      }
    }
    return;
  }
  // Token j (position kv_len - n_q + j) sees rows [lo_j, pos_j]; the chunks
  // cover [lo_0, kv_len).
  const int lo = (a.window > 0) ? max(0, kv_len - n_q + 1 - a.window) : 0;
  const int c0 = lo + split * ch;
  if (c0 >= kv_len) return;
  const int c1 = min(kv_len, c0 + ch);
  const int n_tiles = (c1 - c0 + kRBN - 1) / kRBN;
  const int64_t row0 = a.row_offset[b] + c0;  // cache row of the chunk's first key

  // Descriptors over the chunk's rows of KV head kvh: rows at or past c1 read
  // 0 (their scores are masked, and a zero row keeps P.V finite).
  const int krow = a.Hkv * DK * 2, vrow = a.Hkv * DV * 2;
  const u32x4 kdesc = buffer_desc((const char*)a.k_cache + (row0 * a.Hkv + kvh) * DK * 2,
                                  (uint32_t)((c1 - 1 - c0) * krow + DK * 2));
  const u32x4 vdesc = buffer_desc((const char*)a.v_cache + (row0 * a.Hkv + kvh) * DV * 2,
                                  (uint32_t)((c1 - 1 - c0) * vrow + DV * 2));
  // Block n (n = i*kW + wave) of a tile holds 64 chunks; K rows first, then V
  // rows, each row's chunks XOR-swizzled by (row & 15).
  uint32_t dma_off[DMA_W];
#pragma unroll
  for (int i = 0; i < DMA_W; ++i) {
    const int n = i * kW + wave;
    if (n < C::K_DMA) {
      const int q = n * 64 + lane, r = q / C::KC;
      dma_off[i] = r * krow + ((q % C::KC) ^ (r & 15)) * 16;
    } else {
      const int q = (n - C::K_DMA) * 64 + lane, r = q / C::VC;
      dma_off[i] = r * vrow + ((q % C::VC) ^ (r & 15)) * 16;
    }
  }
  // Tiles past the chunk are issued too (one vmcnt value then covers every
  // step), but at an offset past the descriptors' end: they return zeros
  // without touching memory.
  auto dma_tile = [&](int t, int stage) {
    const int j0 = t * kRBN;
    const uint32_t st = lds_addr(lds) + stage * C::ST;
    const uint32_t far = t < n_tiles ? 0u : 0x80000000u;
#pragma unroll
    for (int i = 0; i < DMA_W; ++i) {
      const int n = i * kW + wave;
      if (i * kW < C::K_DMA)  // same region for every wave (K_DMA % kW == 0)
        dma16<true>(kdesc, st + n * 1024, (dma_off[i] + j0 * krow) | far);
      else
        dma16<true>(vdesc, st + n * 1024, (dma_off[i] + j0 * vrow) | far);
    }
  };
  // Tiles past the chunk's end read zeros without traffic (masked anyway).
#pragma unroll
  for (int i = 0; i < C::AHEAD; ++i) dma_tile(i, i);

  // ---- rotated queries as the B operand: col = head, k = dims -------------
  // The angle of each rotary pair is formed once per wave (one pair per lane,
  // fp64) into a small LDS table; every lane then reads the pairs it holds.
  // (one-token calls only, which have one column group: NGW == 1)
  constexpr int kCS = NGW == 1 ? kW : 1;
  __shared__ float2 cs_tab[kCS][DK / 2];
  bf16x8 qf[DK / 32];
  if (a.q_rotated) {
    const bool hv = col_ok(col);
    const uint16_t* qrow = (const uint16_t*)a.q + col_row(hv ? col : 0) * DK;
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
      u32x4 w = *(const u32x4*)(qrow + 32 * s + 8 * g);
      if (!hv) w = u32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  } else {  // one token per sequence (n_q = 1), turned here at kv_len - 1
    const int qpos = kv_len - 1;
    const double l2t = log2(a.theta);
    for (int p = lane; p < a.rot_pairs; p += 64) {
      float c, sn;
      rope_cos_sin(qpos, rope_freq(p, DK, l2t), &c, &sn);
      cs_tab[wave % kCS][p] = make_float2(c, sn);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const bool hv = col_ok(col);
    const uint16_t* qrow = (const uint16_t*)a.q + col_row(hv ? col : 0) * DK;
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
      const int d0 = 32 * s + 8 * g;
      u32x4 w = *(const u32x4*)(qrow + d0);
      if (d0 / 2 < a.rot_pairs) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (d0 / 2 + e < a.rot_pairs) {
            const float2 t = cs_tab[wave % kCS][d0 / 2 + e];
            const float x0 = bf16_lo(w[e]), x1 = bf16_hi(w[e]);
            w[e] = pack_bf16x2(x0 * t.x - x1 * t.y, x0 * t.y + x1 * t.x);
          }
        }
      }
      if (!hv) w = u32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }
  wait_vm<(C::AHEAD - 1) * DMA_W>();
  lds_barrier();

  // Visible keys of this lane's column, and the tile-uniform bounds inside
  // which no column masks anything.
  const int col_pos = kv_len - n_q + (col_ok(col) ? col_tok(col) : 0);
  const int col_lo = (a.window > 0) ? max(0, col_pos + 1 - a.window) : 0;
  const int col_hi = min(c1, col_pos + 1);
  const int mask_lo = (a.window > 0) ? max(0, kv_len - a.window) : 0;
  const int mask_hi = min(c1, kv_len - n_q + 1);

  // scores to log2 units; kept > 0 so a masked -inf never meets a zero factor
  const float c2 = fmaxf(a.scale * kLog2e, 1e-30f);
  float m_run = -INFINITY, l_run = 0.f;  // per head `col`
  f32x4 oacc[DV / 16];
#pragma unroll
  for (int d = 0; d < DV / 16; ++d) oacc[d] = f32x4{};

  // Per-lane LDS offsets. K: row 16*wave + col, chunk 4s + g, swizzled by
  // col: 4(s ^ (col >> 2)) + (g ^ (col & 3)); s = 4A + B gives 4 bases plus
  // an immediate. V^T: rows 16*wave + 4g + r (r = col >> 2), dims
  // 16d + 4(col & 3) .. + 3; swizzle x = 4g + r, so with d = 8A + B the
  // chunk 2(d ^ (x >> 1)) + (((col & 3) >> 1) ^ (x & 1)) gives 8 bases.
  int ko[4], vo[8];
  {
    const int krow_l = (16 * wr + col) * C::KC * 16 + ((g ^ (col & 3)) << 4);
#pragma unroll
    for (int B = 0; B < 4; ++B) ko[B] = krow_l + ((B ^ (col >> 2)) << 6);
    const int x = 4 * g + (col >> 2), c4 = col & 3;
    const int vrow_l = C::V_OFF + (16 * wr + x) * C::VC * 16 +
                       ((((c4 >> 1) ^ (x & 1))) << 4) + ((c4 & 1) << 3);
#pragma unroll
    for (int B = 0; B < 8; ++B) vo[B] = vrow_l + ((B ^ (x >> 1)) << 5);
  }

  int cur = 0;
  for (int t = 0; t < n_tiles; ++t) {
    dma_tile(t + C::AHEAD, cur == 0 ? C::AHEAD : cur - 1);
    const lds_u8* st = (const lds_u8*)lds + __builtin_amdgcn_readfirstlane(cur * C::ST);
    // S^T[16 keys][16 heads]: lane holds keys 4g + i of head col.
    f32x4 s = f32x4{};
#pragma unroll
    for (int k = 0; k < DK / 32; ++k) {
      const bf16x8 kv = *(const lds_bf16x8*)(st + ko[k % 4] + (k / 4) * 256);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qf[k], s, 0, 0, 0);
    }
    const int key0 = c0 + t * kRBN + 16 * wr + 4 * g;
    // Edge tiles only: the chunk's end, the new tokens' own rows (each sees
    // the rows up to its own) and a window's start (later tokens start later).
    if (c0 + t * kRBN < mask_lo || c0 + (t + 1) * kRBN > mask_hi) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = (key0 + i >= col_lo && key0 + i < col_hi) ? s[i] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = xor32_16_max(mx);
    const float mc = (mx == -INFINITY) ? -INFINITY : mx * c2;
    if (__any(mc > m_run + 8.f)) {  // move the max only when it grows by 2^8
      const float m_new = fmaxf(m_run, mc);
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < DV / 16; ++d) oacc[d] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    f32x4 p;
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -m_use));
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    const s16x4 pb = __builtin_bit_cast(s16x4, __builtin_convertvector(p, bf16x4));
#pragma unroll
    for (int d = 0; d < DV / 16; ++d) {
      const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4*)(st + vo[d % 8] + (d / 8) * 256));
      oacc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, v), pb,
                                                          oacc[d], 0, 0, 0);
    }
    wait_vm<(C::AHEAD - 1) * DMA_W>();  // tile t+1 landed
    lds_barrier();
    cur = cur == C::AHEAD ? 0 : cur + 1;
  }
  wait_vm<0>();
  lds_barrier();  // every wave is done with the ring before it is reused

  // The 4 lanes of a head (col, col+16, col+32, col+48) hold different keys
  // under the same running max: sum their sums.
  l_run = xor32_16_sum(l_run);

  // ---- merge each group's row waves through LDS, write this split's
  // partial; the groups take turns in the same LDS area ------------------------
  float* red = reinterpret_cast<float*>(lds);  // [row wave][16][DV + 2]
  const int RS = DV + 2;
  float* part = reinterpret_cast<float*>(a.workspace);
#pragma unroll
  for (int gi = 0; gi < NGW; ++gi) {
    if (gi > 0) __syncthreads();  // the previous group's reads are done
    if (wg == gi) {
      float* wrp = red + (wr * 16 + col) * RS;
      if (g == 0) {
        wrp[DV] = m_run;
        wrp[DV + 1] = l_run;
      }
      // O^T layout: lane holds dims 16d + 4g + i of head col.
#pragma unroll
      for (int d = 0; d < DV / 16; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) wrp[16 * d + 4 * g + i] = oacc[d][i];
    }
    __syncthreads();
    if (n_split == 1) {  // one chunk per sequence: normalise and write o here
      for (int idx = tid; idx < 16 * DV; idx += kW * 64) {
        const int h = idx / DV, d = idx % DV;
        if (!col_ok_g(gi, h)) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kRW; ++w) M = fmaxf(M, red[(w * 16 + h) * RS + DV]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < kRW; ++w) {
          const float f = exp2f(red[(w * 16 + h) * RS + DV] - M);
          num += f * red[(w * 16 + h) * RS + d];
          den += f * red[(w * 16 + h) * RS + DV + 1];
        }
        ((uint16_t*)a.o)[col_row_g(gi, h) * DV + d] = f32_to_bf16(num / den);
      }
    } else {
      for (int idx = tid; idx < 16 * (DV + 2); idx += kW * 64) {
        const int h = idx / (DV + 2), d = idx % (DV + 2);
        if (!col_ok_g(gi, h)) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kRW; ++w) M = fmaxf(M, red[(w * 16 + h) * RS + DV]);
        float val = 0.f;
        if (d == DV) {
          val = M;
        } else if (M != -INFINITY) {
#pragma unroll
          for (int w = 0; w < kRW; ++w) {
            const float f = exp2f(red[(w * 16 + h) * RS + DV] - M);
            val += f * red[(w * 16 + h) * RS + d];
          }
        }
        const int64_t slot = col_row_g(gi, h) * n_split + split;
        part[slot * (DV + 2) + d] = val;  // d == DV+1 sums the l's by the same rule
      }
    }
  }
}

// Merge the splits of one (sequence, token, query head):
// O = sum_c f_c acc_c / sum_c f_c l_c. A chunk with no row a token sees holds
// m = -inf and adds nothing.
template <int DV>
__global__ __launch_bounds__(DV) void decode_merge_kernel(DecodeArgs a, int ch, int n_split) {
  const int bh = blockIdx.x;  // (b * n_q + j) * Hq + h
  const int b = bh / (a.n_q * a.Hq);
  const int kv_len = a.kv_len[b];
  uint16_t* o = (uint16_t*)a.o + (int64_t)bh * DV;
  const int d = threadIdx.x;
  if (d >= DV) return;
  if (kv_len <= 0 || kv_len > a.max_kv_len || kv_len < a.n_q) {
    // kv_len == 0: no rows, o = 0. Out of range: poison the row (NaN).
    o[d] = (kv_len == 0) ? 0 : 0x7fc0;
    return;
  }
  const int lo = (a.window > 0) ? max(0, kv_len - a.n_q + 1 - a.window) : 0;
  const int n = (kv_len - lo + ch - 1) / ch;
  const float* part = reinterpret_cast<const float*>(a.workspace) + (int64_t)bh * n_split * (DV + 2);
  float M = -INFINITY;
  for (int c = 0; c < n; ++c) M = fmaxf(M, part[c * (DV + 2) + DV]);
  float num = 0.f, den = 0.f;
  for (int c = 0; c < n; ++c) {
    const float* pc = part + c * (DV + 2);
    const float f = exp2f(pc[DV] - M);
    num += f * pc[d];
    den += f * pc[DV + 1];
  }
  o[d] = f32_to_bf16(num / den);
}

// Ring shapes (measured on the decode workload). With one wave per SIMD a
// workgroup's MFMA/LDS latency goes unhidden, so the heavier-per-byte cases
// trade ring depth for more workgroups per CU:
//  * separate 512/256 caches: 2 waves (32-row tiles), 3 stages;
//  * local 256/256 heads: 2 waves (32-row tiles), 2 stages (the local call
//    of the decode workload: 0.089 ms against 0.091-0.093 with 1 wave x 3
//    stages);
//  * one shared cache (K = V): 2 waves (32-row tiles), 2 stages. On the
//    K = V global shape this runs at 6.0 TB/s, 1 wave x 2 stages at 5.7 and
//    2 waves x 4 stages at 4.1;
//  * separate caches with 512-dim values: 1 wave, 2 stages, two workgroups
//    per CU.
template <int DK, int DV, bool SHARED>
using RingCfg = std::conditional_t<
    SHARED, RCfg<DK, DV, 2, 2, SHARED>,
    std::conditional_t<(DK == 512 && DV == 512), RCfg<DK, DV, 1, 2, SHARED>,
    std::conditional_t<(DK == 256 && DV == 256), RCfg<DK, DV, 2, 2>, RCfg<DK, DV, 2, 3>>>>;

template <int DV>
hipError_t launch_merge_dv(const DecodeArgs& a, const SplitPlan& pl, hipStream_t st) {
  hipLaunchKernelGGL((decode_merge_kernel<DV>), dim3(a.B * a.n_q * a.Hq), dim3(DV), 0, st, a,
                     pl.ch, pl.ns);
  return hipGetLastError();
}

template <int DK, int DV, bool SHARED, int NGW>
hipError_t launch_ring(const DecodeArgs& a, const SplitPlan& pl, int ncb, hipStream_t st) {
  using C = RingCfg<DK, DV, SHARED>;
  // Chunk-relative 32-bit buffer offsets: ch rows plus the read-ahead tiles.
  const int64_t row = (int64_t)a.Hkv * (DK > DV ? DK : DV) * 2;
  static_assert((C::STAGES + 1) * C::RBN <= 192, "read-ahead bound of decode_shape_fits");
  if (((int64_t)pl.ch + (C::STAGES + 1) * C::RBN) * row >= ((int64_t)1 << 31))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_ring_kernel<C, DK, DV, NGW>), dim3(a.Hkv * ncb, pl.ns, a.B),
                     dim3(C::RW * NGW * 64), 0, st, a, pl.ch, pl.ns);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.ns == 1) return e;  // one chunk: the ring kernel wrote o
  return launch_merge_dv<DV>(a, pl, st);
}

template <int DK, int DV, int NGW>
hipError_t launch_dk_dv_g(const DecodeArgs& a, int ncb, hipStream_t st) {
  const SplitPlan pl = decode_plan(a.B, a.Hkv * ncb, a.max_kv_len, a.window, a.n_q);
  if (pl.ns > 65535) return hipErrorInvalidValue;
  if constexpr (DK == DV) {
    if (a.k_cache == a.v_cache) return launch_ring<DK, DV, true, NGW>(a, pl, ncb, st);
  }
  return launch_ring<DK, DV, false, NGW>(a, pl, ncb, st);
}

// Column groups per workgroup: up to four when a verify call has more (token,
// head) pairs per KV head than one 16-column group holds (each cache row is
// then read once for all of them), one otherwise.
template <int DK, int DV>
hipError_t launch_dk_dv(const DecodeArgs& a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const int ncb = decode_column_blocks(a.n_q, G);
  const int ngw = decode_groups_per_block(a.n_q, G);
  if (ngw == 4) return launch_dk_dv_g<DK, DV, 4>(a, ncb, st);
  if (ngw == 2) return launch_dk_dv_g<DK, DV, 2>(a, ncb, st);
  return launch_dk_dv_g<DK, DV, 1>(a, ncb, st);
}

// Several new tokens: turn every query once at its own position
// (kv_len - n_q + j) into the workspace, in the arithmetic of the one-token
// path (fp64 angle, fp32 rotation of the bf16 pair, bf16 result).
__global__ __launch_bounds__(256) void verify_rotate_q_kernel(DecodeArgs a, uint32_t* out) {
  const int P = a.Dk / 2;
  const int64_t total = (int64_t)a.B * a.n_q * a.Hq * P;
  const double l2t = log2(a.theta);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int p = (int)(i % P);
    const int64_t bj = i / P / a.Hq;  // b * n_q + j
    const int b = (int)(bj / a.n_q), j = (int)(bj % a.n_q);
    uint32_t w = reinterpret_cast<const uint32_t*>(a.q)[i];
    if (p < a.rot_pairs) {
      const int pos = max(0, a.kv_len[b] - a.n_q + j);
      float c, sn;
      rope_cos_sin(pos, rope_freq(p, a.Dk, l2t), &c, &sn);
      const float x0 = bf16_lo(w), x1 = bf16_hi(w);
      w = pack_bf16x2(x0 * c - x1 * sn, x0 * sn + x1 * c);
    }
    out[i] = w;
  }
}

}  // namespace

hipError_t launch_decode_merge(const DecodeArgs& a, const SplitPlan& pl, hipStream_t st) {
  switch (a.Dv) {
    case 128: return launch_merge_dv<128>(a, pl, st);
    case 256: return launch_merge_dv<256>(a, pl, st);
    case 512: return launch_merge_dv<512>(a, pl, st);
    default: return hipErrorNotSupported;
  }
}

// Scratch of the decode entry point that allocates nothing: the split-K
// partials live in this file-scope device array, one copy per GPU, held until
// the process ends. Host code must never pass the array's name to a kernel
// (on the host it is only a stand-in for the symbol): the device address of
// each GPU's copy comes from hipGetSymbolAddress, taken once per device with
// that device current, and is cached here.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a0, hipStream_t st) {
  if (a0.B == 0) return hipSuccess;
  DecodeArgs a = a0;
  if (a0.n_q > 1) {
    uint32_t* qr = static_cast<uint32_t*>(a0.workspace);
    const int64_t total = (int64_t)a0.B * a0.n_q * a0.Hq * (a0.Dk / 2);
    const int blocks = (int)std::min<int64_t>((total + 255) / 256, 8192);
    hipLaunchKernelGGL(verify_rotate_q_kernel, dim3(blocks), dim3(256), 0, st, a0, qr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.q = qr;
    a.q_rotated = 1;
    a.workspace = static_cast<char*>(a0.workspace) + decode_rotated_q_bytes(a0.B, a0.n_q, a0.Hq, a0.Dk);
  }
#define ATTN_DEC(DK, DV) \
  if (a.Dk == DK && a.Dv == DV) return launch_dk_dv<DK, DV>(a, st);
  ATTN_DEC(512, 256)
  ATTN_DEC(512, 512)
  ATTN_DEC(256, 256)
  ATTN_DEC(128, 128)
  ATTN_DEC(512, 128)
  ATTN_DEC(256, 128)
  ATTN_DEC(128, 256)
#undef ATTN_DEC
  return hipErrorNotSupported;
}

}  // namespace attn
