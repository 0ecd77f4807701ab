// decode.hip — single-token GQA decode over a ragged bf16 KV cache on gfx950:
// split-K partial kernel + log-sum-exp merge kernel.
//
// What it computes (Gemma 4 pages): the new token attends every cached row of
// a global layer or the last W rows of a local one ("Gemma 4: End-to-End
// Architecture Walkthrough", Phase 3 sections 3a-3b: global layers must keep
// K/V for the whole context, which is why decode is bound by reading that
// cache); 8 (global) or 2 (local) query heads share each KV head; the query is
// rotated with (p-)RoPE at its own position (section 3c), cached keys are
// stored already rotated.
//
// Design for CDNA4 (HBM-bound: ~8 FLOP per cache byte with 8 heads/KV head):
//  * Grid = (splits, KV heads, sequences). A workgroup streams one chunk of
//    one sequence's rows for one KV head and serves all G query heads of that
//    KV head from the same bytes.
//  * Q.K^T runs on v_mfma_f32_16x16x32_bf16 with keys as the M dimension and
//    the G heads (padded to 16) as N: each lane loads its K operand (16 bytes
//    of one key row) straight from HBM into registers — no LDS round trip.
//  * V rows are loaded with fully coalesced 16-byte loads into a per-wave LDS
//    tile; the transposed P.V operand is gathered from there in the key order
//    that matches the score layout, so P^T is the lane's own scores.
//  * Each wave keeps its own online-softmax state; the 4 waves merge through
//    LDS at the end into one (max, sum, acc) partial per (sequence, head,
//    split), and a second kernel merges the splits.
#include "attn_common.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kNW = 4;  // waves per workgroup

// Rows of one sequence handled by one workgroup.
__host__ __device__ inline int decode_chunk_rows(int window) { return window > 0 ? 512 : 1024; }

__host__ __device__ inline int decode_splits(int max_kv_len, int window) {
  const int range = (window > 0 && window < max_kv_len) ? window : max_kv_len;
  const int ch = decode_chunk_rows(window);
  return (range + ch - 1) / ch;
}

template <int DK, int DV>
struct DCfg {
  static constexpr int VS = DV + 16;            // V row stride in LDS (elements)
  static constexpr int VTILE = 32 * VS;         // per-wave V tile (elements)
  static constexpr int VCH = 32 * (DV / 8) / 64;  // 16-byte V chunks per lane
};

template <int DK, int DV>
__global__ __launch_bounds__(kNW * 64) void decode_partial_kernel(DecodeArgs a, int n_split) {
  using C = DCfg<DK, DV>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[kNW * C::VTILE];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp4 = lane >> 4;  // MFMA column (head) and k-group
  const int G = a.Hq / a.Hkv;

  const int kv_len = a.kv_len[b];
  if (kv_len <= 0 || kv_len > a.max_kv_len) return;  // merge handles these
  const int lo = (a.window > 0) ? max(0, kv_len - a.window) : 0;
  const int ch = decode_chunk_rows(a.window);
  const int c0 = lo + split * ch;
  if (c0 >= kv_len) return;
  const int c1 = min(kv_len, c0 + ch);
  const int64_t off = a.row_offset[b];
  const int qpos = kv_len - 1;

  // ---- rotated queries as the B operand: col = head, k = dims -------------
  bf16x8 qf[DK / 32];
  {
    const bool hv = col < G;
    const int head = kvh * G + (hv ? col : 0);
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)b * a.Hq + head) * DK;
    const double l2t = log2(a.theta);
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
      const int d0 = 32 * s + 8 * grp4;
      u32x4 w = *(const u32x4*)(qrow + d0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = d0 / 2 + e;
        if (p < a.rot_pairs) {
          float c, sn;
          rope_cos_sin(qpos, rope_freq(p, DK, l2t), &c, &sn);
          const float x0 = bf16_lo(w[e]), x1 = bf16_hi(w[e]);
          w[e] = pack_bf16x2(x0 * c - x1 * sn, x0 * sn + x1 * c);
        }
      }
      if (!hv) w = u32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const uint16_t* kbase = (const uint16_t*)a.k_cache + (off * a.Hkv + kvh) * DK;
  const uint16_t* vbase = (const uint16_t*)a.v_cache + (off * a.Hkv + kvh) * DV;
  const int64_t krs = (int64_t)a.Hkv * DK, vrs = (int64_t)a.Hkv * DV;
  uint16_t* vt = lds + wave * C::VTILE;
  const float c2 = a.scale * kLog2e;

  float m_run = -INFINITY, l_run = 0.f;  // per head `col`
  f32x4 oacc[DV / 16];
#pragma unroll
  for (int d = 0; d < DV / 16; ++d) oacc[d] = f32x4{};

  for (int k0 = c0 + 32 * wave; k0 < c1; k0 += 32 * kNW) {
    // K operands for two 16-key sub-blocks and the V tile, all in flight.
    u32x4 kr[2][DK / 32];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int key = k0 + 16 * sb + col;
      const bool in = key < c1;
      const uint16_t* kp = kbase + (int64_t)(in ? key : c0) * krs + 8 * grp4;
#pragma unroll
      for (int s = 0; s < DK / 32; ++s)
        kr[sb][s] = in ? *(const u32x4*)(kp + 32 * s) : u32x4{0, 0, 0, 0};
    }
    u32x4 vr[C::VCH];
#pragma unroll
    for (int it = 0; it < C::VCH; ++it) {
      const int c = lane + 64 * it;
      const int key = c / (DV / 8), d8 = c % (DV / 8);
      const int kk = k0 + key;
      vr[it] = (kk < c1) ? *(const u32x4*)(vbase + (int64_t)kk * vrs + 8 * d8)
                         : u32x4{0, 0, 0, 0};
    }

    // S^T[16 keys][16 heads] per sub-block; lane holds keys 4*grp4 + i.
    f32x4 s[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      s[sb] = f32x4{};
#pragma unroll
      for (int st = 0; st < DK / 32; ++st)
        s[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, kr[sb][st]), qf[st], s[sb], 0, 0, 0);
    }
    float mx = -INFINITY;
    const bool tail = (k0 + 32 > c1);
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + 16 * sb + 4 * grp4 + i;
        if (tail && key >= c1) s[sb][i] = -INFINITY;
        mx = fmaxf(mx, s[sb][i]);
      }
    mx = xor32_16_max(mx);
    const float m_new = fmaxf(m_run, mx * c2);
    const float alpha = exp2f(m_run - m_new);
    float pv[8], psum = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float p = exp2f(fmaf(s[sb][i], c2, -m_new));
        if (tail && k0 + 16 * sb + 4 * grp4 + i >= c1) p = 0.f;
        pv[4 * sb + i] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < DV / 16; ++d) oacc[d] *= alpha;

    // V tile -> LDS (row-major, padded), then gather the transposed operand:
    // slot (grp4, i) <-> key 16*(i/4) + 4*grp4 + (i%4).
#pragma unroll
    for (int it = 0; it < C::VCH; ++it) {
      const int c = lane + 64 * it;
      const int key = c / (DV / 8), d8 = c % (DV / 8);
      *(u32x4*)(vt + key * C::VS + 8 * d8) = vr[it];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    f32x4 plo = {pv[0], pv[1], pv[2], pv[3]}, phi = {pv[4], pv[5], pv[6], pv[7]};
    const bf16x4 pa = __builtin_convertvector(plo, bf16x4);
    const bf16x4 pb = __builtin_convertvector(phi, bf16x4);
    const bf16x8 pop = __builtin_shufflevector(pa, pb, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int d = 0; d < DV / 16; ++d) {
      const int dim = 16 * d + col;
      uint16_t e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = vt[(16 * (i / 4) + 4 * grp4 + (i % 4)) * C::VS + dim];
      const u32x4 w = {(uint32_t)e[0] | ((uint32_t)e[1] << 16),
                       (uint32_t)e[2] | ((uint32_t)e[3] << 16),
                       (uint32_t)e[4] | ((uint32_t)e[5] << 16),
                       (uint32_t)e[6] | ((uint32_t)e[7] << 16)};
      oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), pop,
                                                        oacc[d], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // Each lane's running sum covers only its own keys; the 4 lanes of a head
  // (col, col+16, col+32, col+48) share the same running max, so sum them.
  l_run = xor32_16_sum(l_run);

  // ---- merge the 4 waves through LDS, write this split's partial ---------
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);  // [wave][16][DV + 2]
  const int RS = DV + 2;
  {
    float* wr = red + (wave * 16 + col) * RS;
    if (grp4 == 0) {
      wr[DV] = m_run;
      wr[DV + 1] = l_run;
    }
    // O^T layout: lane holds dims 16d + 4*grp4 + i of head `col`.
#pragma unroll
    for (int d = 0; d < DV / 16; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) wr[16 * d + 4 * grp4 + i] = oacc[d][i];
  }
  __syncthreads();
  float* part = reinterpret_cast<float*>(a.workspace);
  for (int idx = tid; idx < G * (DV + 2); idx += kNW * 64) {
    const int h = idx / (DV + 2), d = idx % (DV + 2);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, red[(w * 16 + h) * RS + DV]);
    float val = 0.f;
    if (d == DV) {
      val = M;
    } else if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kNW; ++w) {
        const float f = exp2f(red[(w * 16 + h) * RS + DV] - M);
        val += f * red[(w * 16 + h) * RS + d];
      }
    }
    const int64_t slot = ((int64_t)b * a.Hq + kvh * G + h) * n_split + split;
    part[slot * (DV + 2) + d] = val;  // d == DV+1 sums the l's via the same rule
  }
}

// ---- streaming kernel: K/V tiles through an LDS DMA ring -------------------
// Decode is bound by the bytes of the cache, and there is little arithmetic
// per byte, so this kernel is built around keeping bytes in flight: 2 waves
// stream 32-row tiles (K and V) into a 3-stage LDS ring by DMA, two tiles
// ahead, with no staging registers; each wave takes 16 of a tile's rows.
// S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (16 keys x 16 head columns), then
// O^T += V^T P^T on v_mfma_f32_16x16x16_bf16: the P^T operand (keys 4g..4g+3
// of head col) is exactly what the score MFMA left in the lane, and V^T comes
// from one transposing LDS read (ds_read_b64_tr_b16) per MFMA.
constexpr int kRW = 2;    // waves per workgroup
constexpr int kRBN = 32;  // rows per tile (16 per wave)

template <int DK, int DV>
struct RCfg {
  static constexpr int KC = DK / 8, VC = DV / 8;  // 16-byte chunks per row
  static constexpr int KT = kRBN * DK * 2, VT = kRBN * DV * 2;
  static constexpr int ST = KT + VT;
  static constexpr int STAGES = 3;
  static constexpr int LDS = STAGES * ST;
  static constexpr int K_DMA = KT / 1024, N_DMA = ST / 1024;
  static constexpr int DMA_W = N_DMA / kRW;  // DMAs per wave per tile
  static_assert(KC >= 16 && VC >= 16, "row swizzle uses 16 chunk groups");
  static_assert(K_DMA % kRW == 0 && N_DMA % kRW == 0, "uniform DMA counts");
  static_assert(DMA_W < 64 && LDS <= 160 * 1024, "vmcnt / LDS limits");
};

template <int DK, int DV>
__global__ __launch_bounds__(kRW * 64, 1) void decode_ring_kernel(DecodeArgs a, int n_split) {
  using C = RCfg<DK, DV>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int G = a.Hq / a.Hkv;

  const int kv_len = a.kv_len[b];
  if (kv_len <= 0 || kv_len > a.max_kv_len) return;  // the merge handles these
  const int lo = (a.window > 0) ? max(0, kv_len - a.window) : 0;
  const int ch = decode_chunk_rows(a.window);
  const int c0 = lo + split * ch;
  if (c0 >= kv_len) return;
  const int c1 = min(kv_len, c0 + ch);
  const int n_tiles = (c1 - c0 + kRBN - 1) / kRBN;
  const int64_t off = a.row_offset[b];

  // Descriptors over this sequence's rows of KV head kvh: rows past kv_len
  // read 0 (they are never inside [c0, c1) and their scores are masked).
  const int krow = a.Hkv * DK * 2, vrow = a.Hkv * DV * 2;
  const u32x4 kdesc = buffer_desc((const char*)a.k_cache + (off * a.Hkv + kvh) * DK * 2,
                                  (uint32_t)((int64_t)(kv_len - 1) * krow + DK * 2));
  const u32x4 vdesc = buffer_desc((const char*)a.v_cache + (off * a.Hkv + kvh) * DV * 2,
                                  (uint32_t)((int64_t)(kv_len - 1) * vrow + DV * 2));
  // Block n (n = i*kRW + wave) of a tile holds 64 chunks; K rows first, then V
  // rows, each row's chunks XOR-swizzled by (row & 15).
  uint32_t dma_off[C::DMA_W];
#pragma unroll
  for (int i = 0; i < C::DMA_W; ++i) {
    const int n = i * kRW + wave;
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
    const int j0 = c0 + t * kRBN;
    const uint32_t st = lds_addr(lds) + stage * C::ST;
    const uint32_t far = t < n_tiles ? 0u : 0x80000000u;
#pragma unroll
    for (int i = 0; i < C::DMA_W; ++i) {
      const int n = i * kRW + wave;
      if (i * kRW < C::K_DMA)  // same region for both waves (K_DMA % kRW == 0)
        dma16<true>(kdesc, st + n * 1024, (dma_off[i] + j0 * krow) | far);
      else
        dma16<true>(vdesc, st + n * 1024, (dma_off[i] + j0 * vrow) | far);
    }
  };
  dma_tile(0, 0);

  // ---- rotated queries as the B operand: col = head, k = dims -------------
  // The angle of each rotary pair is formed once per wave (one pair per lane,
  // fp64) into a small LDS table; every lane then reads the pairs it holds.
  __shared__ float2 cs_tab[kRW][DK / 2];
  bf16x8 qf[DK / 32];
  {
    const int qpos = kv_len - 1;
    const double l2t = log2(a.theta);
    for (int p = lane; p < a.rot_pairs; p += 64) {
      float c, sn;
      rope_cos_sin(qpos, rope_freq(p, DK, l2t), &c, &sn);
      cs_tab[wave][p] = make_float2(c, sn);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const bool hv = col < G;
    const int head = kvh * G + (hv ? col : 0);
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)b * a.Hq + head) * DK;
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
      const int d0 = 32 * s + 8 * g;
      u32x4 w = *(const u32x4*)(qrow + d0);
      if (d0 / 2 < a.rot_pairs) {  // rot_pairs is a multiple of 4: all 4 pairs turn
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float2 t = cs_tab[wave][d0 / 2 + e];
          const float x0 = bf16_lo(w[e]), x1 = bf16_hi(w[e]);
          w[e] = pack_bf16x2(x0 * t.x - x1 * t.y, x0 * t.y + x1 * t.x);
        }
      }
      if (!hv) w = u32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }
  dma_tile(1, 1);  // may lie past c1: masked, or past kv_len: zeros
  wait_vm<C::DMA_W>();
  lds_barrier();

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
    const int krow_l = (16 * wave + col) * C::KC * 16 + ((g ^ (col & 3)) << 4);
#pragma unroll
    for (int B = 0; B < 4; ++B) ko[B] = krow_l + ((B ^ (col >> 2)) << 6);
    const int x = 4 * g + (col >> 2), c4 = col & 3;
    const int vrow_l = C::KT + (16 * wave + x) * C::VC * 16 +
                       ((((c4 >> 1) ^ (x & 1))) << 4) + ((c4 & 1) << 3);
#pragma unroll
    for (int B = 0; B < 8; ++B) vo[B] = vrow_l + ((B ^ (x >> 1)) << 5);
  }

  int cur = 0;
  for (int t = 0; t < n_tiles; ++t) {
    dma_tile(t + 2, cur == 0 ? 2 : cur - 1);
    const lds_u8* st = (const lds_u8*)lds + __builtin_amdgcn_readfirstlane(cur * C::ST);
    // S^T[16 keys][16 heads]: lane holds keys 4g + i of head col.
    f32x4 s = f32x4{};
#pragma unroll
    for (int k = 0; k < DK / 32; ++k) {
      const bf16x8 kv = *(const lds_bf16x8*)(st + ko[k % 4] + (k / 4) * 256);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qf[k], s, 0, 0, 0);
    }
    const int key0 = c0 + t * kRBN + 16 * wave + 4 * g;
    if (c0 + (t + 1) * kRBN > c1) {  // last tile of the chunk: mask rows >= c1
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = (key0 + i < c1) ? s[i] : -INFINITY;
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
    wait_vm<C::DMA_W>();  // tile t+1 landed
    lds_barrier();
    cur = cur == 2 ? 0 : cur + 1;
  }
  wait_vm<0>();
  lds_barrier();  // every wave is done with the ring before it is reused

  // The 4 lanes of a head (col, col+16, col+32, col+48) hold different keys
  // under the same running max: sum their sums.
  l_run = xor32_16_sum(l_run);

  // ---- merge the 2 waves through LDS, write this split's partial ---------
  float* red = reinterpret_cast<float*>(lds);  // [wave][16][DV + 2]
  const int RS = DV + 2;
  {
    float* wr = red + (wave * 16 + col) * RS;
    if (g == 0) {
      wr[DV] = m_run;
      wr[DV + 1] = l_run;
    }
    // O^T layout: lane holds dims 16d + 4g + i of head col.
#pragma unroll
    for (int d = 0; d < DV / 16; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) wr[16 * d + 4 * g + i] = oacc[d][i];
  }
  __syncthreads();
  float* part = reinterpret_cast<float*>(a.workspace);
  for (int idx = tid; idx < G * (DV + 2); idx += kRW * 64) {
    const int h = idx / (DV + 2), d = idx % (DV + 2);
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
    const int64_t slot = ((int64_t)b * a.Hq + kvh * G + h) * n_split + split;
    part[slot * (DV + 2) + d] = val;  // d == DV+1 sums the l's by the same rule
  }
}

// Merge the splits of one (sequence, query head): O = sum_c f_c acc_c / sum_c f_c l_c.
template <int DV>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a, int n_split) {
  const int bh = blockIdx.x;
  const int b = bh / a.Hq;
  const int kv_len = a.kv_len[b];
  uint16_t* o = (uint16_t*)a.o + (int64_t)bh * DV;
  const int d = threadIdx.x;
  if (d >= DV) return;
  if (kv_len <= 0 || kv_len > a.max_kv_len) {
    // kv_len == 0: no rows, o = 0. Out of range: poison the row (NaN).
    o[d] = (kv_len == 0) ? 0 : 0x7fc0;
    return;
  }
  const int lo = (a.window > 0) ? max(0, kv_len - a.window) : 0;
  const int ch = decode_chunk_rows(a.window);
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

// The streaming kernel addresses one sequence's cache rows with 32-bit
// buffer offsets: kv_len rows (plus two tiles of read-ahead) of all KV heads.
// It also turns the query 4 pairs (one 16-byte chunk) at a time.
template <int DK, int DV>
bool ring_fits(const DecodeArgs& a) {
  const int64_t row = (int64_t)a.Hkv * (DK > DV ? DK : DV) * 2;
  return ((int64_t)a.max_kv_len + 3 * kRBN) * row < ((int64_t)1 << 31) && a.rot_pairs % 4 == 0;
}

template <int DK, int DV>
hipError_t launch_dk_dv(const DecodeArgs& a, hipStream_t st) {
  const int ns = decode_splits(a.max_kv_len, a.window);
  if (ring_fits<DK, DV>(a))
    hipLaunchKernelGGL((decode_ring_kernel<DK, DV>), dim3(ns, a.Hkv, a.B), dim3(kRW * 64), 0,
                       st, a, ns);
  else
    hipLaunchKernelGGL((decode_partial_kernel<DK, DV>), dim3(ns, a.Hkv, a.B),
                       dim3(kNW * 64), 0, st, a, ns);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<DV>), dim3(a.B * a.Hq), dim3(256), 0, st, a, ns);
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int B, int Hq, int Dv, int max_kv_len, int window) {
  if (B <= 0 || Hq <= 0 || Dv <= 0 || max_kv_len <= 0) return 0;
  const int ns = decode_splits(max_kv_len, window);
  return (size_t)B * Hq * ns * (Dv + 2) * sizeof(float);
}

bool decode_supported(int Dk, int Dv, int G) {
  return (Dk == 128 || Dk == 256 || Dk == 512) && (Dv == 128 || Dv == 256) && G >= 1 &&
         G <= 16;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
#define ATTN_DEC(DK, DV) \
  if (a.Dk == DK && a.Dv == DV) return launch_dk_dv<DK, DV>(a, st);
  ATTN_DEC(512, 256)
  ATTN_DEC(256, 256)
  ATTN_DEC(128, 128)
  ATTN_DEC(512, 128)
  ATTN_DEC(256, 128)
  ATTN_DEC(128, 256)
#undef ATTN_DEC
  return hipErrorNotSupported;
}

}  // namespace attn
