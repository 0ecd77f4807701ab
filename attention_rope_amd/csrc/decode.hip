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
__host__ __device__ inline int decode_chunk_rows(int window) { return window > 0 ? 256 : 1024; }

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

template <int DK, int DV>
hipError_t launch_dk_dv(const DecodeArgs& a, hipStream_t st) {
  const int ns = decode_splits(a.max_kv_len, a.window);
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
