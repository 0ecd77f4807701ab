// prefill_general.hip — general causal / sliding-window GQA prefill for any
// supported head shape, fp32 or bf16 (correctness path; the MFMA kernel is
// the fast path for the model's shapes).
//
// Computes softmax(scale * rope(q) rope(k)^T + mask) v as the Gemma 4 pages
// describe it ("Gemma 4: End-to-End Architecture Walkthrough", Phase 3
// sections 3a-3c): query i of a local layer sees keys i-W+1..i, of a global
// layer keys 0..i; query head h reads KV head h / (Hq/Hkv).
//
// One wavefront per (batch, query head, query row). Lane l owns dimension
// pairs l, l+64, ... of q/k and of v/o, so RoPE pairs stay inside a lane. The
// query's angles are formed in fp64 here; K's rotary pairs arrive turned by
// the pre-pass (k_rot).
// Keys stream in order with an online softmax (running max and sum in fp32).
#include "attn_common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int kMaxPairs = 4;  // head dims up to 512

template <bool BF16>
__device__ __forceinline__ float2 load_pair(const void* base, int64_t elem) {
  if constexpr (BF16) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(base)[elem / 2];
    return make_float2(bf16_lo(w), bf16_hi(w));
  } else {
    return reinterpret_cast<const float2*>(base)[elem / 2];
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void prefill_general_kernel(PrefillArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row_id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t n_rows = (int64_t)a.B * a.T * a.Hq;
  if (row_id >= n_rows) return;
  const int h = (int)(row_id % a.Hq);
  const int i = (int)((row_id / a.Hq) % a.T);
  const int b = (int)(row_id / ((int64_t)a.Hq * a.T));
  const int G = a.Hq / a.Hkv;
  const int g = h / G;
  const int PK = a.Dk / 2, PV = a.Dv / 2;

  // The query pairs this lane owns, rotated at position pos0 + i (angles in
  // fp64).
  float2 q[kMaxPairs];
#pragma unroll
  for (int e = 0; e < kMaxPairs; ++e) {
    const int p = lane + 64 * e;
    q[e] = make_float2(0.f, 0.f);
    if (p < PK) {
      float2 x = load_pair<BF16>(a.q, (((int64_t)b * a.T + i) * a.Hq + h) * a.Dk + 2 * p);
      if (a.rope_q && p < a.rot_pairs) {
        float c, sn;
        rope_cos_sin((int64_t)a.pos0 + i, rope_freq(p, a.Dk, a.log2_theta), &c, &sn);
        x = make_float2(x.x * c - x.y * sn, x.x * sn + x.y * c);
      }
      q[e] = x;
    }
  }

  float m = -INFINITY, l = 0.f;
  float2 acc[kMaxPairs];
#pragma unroll
  for (int e = 0; e < kMaxPairs; ++e) acc[e] = make_float2(0.f, 0.f);

  const int lo = (a.window > 0) ? max(0, i - a.window + 1) : 0;
  for (int j = lo; j <= i; ++j) {
    const int64_t kbase = (((int64_t)b * a.T + j) * a.Hkv + g) * a.Dk;
    const int64_t krbase = (((int64_t)b * a.T + j) * a.Hkv + g) * (2 * a.rot_pairs);
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < kMaxPairs; ++e) {
      const int p = lane + 64 * e;
      if (p < PK) {
        // K's rotary pairs come turned from the pre-pass (k_rot).
        const float2 kx = (a.rope_k && p < a.rot_pairs)
                              ? load_pair<BF16>(a.k_rot, krbase + 2 * p)
                              : load_pair<BF16>(a.k, kbase + 2 * p);
        part += q[e].x * kx.x + q[e].y * kx.y;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    const float s = part * a.scale;
    const float m_new = fmaxf(m, s);
    const float alpha = __expf(m - m_new);
    const float p = __expf(s - m_new);
    l = l * alpha + p;
    m = m_new;
    const int64_t vbase = (((int64_t)b * a.T + j) * a.Hkv + g) * a.Dv;
#pragma unroll
    for (int e = 0; e < kMaxPairs; ++e) {
      const int pp = lane + 64 * e;
      if (pp < PV) {
        const float2 vx = load_pair<BF16>(a.v, vbase + 2 * pp);
        acc[e].x = acc[e].x * alpha + p * vx.x;
        acc[e].y = acc[e].y * alpha + p * vx.y;
      }
    }
  }

  const float inv = 1.f / l;
  const int64_t obase = (((int64_t)b * a.T + i) * a.Hq + h) * a.Dv;
#pragma unroll
  for (int e = 0; e < kMaxPairs; ++e) {
    const int pp = lane + 64 * e;
    if (pp < PV) {
      const float y0 = acc[e].x * inv, y1 = acc[e].y * inv;
      if constexpr (BF16)
        reinterpret_cast<uint32_t*>(a.o)[(obase + 2 * pp) / 2] = pack_bf16x2(y0, y1);
      else
        reinterpret_cast<float2*>(a.o)[(obase + 2 * pp) / 2] = make_float2(y0, y1);
    }
  }
}

}  // namespace

hipError_t launch_prefill_general(const PrefillArgs& a, bool bf16, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.T * a.Hq;
  const int64_t blocks = (rows + 3) / 4;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(prefill_general_kernel<true>, dim3((unsigned)blocks), dim3(256),
                       0, st, a);
  else
    hipLaunchKernelGGL(prefill_general_kernel<false>, dim3((unsigned)blocks), dim3(256),
                       0, st, a);
  return hipGetLastError();
}

}  // namespace attn
