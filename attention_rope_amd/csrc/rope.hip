// rope.hip — rotary position embedding kernels for gfx950.
//
// (p-)RoPE as the Gemma 4 pages state it ("Gemma 4: End-to-End Architecture
// Walkthrough", Phase 3 section 3c; "Gemma 4 Architecture Reference",
// "Positional Encoding: Proportional RoPE (p-RoPE)"): the high-frequency
// leading pairs of each head vector turn with the token position, the
// remaining pairs are left alone (p = 0.25 keeps three quarters fixed).
// Pair p = dims (2p, 2p+1) turns by pos * theta^(-2p/D); angles are formed and
// evaluated in fp64, the rotation itself runs in fp32.
#include "attn_common.h"
#include "kernels.h"

namespace attn {

// Cos/sin table for tokens 0..T-1 at positions pos0 + t: tab[t * P + p] =
// (cos, sin) of pair p, P = rotary pairs. One thread per (t, p).
__global__ void rope_table_kernel(float2* __restrict__ tab, int T, int P, int D,
                                  int pos0, double log2_theta) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * P) return;
  const int t = (int)(idx / P), p = (int)(idx % P);
  float c, s;
  rope_cos_sin((int64_t)pos0 + t, rope_freq(p, D, log2_theta), &c, &s);
  tab[idx] = make_float2(c, s);
}

// y[n, h, :] = rope(x[n, h, :], pos[n]) with NH = 1 half, or 2-D RoPE with
// NH = 2: each half of the D dims is a vector of its own, turned by its own
// coordinate (pos[2n] the patch's width coordinate for the first half,
// pos[2n + 1] its height coordinate for the second), pair p of a half by
// coordinate * theta^(-2p/(D/2)) ("Gemma 4: End-to-End Architecture
// Walkthrough", Phase 1 section 1b). One thread per (n, half, pair) forms the
// angle once and applies it to all H heads; a second grid dimension copies
// the untouched dims when y != x.
template <typename T_>
__global__ void prope_kernel(const T_* __restrict__ x, T_* __restrict__ y,
                             const int32_t* __restrict__ pos, int N, int H, int D,
                             int P, int NH, double log2_theta, int in_place) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int DH = D / NH;  // dims per half
  if (blockIdx.y == 0) {
    if (idx >= (int64_t)N * NH * P) return;
    const int n = (int)(idx / (NH * P)), q = (int)(idx % (NH * P));
    const int half = q / P, p = q - half * P;
    float c, s;
    rope_cos_sin(pos[(int64_t)n * NH + half], rope_freq(p, DH, log2_theta), &c, &s);
    for (int h = 0; h < H; ++h) {
      const int64_t off = ((int64_t)n * H + h) * D + half * DH + 2 * p;
      float x0, x1;
      if constexpr (sizeof(T_) == 2) {
        x0 = bf16_to_f32(reinterpret_cast<const uint16_t*>(x)[off]);
        x1 = bf16_to_f32(reinterpret_cast<const uint16_t*>(x)[off + 1]);
      } else {
        x0 = reinterpret_cast<const float*>(x)[off];
        x1 = reinterpret_cast<const float*>(x)[off + 1];
      }
      const float y0 = x0 * c - x1 * s;
      const float y1 = x0 * s + x1 * c;
      if constexpr (sizeof(T_) == 2) {
        reinterpret_cast<uint32_t*>(y)[off / 2] = pack_bf16x2(y0, y1);
      } else {
        reinterpret_cast<float2*>(y)[off / 2] = make_float2(y0, y1);
      }
    }
  } else {
    // Copy dims [2P, DH) of every half of every (n, h) when writing out of place.
    if (in_place) return;
    const int rest = DH - 2 * P;
    if (rest == 0) return;
    const int64_t total = (int64_t)N * H * NH * rest;
    for (int64_t i = idx; i < total; i += (int64_t)gridDim.x * blockDim.x) {
      const int64_t nhh = i / rest;  // (n * H + h) * NH + half
      const int d = (int)(nhh % NH) * DH + 2 * P + (int)(i % rest);
      const int64_t base = (nhh / NH) * D;
      y[base + d] = x[base + d];
    }
  }
}

// K's rotary dims, turned once per key for the MFMA prefill: one thread per
// (token, head, 8-dim chunk c < R/8) turns 4 pairs with the table row of its
// token and writes them to out[b, t, h, 8c .. 8c+7] (bf16, fp32 arithmetic).
__global__ void rope_k_lead_kernel(const uint16_t* __restrict__ k, uint16_t* __restrict__ out,
                                   const float2* __restrict__ tab, int64_t n_chunks, int T,
                                   int H, int D, int RC) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_chunks) return;
  const int c = (int)(idx % RC);
  const int64_t nh = idx / RC;  // (b*T + t)*H + h
  const int t = (int)((nh / H) % T);
  const u32x4 w = *reinterpret_cast<const u32x4*>(k + nh * D + 8 * c);
  const f32x4 t0 = *reinterpret_cast<const f32x4*>(tab + (int64_t)t * (4 * RC) + 4 * c);
  const f32x4 t1 = *reinterpret_cast<const f32x4*>(tab + (int64_t)t * (4 * RC) + 4 * c + 2);
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float cs = (j < 2) ? t0[2 * j] : t1[2 * (j - 2)];
    const float sn = (j < 2) ? t0[2 * j + 1] : t1[2 * (j - 2) + 1];
    const float x0 = bf16_lo(w[j]), x1 = bf16_hi(w[j]);
    r[j] = pack_bf16x2(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
  }
  *reinterpret_cast<u32x4*>(out + nh * (8 * RC) + 8 * c) = r;
}

hipError_t launch_rope_k_lead(const void* k, void* out, const float2* tab, int B, int T,
                              int H, int D, int R, hipStream_t st) {
  if (R % 8 != 0 || D % 8 != 0 || R > D) return hipErrorInvalidValue;
  const int64_t n = (int64_t)B * T * H * (R / 8);
  if (n == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rope_k_lead_kernel, dim3((unsigned)blocks), dim3(threads), 0, st,
                     reinterpret_cast<const uint16_t*>(k), reinterpret_cast<uint16_t*>(out),
                     tab, n, T, H, D, R / 8);
  return hipGetLastError();
}

hipError_t launch_rope_table(float2* tab, int T, int P, int D, int pos0,
                             double theta, hipStream_t st) {
  if ((int64_t)T * P == 0) return hipSuccess;
  const int64_t n = (int64_t)T * P;
  const int threads = 256;
  const int blocks = (int)((n + threads - 1) / threads);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(threads), 0, st, tab, T,
                     P, D, pos0, log2(theta));
  return hipGetLastError();
}

hipError_t launch_prope(const void* x, void* y, const int32_t* pos, int N, int H,
                        int D, int P, int NH, double theta, bool bf16, hipStream_t st) {
  const int64_t n = (int64_t)N * NH * P;
  const int threads = 256;
  int64_t blocks = (n + threads - 1) / threads;
  if (blocks < 1) blocks = 1;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const int in_place = (x == y);
  const int ydim = (in_place || D == 2 * P * NH) ? 1 : 2;
  int bx = (int)blocks;
  if (ydim == 2) {
    // The copy half needs enough blocks for the untouched elements as well.
    const int64_t m = (int64_t)N * H * (D - 2 * P * NH);
    int64_t want = (m + threads - 1) / threads;
    if (want > 65536) want = 65536;
    if (want > bx) bx = (int)want;
  }
  if (bf16)
    hipLaunchKernelGGL(prope_kernel<uint16_t>, dim3(bx, ydim), dim3(threads), 0, st,
                       (const uint16_t*)x, (uint16_t*)y, pos, N, H, D, P, NH, log2(theta),
                       in_place);
  else
    hipLaunchKernelGGL(prope_kernel<float>, dim3(bx, ydim), dim3(threads), 0, st,
                       (const float*)x, (float*)y, pos, N, H, D, P, NH, log2(theta),
                       in_place);
  return hipGetLastError();
}

}  // namespace attn
