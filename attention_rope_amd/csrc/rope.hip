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

// Pair (x0, x1) turned by the angle with cosine c and sine s, in fp32, each
// product rounded before the sum (no fused multiply-add, whose use the
// compiler would otherwise choose per kernel). Every kernel here that turns a
// vector goes through this, so a key turned by any of them has the same bits.
__device__ __forceinline__ float2 turn_pair(float x0, float x1, float c, float s) {
#pragma clang fp contract(off)
  return make_float2(x0 * c - x1 * s, x0 * s + x1 * c);
}

// A 16-byte chunk of E = 16 / sizeof(T_) elements (E / 2 adjacent pairs)
// turned by the pairs' (cos, sin).
template <typename T_>
__device__ __forceinline__ u32x4 turn_chunk(u32x4 w, const float* cs, const float* sn) {
  u32x4 r;
  if constexpr (sizeof(T_) == 2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float2 y = turn_pair(bf16_lo(w[j]), bf16_hi(w[j]), cs[j], sn[j]);
      r[j] = pack_bf16x2(y.x, y.y);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float2 y = turn_pair(__uint_as_float(w[2 * j]), __uint_as_float(w[2 * j + 1]),
                                 cs[j], sn[j]);
      r[2 * j] = __float_as_uint(y.x);
      r[2 * j + 1] = __float_as_uint(y.y);
    }
  }
  return r;
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
      const float2 r = turn_pair(x0, x1, c, s);
      if constexpr (sizeof(T_) == 2) {
        reinterpret_cast<uint32_t*>(y)[off / 2] = pack_bf16x2(r.x, r.y);
      } else {
        reinterpret_cast<float2*>(y)[off / 2] = r;
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
// (token t, 8-dim chunk c < R/8) forms the angles of its 4 pairs at position
// pos0 + t in fp64 once, then turns that chunk of every (batch, head) row of
// the token and writes it to out[b, t, h, 8c .. 8c+7] (bf16, fp32 arithmetic).
// Consecutive threads take consecutive chunks of one token, so each (b, h)
// step reads and writes R/8 contiguous 16-byte pieces.
__global__ void rope_k_lead_kernel(const uint16_t* __restrict__ k, uint16_t* __restrict__ out,
                                   int B, int T, int H, int D, int RC, int pos0,
                                   double log2_theta) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * RC) return;
  const int c = (int)(idx % RC);
  const int t = (int)(idx / RC);
  float cs[4], sn[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    rope_cos_sin((int64_t)pos0 + t, rope_freq(4 * c + j, D, log2_theta), &cs[j], &sn[j]);
  // (b, h) rows n = b * H + h of token t, 8 at a time: all loads first, so
  // every thread keeps 8 reads in flight.
  const int BH = B * H;
  for (int n0 = 0; n0 < BH; n0 += 8) {
    u32x4 w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int n = n0 + u;
      if (n < BH) {
        const int64_t nh = ((int64_t)(n / H) * T + t) * H + n % H;
        w[u] = *reinterpret_cast<const u32x4*>(k + nh * D + 8 * c);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int n = n0 + u;
      if (n < BH) {
        const int64_t nh = ((int64_t)(n / H) * T + t) * H + n % H;
        *reinterpret_cast<u32x4*>(out + nh * (8 * RC) + 8 * c) =
            turn_chunk<uint16_t>(w[u], cs, sn);
      }
    }
  }
}

hipError_t launch_rope_k_chunks(const void* k, void* out, int B, int T, int H, int D, int R,
                                int pos0, double theta, hipStream_t st);

// The same for any even R and either element type (the general prefill path):
// one thread per (token t, pair p) forms the angle once and turns pair p of
// every (batch, head) row of the token into out[b, t, h, 2p .. 2p+1].
template <typename T_>
__global__ void rope_k_pairs_kernel(const T_* __restrict__ k, T_* __restrict__ out, int B,
                                    int T, int H, int D, int P, int pos0, double log2_theta) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * P) return;
  const int p = (int)(idx % P);
  const int t = (int)(idx / P);
  float c, sn;
  rope_cos_sin((int64_t)pos0 + t, rope_freq(p, D, log2_theta), &c, &sn);
  const int BH = B * H;
  for (int n0 = 0; n0 < BH; n0 += 8) {
    float2 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int n = n0 + u;
      if (n < BH) {
        const int64_t nh = ((int64_t)(n / H) * T + t) * H + n % H;
        if constexpr (sizeof(T_) == 2) {
          const uint32_t w = reinterpret_cast<const uint32_t*>(k + nh * D)[p];
          x[u] = make_float2(bf16_lo(w), bf16_hi(w));
        } else {
          x[u] = reinterpret_cast<const float2*>(k + nh * D)[p];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int n = n0 + u;
      if (n < BH) {
        const int64_t nh = ((int64_t)(n / H) * T + t) * H + n % H;
        const float2 y = turn_pair(x[u].x, x[u].y, c, sn);
        if constexpr (sizeof(T_) == 2)
          reinterpret_cast<uint32_t*>(out + nh * (2 * P))[p] = pack_bf16x2(y.x, y.y);
        else
          reinterpret_cast<float2*>(out + nh * (2 * P))[p] = y;
      }
    }
  }
}

hipError_t launch_rope_k_lead(const void* k, void* out, int B, int T, int H, int D, int R,
                              int pos0, double theta, bool bf16, hipStream_t st) {
  if (R % 2 != 0 || R > D || D % 2 != 0) return hipErrorInvalidValue;
  if ((int64_t)T * R == 0 || B == 0 || H == 0) return hipSuccess;
  const int threads = 256;
  if (!bf16 || R % 8 != 0 || D % 8 != 0) {
    const int64_t blocks = ((int64_t)T * (R / 2) + threads - 1) / threads;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (bf16)
      hipLaunchKernelGGL(rope_k_pairs_kernel<uint16_t>, dim3((unsigned)blocks), dim3(threads), 0,
                         st, (const uint16_t*)k, (uint16_t*)out, B, T, H, D, R / 2, pos0,
                         log2(theta));
    else
      hipLaunchKernelGGL(rope_k_pairs_kernel<float>, dim3((unsigned)blocks), dim3(threads), 0,
                         st, (const float*)k, (float*)out, B, T, H, D, R / 2, pos0,
                         log2(theta));
    return hipGetLastError();
  }
  return launch_rope_k_chunks(k, out, B, T, H, D, R, pos0, theta, st);
}

hipError_t launch_rope_k_chunks(const void* k, void* out, int B, int T, int H, int D, int R,
                                int pos0, double theta, hipStream_t st) {
  if (R % 8 != 0 || D % 8 != 0 || R > D) return hipErrorInvalidValue;
  const int64_t n = (int64_t)T * (R / 8);
  if (n == 0 || B == 0 || H == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rope_k_lead_kernel, dim3((unsigned)blocks), dim3(threads), 0, st,
                     reinterpret_cast<const uint16_t*>(k), reinterpret_cast<uint16_t*>(out),
                     B, T, H, D, R / 8, pos0, log2(theta));
  return hipGetLastError();
}

// Prefill's K/V pass that also fills a decode cache. Grid y = 0: one thread
// per (token t, 16-byte chunk c of a key row) forms the angles of the chunk's
// pairs at pos0 + t once (fp64), then for every (b, h) turns the chunk if it
// lies in the leading R dims, writes it to the cache row row_offset[b] + t
// and, if turned, to the workspace the attention kernel reads (the layout of
// launch_rope_k_lead). Grid y = 1: the same for value rows, copied unchanged.
// A batch row whose cache rows would leave [0, cache_rows) is not written to
// the cache (its workspace rows still are).
template <typename T_>
__global__ void prefill_cache_fill_kernel(const T_* __restrict__ k, const T_* __restrict__ v,
                                          T_* __restrict__ k_cache, T_* __restrict__ v_cache,
                                          T_* __restrict__ k_rot,
                                          const int64_t* __restrict__ row_offset,
                                          int64_t cache_rows, int B, int T, int H, int Dk,
                                          int Dv, int R, int pos0, double log2_theta) {
  constexpr int E = 16 / sizeof(T_), NP = E / 2;  // elements, pairs per chunk
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool keys = blockIdx.y == 0;
  const int D = keys ? Dk : Dv, NC = D / E;
  if (idx >= (int64_t)T * NC) return;
  const int c = (int)(idx % NC), t = (int)(idx / NC);
  const bool turn = keys && c * E < R;
  float cs[NP], sn[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    cs[j] = 1.f;
    sn[j] = 0.f;
    if (turn) rope_cos_sin((int64_t)pos0 + t, rope_freq(c * NP + j, Dk, log2_theta), &cs[j], &sn[j]);
  }
  const T_* src = keys ? k : v;
  T_* dst = keys ? k_cache : v_cache;
  for (int b = 0; b < B; ++b) {
    const int64_t r0 = row_offset[b];
    const bool in = r0 >= 0 && r0 <= cache_rows - T;
    for (int h = 0; h < H; ++h) {
      const int64_t n = ((int64_t)b * T + t) * H + h;
      u32x4 w = *reinterpret_cast<const u32x4*>(src + n * D + c * E);
      if (turn) {
        w = turn_chunk<T_>(w, cs, sn);
        *reinterpret_cast<u32x4*>(k_rot + n * R + c * E) = w;
      }
      if (in) *reinterpret_cast<u32x4*>(dst + ((r0 + t) * H + h) * D + c * E) = w;
    }
  }
}

hipError_t launch_prefill_cache_fill(const void* k, const void* v, void* k_cache, void* v_cache,
                                     void* k_rot, const int64_t* row_offset, int64_t cache_rows,
                                     int B, int T, int H, int Dk, int Dv, int R, int pos0,
                                     double theta, bool bf16, hipStream_t st) {
  const int E = bf16 ? 8 : 4;
  if (Dk % E || Dv % E || R % E || R > Dk || (R > 0 && !k_rot)) return hipErrorInvalidValue;
  const int64_t n = (int64_t)T * ((Dk > Dv ? Dk : Dv) / E);
  if (n == 0 || B == 0 || H == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const double l2t = R > 0 ? log2(theta) : 0.0;
  if (bf16)
    hipLaunchKernelGGL(prefill_cache_fill_kernel<uint16_t>, dim3((unsigned)blocks, 2),
                       dim3(threads), 0, st, (const uint16_t*)k, (const uint16_t*)v,
                       (uint16_t*)k_cache, (uint16_t*)v_cache, (uint16_t*)k_rot, row_offset,
                       cache_rows, B, T, H, Dk, Dv, R, pos0, l2t);
  else
    hipLaunchKernelGGL(prefill_cache_fill_kernel<float>, dim3((unsigned)blocks, 2),
                       dim3(threads), 0, st, (const float*)k, (const float*)v,
                       (float*)k_cache, (float*)v_cache, (float*)k_rot, row_offset, cache_rows,
                       B, T, H, Dk, Dv, R, pos0, l2t);
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
