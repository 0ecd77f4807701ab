// prefill_general.hip — general causal / sliding-window GQA prefill for any
// supported head shape, fp32 or bf16 (correctness path; the MFMA kernel is
// the fast path for the model's shapes).
//
// Computes softmax(scale * rope(q) rope(k)^T + mask) v as the Gemma 4 pages
// describe it ("Gemma 4: End-to-End Architecture Walkthrough", Phase 3
// sections 3a-3c): query i of a local layer sees keys i-W+1..i, of a global
// layer keys 0..i; query head h reads KV head h / (Hq/Hkv).
//
// One workgroup of 4 waves per (batch, query row, up to four query heads of
// one KV head): each key and value it loads serves all those heads, so the
// caches are read once per head group rather than once per head. Wave w takes
// key blocks w, w + 4, ... and the four softmax states of each head are
// merged at the end (four shorter dependent chains instead of one). Lane l owns dimension
// pairs l, l+64, ... of q/k and of v/o, so RoPE pairs stay inside a lane. The
// query's angles are formed in fp64 here; K's rotary pairs arrive turned by
// the pre-pass (k_rot).
// Each wave streams its keys 8 at a time with an online softmax (running max
// and sum in fp32).
#include <type_traits>

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

// NE: dimension pairs per lane (ceil(max(Dk, Dv) / 128)). Lanes whose pair
// is past the head read pair 0 and weigh it by 0 (a select, not a branch), so
// every load of a key block goes out before the first is waited on.
constexpr int kWaves = 4;  // waves per query row: each takes every 4th key block

template <bool BF16, int NE, int HG>
__global__ __launch_bounds__(kWaves * 64) void prefill_general_kernel(PrefillArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // One workgroup per (batch, query row, HG consecutive query heads of one KV
  // head): every key and value block it loads serves all HG heads.
  const int64_t row_id = blockIdx.x;
  const int HB = a.Hq / HG;  // head blocks per row
  const int64_t n_rows = (int64_t)a.B * a.T * HB;
  if (row_id >= n_rows) return;
  const int h0 = (int)(row_id % HB) * HG;
  const int i = (int)((row_id / HB) % a.T);
  const int b = (int)(row_id / ((int64_t)HB * a.T));
  const int G = a.Hq / a.Hkv;
  const int g = h0 / G;
  const int PK = a.Dk / 2, PV = a.Dv / 2;

  // The query pairs this lane owns for each head, rotated at position
  // pos0 + i (angles in fp64).
  float2 q[HG][NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int p = lane + 64 * e;
    float c = 1.f, sn = 0.f;
    const bool turn = p < PK && a.rope_q && p < a.rot_pairs;
    if (turn) rope_cos_sin((int64_t)a.pos0 + i, rope_freq(p, a.Dk, a.log2_theta), &c, &sn);
#pragma unroll
    for (int t = 0; t < HG; ++t) {
      q[t][e] = make_float2(0.f, 0.f);
      if (p < PK) {
        float2 x = load_pair<BF16>(a.q, (((int64_t)b * a.T + i) * a.Hq + h0 + t) * a.Dk + 2 * p);
        if (turn) x = make_float2(x.x * c - x.y * sn, x.x * sn + x.y * c);
        q[t][e] = x;
      }
    }
  }

  float m[HG], l[HG];
  float2 acc[HG][NE];
#pragma unroll
  for (int t = 0; t < HG; ++t) {
    m[t] = -INFINITY;
    l[t] = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[t][e] = make_float2(0.f, 0.f);
  }

  // Keys in blocks of KB: the block's loads and reductions are independent,
  // so they overlap; one online-softmax update per block and head. Keys past
  // i (the last block's tail) are read at i and masked out.
  // Keys per block: 8, which the reduction below assumes (16 measured
  // slower).
  constexpr int KB = 8;
  const int lo = (a.window > 0) ? max(0, i - a.window + 1) : 0;
  for (int j0 = lo + KB * wave; j0 <= i; j0 += KB * kWaves) {
    float s[HG][KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int j = min(j0 + u, i);
      const int64_t kbase = (((int64_t)b * a.T + j) * a.Hkv + g) * a.Dk;
      const int64_t krbase = (((int64_t)b * a.T + j) * a.Hkv + g) * (2 * a.rot_pairs);
#pragma unroll
      for (int t = 0; t < HG; ++t) s[t][u] = 0.f;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int p = lane + 64 * e;
        const bool in = p < PK;
        const int pc = in ? p : 0;
        // K's rotary pairs come turned from the pre-pass (k_rot).
        const bool rot = a.rope_k && pc < a.rot_pairs;
        const float2 kx = load_pair<BF16>(rot ? a.k_rot : a.k,
                                          (rot ? krbase : kbase) + 2 * pc);
#pragma unroll
        for (int t = 0; t < HG; ++t)
          s[t][u] += in ? q[t][e].x * kx.x + q[t][e].y * kx.y : 0.f;
      }
    }
    // The block's V rows, loaded before the scores are reduced (they do not
    // depend on them), so their latency runs under the reduction.
    float2 vx[KB][NE];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int j = min(j0 + u, i);
      const int64_t vbase = (((int64_t)b * a.T + j) * a.Hkv + g) * a.Dv;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int pp = lane + 64 * e;
        vx[u][e] = load_pair<BF16>(a.v, vbase + 2 * (pp < PV ? pp : 0));
      }
    }
#pragma unroll
    for (int t = 0; t < HG; ++t) {
      // Sum each key's partial over the 64 lanes by reduce-scatter: halving
      // the keys a lane keeps at lane distances 32, 16 and 8 leaves lane l
      // with key (l >> 3) & 7 summed over 8 lanes; three more steps finish
      // the sum, and lane 8u then holds key u's score (10 exchanges instead
      // of 48).
      {
        const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
        float tt[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float give = b5 ? s[t][k] : s[t][k + 4];
          tt[k] = (b5 ? s[t][k + 4] : s[t][k]) + __shfl_xor(give, 32);
        }
        float w[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float give = b4 ? tt[k] : tt[k + 2];
          w[k] = (b4 ? tt[k + 2] : tt[k]) + __shfl_xor(give, 16);
        }
        float x = (b3 ? w[1] : w[0]) + __shfl_xor(b3 ? w[0] : w[1], 8);
        x += __shfl_xor(x, 4);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 1);
#pragma unroll
        for (int u = 0; u < KB; ++u)
          s[t][u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 8 * u));
      }
      float m_blk = -INFINITY;
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        s[t][u] = (j0 + u <= i) ? s[t][u] * a.scale : -INFINITY;
        m_blk = fmaxf(m_blk, s[t][u]);
      }
      const float m_new = fmaxf(m[t], m_blk);
      const float alpha = __expf(m[t] - m_new);
      float pr[KB];
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        pr[u] = __expf(s[t][u] - m_new);
        psum += pr[u];
      }
      l[t] = l[t] * alpha + psum;
      m[t] = m_new;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        acc[t][e].x *= alpha;
        acc[t][e].y *= alpha;
      }
#pragma unroll
      for (int u = 0; u < KB; ++u) {
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const float w = (lane + 64 * e < PV) ? pr[u] : 0.f;
          acc[t][e].x += w * vx[u][e].x;
          acc[t][e].y += w * vx[u][e].y;
        }
      }
    }
  }

  // The waves' online-softmax states (m, l, acc) of each head merged by
  // log-sum-exp: each is rescaled to the largest m (a wave that saw no key
  // has m = -inf and weighs 0; wave 0 always sees key lo). Wave t % kWaves
  // merges and writes head t.
  __shared__ float s_m[kWaves][HG], s_l[kWaves][HG];
  __shared__ float2 s_acc[kWaves][HG][NE * 64];
#pragma unroll
  for (int t = 0; t < HG; ++t) {
#pragma unroll
    for (int e = 0; e < NE; ++e) s_acc[wave][t][e * 64 + lane] = acc[t][e];
    if (lane == 0) {
      s_m[wave][t] = m[t];
      s_l[wave][t] = l[t];
    }
  }
  __syncthreads();
  for (int t = wave; t < HG; t += kWaves) {
    float mm = s_m[0][t];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mm = fmaxf(mm, s_m[w][t]);
    float ll = 0.f;
    float2 ac[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) ac[e] = make_float2(0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = s_m[w][t] == -INFINITY ? 0.f : __expf(s_m[w][t] - mm);
      ll += s_l[w][t] * f;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const float2 x = s_acc[w][t][e * 64 + lane];
        ac[e].x += x.x * f;
        ac[e].y += x.y * f;
      }
    }
    const float inv = 1.f / ll;
    const int64_t obase = (((int64_t)b * a.T + i) * a.Hq + h0 + t) * a.Dv;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int pp = lane + 64 * e;
      if (pp < PV) {
        const float y0 = ac[e].x * inv, y1 = ac[e].y * inv;
        if constexpr (BF16)
          reinterpret_cast<uint32_t*>(a.o)[(obase + 2 * pp) / 2] = pack_bf16x2(y0, y1);
        else
          reinterpret_cast<float2*>(a.o)[(obase + 2 * pp) / 2] = make_float2(y0, y1);
      }
    }
  }
}

}  // namespace

#ifdef ATTN_DEBUG_TILES
static __device__ unsigned long long g_dbg_visits[2];

hipError_t debug_visits_ptr(unsigned long long** p) {
  return hipGetSymbolAddress(reinterpret_cast<void**>(p), HIP_SYMBOL(g_dbg_visits));
}
#endif

hipError_t launch_prefill_general(const PrefillArgs& a, bool bf16, hipStream_t st) {
  const int ne = ((a.Dk > a.Dv ? a.Dk : a.Dv) / 2 + 63) / 64;
  if (ne < 1 || ne > kMaxPairs) return hipErrorInvalidValue;
  // Query heads per workgroup: the largest of 4, 2, 1 that divides the heads
  // per KV head, with at most 8 dim pairs per lane over all of them (8 heads
  // measured slower: too few workgroups, and twice the registers).
  const int G = a.Hkv > 0 ? a.Hq / a.Hkv : 1;
  int hg = 1;
  for (int c : {4, 2})
    if (G % c == 0 && c * ne <= 8) {
      hg = c;
      break;
    }
  const int64_t blocks = (int64_t)a.B * a.T * (a.Hq / hg);  // one (row, head block) each
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kWaves * 64), 0, st, a);
  };
  auto by_hg = [&](auto BF_, auto NE_) {
    constexpr bool BF = decltype(BF_)::value;
    constexpr int N = decltype(NE_)::value;
    if constexpr (4 * N <= 8) {
      if (hg == 4) return go(prefill_general_kernel<BF, N, 4>);
    }
    if constexpr (2 * N <= 8) {
      if (hg == 2) return go(prefill_general_kernel<BF, N, 2>);
    }
    go(prefill_general_kernel<BF, N, 1>);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  auto by_ne = [&](auto BF_) {
    if (ne == 1) by_hg(BF_, std::integral_constant<int, 1>{});
    else if (ne == 2) by_hg(BF_, std::integral_constant<int, 2>{});
    else if (ne == 3) by_hg(BF_, std::integral_constant<int, 3>{});
    else by_hg(BF_, std::integral_constant<int, 4>{});
  };
  if (bf16) by_ne(T_{});
  else by_ne(F_{});
  return hipGetLastError();
}

}  // namespace attn
