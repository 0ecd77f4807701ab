/*
 * attn_oracle.c — plain, slow, obviously-correct fp64 CPU oracle for the hybrid
 * attention of the Gemma 4 decoder (local sliding-window GQA, global GQA with
 * widened keys, proportional RoPE).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do. It shares no code, header, table or helper with the HIP library.
 *
 * Everything is fp64, computed naively in the order the definition states:
 * no tiling, no online softmax, no fusion. Inputs are fp64 arrays (bf16 and
 * fp32 values convert to fp64 exactly, so the oracle sees the stored values).
 *
 * Sources (the pages this follows):
 *  - "Gemma 4: End-to-End Architecture Walkthrough", Phase 3, section 3a
 *    (local layers attend a fixed recent window, global layers the whole
 *    preceding context), section 3b (8 query heads share one KV head in global
 *    layers, 2 in local ones; wider global keys) and section 3c (p-RoPE: only
 *    the first quarter of the rotary dimension pairs — the high-frequency ones —
 *    rotate; the rest get no rotation).
 *  - "Gemma 4 Architecture Reference", sections "Attention Architecture" and
 *    "Positional Encoding: Proportional RoPE (p-RoPE)" (p = 0.25, theta = 1e6,
 *    global layers only).
 *  - "Gemma 4 Technical Report" (paperglide reader), "Core Model
 *    Architecture": attention computes Q K^T, softmax, then weights the values.
 *
 * Readings taken where the pages leave a step open (each also listed in the
 * design notes):
 *  - Rotary pairs are adjacent dims (2p, 2p+1); pair p turns by
 *    pos * theta^(-2p/D), D = full head dim; pairs p >= rotary_dims/2 do not
 *    turn (the "zero out" reading of p-RoPE). parity unpinned: the pages do not
 *    fix adjacent-vs-half-split pairing, and either layout passes every
 *    invariant the pages state.
 *  - Window W (W > 0): query i may attend key j iff j <= i and i - j < W
 *    (self included, W keys). W <= 0 means full causal.
 *  - GQA grouping is contiguous: query head h reads KV head h / (Hq / Hkv).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Rotate one head vector x[0..D) at integer position `pos` into y (may alias).
 * Pair p < rotary_dims/2 of dims (2p, 2p+1) turns by angle pos * w_p with
 * w_p = theta^(-2p/D); other dims are copied unchanged. */
static void rope_vec(const double *x, double *y, int D, int rotary_dims,
                     double theta, int64_t pos) {
  for (int d = 0; d < D; ++d) y[d] = x[d];
  for (int p = 0; p < rotary_dims / 2; ++p) {
    double w = pow(theta, -2.0 * (double)p / (double)D);
    double a = (double)pos * w;
    double c = cos(a), s = sin(a);
    double x0 = x[2 * p], x1 = x[2 * p + 1];
    y[2 * p] = x0 * c - x1 * s;
    y[2 * p + 1] = x0 * s + x1 * c;
  }
}

/* x, y: [N, H, D]; positions: [N]. y may equal x. */
void oracle_rope(const double *x, double *y, const int64_t *positions,
                 int64_t N, int H, int D, int rotary_dims, double theta) {
  for (int64_t n = 0; n < N; ++n)
    for (int h = 0; h < H; ++h) {
      size_t off = ((size_t)n * H + h) * D;
      rope_vec(x + off, y + off, D, rotary_dims, theta, positions[n]);
    }
}

/* Is key j visible from query i under window W (W <= 0: full causal)? */
static int allowed(int64_t i, int64_t j, int64_t W) {
  if (j > i) return 0;
  if (W > 0 && i - j >= W) return 0;
  return 1;
}

/* Attention for one query vector (already rotated) over n_keys replicated
 * key/value rows of one head: two passes, exact max-subtracted softmax.
 * keys:   row t at keys + t*kstride,   Dk values
 * values: row t at values + t*vstride, Dv values
 * vis[t] != 0 marks the allowed keys. Writes Dv outputs. */
static void attend_row(const double *q, const double *keys, size_t kstride,
                       const double *values, size_t vstride, const char *vis,
                       int64_t n_keys, int Dk, int Dv, double scale,
                       double *scores, double *out) {
  double m = -INFINITY;
  for (int64_t t = 0; t < n_keys; ++t) {
    if (!vis[t]) continue;
    const double *k = keys + (size_t)t * kstride;
    double s = 0.0;
    for (int d = 0; d < Dk; ++d) s += q[d] * k[d];
    s *= scale;
    scores[t] = s;
    if (s > m) m = s;
  }
  for (int d = 0; d < Dv; ++d) out[d] = 0.0;
  if (m == -INFINITY) return; /* nothing visible: output zero */
  double denom = 0.0;
  for (int64_t t = 0; t < n_keys; ++t) {
    if (!vis[t]) continue;
    double p = exp(scores[t] - m);
    denom += p;
    const double *v = values + (size_t)t * vstride;
    for (int d = 0; d < Dv; ++d) out[d] += p * v[d];
  }
  for (int d = 0; d < Dv; ++d) out[d] /= denom;
}

/*
 * Prefill: q [B, n_rows, Hq, Dk] holds the query rows listed in rows[] (query
 * positions i = rows[r] in 0..T-1; rows == NULL means all T rows in order),
 * k [B, T, Hkv, Dk], v [B, T, Hkv, Dv] unrotated, o [B, n_rows, Hq, Dv].
 * Token t sits at position pos0 + t. rope_mask bit 1 rotates q, bit 2 rotates k.
 * Returns 0, or -1 on bad arguments / out of memory.
 */
int oracle_prefill(const double *q, const double *k, const double *v, double *o,
                   int B, int T, int Hq, int Hkv, int Dk, int Dv, int window,
                   double scale, int rotary_dims, double theta, int rope_mask,
                   int64_t pos0, const int32_t *rows, int n_rows, int nthreads) {
  if (B < 0 || T < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || Dk <= 0 || Dv <= 0)
    return -1;
  if (rows == NULL) n_rows = T;
  if (B == 0 || T == 0 || n_rows == 0) return 0;
  const int G = Hq / Hkv;
  const size_t BT = (size_t)B * T;

  /* Step 1: rotate the keys at their own positions. */
  double *k_rot = (double *)malloc(BT * Hkv * Dk * sizeof(double));
  /* Step 2: explicit per-head replication, K_rep[b,t,h] = K[b,t,h/G]. */
  double *k_rep = (double *)malloc(BT * Hq * Dk * sizeof(double));
  double *v_rep = (double *)malloc(BT * Hq * Dv * sizeof(double));
  if (!k_rot || !k_rep || !v_rep) {
    free(k_rot); free(k_rep); free(v_rep);
    return -1;
  }
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t bt = 0; bt < (int64_t)BT; ++bt) {
    int64_t t = bt % T;
    for (int g = 0; g < Hkv; ++g) {
      const double *src = k + ((size_t)bt * Hkv + g) * Dk;
      double *dst = k_rot + ((size_t)bt * Hkv + g) * Dk;
      if (rope_mask & 2)
        rope_vec(src, dst, Dk, rotary_dims, theta, pos0 + t);
      else
        memcpy(dst, src, Dk * sizeof(double));
    }
    for (int h = 0; h < Hq; ++h) {
      int g = h / G;
      memcpy(k_rep + ((size_t)bt * Hq + h) * Dk,
             k_rot + ((size_t)bt * Hkv + g) * Dk, Dk * sizeof(double));
      memcpy(v_rep + ((size_t)bt * Hq + h) * Dv,
             v + ((size_t)bt * Hkv + g) * Dv, Dv * sizeof(double));
    }
  }
  free(k_rot);

  /* Step 3: each (b, row, head) independently. */
  int failed = 0;
#pragma omp parallel num_threads(nthreads)
  {
    double *scores = (double *)malloc((size_t)T * sizeof(double));
    double *qr = (double *)malloc((size_t)Dk * sizeof(double));
    char *vis = (char *)malloc((size_t)T);
    const int ok = scores && qr && vis;
    if (!ok) {
#pragma omp atomic write
      failed = 1;
    }
    /* Every thread enters the work-sharing loop; one without buffers skips. */
#pragma omp for schedule(dynamic, 4)
    for (int64_t idx = 0; idx < (int64_t)B * n_rows * Hq; ++idx) {
      if (ok) {
        int h = (int)(idx % Hq);
        int64_t r = (idx / Hq) % n_rows;
        int64_t b = idx / ((int64_t)Hq * n_rows);
        int64_t i = rows ? rows[r] : r;
        const double *qin = q + (((size_t)b * n_rows + r) * Hq + h) * Dk;
        if (rope_mask & 1)
          rope_vec(qin, qr, Dk, rotary_dims, theta, pos0 + i);
        else
          memcpy(qr, qin, Dk * sizeof(double));
        for (int64_t j = 0; j < T; ++j) vis[j] = (char)allowed(i, j, window);
        attend_row(qr, k_rep + ((size_t)b * T * Hq + h) * Dk, (size_t)Hq * Dk,
                   v_rep + ((size_t)b * T * Hq + h) * Dv, (size_t)Hq * Dv, vis,
                   T, Dk, Dv, scale, scores,
                   o + (((size_t)b * n_rows + r) * Hq + h) * Dv);
      }
    }
    free(scores); free(qr); free(vis);
  }
  free(k_rep); free(v_rep);
  return failed ? -1 : 0;
}

/*
 * Decode for ONE sequence. The sequence holds kv_len cache rows; the new
 * token's query q [Hq, Dk] (unrotated) sits at position L = kv_len - 1 and may
 * attend row j iff allowed(L, j, window). Only rows row0 .. kv_len-1 are passed:
 * kc [kv_len - row0, Hkv, Dk] (keys stored already rotated), vc [.., Hkv, Dv].
 * Rows before row0 must all be invisible (row0 <= kv_len - window when a window
 * is set, else row0 == 0); otherwise the call fails. o [Hq, Dv]. kv_len == 0
 * gives o = 0. The query is rotated at position L (rotary_dims == 0: no
 * rotation). Heads run one after another; the replicated key/value rows of the
 * current head are materialised explicitly.
 */
int oracle_decode_one(const double *q, const double *kc, const double *vc,
                      int64_t row0, int64_t kv_len, double *o, int Hq, int Hkv,
                      int Dk, int Dv, int window, double scale, int rotary_dims,
                      double theta, int nthreads) {
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv || Dk <= 0 || Dv <= 0 || kv_len < 0 ||
      row0 < 0 || row0 > kv_len)
    return -1;
  if (kv_len == 0) {
    memset(o, 0, (size_t)Hq * Dv * sizeof(double));
    return 0;
  }
  const int64_t L = kv_len - 1;
  if (row0 > 0 && allowed(L, row0 - 1, window)) return -1;
  const int G = Hq / Hkv;
  const int64_t n = kv_len - row0;
  double *k_rep = (double *)malloc((size_t)n * Dk * sizeof(double));
  double *v_rep = (double *)malloc((size_t)n * Dv * sizeof(double));
  double *p = (double *)malloc((size_t)n * sizeof(double));
  double *qr = (double *)malloc((size_t)Dk * sizeof(double));
  if (!k_rep || !v_rep || !p || !qr) {
    free(k_rep); free(v_rep); free(p); free(qr);
    return -1;
  }
  for (int h = 0; h < Hq; ++h) {
    const int g = h / G;
    /* Explicit replication: this head's copy of KV head g. */
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t t = 0; t < n; ++t) {
      memcpy(k_rep + (size_t)t * Dk, kc + ((size_t)t * Hkv + g) * Dk,
             Dk * sizeof(double));
      memcpy(v_rep + (size_t)t * Dv, vc + ((size_t)t * Hkv + g) * Dv,
             Dv * sizeof(double));
    }
    rope_vec(q + (size_t)h * Dk, qr, Dk, rotary_dims, theta, L);
    /* Pass 1: scaled scores of the visible rows and their maximum. */
    double m = -INFINITY;
#pragma omp parallel for num_threads(nthreads) schedule(static) reduction(max : m)
    for (int64_t t = 0; t < n; ++t) {
      if (!allowed(L, row0 + t, window)) continue;
      double s = 0.0;
      for (int d = 0; d < Dk; ++d) s += qr[d] * k_rep[(size_t)t * Dk + d];
      s *= scale;
      p[t] = s;
      if (s > m) m = s;
    }
    /* Pass 2: exponentials and their sum. */
    double denom = 0.0;
#pragma omp parallel for num_threads(nthreads) schedule(static) reduction(+ : denom)
    for (int64_t t = 0; t < n; ++t) {
      if (!allowed(L, row0 + t, window)) continue;
      p[t] = exp(p[t] - m);
      denom += p[t];
    }
    /* Pass 3: probability-weighted values. */
    double *out = o + (size_t)h * Dv;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int d = 0; d < Dv; ++d) {
      double acc = 0.0;
      for (int64_t t = 0; t < n; ++t)
        if (allowed(L, row0 + t, window)) acc += p[t] * v_rep[(size_t)t * Dv + d];
      out[d] = acc / denom;
    }
  }
  free(k_rep); free(v_rep); free(p); free(qr);
  return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
