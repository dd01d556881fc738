/*
 * fa_oracle.c - plain, slow, fp64 CPU oracle for fused attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke check
 * and the CPU-baseline leg of the benchmark do. It shares no code, header or
 * constant with the HIP library.
 *
 * The method on the pages (tiling with a running max, running sum and a
 * rescaled accumulator - "Real-time inference optimisation", section "Flash
 * Attention optimisation") reaches, in exact arithmetic, exactly the plain
 * softmax attention. So this oracle is that plain definition written out:
 * materialise one row of scores, take its max, exponentiate, sum, divide, and
 * multiply by V. No tiling, no online rescale, no split, no reordering:
 * every reduction runs over ascending indices.
 *
 * Readings of points the pages leave open (each one is also listed in the
 * design notes):
 *   - the scale multiplies the raw dot product q.k (the page's kernel scales
 *     after the dot; its 1/sqrt(K) is garbled, so the scale is an argument);
 *   - causal alignment is bottom-right: row i sees keys j <= i + Skv - Sq;
 *   - kv head of query head h is floor(h * Hkv / Hq);
 *   - decode: the one query sees all seqlens[b] cached tokens; a sequence of
 *     length 0 has output 0 and log-sum-exp -inf;
 *   - paged cache: page size is a parameter (16 in every workload, as on the
 *     real-time inference page's paged sketch); token t of sequence b lives in
 *     page block_table[b][t / page] at slot t % page.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared (no -ffast-math: the oracle keeps
 * IEEE double semantics). OpenMP only distributes independent (b, h) rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* One output row: scores s[0..n) already materialised (already scaled).
 * Writes o[0..d) and returns lse = m + log(sum exp(s - m)). The value rows are
 * given by an array of row pointers so that the caller does its own gather. */
static double softmax_times_v(const double* s, int n, const double* const* vrow, int d, double* o) {
  if (n == 0) {
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    return -INFINITY;
  }
  double m = s[0];
  for (int j = 1; j < n; ++j)
    if (s[j] > m) m = s[j];
  double* e = (double*)malloc(sizeof(double) * (size_t)n);
  double L = 0.0;
  for (int j = 0; j < n; ++j) {
    e[j] = exp(s[j] - m);
    L += e[j];
  }
  for (int c = 0; c < d; ++c) o[c] = 0.0;
  for (int j = 0; j < n; ++j) {
    const double p = e[j] / L;
    const double* vj = vrow[j];
    for (int c = 0; c < d; ++c) o[c] += p * vj[c];
  }
  free(e);
  return m + log(L);
}

static double dot(const double* a, const double* b, int d) {
  double acc = 0.0;
  for (int c = 0; c < d; ++c) acc += a[c] * b[c];
  return acc;
}

/*
 * Full attention (prefill). q, o: [B, Hq, Sq, d]; k, v: [B, Hkv, Skv, d].
 * lse (optional, may be NULL): [B, Hq, Sq] natural-log log-sum-exp of the
 * scaled scores of each row. Returns 0, or -1 on invalid shapes.
 */
int oracle_attention_f64(const double* q, const double* k, const double* v, double* o, double* lse,
                         int B, int Hq, int Hkv, int Sq, int Skv, int d, double scale, int causal) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Sq < 0 || Skv < 0 || d <= 0) return -1;
  if (Hq % Hkv != 0) return -1;
  if (causal && Sq > Skv) return -1;
  const long nbh = (long)B * Hq;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
    const double** vrow = (const double**)malloc(sizeof(double*) * (size_t)(Skv > 0 ? Skv : 1));
#pragma omp for schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
      const int b = (int)(bh / Hq), h = (int)(bh % Hq);
      const int g = (int)((long)h * Hkv / Hq);
      const double* kb = k + ((size_t)b * Hkv + g) * (size_t)Skv * d;
      const double* vb = v + ((size_t)b * Hkv + g) * (size_t)Skv * d;
      for (int i = 0; i < Sq; ++i) {
        const double* qi = q + (((size_t)b * Hq + h) * Sq + i) * d;
        int n = Skv;
        if (causal) n = i + (Skv - Sq) + 1; /* keys 0 .. i + Skv - Sq */
        for (int j = 0; j < n; ++j) {
          s[j] = scale * dot(qi, kb + (size_t)j * d, d);
          vrow[j] = vb + (size_t)j * d;
        }
        double* oi = o + (((size_t)b * Hq + h) * Sq + i) * d;
        const double l = softmax_times_v(s, n, vrow, d, oi);
        if (lse) lse[((size_t)b * Hq + h) * Sq + i] = l;
      }
    }
    free(s);
    free(vrow);
  }
  return 0;
}

/*
 * Decode: one query per sequence over its cached tokens.
 *   q, o      : [B, Hq, d]
 *   block_table == NULL: kc, vc are [B, max_kv_len, Hkv, d]
 *   block_table != NULL: kc, vc are [num_pages, page, Hkv, d] and block_table is
 *                        [B, pages_per_seq]; token t of sequence b is row
 *                        block_table[b*pages_per_seq + t/page]*page + t%page.
 *   seqlens   : [B]; clamped to [0, max_kv_len].
 *   lse       : optional [B, Hq].
 * Returns 0, or -1 on invalid shapes.
 */
int oracle_decode_f64(const double* q, const double* kc, const double* vc, const int32_t* block_table,
                      int pages_per_seq, const int32_t* seqlens, double* o, double* lse, int B, int Hq,
                      int Hkv, int d, int max_kv_len, int page, double scale) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || max_kv_len < 0 || page <= 0) return -1;
  if (Hq % Hkv != 0) return -1;
  const long nbh = (long)B * Hq;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(max_kv_len > 0 ? max_kv_len : 1));
    const double** vrow = (const double**)malloc(sizeof(double*) * (size_t)(max_kv_len > 0 ? max_kv_len : 1));
#pragma omp for schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
      const int b = (int)(bh / Hq), h = (int)(bh % Hq);
      const int g = (int)((long)h * Hkv / Hq);
      int n = seqlens[b];
      if (n < 0) n = 0;
      if (n > max_kv_len) n = max_kv_len;
      const double* qh = q + ((size_t)b * Hq + h) * d;
      for (int t = 0; t < n; ++t) {
        size_t row;
        if (block_table)
          row = (size_t)block_table[(size_t)b * pages_per_seq + t / page] * page + (size_t)(t % page);
        else
          row = (size_t)b * max_kv_len + t;
        const double* kt = kc + (row * Hkv + g) * d;
        s[t] = scale * dot(qh, kt, d);
        vrow[t] = vc + (row * Hkv + g) * d;
      }
      const double l = softmax_times_v(s, n, vrow, d, o + ((size_t)b * Hq + h) * d);
      if (lse) lse[(size_t)b * Hq + h] = l;
    }
    free(s);
    free(vrow);
  }
  return 0;
}

/*
 * Log-sum-exp merge of S partial results per row (R rows):
 *   o_parts [R, S, d] (each normalised by its own softmax sum), lse_parts [R, S].
 *   M = max_s lse_s; w_s = exp(lse_s - M); o = sum_s w_s o_s / sum_s w_s;
 *   lse = M + log(sum_s w_s). Parts with lse = -inf are empty and skipped;
 *   an all-empty row gives o = 0, lse = -inf.
 * This is the combination rule of log-sum-exp algebra: a softmax over the union
 * of disjoint key sets, written from the partial sums. Returns 0.
 */
int oracle_merge_f64(const double* o_parts, const double* lse_parts, double* o, double* lse, int R, int S,
                     int d) {
  for (int r = 0; r < R; ++r) {
    const double* ls = lse_parts + (size_t)r * S;
    double M = -INFINITY;
    for (int s = 0; s < S; ++s)
      if (ls[s] > M) M = ls[s];
    double* orow = o + (size_t)r * d;
    for (int c = 0; c < d; ++c) orow[c] = 0.0;
    if (M == -INFINITY) {
      if (lse) lse[r] = -INFINITY;
      continue;
    }
    double W = 0.0;
    for (int s = 0; s < S; ++s) {
      if (ls[s] == -INFINITY) continue;
      const double w = exp(ls[s] - M);
      W += w;
      const double* os = o_parts + ((size_t)r * S + s) * d;
      for (int c = 0; c < d; ++c) orow[c] += w * os[c];
    }
    for (int c = 0; c < d; ++c) orow[c] /= W;
    if (lse) lse[r] = M + log(W);
  }
  return 0;
}

/* Number of OpenMP threads the oracle runs with (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
