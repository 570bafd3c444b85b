/*
 * TEST INFRASTRUCTURE ONLY — the fp64 CPU oracle for chunked-prefill causal
 * attention.  Only tests, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The GPU library shares no code, header, table or
 * helper with it.
 *
 * What it computes (the plain definition, not an algorithm under test):
 *
 *   VPP: Virtual Pipeline Parallelism for Efficient Chunked Prefill in
 *   Long-Context LLM Inference — technical review (English edition):
 *     §2.2, Eq. (1): Attn(Q,K,V) = softmax(Q K^T / sqrt(d)) V;
 *     §2.2, causal rule: token i attends only to tokens at positions <= i;
 *     §2.3, chunked prefill: a later chunk attends to the KV cache of every
 *           preceding chunk plus itself.
 *
 * So a query row (token i of a chunk that starts at absolute position
 * past_len, query head h) sits at absolute position p = past_len + i and sees
 * keys j = 0..p of the logical cache.  Grouped-query attention maps query
 * head h to KV head h / (Hq / Hkv) (contiguous groups).  The scale is a
 * parameter (1/sqrt(head_dim) in every workload).
 *
 * Computation per row, in IEEE fp64, two passes, no fast-math:
 *   pass 1: s_j = scale * sum_e q[e] k_j[e],  m = max_j s_j
 *   pass 2: w_j = exp(s_j - m),  l = sum_j w_j,  o = (sum_j w_j v_j) / l
 *   lse = m + ln(l)   (natural log)
 *
 * A key range [key_lo, key_hi) restricts j further (the partial attention of
 * one key split).  An empty range yields o = 0 and lse = -inf.
 *
 * orc_merge combines partials by log-sum-exp weights: the result over a key
 * partition equals the result over the union (the merge that decode context
 * parallelism needs from an attention backend returning LSE; GLM5.3 PP-split
 * deployment notes, §7).
 *
 * Inputs are read as stored: fp32, or bf16 bit patterns widened exactly to
 * fp64.  Nothing is rounded on the way in.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };

static double orc_load(const void* base, int dtype, int64_t idx) {
  if (dtype == ORC_F32) return (double)((const float*)base)[idx];
  if (dtype == ORC_F64) return ((const double*)base)[idx];
  uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

int orc_version(void) { return 1; }

/*
 * Attention for an explicit list of query rows.
 *   q      [chunk_len, Hq, d]       (row-major, token-major)
 *   k      [kv_len,    Hkv, d]      logical cache, positions 0..kv_len-1
 *   v      [kv_len,    Hkv, dv]
 *   rows   n_rows pairs (tok[r], head[r])
 *   out    [n_rows, dv] fp64,  lse [n_rows] fp64
 * Returns 0, or -1 on an argument error (row out of range, key beyond kv_len).
 */
int orc_attend_rows(const void* q, const void* k, const void* v, int dtype,
                    int64_t chunk_len, int64_t kv_len, int32_t Hq, int32_t Hkv,
                    int32_t d, int32_t dv, double scale, int64_t past_len,
                    int64_t n_rows, const int64_t* tok, const int32_t* head,
                    int64_t key_lo, int64_t key_hi,
                    double* out, double* lse, int32_t nthreads) {
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || dv <= 0) return -1;
  const int32_t group = Hq / Hkv;
  for (int64_t r = 0; r < n_rows; ++r) {
    if (tok[r] < 0 || tok[r] >= chunk_len || head[r] < 0 || head[r] >= Hq) return -1;
    if (past_len + tok[r] >= kv_len) return -1;
  }
  int err = 0;
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(kv_len > 0 ? kv_len : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!s || !acc) {
#pragma omp atomic write
      err = -1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t i = tok[r];
        const int32_t h = head[r];
        const int32_t g = h / group;
        const int64_t p = past_len + i;           /* absolute query position */
        int64_t lo = key_lo < 0 ? 0 : key_lo;
        int64_t hi = p + 1;                       /* causal: keys 0..p */
        if (key_hi >= 0 && key_hi < hi) hi = key_hi;
        double* o = out + r * dv;
        if (hi <= lo) {
          for (int32_t e = 0; e < dv; ++e) o[e] = 0.0;
          lse[r] = -INFINITY;
          continue;
        }
        const int64_t qoff = (i * Hq + h) * (int64_t)d;
        /* pass 1: logits and their maximum */
        double m = -INFINITY;
        for (int64_t j = lo; j < hi; ++j) {
          const int64_t koff = (j * Hkv + g) * (int64_t)d;
          double dot = 0.0;
          for (int32_t e = 0; e < d; ++e)
            dot += orc_load(q, dtype, qoff + e) * orc_load(k, dtype, koff + e);
          s[j - lo] = scale * dot;
          if (s[j - lo] > m) m = s[j - lo];
        }
        /* pass 2: weights, normaliser, weighted sum of values */
        double l = 0.0;
        for (int32_t e = 0; e < dv; ++e) acc[e] = 0.0;
        for (int64_t j = lo; j < hi; ++j) {
          const double w = exp(s[j - lo] - m);
          l += w;
          const int64_t voff = (j * Hkv + g) * (int64_t)dv;
          for (int32_t e = 0; e < dv; ++e) acc[e] += w * orc_load(v, dtype, voff + e);
        }
        for (int32_t e = 0; e < dv; ++e) o[e] = acc[e] / l;
        lse[r] = m + log(l);
      }
    }
    free(s);
    free(acc);
  }
  return err;
}

/*
 * Log-sum-exp merge of n_parts partial results over disjoint key ranges.
 *   o_parts  [n_parts, n_rows, dv],  lse_parts [n_parts, n_rows]
 *   out      [n_rows, dv],           lse       [n_rows]
 * A part with lse = -inf (empty range) carries weight 0.
 */
int orc_merge(int32_t n_parts, int64_t n_rows, int32_t dv,
              const double* o_parts, const double* lse_parts,
              double* out, double* lse) {
  if (n_parts <= 0 || dv <= 0) return -1;
  for (int64_t r = 0; r < n_rows; ++r) {
    double M = -INFINITY;
    for (int32_t s = 0; s < n_parts; ++s)
      if (lse_parts[s * n_rows + r] > M) M = lse_parts[s * n_rows + r];
    double* o = out + r * dv;
    for (int32_t e = 0; e < dv; ++e) o[e] = 0.0;
    if (M == -INFINITY) { lse[r] = -INFINITY; continue; }
    double W = 0.0;
    for (int32_t s = 0; s < n_parts; ++s) {
      const double ls = lse_parts[s * n_rows + r];
      if (ls == -INFINITY) continue;
      const double w = exp(ls - M);
      W += w;
      const double* os = o_parts + ((int64_t)s * n_rows + r) * dv;
      for (int32_t e = 0; e < dv; ++e) o[e] += w * os[e];
    }
    for (int32_t e = 0; e < dv; ++e) o[e] /= W;
    lse[r] = M + log(W);
  }
  return 0;
}
