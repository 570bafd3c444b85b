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

/* Elements idx .. idx+n-1 of a tensor stored as dtype, widened exactly to fp64. */
static void orc_widen(const void* base, int dtype, int64_t idx, int32_t n, double* dst) {
  if (dtype == ORC_F64) {
    memcpy(dst, (const double*)base + idx, sizeof(double) * (size_t)n);
  } else if (dtype == ORC_F32) {
    const float* src = (const float*)base + idx;
    for (int32_t e = 0; e < n; ++e) dst[e] = (double)src[e];
  } else {
    const uint16_t* src = (const uint16_t*)base + idx;   /* bf16: the upper half of an fp32 */
    for (int32_t e = 0; e < n; ++e) {
      const uint32_t bits = (uint32_t)src[e] << 16;
      float f;
      memcpy(&f, &bits, sizeof f);
      dst[e] = (double)f;
    }
  }
}

/* Rows are independent.  They are evaluated in blocks of up to ORC_ROWS rows
 * that read the same KV head (taken in order of query position), key by key,
 * so a block reads each key's K and V rows once instead of once per row.
 * Every row's arithmetic is the one-row definition above, in the same order:
 * each dot product adds its terms in feature order, and the maximum, the
 * normaliser and the weighted sum of values run over keys in key order.  So
 * the blocking changes no value; it only spares host memory traffic. */
enum { ORC_ROWS = 16 };

int orc_version(void) { return 2; }

typedef struct {
  int32_t g;        /* KV head */
  int64_t pos;      /* absolute query position */
  int64_t r;        /* index into the caller's row list */
} orc_row;

static int orc_row_cmp(const void* a, const void* b) {
  const orc_row* x = (const orc_row*)a;
  const orc_row* y = (const orc_row*)b;
  if (x->g != y->g) return x->g < y->g ? -1 : 1;
  if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;
  return x->r < y->r ? -1 : (x->r > y->r);
}

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
  if (n_rows == 0) return 0;
  orc_row* order = (orc_row*)malloc(sizeof(orc_row) * (size_t)n_rows);
  int64_t* block_start = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_rows + 1));
  if (!order || !block_start) {
    free(order);
    free(block_start);
    return -1;
  }
  for (int64_t r = 0; r < n_rows; ++r) {
    order[r].g = head[r] / group;
    order[r].pos = past_len + tok[r];
    order[r].r = r;
  }
  qsort(order, (size_t)n_rows, sizeof(orc_row), orc_row_cmp);
  int64_t n_blocks = 0;
  for (int64_t r = 0; r < n_rows; ++r)
    if (r == 0 || order[r].g != order[r - 1].g || r - block_start[n_blocks - 1] == ORC_ROWS)
      block_start[n_blocks++] = r;
  block_start[n_blocks] = n_rows;

  int err = 0;
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
  {
    const int64_t span = kv_len > 0 ? kv_len : 1;
    double* s = (double*)malloc(sizeof(double) * (size_t)span * ORC_ROWS);      /* logits, [row][key] */
    double* acc = (double*)malloc(sizeof(double) * (size_t)dv * ORC_ROWS);     /* weighted sums, [row][e] */
    double* qt = (double*)malloc(sizeof(double) * (size_t)d * ORC_ROWS);      /* queries, [e][row] */
    double* kd = (double*)malloc(sizeof(double) * (size_t)d);
    double* vd = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!s || !acc || !qt || !kd || !vd) {
#pragma omp atomic write
      err = -1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t b = 0; b < n_blocks; ++b) {
        const orc_row* rows = order + block_start[b];
        const int32_t nr = (int32_t)(block_start[b + 1] - block_start[b]);
        const int32_t g = rows[0].g;
        int64_t lo[ORC_ROWS], hi[ORC_ROWS];
        double m[ORC_ROWS], l[ORC_ROWS], dot[ORC_ROWS];
        int64_t j_lo = -1, j_hi = 0;
        for (int32_t t = 0; t < nr; ++t) {
          lo[t] = key_lo < 0 ? 0 : key_lo;
          hi[t] = rows[t].pos + 1;                         /* causal: keys 0..pos */
          if (key_hi >= 0 && key_hi < hi[t]) hi[t] = key_hi;
          if (hi[t] > lo[t]) {
            if (j_lo < 0 || lo[t] < j_lo) j_lo = lo[t];
            if (hi[t] > j_hi) j_hi = hi[t];
          }
          m[t] = -INFINITY;
          l[t] = 0.0;
          const int64_t i = rows[t].pos - past_len;
          const int32_t h = head[rows[t].r];
          for (int32_t e = 0; e < d; ++e) qt[(int64_t)e * ORC_ROWS + t] = orc_load(q, dtype, (i * Hq + h) * (int64_t)d + e);
          for (int32_t e = 0; e < dv; ++e) acc[(int64_t)t * dv + e] = 0.0;
        }
        /* pass 1: logits and their maxima */
        for (int64_t j = (j_lo < 0 ? 0 : j_lo); j < j_hi; ++j) {
          orc_widen(k, dtype, (j * Hkv + g) * (int64_t)d, d, kd);
          for (int32_t t = 0; t < nr; ++t) dot[t] = 0.0;
          for (int32_t e = 0; e < d; ++e) {
            const double ke = kd[e];
            const double* qe = qt + (int64_t)e * ORC_ROWS;
            for (int32_t t = 0; t < nr; ++t) dot[t] += qe[t] * ke;
          }
          for (int32_t t = 0; t < nr; ++t) {
            if (j < lo[t] || j >= hi[t]) continue;
            const double sj = scale * dot[t];
            s[(int64_t)t * span + j] = sj;
            if (sj > m[t]) m[t] = sj;
          }
        }
        /* pass 2: weights, normalisers, weighted sums of values */
        for (int64_t j = (j_lo < 0 ? 0 : j_lo); j < j_hi; ++j) {
          orc_widen(v, dtype, (j * Hkv + g) * (int64_t)dv, dv, vd);
          for (int32_t t = 0; t < nr; ++t) {
            if (j < lo[t] || j >= hi[t]) continue;
            const double w = exp(s[(int64_t)t * span + j] - m[t]);
            l[t] += w;
            double* a = acc + (int64_t)t * dv;
            for (int32_t e = 0; e < dv; ++e) a[e] += w * vd[e];
          }
        }
        for (int32_t t = 0; t < nr; ++t) {
          const int64_t r = rows[t].r;
          double* o = out + r * dv;
          if (hi[t] <= lo[t]) {
            for (int32_t e = 0; e < dv; ++e) o[e] = 0.0;
            lse[r] = -INFINITY;
            continue;
          }
          for (int32_t e = 0; e < dv; ++e) o[e] = acc[(int64_t)t * dv + e] / l[t];
          lse[r] = m[t] + log(l[t]);
        }
      }
    }
    free(s);
    free(acc);
    free(qt);
    free(kd);
    free(vd);
  }
  free(order);
  free(block_start);
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
