// Online attention-latency predictor (host code, no GPU).
//
// "Revisiting Pipeline Parallelism for LLM Serving" paper notes, §2.3: the
// ALP predictor models the attention share of an iteration with three
// features summed over the batch — new prefill tokens against the existing
// context (L_past * L_pre), the chunk against itself (L_pre^2), and decode
// requests reading their context (L_dec) — and adapts their coefficients
// online by recursive least squares with a forgetting factor.  Here the model
// is the attention kernel alone, so a constant (launch and tail cost) takes
// the place of the notes' offline token-linear term:
//
//   T = theta0 + theta1 * sum(L_past L_pre) / 1e6 + theta2 * sum(L_pre^2) / 1e6
//       + theta3 * sum(L_dec) / 1e3 + theta4 * fill
//
// (features scaled to millions / thousands of tokens).  The fill term is this
// library's addition: a prefill launch of W workgroups (one per CU) on 256 CUs
// runs ceil(W / 256) rounds, and a short chunk leaves most of its last round
// idle, which no term linear in the pages' features expresses.  fill = (ceil(W /
// 256) * 256 / W - 1) x the launch's causal pairs / 1e6: the work the idle CUs
// stand for.  The least-squares fit
// is recursive with a forgetting factor lambda, kept in information form: the
// exponentially weighted normal equations
//   R <- lambda R + x x',  b <- lambda b + x y,  R_0 = I / delta,
// are updated per observation and theta solves R theta = b (4 x 4 Cholesky).
// This is the same estimate as the gain form of RLS (whose covariance is
// R^-1) but keeps full precision when delta is large, where the gain form
// cancels away most digits in its first updates.
#include <cmath>
#include <cstdint>

#include "chunkattn.h"

namespace chunkattn {
void set_error(const char* fmt, ...);
void clear_error();
int64_t varlen_prefill_workgroups(int q_len, int heads, int kv_heads);
int num_cus();
}

using chunkattn::clear_error;
using chunkattn::set_error;

namespace {
constexpr int kF = CA_ALP_FEATURES;
bool finite_vec(const double* x, int n) {
  for (int i = 0; i < n; ++i)
    if (!std::isfinite(x[i])) return false;
  return true;
}
}  // namespace

extern "C" ca_status chunkattn_alp_features(int32_t num_seqs, const int32_t* q_lens, const int32_t* kv_lens,
                                            int32_t heads, int32_t kv_heads, double* x) {
  if (num_seqs < 0 || !x || (num_seqs > 0 && (!q_lens || !kv_lens))) {
    set_error("chunkattn_alp_features: need num_seqs >= 0, q_lens, kv_lens and x");
    return CA_EINVAL;
  }
  if (heads <= 0 || kv_heads <= 0 || heads % kv_heads != 0) {
    set_error("chunkattn_alp_features: heads (%d) must be a positive multiple of kv_heads (%d)", heads, kv_heads);
    return CA_EINVAL;
  }
  double past_pre = 0.0, pre_sq = 0.0, dec = 0.0, fill_pairs = 0.0;
  int64_t wgs = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t q = q_lens[s], kv = kv_lens[s];
    if (q < 0 || kv < q) {
      set_error("chunkattn_alp_features: sequence %d has q_len %lld and kv_len %lld", s, (long long)q,
                (long long)kv);
      return CA_EINVAL;
    }
    if (q == 1) {
      dec += (double)kv;
    } else if (q > 1) {
      past_pre += (double)(kv - q) * (double)q;
      pre_sq += (double)q * (double)q;
    }
    const int64_t w = chunkattn::varlen_prefill_workgroups((int)q, heads, kv_heads);
    if (w) {
      wgs += w;
      fill_pairs += (double)(kv - q) * (double)q + (double)q * (double)(q + 1) / 2.0;
    }
  }
  const int64_t cus = chunkattn::num_cus();
  const double idle = wgs ? (double)((wgs + cus - 1) / cus * cus) / (double)wgs - 1.0 : 0.0;
  x[0] = 1.0;
  x[1] = past_pre / 1e6;
  x[2] = pre_sq / 1e6;
  x[3] = dec / 1e3;
  x[4] = idle * fill_pairs / 1e6;
  clear_error();
  return CA_OK;
}

extern "C" ca_status chunkattn_alp_init(ca_alp_state* st, double lambda, double delta) {
  if (!st || !(lambda > 0.0 && lambda <= 1.0) || !(delta > 0.0) || !std::isfinite(delta)) {
    set_error("chunkattn_alp_init: need a state, 0 < lambda <= 1 and finite delta > 0");
    return CA_EINVAL;
  }
  for (int i = 0; i < kF; ++i) {
    st->theta[i] = 0.0;
    st->rhs[i] = 0.0;
    for (int j = 0; j < kF; ++j) st->info[i * kF + j] = i == j ? 1.0 / delta : 0.0;
  }
  st->lambda = lambda;
  st->n_obs = 0;
  clear_error();
  return CA_OK;
}

extern "C" double chunkattn_alp_predict(const ca_alp_state* st, const double* x) {
  if (!st || !x) return NAN;
  double y = 0.0;
  for (int i = 0; i < kF; ++i) y += st->theta[i] * x[i];
  return y;
}

extern "C" ca_status chunkattn_alp_update(ca_alp_state* st, const double* x, double measured, double* prior_error) {
  if (!st || !x || !finite_vec(x, kF) || !std::isfinite(measured)) {
    set_error("chunkattn_alp_update: need a state, finite features and a finite measurement");
    return CA_EINVAL;
  }
  const double err = measured - chunkattn_alp_predict(st, x);
  double r[kF * kF], rhs[kF];
  for (int i = 0; i < kF; ++i) {
    rhs[i] = st->lambda * st->rhs[i] + x[i] * measured;
    for (int j = 0; j < kF; ++j) r[i * kF + j] = st->lambda * st->info[i * kF + j] + x[i] * x[j];
  }
  // Cholesky R = L L' (R is symmetric positive definite: I / delta scaled by lambda^n plus a Gram sum)
  double l[kF * kF] = {};
  for (int j = 0; j < kF; ++j) {
    double d = r[j * kF + j];
    for (int k = 0; k < j; ++k) d -= l[j * kF + k] * l[j * kF + k];
    if (!(d > 0.0)) {
      set_error("chunkattn_alp_update: the normal equations lost positive definiteness");
      return CA_ERANGE;
    }
    l[j * kF + j] = std::sqrt(d);
    for (int i = j + 1; i < kF; ++i) {
      double v = r[i * kF + j];
      for (int k = 0; k < j; ++k) v -= l[i * kF + k] * l[j * kF + k];
      l[i * kF + j] = v / l[j * kF + j];
    }
  }
  double z[kF], th[kF];
  for (int i = 0; i < kF; ++i) {                 // L z = rhs
    double v = rhs[i];
    for (int k = 0; k < i; ++k) v -= l[i * kF + k] * z[k];
    z[i] = v / l[i * kF + i];
  }
  for (int i = kF - 1; i >= 0; --i) {            // L' theta = z
    double v = z[i];
    for (int k = i + 1; k < kF; ++k) v -= l[k * kF + i] * th[k];
    th[i] = v / l[i * kF + i];
  }
  for (int i = 0; i < kF; ++i) {
    st->theta[i] = th[i];
    st->rhs[i] = rhs[i];
    for (int j = 0; j < kF; ++j) st->info[i * kF + j] = r[i * kF + j];
  }
  st->n_obs += 1;
  if (prior_error) *prior_error = err;
  clear_error();
  return CA_OK;
}
