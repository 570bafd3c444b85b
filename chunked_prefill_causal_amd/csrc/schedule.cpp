// Two-rank pipeline schedules that chunked prefill feeds (host code, no GPU).
//
// VPP technical review (English edition):
//  * §4.1 Eq. (2): the per-stage latency tau_k of chunk k grows near-linearly
//    with k when attention dominates; here tau comes from the caller (for
//    example the measured per-chunk latency of the prefill kernel).
//  * §2.4 / §4.2: the conventional layout ("CPP") runs stages s0, s1 on pp0 and
//    s2, s3 on pp1, chunk after chunk.
//  * §4.2 Alg. 1, Eq. (3a)/(3b): the V-shaped layout runs s0, s3 on pp0 and
//    s1, s2 on pp1; while pp1 runs chunk k's middle stages, pp0 runs s3 of
//    chunk k-1 then s0 of chunk k+1.
//  * §4.4: VPP-Async issues pp0's pair the other way round (s0 of k+1 first).
//  * §4.5 Alg. 2, Eq. (4a): the next request's leading chunks are packed into
//    the (N+1)t drain window, greedily while they fit.
//
// Model: every virtual stage of chunk k takes tau[k]; a hand-off between
// ranks delays the receiving stage by `comm` without occupying either rank;
// stages run in a fixed per-rank order, each starting once its rank is free
// and its predecessor stage has ended.  Without packing a request's first
// stage also waits for the previous request's last stage.
#include <cmath>
#include <cstdint>
#include <vector>

#include "chunkattn.h"

namespace chunkattn {
void set_error(const char* fmt, ...);
void clear_error();
}

namespace {

using chunkattn::clear_error;
using chunkattn::set_error;

struct Stage {
  int32_t chunk;
  int8_t index;   // virtual stage 0..3
};

// rank holding each virtual stage, per layout
constexpr int8_t kRank[3][4] = {{0, 0, 1, 1}, {0, 1, 1, 0}, {0, 1, 1, 0}};

// Greedy packing of Alg. 2: leading chunks of the next request whose tau fits
// in what is left of the (n + 1) t window.
int32_t pack_count(int32_t n, double t, int32_t n_next, const double* tau_next, double* left) {
  double window = (double)(n + 1) * t;
  int32_t j = 0;
  while (j < n_next && tau_next[j] <= window) {
    window -= tau_next[j];
    ++j;
  }
  if (left) *left = window;
  return j;
}

// Appends one request's per-rank stage order (chunks k0 .. k0+n-1).
void append_request(int kind, int32_t k0, int32_t n, std::vector<Stage>* pp0, std::vector<Stage>* pp1) {
  if (kind == CA_SCHED_CPP) {
    for (int32_t k = k0; k < k0 + n; ++k) {
      pp0->push_back({k, 0});
      pp0->push_back({k, 1});
      pp1->push_back({k, 2});
      pp1->push_back({k, 3});
    }
    return;
  }
  for (int32_t k = k0; k < k0 + n; ++k) {
    pp1->push_back({k, 1});
    pp1->push_back({k, 2});
  }
  pp0->push_back({k0, 0});
  for (int32_t i = 0; i < n; ++i) {          // pp1 on chunk k0+i's middle stages
    const bool tail = i >= 1, head = i + 1 < n;
    if (kind == CA_SCHED_VPP_ASYNC) {
      if (head) pp0->push_back({k0 + i + 1, 0});
      if (tail) pp0->push_back({k0 + i - 1, 3});
    } else {
      if (tail) pp0->push_back({k0 + i - 1, 3});
      if (head) pp0->push_back({k0 + i + 1, 0});
    }
  }
  pp0->push_back({k0 + n - 1, 3});
}

}  // namespace

extern "C" int32_t chunkattn_sched_drain_pack(int32_t n_chunks, double t, int32_t n_next, const double* tau_next,
                                              double* window_left) {
  if (n_chunks < 0 || n_next < 0 || !(t >= 0.0) || !std::isfinite(t) || (n_next > 0 && !tau_next)) {
    set_error("chunkattn_sched_drain_pack: need n_chunks, n_next >= 0, finite t >= 0 and tau_next");
    return CA_EINVAL;
  }
  for (int32_t j = 0; j < n_next; ++j)
    if (!(tau_next[j] >= 0.0) || !std::isfinite(tau_next[j])) {
      set_error("chunkattn_sched_drain_pack: tau_next[%d] is negative or not finite", j);
      return CA_EINVAL;
    }
  clear_error();
  return pack_count(n_chunks, t, n_next, tau_next, window_left);
}

extern "C" ca_status chunkattn_sched_simulate(int32_t kind, int32_t n_chunks, const double* tau, const int32_t* request,
                                              double comm, int32_t pack, double* stage_start, double* stage_end,
                                              double* rank_busy, double* makespan) {
  if (kind < CA_SCHED_CPP || kind > CA_SCHED_VPP_ASYNC) {
    set_error("chunkattn_sched_simulate: unknown schedule kind %d", kind);
    return CA_EINVAL;
  }
  if (n_chunks < 0 || (n_chunks > 0 && !tau) || !makespan || !(comm >= 0.0) || !std::isfinite(comm)) {
    set_error("chunkattn_sched_simulate: need n_chunks >= 0, tau, makespan and finite comm >= 0");
    return CA_EINVAL;
  }
  for (int32_t k = 0; k < n_chunks; ++k) {
    if (!(tau[k] >= 0.0) || !std::isfinite(tau[k])) {
      set_error("chunkattn_sched_simulate: tau[%d] is negative or not finite", k);
      return CA_EINVAL;
    }
    if (request && k > 0 && request[k] < request[k - 1]) {
      set_error("chunkattn_sched_simulate: request ids must not decrease (chunk %d)", k);
      return CA_EINVAL;
    }
  }
  // requests as [first chunk, count)
  std::vector<int32_t> first, count;
  for (int32_t k = 0; k < n_chunks; ++k) {
    if (k == 0 || (request && request[k] != request[k - 1])) {
      first.push_back(k);
      count.push_back(0);
    }
    ++count.back();
  }
  std::vector<Stage> order[2];
  std::vector<char> moved(n_chunks, 0);      // entry stages already placed in a drain slot
  for (size_t r = 0; r < first.size(); ++r) {
    std::vector<Stage> pp0, pp1;
    append_request(kind, first[r], count[r], &pp0, &pp1);
    std::vector<Stage> heads;
    if (pack && kind != CA_SCHED_CPP && r + 1 < first.size()) {
      const int32_t j = pack_count(count[r], tau[first[r]], count[r + 1], tau + first[r + 1], nullptr);
      for (int32_t i = 0; i < j; ++i) heads.push_back({first[r + 1] + i, 0});
    }
    for (size_t i = 0; i < pp0.size(); ++i) {
      const Stage st = pp0[i];
      if (i + 1 == pp0.size())
        for (const Stage& h : heads) {       // drain slot: before the last exit stage
          order[0].push_back(h);
          moved[h.chunk] = 1;
        }
      if (st.index == 0 && moved[st.chunk]) continue;   // issued in the previous drain slot
      order[0].push_back(st);
    }
    order[1].insert(order[1].end(), pp1.begin(), pp1.end());
  }

  // list scheduling: advance whichever rank can start its next stage
  std::vector<double> t0(4 * (size_t)n_chunks, -1.0), t1(4 * (size_t)n_chunks, -1.0);
  size_t next[2] = {0, 0};
  double free_at[2] = {0.0, 0.0}, busy[2] = {0.0, 0.0};
  std::vector<int32_t> request_of(n_chunks), last_of_prev(n_chunks, -1);
  for (size_t r = 0; r < first.size(); ++r)
    for (int32_t k = first[r]; k < first[r] + count[r]; ++k) {
      request_of[k] = (int32_t)r;
      last_of_prev[k] = r > 0 ? first[r] - 1 : -1;
    }
  const int8_t* rank_of = kRank[kind];
  size_t remaining = order[0].size() + order[1].size();
  while (remaining > 0) {
    bool advanced = false;
    for (int rk = 0; rk < 2; ++rk) {
      if (next[rk] >= order[rk].size()) continue;
      const Stage st = order[rk][next[rk]];
      double ready = free_at[rk];
      if (st.index > 0) {
        const double prev_end = t1[4 * (size_t)st.chunk + st.index - 1];
        if (prev_end < 0.0) continue;
        const double hop = rank_of[st.index - 1] != rank_of[st.index] ? comm : 0.0;
        if (prev_end + hop > ready) ready = prev_end + hop;
      } else if (!pack && st.chunk == first[request_of[st.chunk]] && last_of_prev[st.chunk] >= 0) {
        const double prev_req_end = t1[4 * (size_t)last_of_prev[st.chunk] + 3];
        if (prev_req_end < 0.0) continue;
        if (prev_req_end > ready) ready = prev_req_end;
      }
      const size_t slot = 4 * (size_t)st.chunk + st.index;
      t0[slot] = ready;
      t1[slot] = ready + tau[st.chunk];
      free_at[rk] = t1[slot];
      busy[rk] += tau[st.chunk];
      ++next[rk];
      --remaining;
      advanced = true;
    }
    if (!advanced) {
      set_error("chunkattn_sched_simulate: the stage order deadlocked");
      return CA_EINVAL;
    }
  }
  double span = 0.0;
  for (size_t i = 0; i < t1.size(); ++i) span = t1[i] > span ? t1[i] : span;
  if (stage_start)
    for (size_t i = 0; i < t0.size(); ++i) stage_start[i] = t0[i];
  if (stage_end)
    for (size_t i = 0; i < t1.size(); ++i) stage_end[i] = t1[i];
  if (rank_busy) {
    rank_busy[0] = busy[0];
    rank_busy[1] = busy[1];
  }
  *makespan = span;
  clear_error();
  return CA_OK;
}
