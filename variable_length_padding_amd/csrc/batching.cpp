// Batch planning over a queue of variable-length requests (host only).
//
// The announcement article's "Serving" section and the README's "Batching"
// section: the queue is packed into batches by how fast the machine runs
// them, following TurboTransformers' dynamic programming scheduler, and the
// batch with the highest priority (waiting time, batch size, room to grow at
// its padded length) runs first.  FIFO packing, each batch padded to its
// longest request, is the baseline of the "Performance tests" section.
//
// Dynamic programming: with the requests ordered by length, a batch that is
// a contiguous run [j, i) of that order is padded to the length of request
// i-1, and best[i] = min over j of best[j] + cost(run [j, i)).  Costs are
// sums of products of doubles evaluated in a fixed order, with contraction
// into fused multiply-adds disabled, so every caller that evaluates the same
// formula in the same order gets the same bits and the same tie decisions.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <numeric>
#include <vector>

#include "internal.h"

#pragma clang fp contract(off)

namespace {

struct Run {
  int64_t B, P, tokens;  // requests, padded length, sum of lengths
  double pairs;          // sum len (len + 1) / 2
};

double run_cost(const ee_batch_cost& c, const Run& r) {
  double tok, pairs;
  if (c.padded_compute) {
    tok = (double)(r.B * r.P);
    pairs = (double)r.B * ((double)r.P * (double)(r.P + 1) / 2.0);
  } else {
    tok = (double)r.tokens;
    pairs = r.pairs;
  }
  const double q = c.token_quantum > 1 ? (double)c.token_quantum : 1.0;
  if (c.token_quantum > 1) tok = std::ceil(tok / q) * q;
  double s;
  if (c.token_table && c.token_table_len >= 1) {
    const int64_t k = (int64_t)(tok / q) - 1;  // entry of this token count
    const int64_t last = c.token_table_len - 1;
    if (k < 0)
      s = 0.0;
    else if (k <= last)
      s = c.token_table[k];
    else if (last >= 1)
      s = c.token_table[last] + (double)(k - last) * (c.token_table[last] - c.token_table[last - 1]);
    else
      s = c.token_table[0] * (double)(k + 1);
  } else {
    s = c.t_token * tok;
  }
  return c.t_batch + s + c.t_row * (double)(r.B * r.P) + c.t_pair * pairs;
}

ee_status check_lens(const int32_t* lens, int32_t n) {
  if (n < 0) return ee::set_error(EE_ERR_INVALID_ARG, "n < 0");
  if (n > 0 && !lens) return ee::set_error(EE_ERR_INVALID_ARG, "lens is NULL");
  for (int32_t i = 0; i < n; ++i)
    if (lens[i] < 1) return ee::set_error(EE_ERR_INVALID_ARG, "request length < 1");
  return EE_OK;
}

ee_status check_cost(const ee_batch_cost* c) {
  if (!c) return ee::set_error(EE_ERR_INVALID_ARG, "cost is NULL");
  if (!(c->t_batch >= 0 && c->t_token >= 0 && c->t_row >= 0 && c->t_pair >= 0) || c->token_quantum < 0 ||
      c->token_table_len < 0)
    return ee::set_error(EE_ERR_INVALID_ARG, "cost coefficients must be finite and >= 0");
  for (int32_t k = 0; c->token_table && k < c->token_table_len; ++k)
    if (!(c->token_table[k] >= 0)) return ee::set_error(EE_ERR_INVALID_ARG, "token_table entries must be >= 0");
  return EE_OK;
}

}  // namespace

extern "C" {

EE_API ee_status ee_batch_cost_eval(const int32_t* lens, int32_t n, const ee_batch_cost* cost, double* out) {
  if (ee_status s = check_lens(lens, n)) return s;
  if (ee_status s = check_cost(cost)) return s;
  if (n < 1 || !out) return ee::set_error(EE_ERR_INVALID_ARG, "need n >= 1 and an output");
  Run r{n, 0, 0, 0.0};
  for (int32_t i = 0; i < n; ++i) {
    r.P = std::max<int64_t>(r.P, lens[i]);
    r.tokens += lens[i];
    r.pairs += (double)lens[i] * (double)(lens[i] + 1) / 2.0;
  }
  *out = run_cost(*cost, r);
  return EE_OK;
}

EE_API ee_status ee_plan_fifo(const int32_t* lens, int32_t n, int32_t max_batch, int32_t* batch_of,
                              int32_t* n_batches) {
  if (ee_status s = check_lens(lens, n)) return s;
  if (max_batch < 1) return ee::set_error(EE_ERR_INVALID_ARG, "max_batch < 1");
  if ((n > 0 && !batch_of) || !n_batches) return ee::set_error(EE_ERR_INVALID_ARG, "NULL output");
  for (int32_t i = 0; i < n; ++i) batch_of[i] = i / max_batch;
  *n_batches = (n + max_batch - 1) / max_batch;
  return EE_OK;
}

EE_API ee_status ee_plan_dynamic(const int32_t* lens, const double* wait, int32_t n, int32_t max_batch,
                                 int64_t max_tokens, const ee_batch_cost* cost, int32_t* batch_of,
                                 int32_t* n_batches, double* total_cost) {
  if (ee_status s = check_lens(lens, n)) return s;
  if (ee_status s = check_cost(cost)) return s;
  if (max_batch < 1) return ee::set_error(EE_ERR_INVALID_ARG, "max_batch < 1");
  if ((n > 0 && !batch_of) || !n_batches) return ee::set_error(EE_ERR_INVALID_ARG, "NULL output");
  for (int32_t i = 0; i < n; ++i)
    if (max_tokens > 0 && lens[i] > max_tokens)
      return ee::set_error(EE_ERR_INVALID_ARG, "a request is longer than max_tokens");
  if (n == 0) {
    *n_batches = 0;
    if (total_cost) *total_cost = 0.0;
    return EE_OK;
  }

  // requests by length, arrival order breaking ties
  std::vector<int32_t> ord(n);
  std::iota(ord.begin(), ord.end(), 0);
  std::stable_sort(ord.begin(), ord.end(), [&](int32_t a, int32_t b) { return lens[a] < lens[b]; });
  std::vector<int64_t> tok(n + 1, 0);
  std::vector<double> pairs(n + 1, 0.0);
  for (int32_t i = 0; i < n; ++i) {
    const int64_t L = lens[ord[i]];
    tok[i + 1] = tok[i] + L;
    pairs[i + 1] = pairs[i] + (double)L * (double)(L + 1) / 2.0;
  }

  // best[i]: least cost of serving the first i requests of the order;
  // from[i]: start of the last batch in that plan
  const double inf = INFINITY;
  std::vector<double> best(n + 1, inf);
  std::vector<int32_t> from(n + 1, -1);
  best[0] = 0.0;
  for (int32_t i = 1; i <= n; ++i) {
    const int64_t P = lens[ord[i - 1]];
    for (int32_t j = std::max(0, i - max_batch); j < i; ++j) {  // longest last batch first
      if (best[j] == inf) continue;
      const int64_t B = i - j;
      const int64_t rows = cost->padded_compute ? B * P : tok[i] - tok[j];
      if (max_tokens > 0 && rows > max_tokens) continue;
      const Run r{B, P, tok[i] - tok[j], pairs[i] - pairs[j]};
      const double c = best[j] + run_cost(*cost, r);
      if (c < best[i]) {
        best[i] = c;
        from[i] = j;
      }
    }
  }
  if (best[n] == inf) return ee::set_error(EE_ERR_INVALID_ARG, "no feasible batch plan");

  struct Batch {
    int32_t lo, hi;     // run [lo, hi) of the length order
    double max_wait;
    int32_t first;      // earliest arrival index
  };
  std::vector<Batch> batches;
  for (int32_t i = n; i > 0; i = from[i]) {
    Batch b{from[i], i, 0.0, n};
    for (int32_t k = b.lo; k < b.hi; ++k) {
      b.max_wait = std::max(b.max_wait, wait ? wait[ord[k]] : 0.0);
      b.first = std::min(b.first, ord[k]);
    }
    batches.push_back(b);
  }
  // priority: longest wait, then more requests, then earliest arrival
  std::sort(batches.begin(), batches.end(), [](const Batch& a, const Batch& b) {
    if (a.max_wait != b.max_wait) return a.max_wait > b.max_wait;
    if (a.hi - a.lo != b.hi - b.lo) return a.hi - a.lo > b.hi - b.lo;
    return a.first < b.first;
  });
  for (size_t q = 0; q < batches.size(); ++q)
    for (int32_t k = batches[q].lo; k < batches[q].hi; ++k) batch_of[ord[k]] = (int32_t)q;
  *n_batches = (int32_t)batches.size();
  if (total_cost) *total_cost = best[n];
  return EE_OK;
}

}  // extern "C"
