// Accept tests and first-rejection scan of one request over one phase of its
// draft positions, by one wavefront (lane i = position j_begin + i).
//
//  - p(x*) = exp2(l(x*) c - shift) / sum in fp64 from the merged row partials;
//    accept iff u_j q(x*) < p(x*), u_j the Philox accept uniform, q(x*) = 1
//    without draft probabilities [第12章 投机解码：以小博大 §12.2.1, §12.2.3;
//    投机解码（Speculative Decoding）端到端深挖 §7.3 (coin * q < p)].
//  - greedy requests accept iff x* == argmax [§12.2.4; 端到端深挖 §7.1].
//  - the first rejected position n ends the request: later drafts are
//    discarded [§12.9; vllm v1 源码精读（五） §7]; a ballot finds it.
//  - a request with top-k / top-p takes shift, sum and the threshold tau of
//    each row from the filter's record: p'(x*) = 0 when l(x*) < tau
//    [§12.2.3; §12.9 (compute_probs)].  COH_FREC: the records were written by
//    other workgroups of the same kernel (the fused filter + scan kernel) and
//    are read with agent-coherent loads.
//  - if no position of the phase rejects and the bonus row K lies in it,
//    n = K (bonus) [§12.3.2]; otherwise the request stays active for the
//    next phase.
// Greedy requests get their output row here; random ones get a record for
// the race.  Requests whose metadata is out of range get a -1 row.
#pragma once

#include "common.hpp"
#include "filter.hpp"
#include "philox.hpp"
#include "row_pass.hpp"

namespace rsv {

template <typename Elem, bool COH_FREC = false>
__device__ __forceinline__ void scan_phase(
    int32_t b, const float* __restrict__ q, const int32_t* __restrict__ draft, const int32_t* __restrict__ cu,
    const float* __restrict__ temperature, int32_t greedy_all, int32_t D, int32_t max_k, int32_t V, int32_t nsplit,
    uint64_t seed, const RowPartial* __restrict__ partials, const Gathered* __restrict__ gath, int32_t j_begin,
    int32_t j_end, int32_t phase, ReqRecord* __restrict__ records, int32_t* __restrict__ out,
    int32_t* __restrict__ num_accepted, double* __restrict__ dbg_p, const int32_t* __restrict__ top_k,
    const float* __restrict__ top_p, const FilterRec* __restrict__ frec) {
  const int lane = threadIdx.x & 63;
  // Loads are grouped by what their addresses depend on (b, then cu[b]) so
  // each group's latencies overlap.
  const int32_t s = cu[b], e = cu[b + 1];
  const float T = greedy_all ? 0.f : temperature[b];
  if (j_begin > 0 && records[b].mode != kModeActive) return;  // decided in an earlier phase
  int32_t* ob = out + (int64_t)b * (max_k + 1);
  if (j_begin == 0 && !request_valid(s, e, D, max_k)) {
    if (lane <= max_k) ob[lane] = -1;
    if (lane == 0) {
      num_accepted[b] = -1;
      records[b].mode = kModeDone;
    }
    return;
  }
  const int32_t K = e - s;
  const bool greedy = !(T > 0.f);
  const float cs = greedy ? 0.f : scale_of(T);
  const int32_t j = j_begin + lane;
  const bool in_phase = j < j_end && j <= K;
  // Phase 1 reads every draft id (lane = position) to validate the request.
  const int32_t x = (j < K && (in_phase || j_begin == 0)) ? draft[s + j] : -1;
  const bool filt = !greedy && filter_on(top_k, top_p, b, V);
  float shift = -INFINITY, tau = -INFINITY;
  double S = 0.0;
  int32_t amax = -1;
  double ps = __builtin_nan("");
  bool accept = false;
  if (in_phase) {
    const int64_t row = (int64_t)s + b + j;
    const RowPartial* P = partials + row * nsplit;
    if (greedy) {
      amax = merge_greedy(P, nsplit);
      accept = (j < K) && (x == amax);
    } else {
      const double u = j < K ? accept_uniform(seed, b, j) : 0.0;
      const Gathered g = j < K ? gath[s + j] : Gathered{0.f, 0.f};
      if (filt) {  // p' from the row's filter record; p'(x*) = 0 below the threshold
        const FilterRec f = load_frec<COH_FREC>(frec + row);
        shift = f.shift;
        S = f.sum;
        tau = f.tau;
      } else {
        merge_random(P, nsplit, shift, S);
      }
      if (j < K) {
        ps = g.lstar >= tau ? exp2((double)g.lstar * (double)cs - (double)shift) / S : 0.0;
        accept = u * (double)g.qstar < ps;
      }
    }
  }
  if (j_begin == 0 && __ballot(j < K && (x < 0 || x >= V))) {  // a draft id out of range
    if (lane <= max_k) ob[lane] = -1;
    if (lane == 0) {
      num_accepted[b] = -1;
      records[b].mode = kModeDone;
    }
    return;
  }
  if (dbg_p && in_phase && j < K) dbg_p[s + j] = ps;
  const unsigned long long rej = __ballot(in_phase && j < K && !accept);
  int32_t n;
  if (rej) {
    n = j_begin + (__ffsll((long long)rej) - 1);
  } else if (K < j_end) {
    n = K;
  } else {
    if (lane == 0) records[b].mode = kModeActive;
    return;
  }
  const int src = n - j_begin;
  const float shift_n = __shfl(shift, src);
  const float tau_n = __shfl(tau, src);
  const double S_n = __shfl(S, src);
  const int32_t amax_n = __shfl(amax, src);
  const int32_t x_n = __shfl(x, src);

  if (greedy) {
    if (lane <= max_k) ob[lane] = lane < n ? draft[s + lane] : (lane == n ? amax_n : -1);
    if (lane == 0) {
      num_accepted[b] = n;
      records[b].mode = kModeDone;
    }
    return;
  }
  if (lane == 0) {
    ReqRecord r;
    r.mode = n < K ? (q ? kModeResampleQ : kModeResampleOneHot) : kModeBonus;
    r.phase = phase;
    r.n = n;
    r.row = s + b + n;
    r.slot0 = s;
    r.exclude = (n < K && !q) ? x_n : -1;
    r.c = cs;
    r.shift = shift_n;
    r.inv_sum = (float)(1.0 / S_n);
    r.tau = tau_n;
    r.pad[0] = r.pad[1] = 0;
    records[b] = r;
  }
}

}  // namespace rsv
