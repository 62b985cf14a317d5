// Stream path: rows, decisions and races in one streaming kernel, with a
// small kernel before it (per-request set-up) and one after it (race chunks
// the stream kernel did not get to).  No workgroup waits on another beyond a
// short bounded poll.
//
// Tasks of the stream kernel, one workgroup each, in launch order: the row
// statistics of every (position, request, V-chunk), position-major, with the
// race tasks (queue slot, V-chunk) interleaved one for one after the first P
// positions.
//
// The last chunk of a row to finish runs that position's accept test and
// publishes it in the request's accept / reject bit masks.  Whoever sees a
// first rejection with every earlier position accepted -- or every position
// and the bonus row done -- claims the decision with a compare-and-swap; the
// winner writes a greedy request's output row, or a random request's race
// record, and appends the request to the race queue.  A row task whose
// request is already decided before its position is skipped: the drafts
// behind a rejected one are discarded [第12章 投机解码：以小博大 §12.9;
// vllm v1 源码精读（五） §7], so those rows cannot change the output.  Rows
// started before the decision is known are read speculatively.
//
// Race work is handed out in chunks through a per-request claim counter, and
// three kinds of workgroup claim it:
//   * a row task that finds its request already decided before its position
//     (and the race record written) races a chunk of that request instead of
//     leaving: the skipped rows of early-rejecting requests carry most of the
//     race, overlapped with the row streaming of other requests;
//   * race tasks (queue slot, chunk), interleaved with the rows of the last
//     position, take the requests in the order they were decided, after a
//     short bounded poll of an empty slot;
//   * the tail kernel, launched when every request is decided, claims every
//     chunk still unclaimed (one workgroup per queue slot, looping).
// The last chunk of a request to be raced writes its output row.
#pragma once

#include "common.hpp"
#include "philox.hpp"
#include "race.hpp"
#include "row_pass.hpp"

namespace rsv {

// Per-request state word: undecided, invalid, or decided with n accepted
// drafts (2 + n), plus kStateReady once a random request's race record is
// written.
constexpr int32_t kStateUndecided = 0;
constexpr int32_t kStateInvalid = 1;
constexpr int32_t kStateReady = 64;
constexpr int32_t kQueueSkip = 0x7FFFFFFF;  // queue entry of a request with no race
constexpr int kRaceCtlStride = 32;          // per request: arrivals at [0], claims at [16] (own 64-B lines)
constexpr int32_t kPollLimit = 32;          // polls of an empty queue slot before leaving the chunk

template <typename Elem>
struct StreamArgs {
  const Elem* logits;
  const float* q;
  const int32_t* draft;
  const int32_t* cu;
  const float* temperature;
  uint64_t seed;
  int32_t greedy_all, B, D, max_k, V;
  int32_t nsplit, race_chunks;
  int64_t n_lead, n_rows, n_race, n_tasks;
  RowPartial* partials;
  Gathered* gath;
  ReqRecord* records;
  unsigned long long* cand;
  uint32_t* row_count;        // [R] chunk arrivals per row
  unsigned long long* masks;  // [B][2] accepted / rejected positions
  int32_t* state;             // [B]
  uint32_t* race_ctl;         // [B * kRaceCtlStride] race chunk arrivals and claims
  int32_t* queue;             // [B] b + 1 or kQueueSkip, in decision order
  uint32_t* tail;             // queue length
  int32_t* out;
  int32_t* nacc;
  double* dbg_p;
};

__device__ __forceinline__ void store_record(ReqRecord* dst, const ReqRecord& v) {
  unsigned long long w[sizeof(ReqRecord) / 8];
  __builtin_memcpy(w, &v, sizeof(ReqRecord));
#pragma unroll
  for (int i = 0; i < (int)(sizeof(ReqRecord) / 8); ++i)
    store_coherent(reinterpret_cast<unsigned long long*>(dst) + i, w[i]);
}
__device__ __forceinline__ ReqRecord load_record(const ReqRecord* src) {
  unsigned long long w[sizeof(ReqRecord) / 8];
#pragma unroll
  for (int i = 0; i < (int)(sizeof(ReqRecord) / 8); ++i)
    w[i] = load_coherent(reinterpret_cast<const unsigned long long*>(src) + i);
  ReqRecord r;
  __builtin_memcpy(&r, w, sizeof(ReqRecord));
  return r;
}

template <typename Elem>
__device__ __forceinline__ void enqueue(const StreamArgs<Elem>& a, int32_t v) {
  const uint32_t slot = __hip_atomic_fetch_add(a.tail, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (slot < (uint32_t)a.B) store_coherent32(a.queue + slot, v);
}

// Request b is decided with n accepted drafts (wavefront 0 of the claiming
// workgroup).  shift / S / amax are row j's statistics, reused when n == j.
template <typename Elem>
__device__ __forceinline__ void stream_decide(const StreamArgs<Elem>& a, int32_t b, int32_t n, int32_t j, int32_t s,
                                              int32_t K, bool greedy, float cs, float shift, double S,
                                              int32_t amax) {
  const int lane = threadIdx.x & 63;
  const int64_t row_n = (int64_t)s + b + n;
  if (greedy) {
    const int32_t amax_n = n == j ? amax : merge_greedy<true>(a.partials + row_n * a.nsplit, a.nsplit);
    int32_t* ob = a.out + (int64_t)b * (a.max_k + 1);
    if (lane <= a.max_k) ob[lane] = lane < n ? a.draft[s + lane] : (lane == n ? amax_n : -1);
    if (lane == 0) {
      a.nacc[b] = n;
      if (a.n_race > 0) enqueue(a, kQueueSkip);
    }
    return;
  }
  float sh = shift;
  double Sn = S;
  if (n != j) merge_random<true>(a.partials + row_n * a.nsplit, a.nsplit, sh, Sn);
  if (lane == 0) {
    ReqRecord r;
    r.mode = n < K ? (a.q ? kModeResampleQ : kModeResampleOneHot) : kModeBonus;
    r.phase = 0;
    r.n = n;
    r.row = (int32_t)row_n;
    r.slot0 = s;
    r.exclude = (n < K && !a.q) ? a.draft[s + n] : -1;
    r.c = cs;
    r.shift = sh;
    r.inv_sum = (float)(1.0 / Sn);
    r.tau = -INFINITY;
    r.pad[0] = r.pad[1] = 0;
    store_record(a.records + b, r);
    wait_memory();  // the record is visible before the state or the queue points to it
    store_coherent32(a.state + b, 2 + n + kStateReady);
    enqueue(a, b + 1);
  }
}

// Row j of request b is complete (wavefront 0 of the workgroup whose chunk
// arrived last): accept test of position j, publication, decision.
template <typename Elem>
__device__ __forceinline__ void stream_row_complete(const StreamArgs<Elem>& a, int32_t b, int32_t j, int32_t s,
                                                    int32_t K, float T) {
  const int lane = threadIdx.x & 63;
  const bool greedy = !(T > 0.f);
  const float cs = greedy ? 0.f : scale_of(T);
  const RowPartial* P = a.partials + ((int64_t)s + b + j) * a.nsplit;
  float shift = -INFINITY;
  double S = 0.0;
  int32_t amax = -1;
  bool accept = true;  // the bonus row (j == K) only has to be done
  if (greedy) {
    amax = merge_greedy<true>(P, a.nsplit);
    if (j < K) {
      accept = a.draft[s + j] == amax;
      if (a.dbg_p && lane == 0) a.dbg_p[s + j] = __builtin_nan("");
    }
  } else {
    merge_random<true>(P, a.nsplit, shift, S);
    if (j < K) {
      const Gathered g = load_gathered<true>(a.gath + s + j);
      const double u = accept_uniform(a.seed, b, j);
      const double ps = exp2((double)g.lstar * (double)cs - (double)shift) / S;
      accept = u * (double)g.qstar < ps;
      if (a.dbg_p && lane == 0) a.dbg_p[s + j] = ps;
    }
  }
  unsigned long long acc = 0ull, rej = 0ull;
  if (lane == 0) {
    const unsigned long long bit = 1ull << j;
    unsigned long long* m = a.masks + 2 * (int64_t)b;
    if (accept) {
      acc = atomic_or64(m, bit) | bit;
      rej = load_coherent(m + 1);
    } else {
      rej = atomic_or64(m + 1, bit) | bit;
      acc = load_coherent(m);
    }
  }
  acc = __shfl(acc, 0);
  rej = __shfl(rej, 0);
  // n = the first rejection if every earlier position is accepted, or K if
  // positions 0 .. K (bonus row included) are all done and accepted.  Each
  // publisher reads the other mask after its own update, so whichever update
  // completes the pattern sees all of it.
  const int32_t open = __ffsll((long long)~acc) - 1;
  const int32_t first_rej = rej ? __ffsll((long long)rej) - 1 : 64;
  int32_t n = -1;
  if (rej && open >= first_rej)
    n = first_rej;
  else if (open > K)
    n = K;
  if (n < 0) return;
  int won = 0;
  if (lane == 0) won = atomic_cas32(a.state + b, kStateUndecided, 2 + n);
  if (!__shfl(won, 0)) return;
  stream_decide(a, b, n, j, s, K, greedy, cs, shift, S, amax);
}

// Claim and race one chunk of request b's race (whole workgroup); the last
// chunk raced writes the output row.  Returns false, without work, once every
// chunk is claimed (the same answer in every thread).
template <typename Elem, int TPT>
__device__ __forceinline__ bool stream_race_claim(const StreamArgs<Elem>& a, int32_t b, int32_t* s_word) {
  const int tid = threadIdx.x;
  uint32_t* ctl = a.race_ctl + (int64_t)b * kRaceCtlStride;
  if (tid == 0)
    *s_word = (int32_t)__hip_atomic_fetch_add(ctl + 16, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int32_t c = *s_word;  // every thread reads it before race_chunk's barriers
  if (c >= a.race_chunks) return false;
  const ReqRecord rec = load_record(a.records + b);
  const unsigned long long packed = race_chunk<Elem, TPT, true>(a.logits, a.q, a.V, a.seed, rec, b, c);
  if (tid < 64) {  // wavefront 0 reports the chunk winner
    int last = 0;
    if (tid == 0) {
      store_coherent(a.cand + (int64_t)b * a.race_chunks + c, packed);
      wait_memory();
      last = arrive_last(ctl, (uint32_t)a.race_chunks);
    }
    if (__shfl(last, 0))
      finish_request<Elem>(a.logits, a.draft, a.max_k, a.V, a.race_chunks, a.seed, rec, b, a.cand, a.out, a.nacc);
  }
  return true;
}

// Chunk c of row j of request b, unless the request is invalid, has fewer
// positions or was decided before j -- then, once the race record is written,
// a chunk of its race instead.
template <typename Elem, int NV, int TPT>
__device__ __forceinline__ void stream_row_task(const StreamArgs<Elem>& a, int32_t j, int32_t b, int32_t c,
                                                int32_t* s_word) {
  const int tid = threadIdx.x;
  // Waves issue their loads at raised priority (a wave's arbitration priority
  // among the waves of its SIMD) and do their arithmetic at the default, so
  // the loads of every task go out as early as possible while the arithmetic
  // of others fills the gaps: row tasks here until their loads are issued
  // (chunk_task drops it), race chunks around their loads.  At B=256 K=8
  // V=151936 the call went from 121.3 to 120.2 us with raised row tasks and
  // to ~117 us with the drop after the loads.
  __builtin_amdgcn_s_setprio(1);
  const int32_t s = a.cu[b], e = a.cu[b + 1];
  const float T = a.greedy_all ? 0.f : a.temperature[b];
  // The workgroup agrees on one reading of the request's state.
  if (tid == 0) *s_word = load_coherent32(a.state + b);
  __syncthreads();
  const int32_t st = *s_word;
  __syncthreads();  // s_word is reused below
  if (st == kStateInvalid) {  // the task of chunk 0 of position 0 queues it
    if (j == 0 && c == 0 && tid == 0 && a.n_race > 0) enqueue(a, kQueueSkip);
    return;
  }
  const int32_t K = e - s;  // in range: the init kernel validated the request
  if (j > K) return;
  if (st >= 2 && ((st - 2) & (kStateReady - 1)) < j) {  // decided before position j: row not needed
    __builtin_amdgcn_s_setprio(0);
    if (st >= kStateReady) (void)stream_race_claim<Elem, TPT>(a, b, s_word);
    return;
  }
  const int32_t xstar = (c == 0 && j < K && T > 0.f) ? a.draft[s + j] : -1;
  const int64_t row = (int64_t)s + b + j;
  chunk_task<Elem, NV, true, true>(a.logits, a.q, row, T, a.V, a.nsplit, c, xstar, (int64_t)s + j,
                             a.partials + row * a.nsplit, a.gath);
  if (tid >= 64) return;  // wavefront 0 reports the chunk
  int last = 0;
  if (tid == 0) {
    wait_memory();  // the partial is visible before it is counted
    last = arrive_last(a.row_count + row, (uint32_t)a.nsplit);
  }
  if (__shfl(last, 0)) stream_row_complete(a, b, j, s, K, T);
}

// Race task of queue slot `slot`: the request decided slot-th.  In the stream
// kernel (tail == false) an empty slot is polled briefly and then left to the
// tail kernel, where every slot is filled and the workgroup races chunks of
// its request until none is left to claim.
template <typename Elem, int TPT>
__device__ __forceinline__ void stream_race_task(const StreamArgs<Elem>& a, int32_t slot, bool tail,
                                                 int32_t* s_word) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    int32_t v = load_coherent32(a.queue + slot);
    for (int32_t i = 0; !tail && v == 0 && i < kPollLimit; ++i) {
      __builtin_amdgcn_s_sleep(16);
      v = load_coherent32(a.queue + slot);
    }
    *s_word = v;
  }
  __syncthreads();
  const int32_t v = *s_word;
  __syncthreads();  // s_word is reused below
  if (v == 0 || v == kQueueSkip) return;  // empty (left to the tail kernel) or nothing to race
  if (!tail) {
    (void)stream_race_claim<Elem, TPT>(a, v - 1, s_word);
    return;
  }
  while (stream_race_claim<Elem, TPT>(a, v - 1, s_word)) {
  }
}

// Wavefronts per SIMD: the kernel's time is the sum of its tasks' durations
// over the resident workgroups.  With bf16 logits 5 rather than 4 fit in 96
// VGPRs without spills and took the call from 122 to 117 us at B=256 K=8
// V=151936 (6 spill and are slower); the fp32 race chunk would spill at 5.
template <typename Elem>
constexpr int stream_waves_per_simd() {
  return sizeof(Elem) == 2 ? 5 : 4;
}

template <typename Elem, int NV, int TPT>
__global__ __launch_bounds__(kRowThreads, stream_waves_per_simd<Elem>()) void stream_kernel(StreamArgs<Elem> a) {
  __shared__ int32_t s_word;
  const int64_t t = blockIdx.x;
  int64_t k = t;  // row task index
  if (t >= a.n_lead) {  // rows of later positions interleaved with race tasks
    const int64_t rest = a.n_rows - a.n_lead;
    const int64_t both = rest < a.n_race ? rest : a.n_race;
    const int64_t u = t - a.n_lead;
    bool is_row;
    int64_t i;
    if (u < 2 * both) {
      is_row = (u & 1) == 0;
      i = u >> 1;
    } else {
      i = both + (u - 2 * both);
      is_row = rest > both;
    }
    if (!is_row) {
      stream_race_task<Elem, TPT>(a, (int32_t)(i / a.race_chunks), false, &s_word);
      return;
    }
    k = a.n_lead + i;
  }
  const int64_t per_pos = (int64_t)a.B * a.nsplit;
  stream_row_task<Elem, NV, TPT>(a, (int32_t)(k / per_pos), (int32_t)((k / a.nsplit) % a.B),
                                 (int32_t)(k % a.nsplit), &s_word);
}

// Every race chunk still unclaimed after the stream kernel: one workgroup per
// queue slot races the chunks of its request that nobody claimed yet.
template <typename Elem, int TPT>
__global__ __launch_bounds__(kRaceThreads) void stream_race_tail_kernel(StreamArgs<Elem> a) {
  __shared__ int32_t s_word;
  stream_race_task<Elem, TPT>(a, (int32_t)blockIdx.x, true, &s_word);
}

// One wavefront per request: validity, counters, masks, state; -1 row for an
// invalid request; clears race slot b.  Block 0 also empties the race queue.
__global__ __launch_bounds__(64) void stream_init_kernel(const int32_t* __restrict__ draft,
                                                         const int32_t* __restrict__ cu, int32_t B, int32_t D,
                                                         int32_t max_k, int32_t V, uint32_t* __restrict__ row_count,
                                                         unsigned long long* __restrict__ masks,
                                                         int32_t* __restrict__ state, uint32_t* __restrict__ race_ctl,
                                                         int32_t* __restrict__ queue, uint32_t* __restrict__ tail,
                                                         int32_t* __restrict__ out, int32_t* __restrict__ nacc) {
  const int32_t b = blockIdx.x;
  const int lane = threadIdx.x;
  if (b == 0 && lane == 0) *tail = 0u;
  if (lane == 0) queue[b] = 0;
  if (lane < kRaceCtlStride) race_ctl[(int64_t)b * kRaceCtlStride + lane] = 0u;
  if (lane < 2) masks[2 * (int64_t)b + lane] = 0ull;
  const int32_t s = cu[b], e = cu[b + 1];
  bool valid = request_valid(s, e, D, max_k);
  const int32_t K = valid ? e - s : 0;
  int32_t x = 0;
  if (valid && lane < K) x = draft[s + lane];
  valid = valid && __ballot(lane < K && (x < 0 || x >= V)) == 0ull;
  if (valid && lane <= K) row_count[(int64_t)s + b + lane] = 0u;
  if (lane == 0) state[b] = valid ? kStateUndecided : kStateInvalid;
  if (!valid) {
    if (lane <= max_k) out[(int64_t)b * (max_k + 1) + lane] = -1;
    if (lane == 0) nacc[b] = -1;
  }
}

}  // namespace rsv
