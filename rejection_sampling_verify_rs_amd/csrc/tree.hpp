// Tree verify: the walk over a request's draft tree, spread over the GPU.
//
// The drafts of a request form a tree -- each node one draft token, its parent
// earlier in the node order or -1 for a child of the last prefix position --
// and the target scored the prefix position (row 0) and every node (row
// 1 + i), row r predicting the children of its node [投机解码深度实战 §四: one
// target forward over the whole tree].  The walk goes one depth at a time
// from the root: it takes the current node's row statistics, looks for an
// accepted child among the current layer's siblings, descends into it, and
// stops at the first depth where none is accepted; one extra token then
// comes from the stop node's row [投机解码（Speculative Decoding）端到端深挖 §6.2].
//   greedy (T <= 0): the child whose token is the row's argmax (the first
//     such child; lowest index on argmax ties) [§7.1]; else the argmax is
//     emitted.
//   random: p = softmax(row / T); one coin u_d per depth (the accept uniform
//     of position d); children in node order, a repeated sibling token
//     skipped; child i is accepted iff u_d < the sum of p over the siblings
//     up to and including i [§7.2: one coin against the accumulated target
//     probabilities, both thresholds at their default 1]; if none, the extra
//     token is the exponential race over p without the children's tokens
//     (exponentials of depth d); a childless stop node races over p.
// Each sibling is thus accepted with probability p(its token) and the
// residual is p without the siblings, so every emitted token follows p; a
// one-child-per-node tree is the chain with one-hot q and uses the same
// random numbers.
//
// Layout of the work: one launch (tree_walk_kernel, after tree_init_kernel)
// of K workgroups per request.  Each request has
// a list of entries that its workgroups work through in order:
//   a row entry (node x, step d): stream the row of x (the root: -1) in
//     chunks of 8 vectors per thread into that row's partial statistics;
//   a race entry (stop node, step d): race the stop row in 10240-token chunks
//     (p without the stop node's children, or max(0, p - q) with the stop
//     node's draft row q);
//   an exit entry: the request is finished;
//   a no-op entry (a decided step's slot that holds nothing else).
// A workgroup claims chunks of the entry it is at from that entry's counter
// (the first claim is made while the entry may still be unwritten), so a row
// is streamed by many workgroups at once and a workgroup that is deciding
// holds no chunk back.  The init kernel writes the
// first entries: the root row and the rows of the first kTreeSpec children of
// the root.  Step d's decider writes the next ones: when it accepts node x,
// the row of x if it was not streamed ahead and the rows of the first
// kTreeSpec children of x (needed one step later); when a random walk stops,
// the race entry; when the request is finished, the exit entry.
// A row's counter word holds its arrived chunks and a "chosen" bit that the
// decider sets when it reaches the row's node.  Both sides update the word
// with one atomic; the one whose update completes the pair (all chunks in and
// chosen) decides the row's step, so exactly one does.  A decider that finds
// the next row already complete goes on deciding, step after step.
// Only a request's own workgroups touch its state, and no global counter is
// updated.  A row entry the walk can no longer need (the walk stopped, or
// reached another node at that step; the walk word only moves forward) is
// skipped.  A workgroup waits only for its request's next entry, by a bounded
// poll; a request that never finishes (not expected) keeps num_accepted = -1.
#pragma once

#include "common.hpp"
#include "philox.hpp"
#include "race.hpp"
#include "row_pass.hpp"

namespace rsv {

constexpr int kTreeMaxNodes = 64;               // one wavefront lane per node
constexpr int kTreeRows = kTreeMaxNodes + 1;    // the root row and one per node
// every row at most once, up to kTreeSpec slots per decided step (a no-op
// when it holds nothing else), the race and the exit
constexpr int kTreeEntries = 2 * kTreeRows + 2;
constexpr int kTreeRaceTPT = 40;                // tokens per thread of a race chunk (10240 per chunk)
constexpr int kTreeNV = 8;                      // 16-byte vectors per thread of a row chunk
// bf16 rows when a request has at most kTreeWideK workgroups (B >= ~86 on a
// 256-CU device): fewer, larger chunks per row, so a row takes fewer rounds of
// claims on those workgroups (B=128: 86 -> 81 us, B=256: 151 -> 139 us; B=48:
// 55 against 58 us with the smaller chunks)
constexpr int kTreeNVWide = 12;
constexpr int32_t kTreeWideK = 12;
constexpr int kTreeSpec = 1;                    // children rows streamed before their parent is reached
constexpr int32_t kTreeMaxK = 64;               // workgroups per request, at most
constexpr int32_t kTreePollLimit = 1 << 18;     // polls before a workgroup stops waiting for an entry
constexpr uint32_t kChosen = 0x80000000u;       // row counter: the row's node was reached
// Per-request mailbox of 2 KiB, the words a request's workgroups poll and
// update: the walk word (byte 0), the entry tail (byte 8), the entries (from
// byte 128) and the entries' chunk claims (from byte 1024).  Each request's
// words sit on lines of their own, away from other requests'.
constexpr int kMailboxWords = 512;   // 8-byte words per mailbox
constexpr int kMailboxEntries = 16;  // first entry word
constexpr int kMailboxClaims = kMailboxEntries + kTreeEntries;  // first word of the 32-bit claim counters
static_assert(kMailboxEntries + kTreeEntries <= kMailboxClaims, "entries fit the mailbox");
static_assert(kMailboxClaims + (kTreeEntries + 1) / 2 <= kMailboxWords, "claims fit the mailbox");

// Walk word of a request: step (bits 0-7), node + 1 (bits 8-15), status
// (bits 16-23).  Walking: step `step` decides among the children of `node`.
// Stopped: the walk ended at `step` on `node`, whose row is being raced.
// Done: the output row is written.  Invalid: -1 row written by the init kernel.
constexpr uint32_t kWalking = 1, kStopped = 2, kWalkDone = 3, kWalkInvalid = 4;
__device__ __forceinline__ unsigned long long walk_word(uint32_t step, int32_t node, uint32_t status) {
  return (unsigned long long)step | ((unsigned long long)(uint32_t)(node + 1) << 8) | ((unsigned long long)status << 16);
}
__device__ __forceinline__ uint32_t walk_step(unsigned long long w) { return (uint32_t)(w & 0xFF); }
__device__ __forceinline__ int32_t walk_node(unsigned long long w) { return (int32_t)((w >> 8) & 0xFF) - 1; }
__device__ __forceinline__ uint32_t walk_status(unsigned long long w) { return (uint32_t)((w >> 16) & 0xFF); }

// Entry word: node + 1 (bits 0-7), step (8-15), chunks (16-39), kind
// (40-41), bit 63 set (a zero word is an entry not yet written).
constexpr uint32_t kEntryRow = 0, kEntryRace = 1, kEntryExit = 2, kEntryNone = 3;
__device__ __forceinline__ unsigned long long entry_word(uint32_t kind, int32_t node, int32_t d, int32_t chunks) {
  return (1ull << 63) | ((unsigned long long)kind << 40) | ((unsigned long long)(uint32_t)chunks << 16) |
         ((unsigned long long)(uint32_t)d << 8) | (uint32_t)(node + 1);
}
__device__ __forceinline__ int32_t entry_node(unsigned long long e) { return (int32_t)(e & 0xFF) - 1; }
__device__ __forceinline__ int32_t entry_step(unsigned long long e) { return (int32_t)((e >> 8) & 0xFF); }
__device__ __forceinline__ int32_t entry_chunks(unsigned long long e) { return (int32_t)((e >> 16) & 0xFFFFFF); }
__device__ __forceinline__ uint32_t entry_kind(unsigned long long e) { return (uint32_t)((e >> 40) & 3u); }

template <typename Args>
__device__ __forceinline__ unsigned long long* walk_of(const Args& a, int32_t b) {
  return a.mail + (int64_t)b * kMailboxWords;
}
template <typename Args>
__device__ __forceinline__ uint32_t* tail_of(const Args& a, int32_t b) {
  return reinterpret_cast<uint32_t*>(a.mail + (int64_t)b * kMailboxWords + 1);
}
template <typename Args>
__device__ __forceinline__ unsigned long long* entries_of(const Args& a, int32_t b) {
  return a.mail + (int64_t)b * kMailboxWords + kMailboxEntries;
}
template <typename Args>
__device__ __forceinline__ uint32_t* claims_of(const Args& a, int32_t b) {
  return reinterpret_cast<uint32_t*>(a.mail + (int64_t)b * kMailboxWords + kMailboxClaims);
}

// Lane k's value to every lane (k wavefront-uniform).
__device__ __forceinline__ int32_t lane_i32(int32_t v, int32_t k) { return __builtin_amdgcn_readlane(v, k); }
__device__ __forceinline__ double lane_f64(double v, int32_t k) {
  const unsigned long long x = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int32_t)(uint32_t)x, k);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int32_t)(uint32_t)(x >> 32), k);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Index of the i-th set bit of m (-1: fewer than i + 1 bits).
__device__ __forceinline__ int32_t nth_bit(unsigned long long m, int32_t i) {
  for (int32_t k = 0; k < i && m; ++k) m &= m - 1ull;
  return m ? __ffsll((long long)m) - 1 : -1;
}

template <typename Elem>
struct TreeArgs {
  const Elem* logits;
  const float* q;  // draft distributions, one row per tree position (NULL: none)
  const int32_t* tokens;
  const int32_t* parents;
  const int32_t* cu;
  const float* temperature;
  uint64_t seed;
  int32_t B, N, max_nodes, max_depth, V;
  int32_t nsplit;        // row chunks per row
  int32_t race_chunks;   // race chunks per row
  int32_t K;             // workgroups per request
  int32_t* out;          // [B, max_depth + 1]
  int32_t* path;         // [B, max_depth]
  int32_t* nacc;         // [B]
  unsigned long long* mail;     // [B * kMailboxWords] walk word, entry tail, entries
  uint32_t* count;              // [B * kTreeRows] arrived chunks | kChosen, per row
  uint32_t* race_count;         // [B] arrived race chunks
  RowPartial* partials;         // [B * kTreeRows * nsplit]
  unsigned long long* cand;     // [B * race_chunks] packed race winners
};

// One workgroup per request: validates the tree (sizes, parents before
// children, tokens in range, every node shallower than max_depth), fills the
// request's output rows with -1 (a valid walk overwrites them as it goes),
// clears its counters and writes its first entries: the root row and the
// rows of the root's first children, with the root row chosen; an invalid
// request gets only the exit entry.
template <typename Elem>
__global__ __launch_bounds__(kRowThreads) void tree_init_kernel(TreeArgs<Elem> a) {
  __shared__ int s_ok;
  __shared__ unsigned long long s_kids;
  const int32_t b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 64) {
    const int32_t s = a.cu[b], e = a.cu[b + 1];
    const int32_t n = e - s;
    bool ok = s >= 0 && s <= e && e <= a.N && n <= a.max_nodes;
    int32_t tk = 0, pr = -1;
    if (ok && lane < n) {
      tk = a.tokens[s + lane];
      pr = a.parents[s + lane];
    }
    ok = ok && __ballot(lane < n && (pr < -1 || pr >= lane || tk < 0 || tk >= a.V)) == 0ull;
    int32_t dep = 0;  // depth of node lane: a parent's depth is final after (its depth + 1) rounds
    for (int32_t r = 0; ok && r < n; ++r) {
      const int32_t dp = __shfl(dep, pr < 0 ? lane : pr);
      dep = pr < 0 ? 0 : dp + 1;
    }
    ok = ok && __ballot(lane < n && dep >= a.max_depth) == 0ull;
    const unsigned long long kids = __ballot(ok && lane < n && pr == -1);
    if (tid == 0) {
      s_ok = ok;
      s_kids = kids;
    }
  }
  __syncthreads();
  const bool ok = s_ok;
  const unsigned long long kids = s_kids;
  const int32_t nspec = ok ? min(__popcll(kids), kTreeSpec) : 0;
  unsigned long long* E = entries_of(a, b);
  for (int32_t i = tid; i < kTreeEntries; i += kRowThreads) {
    unsigned long long w = 0ull;
    if (!ok)
      w = i == 0 ? entry_word(kEntryExit, -1, 0, 0) : 0ull;
    else if (i == 0)
      w = entry_word(kEntryRow, -1, 0, a.nsplit);
    else if (i <= nspec)
      w = entry_word(kEntryRow, nth_bit(kids, i - 1), 1, a.nsplit);
    E[i] = w;
  }
  for (int32_t i = tid; i < kTreeRows; i += kRowThreads)
    a.count[(int64_t)b * kTreeRows + i] = (i == 0 && ok) ? kChosen : 0u;
  for (int32_t i = tid; i < kTreeEntries; i += kRowThreads) claims_of(a, b)[i] = 0u;
  for (int32_t i = tid; i <= a.max_depth; i += kRowThreads) a.out[(int64_t)b * (a.max_depth + 1) + i] = -1;
  for (int32_t i = tid; i < a.max_depth; i += kRowThreads) a.path[(int64_t)b * a.max_depth + i] = -1;
  if (tid == 0) {
    a.nacc[b] = -1;
    a.race_count[b] = 0u;
    *tail_of(a, b) = ok ? (uint32_t)(1 + nspec) : 1u;
    *walk_of(a, b) = ok ? walk_word(0, -1, kWalking) : walk_word(0, -1, kWalkInvalid);
  }
}

// Rank of node x among the children of its parent (lanes hold the nodes'
// parents).
__device__ __forceinline__ int32_t child_rank(int32_t par, int32_t n, int32_t x) {
  const int lane = threadIdx.x & 63;
  const int32_t px = lane_i32(par, x);
  const unsigned long long sib = __ballot(lane < n && par == px);
  return __popcll(sib & ((1ull << x) - 1ull));
}

__device__ __forceinline__ RowPartial* tree_partials(RowPartial* p, int32_t b, int32_t x, int32_t nsplit) {
  return p + ((int64_t)b * kTreeRows + x + 1) * nsplit;
}

// A row's statistics from its chunk partials, one wavefront: random rows
// get the common shift (largest chunk shift) and the fp64 sum rescaled to it,
// summed in chunk order; greedy rows the largest value, lowest index on ties.
// The chunks' partials are loaded across lanes and folded through lane reads
// (a short scalar loop, no shuffle chain).  The decider and the race chunks
// call it on the same partials and so get the same numbers.
__device__ __forceinline__ void tree_merge(const RowPartial* P, int32_t nsplit, bool greedy, float& shift,
                                           double& S, int32_t& amax) {
  const int lane = threadIdx.x & 63;
  float sh = -INFINITY;
  double acc = 0.0;
  float m = -INFINITY;
  int32_t idx = INT_MAX;
  for (int32_t c0 = 0; c0 < nsplit; c0 += 64) {
    const int32_t nc = min(64, nsplit - c0);
    RowPartial r;
    r.shift = -INFINITY;
    r.argmax = -1;
    r.sum = 0.0;
    if (lane < nc) r = load_partial<true>(P + c0 + lane);
    if (greedy) {
      for (int32_t c = 0; c < nc; ++c) {
        const int32_t ac = lane_i32(r.argmax, c);
        const float mc = __int_as_float(lane_i32(__float_as_int(r.shift), c));
        if (ac >= 0 && (mc > m || (mc == m && ac < idx))) {
          m = mc;
          idx = ac;
        }
      }
      continue;
    }
    float shc = -INFINITY;  // this batch's shift, then the running one
    for (int32_t c = 0; c < nc; ++c) shc = fmaxf(shc, __int_as_float(lane_i32(__float_as_int(r.shift), c)));
    if (shc > sh) {  // rescale what was summed so far
      if (acc > 0.0) acc *= exp2((double)sh - (double)shc);
      sh = shc;
    }
    const double t = r.sum > 0.0 ? r.sum * exp2((double)r.shift - (double)sh) : 0.0;
    for (int32_t c = 0; c < nc; ++c) acc += lane_f64(t, c);
  }
  if (greedy) {
    amax = idx == INT_MAX ? -1 : idx;
    return;
  }
  shift = sh;
  S = acc;
}

// Appends one entry to request b's list (one wavefront, lane 0).
template <typename Elem>
__device__ __forceinline__ void tree_append(const TreeArgs<Elem>& a, int32_t b, unsigned long long e) {
  if ((threadIdx.x & 63) != 0) return;
  const uint32_t r = __hip_atomic_fetch_add(tail_of(a, b), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (r < (uint32_t)kTreeEntries) store_coherent(entries_of(a, b) + r, e);
}

// Marks request b finished (one wavefront; its output row is written).
template <typename Elem>
__device__ __forceinline__ void tree_finish(const TreeArgs<Elem>& a, int32_t b, int32_t d, int32_t cur) {
  if ((threadIdx.x & 63) == 0) store_coherent(walk_of(a, b), walk_word((uint32_t)d, cur, kWalkDone));
  tree_append(a, b, entry_word(kEntryExit, -1, 0, 0));
}

// Decisions of request b from step d on (wavefront 0 of the workgroup that
// completed the pair for step d): merge the row's partials, choose the child
// or stop, write the step's output and the entries that come next; while the
// next row is already complete, decide it too.  Each step reserves
// kTreeSpec entry slots with one atomic issued together with the row's loads:
// they take the race or the exit when the walk stops, the rows of the chosen
// node's first children (streamed one step ahead) when its own row was
// streamed ahead, else its own row (the children's rows then take further
// slots); a slot left over holds a no-op.  The chosen node's row counter is
// read with those loads too: a row that is already complete needs no
// handshake, since its last chunk has arrived without finding the chosen bit.
template <typename Elem>
__device__ __forceinline__ void tree_decide(const TreeArgs<Elem>& a, int32_t b, int32_t d, int32_t cur, int32_t s,
                                            int32_t n, float T, int32_t tok, int32_t par) {
  static_assert(kTreeSpec >= 1, "a step's slots hold at least the race or the exit");
  const int lane = threadIdx.x & 63;
  const bool greedy = !(T > 0.f);
  const float cs = greedy ? 0.f : scale_of(T);
  int32_t* ob = a.out + (int64_t)b * (a.max_depth + 1);
  int32_t* pb = a.path + (int64_t)b * a.max_depth;
  unsigned long long* E = entries_of(a, b);
  uint32_t* rc = a.count + (int64_t)b * kTreeRows + 1;  // row counter of node x: rc[x]
  // The decisions are the request's critical path: the deciding wave gets
  // issue priority over chunk waves on its SIMD (kept for the rest of the
  // workgroup's work; ~0.7 us per call for B=64 EAGLE trees).
  __builtin_amdgcn_s_setprio(2);
  for (;;) {
    const int64_t row = (int64_t)s + b + 1 + cur;
    const Elem* prow = a.logits + row * (int64_t)a.V;
    const bool child = lane < n && par == cur;
    // the children's logits and row counters, the partials and the slots are requested together
    const float lt = (!greedy && child) ? to_f32(prow[tok]) : -INFINITY;
    const uint32_t early = child ? __hip_atomic_load(rc + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    uint32_t base = 0u;
    if (lane == 0)
      base = __hip_atomic_fetch_add(tail_of(a, b), (uint32_t)kTreeSpec, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float shift = -INFINITY;
    double S = 0.0;
    int32_t amax = -1, next = -1;
    tree_merge(tree_partials(a.partials, b, cur, a.nsplit), a.nsplit, greedy, shift, S, amax);
    if (greedy) {
      const unsigned long long m = __ballot(child && tok == amax);
      next = m ? __ffsll((long long)m) - 1 : -1;
    } else {
      const unsigned long long kids = __ballot(child);
      bool dup = false;  // a repeat of an earlier sibling's token
      for (unsigned long long m = kids; m; m &= m - 1ull) {
        const int32_t k = __ffsll((long long)m) - 1;
        dup = dup || (k < lane && lane_i32(tok, k) == tok);
      }
      const unsigned long long take = __ballot(child && !dup);
      const double pk = exp2((double)lt * (double)cs - (double)shift) / S;
      // the siblings in node order, each adding its p to the accumulated sum
      const double u = accept_uniform(a.seed, b, d);
      double cum = 0.0;
      for (unsigned long long m = take; m; m &= m - 1ull) {
        const int32_t k = __ffsll((long long)m) - 1;
        cum += lane_f64(pk, k);
        if (u < cum) {
          next = k;
          break;
        }
      }
    }
    base = (uint32_t)lane_i32((int32_t)base, 0);
    if (next < 0) {  // stop at step d
      if (lane == 0) {
        if (greedy) {
          ob[d] = amax;
          a.nacc[b] = d;
          store_coherent(walk_of(a, b), walk_word((uint32_t)d, cur, kWalkDone));
        } else {  // the extra token: the race over p without the stop node's children
          store_coherent(walk_of(a, b), walk_word((uint32_t)d, cur, kStopped));
        }
      }
      if (lane < kTreeSpec && base + lane < (uint32_t)kTreeEntries)
        store_coherent(E + base + lane, lane > 0  ? entry_word(kEntryNone, -1, d, 0)
                                        : greedy ? entry_word(kEntryExit, -1, 0, 0)
                                                 : entry_word(kEntryRace, cur, d, a.race_chunks));
      return;
    }
    // descend: the accepted node is emitted, and step d + 1 decides among its children
    const int32_t ntok = lane_i32(tok, next);
    const bool own = child_rank(par, n, next) >= kTreeSpec;  // next's row was not streamed ahead
    const unsigned long long nkids = __ballot(lane < n && par == next);
    const int32_t nspec = min(__popcll(nkids), kTreeSpec);  // next's first children, streamed one step ahead
    if (lane == 0) {
      ob[d] = ntok;
      pb[d] = next;
      store_coherent(walk_of(a, b), walk_word((uint32_t)d + 1, next, kWalking));
    }
    // the reserved slots: next's row (if not streamed ahead), then its first children's rows, no-ops after
    const int32_t nent = (own ? 1 : 0) + nspec;
    if (lane < kTreeSpec && base + lane < (uint32_t)kTreeEntries) {
      const int32_t x = lane < nent ? (own && lane == 0 ? next : nth_bit(nkids, lane - (own ? 1 : 0))) : -1;
      store_coherent(E + base + lane, x < 0 ? entry_word(kEntryNone, -1, d, 0)
                                            : entry_word(kEntryRow, x, x == next ? d + 1 : d + 2, a.nsplit));
    }
    if (nent > kTreeSpec) {  // the rest (next's own row took a slot)
      uint32_t b2 = 0u;
      if (lane == 0)
        b2 = __hip_atomic_fetch_add(tail_of(a, b), (uint32_t)(nent - kTreeSpec), __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
      b2 = (uint32_t)lane_i32((int32_t)b2, 0);
      if (lane >= kTreeSpec && lane < nent && b2 + (lane - kTreeSpec) < (uint32_t)kTreeEntries)
        store_coherent(E + b2 + (lane - kTreeSpec), entry_word(kEntryRow, nth_bit(nkids, lane - 1), d + 2, a.nsplit));
    }
    const bool complete = !own && (uint32_t)lane_i32((int32_t)early, next) == (uint32_t)a.nsplit;
    if (!complete) {  // next is reached: its row's last chunk, or this decider, decides step d + 1
      uint32_t old = 0u;
      if (lane == 0)
        old = __hip_atomic_fetch_or(rc + next, kChosen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      old = (uint32_t)lane_i32((int32_t)old, 0);
      if (old != (uint32_t)a.nsplit) return;  // the row is still streaming
    }
    ++d;
    cur = next;
  }
}

// Row chunk c of the row of node x (root: -1), decided at step d.
template <typename Elem, int NV>
__device__ __forceinline__ void tree_row_chunk(const TreeArgs<Elem>& a, int32_t b, int32_t d, int32_t x, int32_t c,
                                               int32_t s, int32_t n, float T, int32_t tok, int32_t par,
                                               uint32_t* claim, uint32_t* s_c) {
  const int tid = threadIdx.x;
  chunk_task<Elem, NV, true>(a.logits, nullptr, (int64_t)s + b + 1 + x, T, a.V, a.nsplit, c, -1, 0,
                             tree_partials(a.partials, b, x, a.nsplit), nullptr);
  if (tid >= 64) return;
  int go = 0;
  if (tid == 0) {
    wait_memory();  // the partial is visible before it is counted
    const uint32_t old = __hip_atomic_fetch_add(a.count + (int64_t)b * kTreeRows + x + 1, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    *s_c = __hip_atomic_fetch_add(claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    go = old == (kChosen | (uint32_t)(a.nsplit - 1));
  }
  if (lane_i32(go, 0)) tree_decide(a, b, d, x, s, n, T, tok, par);
}

// Race chunk rc (kRaceThreads * kTreeRaceTPT tokens) of request b's stop row
// (node cur, step d), the stop node's children (those with a token in the
// chunk) marked in an LDS bitmap and given weight 0 -- or, with draft
// distributions, every token weighted max(0, p - q) with the stop node's
// draft row.  The row's statistics are merged at a workgroup's first chunk of
// the entry (`merged`) and kept.  The last chunk to arrive writes the extra
// token; if no token had weight it races over p instead.
template <typename Elem>
__device__ __forceinline__ void tree_race_chunk(const TreeArgs<Elem>& a, int32_t b, int32_t d, int32_t cur,
                                                int32_t rc, int32_t s, int32_t n, float T, int32_t tok, int32_t par,
                                                bool& merged, float& shift, float& inv_sum, uint32_t* claim,
                                                uint32_t* s_c) {
  constexpr int NG = kTreeRaceTPT / 4;  // groups of four tokens per thread
  constexpr int kChunk = kRaceThreads * kTreeRaceTPT;
  using R4 = Raw4<Elem>;
  __shared__ uint32_t bits[kChunk / 32];
  __shared__ unsigned long long lds_u[kRaceThreads / 64];
  __shared__ int s_kids;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t row = (int64_t)s + b + 1 + cur;
  const float cs = scale_of(T);
  const Elem* lrow = a.logits + row * a.V;
  bool kids = false;
  if (a.q) {  // only a node whose children were turned down races max(0, p - q); a childless one races p
    if (tid < 64) {  // wavefront 0 holds the nodes
      const bool k = __ballot(lane < n && par == cur) != 0ull;
      if (lane == 0) s_kids = k;
    }
    __syncthreads();
    kids = s_kids != 0;
  }
  const float* qrow = kids ? a.q + row * a.V : nullptr;  // the stop node's draft row
  const bool fast = ((uintptr_t)lrow % sizeof(typename R4::T)) == 0 && ((uintptr_t)qrow % 16) == 0;
  const int32_t Gend = (a.V + 3) / 4, Gfull = fast ? a.V / 4 : 0;
  const int32_t G0 = rc * (kRaceThreads * NG);
  typename R4::T lw[NG];
  if (Gfull > 0) {  // unconditional loads (index clamped into the vector part): all in flight together
#pragma unroll
    for (int i = 0; i < NG; ++i)
      lw[i] = reinterpret_cast<const typename R4::T*>(lrow)[min(G0 + tid + i * kRaceThreads, Gfull - 1)];
  }
  if (!merged) {  // while the chunk's loads are in flight
    double S = 0.0;
    int32_t amax = -1;
    tree_merge(tree_partials(a.partials, b, cur, a.nsplit), a.nsplit, false, shift, S, amax);
    inv_sum = (float)(1.0 / S);
    merged = true;
  }
  const int32_t x0 = rc * kChunk;
  if (!qrow) {  // the stop node's children leave the race (LDS bitmap of the chunk)
    for (int i = tid; i < kChunk / 32; i += kRaceThreads) bits[i] = 0u;
    __syncthreads();
    if (tid < 64 && lane < n && par == cur) {  // wavefront 0 holds the nodes
      const int32_t x = tok - x0;
      if (x >= 0 && x < kChunk) atomicOr(bits + (x >> 5), 1u << (x & 31));
    }
    __syncthreads();
  }
  const uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32);
  float best_key = 0.f;
  int32_t best_x = INT_MAX;
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int32_t G = G0 + tid + i * kRaceThreads;
    if (G >= Gend) continue;
    float l[4], qv[4] = {0.f, 0.f, 0.f, 0.f};
    if (G < Gfull) {
      R4::unpack(lw[i], l);
      if (qrow) {
        const float4 q4 = stream_load(reinterpret_cast<const float4*>(qrow) + G);
        qv[0] = q4.x;
        qv[1] = q4.y;
        qv[2] = q4.z;
        qv[3] = q4.w;
      }
    } else {
      load_group_scalar(lrow, qrow, G, a.V, l, qv);
    }
    if (qrow) {
      race_group_m<kModeResampleQ, false>(l, qv, -1, cs, shift, inv_sum, -INFINITY, k0, k1, (uint32_t)d, (uint32_t)b,
                                          G, best_key, best_x);
    } else {
      const int32_t xl = 4 * G - x0;  // the group's offset in the chunk: bits 4 (G - G0) .. + 3
      const uint32_t mb = bits[xl >> 5] >> (xl & 31);
#pragma unroll
      for (int k = 0; k < 4; ++k) l[k] = ((mb >> k) & 1u) ? -INFINITY : l[k];
      race_group_m<kModeBonus, false>(l, qv, -1, cs, shift, inv_sum, -INFINITY, k0, k1, (uint32_t)d, (uint32_t)b, G,
                                      best_key, best_x);
    }
  }
  const unsigned long long win = block_reduce<kRaceThreads>(pack_key(best_key, best_x), lds_u, MaxOp());
  if (tid >= 64) return;
  int last = 0;
  if (tid == 0) {
    store_coherent(a.cand + (int64_t)b * a.race_chunks + rc, win);
    wait_memory();
    last = arrive_last(a.race_count + b, (uint32_t)a.race_chunks);
    *s_c = __hip_atomic_fetch_add(claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!lane_i32(last, 0)) return;
  unsigned long long best = 0ull;
  for (int32_t c = lane; c < a.race_chunks; c += 64) {
    const unsigned long long v = load_coherent(a.cand + (int64_t)b * a.race_chunks + c);
    best = v > best ? v : best;
  }
  best = wave_max(best);
  if (best == 0ull) {  // no token had weight (every token with mass a child, or p <= q everywhere): race over p
    float bk = 0.f;
    int32_t bx = INT_MAX;
    for (int32_t G = lane; G < Gend; G += 64) {
      float l[4], qd[4];
      load_group_scalar(lrow, (const float*)nullptr, G, a.V, l, qd);
      race_group(l, qd, kModeBonus, -1, cs, shift, inv_sum, -INFINITY, k0, k1, (uint32_t)d, (uint32_t)b, G, bk, bx);
    }
    best = wave_max(pack_key(bk, bx));
  }
  if (lane == 0) {
    a.out[(int64_t)b * (a.max_depth + 1) + d] = unpack_token(best);
    a.nacc[b] = d;
  }
  tree_finish(a, b, d, cur);
}

// Workgroup k of request b = blockIdx / K: works through the request's
// entries in order, claiming chunks of each until none is left.  bf16 rows
// fit four workgroups per CU (128 VGPRs): more workgroups per request, so a
// 151936-token race (15 chunks) finishes in one round of claims.
template <typename Elem, int NV>
__global__ __launch_bounds__(kRowThreads, sizeof(Elem) == 2 ? 4 : 3) void tree_walk_kernel(TreeArgs<Elem> a) {
  __shared__ unsigned long long s_e, s_w;
  __shared__ uint32_t s_c;
  const int32_t b = (int32_t)(blockIdx.x / a.K);
  const int tid = threadIdx.x, lane = tid & 63;
  // The request's nodes once for all its entries (lane i = node i, wavefront
  // 0, for the decisions); loaded only if the range is in bounds (the init
  // kernel validated the rest; an invalid request gets no row entry).
  const int32_t s = a.cu[b], e = a.cu[b + 1];
  const int32_t n = e - s;
  const float T = a.temperature[b];
  int32_t tok = 0, par = -2;
  if (tid < 64 && s >= 0 && s <= e && e <= a.N && n <= kTreeMaxNodes && lane < n) {
    tok = a.tokens[s + lane];
    par = a.parents[s + lane];
  }
  const unsigned long long* E = entries_of(a, b);
  uint32_t* C = claims_of(a, b);
  for (int32_t r = 0; r < kTreeEntries; ++r) {
    if (tid == 0) {
      // a chunk of entry r is claimed at once; the entry and the walk word are polled together
      s_c = __hip_atomic_fetch_add(C + r, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      unsigned long long ent = load_coherent(E + r), w = load_coherent(walk_of(a, b));
      for (int32_t i = 0; !ent && i < kTreePollLimit; ++i) {
        __builtin_amdgcn_s_sleep(4);
        ent = load_coherent(E + r);
        w = load_coherent(walk_of(a, b));
      }
      s_e = ent;
      s_w = w;
    }
    __syncthreads();
    const unsigned long long ent = s_e, w = s_w;
    uint32_t c = s_c;
    __syncthreads();  // s_e, s_w and s_c are rewritten below
    if (!ent || entry_kind(ent) == kEntryExit) return;
    if (entry_kind(ent) == kEntryNone) continue;
    const uint32_t chunks = (uint32_t)entry_chunks(ent);
    const int32_t x = entry_node(ent), d = entry_step(ent);
    const bool race = entry_kind(ent) == kEntryRace;
    bool merged = false;  // a race entry's row statistics, once per workgroup
    float shift = 0.f, inv_sum = 0.f;
    // a row the walk can no longer need: it stopped, passed step d, or reached another node at it
    const uint32_t step = walk_step(w);
    if (!race && (walk_status(w) != kWalking || step > (uint32_t)d || (step == (uint32_t)d && walk_node(w) != x)))
      continue;
    while (c < chunks) {
      // thread 0 claims the next chunk as the finished one is counted (the two
      // atomics travel together), into s_c
      if (race)
        tree_race_chunk<Elem>(a, b, d, x, (int32_t)c, s, n, T, tok, par, merged, shift, inv_sum, C + r, &s_c);
      else
        tree_row_chunk<Elem, NV>(a, b, d, x, (int32_t)c, s, n, T, tok, par, C + r, &s_c);
      __syncthreads();
      c = s_c;
      __syncthreads();
    }
  }
}

}  // namespace rsv
