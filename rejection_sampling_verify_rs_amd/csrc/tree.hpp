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
// Layout of the work (one launch, tree_walk_kernel, after tree_init_kernel).
// Step d of a walk decides among the children of the node reached at step d
// (the root at step 0) from that node's row.  The rows are streamed by walk
// blocks in 16-vector chunks, ahead of the decisions that need them:
//   layer 0: the root row.
//   layer d >= 1: kTreeSpec speculative slots stream the rows of the first
//     kTreeSpec children of the node reached at step d - 1 as soon as it is
//     known (before step d - 1 picks one of them), and one on-demand slot
//     streams the chosen child's row if it is not among them.
//   race blocks, after the walk blocks: (request, 8192-token chunk) pairs
//     that wait for their request's walk to stop and race their chunk of the
//     stop row with the stop node's children masked out; the last one to
//     arrive writes the extra token.
// Step d is decided once both its node is known (step d - 1 decided) and that
// node's row is complete: the step d - 1 decider, after publishing the node,
// checks the row's chunk count; the row's last chunk, after counting itself,
// checks the walk word.  Each stores, waits for the store, then loads, so at
// least one of them sees both; a compare-and-swap on the step's claim word
// lets exactly one decide.  A decider that finds the next row complete goes
// on deciding, step after step.
// A block only ever waits on blocks with smaller indices (earlier layers),
// which were dispatched before it, and every wait is a bounded poll: a walk
// that does not reach a block's step within the bound writes the request as
// invalid (-1 row) instead of hanging.
#pragma once

#include "common.hpp"
#include "philox.hpp"
#include "race.hpp"
#include "row_pass.hpp"

namespace rsv {

constexpr int kTreeMaxNodes = 64;  // one wavefront lane per node
constexpr int kTreeRaceTPT = 32;   // tokens per thread of a race block (8192 tokens per chunk)
constexpr int kTreeNV = 16;        // 16-byte vectors per thread of a walk block
constexpr int kTreeMaxLayers = kTreeMaxNodes + 1;  // steps 0 .. max_depth, max_depth <= max_nodes
constexpr int kTreeSpec = 4;                       // children rows streamed before their parent's step decides
constexpr int kTreeSlots = kTreeSpec + 1;          // plus one on-demand slot per layer
constexpr int32_t kTreePollLimit = 1 << 17;        // polls (about 1 us each) before a block gives up

// Walk word of a request: step (bits 0-7), node + 1 (bits 8-15), status
// (bits 16-23).  Walking: the row of `node` is streamed at `step`.  Stopped:
// the walk ended at `step` on `node`, whose row is raced.  Done: the output
// row is written (greedy stop).  Invalid: -1 row written.
constexpr uint32_t kWalking = 1, kStopped = 2, kWalkDone = 3, kWalkInvalid = 4;
__device__ __forceinline__ unsigned long long walk_word(uint32_t step, int32_t node, uint32_t status) {
  return (unsigned long long)step | ((unsigned long long)(uint32_t)(node + 1) << 8) | ((unsigned long long)status << 16);
}
__device__ __forceinline__ uint32_t walk_step(unsigned long long w) { return (uint32_t)(w & 0xFF); }
__device__ __forceinline__ int32_t walk_node(unsigned long long w) { return (int32_t)((w >> 8) & 0xFF) - 1; }
__device__ __forceinline__ uint32_t walk_status(unsigned long long w) { return (uint32_t)((w >> 16) & 0xFF); }

template <typename Elem>
struct TreeArgs {
  const Elem* logits;
  const int32_t* tokens;
  const int32_t* parents;
  const int32_t* cu;
  const float* temperature;
  uint64_t seed;
  int32_t B, N, max_nodes, max_depth, V;
  int32_t nsplit;       // chunks per row of a walk block
  int32_t race_chunks;  // race blocks per request
  int32_t* out;         // [B, max_depth + 1]
  int32_t* path;        // [B, max_depth]
  int32_t* nacc;        // [B]
  unsigned long long* walk;  // [B]
  uint32_t* count;           // [B * (max_depth + 1) * kTreeSlots] chunk arrivals per (step, slot)
  uint32_t* claim;           // [B * (max_depth + 1)] a step's decision claimed
  uint32_t* race_count;      // [B] race chunk arrivals
  RowPartial* partials;      // [B * (max_depth + 1) * kTreeSlots * nsplit]
  unsigned long long* cand;  // [B * race_chunks] packed race winners
  ReqRecord* records;        // [B] the stop row's race
};

// One wavefront per request: validates the tree (sizes, parents before
// children, tokens in range, every node shallower than max_depth), writes -1
// rows for an invalid one, clears the request's counters and starts its walk.
__global__ __launch_bounds__(64) void tree_init_kernel(const int32_t* __restrict__ tokens,
                                                       const int32_t* __restrict__ parents,
                                                       const int32_t* __restrict__ cu, int32_t N, int32_t max_nodes,
                                                       int32_t max_depth, int32_t V, int32_t* __restrict__ out,
                                                       int32_t* __restrict__ path, int32_t* __restrict__ nacc,
                                                       unsigned long long* __restrict__ walk,
                                                       uint32_t* __restrict__ count, uint32_t* __restrict__ claim,
                                                       uint32_t* __restrict__ race_count) {
  const int32_t b = blockIdx.x;
  const int lane = threadIdx.x;
  const int32_t s = cu[b], e = cu[b + 1];
  const int32_t n = e - s;
  bool ok = s >= 0 && s <= e && e <= N && n <= max_nodes;
  int32_t tk = 0, pr = -1;
  if (ok && lane < n) {
    tk = tokens[s + lane];
    pr = parents[s + lane];
  }
  ok = ok && __ballot(lane < n && (pr < -1 || pr >= lane || tk < 0 || tk >= V)) == 0ull;
  int32_t dep = 0;  // depth of node lane: a parent's depth is final after (its depth + 1) rounds
  for (int32_t r = 0; ok && r < n; ++r) {
    const int32_t dp = __shfl(dep, pr < 0 ? lane : pr);
    dep = pr < 0 ? 0 : dp + 1;
  }
  ok = ok && __ballot(lane < n && dep >= max_depth) == 0ull;
  for (int32_t i = lane; i < (max_depth + 1) * kTreeSlots; i += 64)
    count[(int64_t)b * (max_depth + 1) * kTreeSlots + i] = 0u;
  for (int32_t d = lane; d <= max_depth; d += 64) claim[(int64_t)b * (max_depth + 1) + d] = 0u;
  if (lane == 0) {
    race_count[b] = 0u;
    walk[b] = ok ? walk_word(0, -1, kWalking) : walk_word(0, -1, kWalkInvalid);
  }
  if (!ok) {
    for (int32_t i = lane; i <= max_depth; i += 64) out[(int64_t)b * (max_depth + 1) + i] = -1;
    for (int32_t i = lane; i < max_depth; i += 64) path[(int64_t)b * max_depth + i] = -1;
    if (lane == 0) nacc[b] = -1;
  }
}

// Gives up on a request whose walk did not progress within the poll bound
// (never expected: the blocks waited on were dispatched earlier): -1 row.
template <typename Elem>
__device__ __forceinline__ void tree_give_up(const TreeArgs<Elem>& a, int32_t b) {
  const int lane = threadIdx.x & 63;
  for (int32_t i = lane; i <= a.max_depth; i += 64) a.out[(int64_t)b * (a.max_depth + 1) + i] = -1;
  for (int32_t i = lane; i < a.max_depth; i += 64) a.path[(int64_t)b * a.max_depth + i] = -1;
  if (lane == 0) a.nacc[b] = -1;
}

// Thread 0 polls the walk word of request b until `ready` holds; every thread
// gets the word (0 when the bound expired).
template <typename Ready>
__device__ __forceinline__ unsigned long long tree_wait(const unsigned long long* walk, int32_t b,
                                                        unsigned long long* s_w, Ready ready) {
  if (threadIdx.x == 0) {
    unsigned long long w = load_coherent(walk + b);
    int32_t i = 0;
    for (; !ready(w) && i < kTreePollLimit; ++i) {
      __builtin_amdgcn_s_sleep(2);
      w = load_coherent(walk + b);
    }
    *s_w = ready(w) ? w : 0ull;
  }
  __syncthreads();
  const unsigned long long w = *s_w;
  __syncthreads();  // s_w is reused
  return w;
}

__device__ __forceinline__ int64_t tree_slot_index(int32_t b, int32_t max_depth, int32_t d, int32_t slot) {
  return ((int64_t)b * (max_depth + 1) + d) * kTreeSlots + slot;
}

// Rank of node x among the children of its parent (lanes hold the nodes'
// parents), and the node of rank i among the children of `cur` (-1: none).
__device__ __forceinline__ int32_t child_rank(int32_t par, int32_t n, int32_t x) {
  const int lane = threadIdx.x & 63;
  const int32_t px = __shfl(par, x);
  const unsigned long long sib = __ballot(lane < n && par == px);
  return __popcll(sib & ((1ull << x) - 1ull));
}
__device__ __forceinline__ int32_t nth_child(int32_t par, int32_t n, int32_t cur, int32_t i) {
  const int lane = threadIdx.x & 63;
  unsigned long long kids = __ballot(lane < n && par == cur);
  for (int32_t k = 0; k < i && kids; ++k) kids &= kids - 1ull;
  return kids ? __ffsll((long long)kids) - 1 : -1;
}

// Decisions of request b from step d on (wavefront 0 of the block that
// claimed step d): merge the row's partial statistics, choose the child or
// stop, write the step's output and publish the walk word; while the next
// step's row is already complete, claim and decide it too.
template <typename Elem>
__device__ __forceinline__ void tree_decide(const TreeArgs<Elem>& a, int32_t b, int32_t d, int32_t cur, int32_t slot,
                                            int32_t s, int32_t n, float T, int32_t tok, int32_t par) {
  const int lane = threadIdx.x & 63;
  const bool greedy = !(T > 0.f);
  const float cs = greedy ? 0.f : scale_of(T);
  int32_t* ob = a.out + (int64_t)b * (a.max_depth + 1);
  int32_t* pb = a.path + (int64_t)b * a.max_depth;
  for (;;) {
    const int64_t row = (int64_t)s + b + 1 + cur;
    const Elem* prow = a.logits + row * (int64_t)a.V;
    const bool child = lane < n && par == cur;
    // the children's logits and the partials are loaded together
    const float lt = (!greedy && child) ? to_f32(prow[tok]) : -INFINITY;
    const RowPartial* P = a.partials + tree_slot_index(b, a.max_depth, d, slot) * a.nsplit;
    float shift = -INFINITY;
    double S = 0.0;
    int32_t amax = -1, next = -1;
    if (greedy) {
      amax = merge_greedy<true>(P, a.nsplit);
      const unsigned long long m = __ballot(child && tok == amax);
      next = m ? __ffsll((long long)m) - 1 : -1;
    } else {
      merge_random<true>(P, a.nsplit, shift, S);
      const unsigned long long kids = __ballot(child);
      bool dup = false;  // a repeat of an earlier sibling's token
      for (int k = 0; k < 63; ++k) {
        const int32_t tk = __shfl(tok, k);
        dup = dup || (k < lane && ((kids >> k) & 1ull) && tk == tok);
      }
      const bool take = child && !dup;
      double cum = take ? exp2((double)lt * (double)cs - (double)shift) / S : 0.0;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {  // inclusive prefix sum in node order
        const double v = __shfl_up(cum, o);
        if (lane >= o) cum += v;
      }
      const double u = accept_uniform(a.seed, b, d);
      const unsigned long long m = __ballot(take && u < cum);
      next = m ? __ffsll((long long)m) - 1 : -1;
    }
    if (next < 0) {  // stop at step d
      for (int32_t i = d + lane; i < a.max_depth; i += 64) pb[i] = -1;
      for (int32_t i = d + 1 + lane; i <= a.max_depth; i += 64) ob[i] = -1;
      if (greedy) {
        if (lane == 0) {
          ob[d] = amax;
          a.nacc[b] = d;
          store_coherent(a.walk + b, walk_word((uint32_t)d, cur, kWalkDone));
        }
        return;
      }
      if (lane == 0) {  // the race over p without the stop node's children, by the race blocks
        ReqRecord r;
        r.mode = kModeBonus;
        r.phase = 0;
        r.n = d;
        r.row = (int32_t)row;
        r.slot0 = s;
        r.exclude = cur;  // the stop node (-1: the root); its children leave the race
        r.c = cs;
        r.shift = shift;
        r.inv_sum = (float)(1.0 / S);
        r.tau = -INFINITY;
        r.pad[0] = n;
        r.pad[1] = 0;
        unsigned long long w[sizeof(ReqRecord) / 8];
        __builtin_memcpy(w, &r, sizeof(ReqRecord));
#pragma unroll
        for (int i = 0; i < (int)(sizeof(ReqRecord) / 8); ++i)
          store_coherent(reinterpret_cast<unsigned long long*>(a.records + b) + i, w[i]);
        wait_memory();  // the record is visible before the walk word says "stopped"
        store_coherent(a.walk + b, walk_word((uint32_t)d, cur, kStopped));
      }
      return;
    }
    // descend: the accepted node is emitted, and step d + 1 decides among its children
    const int32_t ntok = __shfl(tok, next);
    const int32_t rank = child_rank(par, n, next);
    int go = 0;
    if (lane == 0) {
      ob[d] = ntok;
      pb[d] = next;
      store_coherent(a.walk + b, walk_word((uint32_t)d + 1, next, kWalking));
      wait_memory();  // published before the next row's count is read
      if (rank < kTreeSpec &&
          __hip_atomic_load(a.count + tree_slot_index(b, a.max_depth, d + 1, rank), __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)a.nsplit)
        go = atomic_cas32(reinterpret_cast<int32_t*>(a.claim) + (int64_t)b * (a.max_depth + 1) + d + 1, 0, 1);
    }
    if (!__shfl(go, 0)) return;
    ++d;
    cur = next;
    slot = rank;
  }
}

// Walk block: chunk c of the row in slot `slot` of layer d of request b (see
// the layout above).
template <typename Elem, int NV>
__device__ __forceinline__ void tree_walk_block(const TreeArgs<Elem>& a, int32_t d, int32_t b, int32_t slot,
                                                int32_t c, unsigned long long* s_w) {
  const int tid = threadIdx.x, lane = tid & 63;
  // Layer 0 streams the root row at once; a speculative slot waits for the
  // node of step d - 1, the on-demand slot for the node of step d.
  const uint32_t need = slot < kTreeSpec ? (uint32_t)(d > 0 ? d - 1 : 0) : (uint32_t)d;
  unsigned long long w;
  if (d > 0) {
    w = tree_wait(a.walk, b, s_w, [need](unsigned long long v) {
      return walk_status(v) != kWalking || walk_step(v) >= need;
    });
    if (w == 0ull) {  // gave up: the walk never reached the step
      if (tid < 64) tree_give_up(a, b);
      return;
    }
  } else {
    if (tid == 0) *s_w = load_coherent(a.walk + b);
    __syncthreads();
    w = *s_w;
    __syncthreads();
  }
  if (walk_status(w) != kWalking) return;  // ended, or invalid (never streamed)
  // The request's nodes, lane i = node i, in every wavefront (each computes
  // the same row to stream; wavefront 0 also takes the decisions).  The init
  // kernel validated the tree.
  const int32_t s = a.cu[b], n = a.cu[b + 1] - s;
  int32_t tok = 0, par = -2;
  if (lane < n) {
    tok = a.tokens[s + lane];
    par = a.parents[s + lane];
  }
  const uint32_t step = walk_step(w);
  int32_t node;
  if (d == 0) {
    node = -1;
  } else if (slot < kTreeSpec) {
    if (step > (uint32_t)d) return;  // step d already decided: its row was complete
    // the slot-th child of the node of step d - 1: the current node, or, once
    // step d - 1 is decided, the parent of the current node
    int32_t prev = walk_node(w);
    if (step == (uint32_t)d) prev = __shfl(par, prev);
    node = nth_child(par, n, prev, slot);
    if (node < 0 || (step == (uint32_t)d && node != walk_node(w))) return;  // no such child / not the chosen one
  } else {
    if (step != (uint32_t)d) return;
    node = walk_node(w);
    if (child_rank(par, n, node) < kTreeSpec) return;  // a speculative slot streams it
  }
  const float T = a.temperature[b];
  const int64_t row = (int64_t)s + b + 1 + node;
  chunk_task<Elem, NV, true>(a.logits, nullptr, row, T, a.V, a.nsplit, c, -1, 0,
                             a.partials + tree_slot_index(b, a.max_depth, d, slot) * a.nsplit, nullptr);
  if (tid >= 64) return;
  int go = 0;
  if (tid == 0) {
    wait_memory();  // the partial is visible before it is counted
    if (arrive_last(a.count + tree_slot_index(b, a.max_depth, d, slot), (uint32_t)a.nsplit)) {
      // the row is complete: decide step d if its node is this row's
      const unsigned long long v = load_coherent(a.walk + b);
      if (walk_status(v) == kWalking && walk_step(v) == (uint32_t)d && walk_node(v) == node)
        go = atomic_cas32(reinterpret_cast<int32_t*>(a.claim) + (int64_t)b * (a.max_depth + 1) + d, 0, 1);
    }
  }
  if (__shfl(go, 0)) tree_decide(a, b, d, node, slot, s, n, T, tok, par);
}

// Race block: chunk rc (kRaceThreads * kTreeRaceTPT tokens) of request b's
// stop row, the stop node's children (those with a token in the chunk)
// marked in an LDS bitmap and given weight 0.  The last chunk to arrive
// writes the extra token; if every token with mass was a child of the stop
// node it races over p instead.
template <typename Elem>
__device__ __forceinline__ void tree_race_block(const TreeArgs<Elem>& a, int32_t b, int32_t rc,
                                                unsigned long long* s_w) {
  constexpr int NG = kTreeRaceTPT / 4;  // groups of four tokens per thread
  constexpr int kChunk = kRaceThreads * kTreeRaceTPT;
  using R4 = Raw4<Elem>;
  __shared__ uint32_t bits[kChunk / 32];
  __shared__ unsigned long long lds_u[kRaceThreads / 64];
  const int tid = threadIdx.x;
  const unsigned long long w =
      tree_wait(a.walk, b, s_w, [](unsigned long long v) { return walk_status(v) != kWalking; });
  if (w == 0ull) {
    if (tid < 64) tree_give_up(a, b);
    return;
  }
  if (walk_status(w) != kStopped) return;  // greedy, invalid, or done
  ReqRecord rec;
  {
    unsigned long long r[sizeof(ReqRecord) / 8];
#pragma unroll
    for (int i = 0; i < (int)(sizeof(ReqRecord) / 8); ++i)
      r[i] = load_coherent(reinterpret_cast<const unsigned long long*>(a.records + b) + i);
    __builtin_memcpy(&rec, r, sizeof(ReqRecord));
  }
  const int32_t x0 = rc * kChunk;
  for (int i = tid; i < kChunk / 32; i += kRaceThreads) bits[i] = 0u;
  __syncthreads();
  if (tid < rec.pad[0] && a.parents[rec.slot0 + tid] == rec.exclude) {
    const int32_t x = a.tokens[rec.slot0 + tid] - x0;
    if (x >= 0 && x < kChunk) atomicOr(bits + (x >> 5), 1u << (x & 31));
  }
  __syncthreads();
  const Elem* lrow = a.logits + (int64_t)rec.row * a.V;
  const bool fast = ((uintptr_t)lrow % sizeof(typename R4::T)) == 0;
  const int32_t Gend = (a.V + 3) / 4, Gfull = fast ? a.V / 4 : 0;
  const int32_t G0 = rc * (kRaceThreads * NG);
  const uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32);
  typename R4::T lw[NG];
  if (Gfull > 0) {  // unconditional loads (index clamped into the vector part): all in flight together
#pragma unroll
    for (int i = 0; i < NG; ++i)
      lw[i] = reinterpret_cast<const typename R4::T*>(lrow)[min(G0 + tid + i * kRaceThreads, Gfull - 1)];
  }
  float best_key = 0.f;
  int32_t best_x = INT_MAX;
  const float qz[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int32_t G = G0 + tid + i * kRaceThreads;
    if (G >= Gend) continue;
    float l[4];
    if (G < Gfull) {
      R4::unpack(lw[i], l);
    } else {
      float qd[4];
      load_group_scalar(lrow, (const float*)nullptr, G, a.V, l, qd);
    }
    const int32_t xl = 4 * G - x0;  // the group's offset in the chunk: bits 4 (G - G0) .. + 3
    const uint32_t mb = bits[xl >> 5] >> (xl & 31);
#pragma unroll
    for (int k = 0; k < 4; ++k) l[k] = ((mb >> k) & 1u) ? -INFINITY : l[k];
    race_group_m<kModeBonus, false>(l, qz, -1, rec.c, rec.shift, rec.inv_sum, -INFINITY, k0, k1, (uint32_t)rec.n,
                                    (uint32_t)b, G, best_key, best_x);
  }
  const unsigned long long win = block_reduce<kRaceThreads>(pack_key(best_key, best_x), lds_u, MaxOp());
  if (tid >= 64) return;
  int last = 0;
  if (tid == 0) {
    store_coherent(a.cand + (int64_t)b * a.race_chunks + rc, win);
    wait_memory();
    last = arrive_last(a.race_count + b, (uint32_t)a.race_chunks);
  }
  if (!__shfl(last, 0)) return;
  unsigned long long best = 0ull;
  for (int32_t c = tid; c < a.race_chunks; c += 64) {
    const unsigned long long v = load_coherent(a.cand + (int64_t)b * a.race_chunks + c);
    best = v > best ? v : best;
  }
  best = wave_max(best);
  if (best == 0ull) {  // every token with mass is a child of the stop node: race over p
    float bk = 0.f;
    int32_t bx = INT_MAX;
    for (int32_t G = tid; G < Gend; G += 64) {
      float l[4], qd[4];
      load_group_scalar(lrow, (const float*)nullptr, G, a.V, l, qd);
      race_group(l, qd, kModeBonus, -1, rec.c, rec.shift, rec.inv_sum, -INFINITY, k0, k1, (uint32_t)rec.n,
                 (uint32_t)b, G, bk, bx);
    }
    best = wave_max(pack_key(bk, bx));
  }
  if (tid == 0) {
    a.out[(int64_t)b * (a.max_depth + 1) + rec.n] = unpack_token(best);
    a.nacc[b] = rec.n;
  }
}

template <typename Elem, int NV>
__global__ __launch_bounds__(kRowThreads) void tree_walk_kernel(TreeArgs<Elem> a) {
  __shared__ unsigned long long s_w;
  int64_t k = blockIdx.x;
  const int64_t layer0 = (int64_t)a.B * a.nsplit;                 // root rows
  const int64_t per_layer = (int64_t)a.B * kTreeSlots * a.nsplit;  // layers 1 .. max_depth
  if (k < layer0) {
    tree_walk_block<Elem, NV>(a, 0, (int32_t)(k / a.nsplit), 0, (int32_t)(k % a.nsplit), &s_w);
    return;
  }
  k -= layer0;
  if (k < per_layer * a.max_depth) {
    const int32_t d = 1 + (int32_t)(k / per_layer);
    const int64_t r = k % per_layer;  // request, then slot, then chunk
    tree_walk_block<Elem, NV>(a, d, (int32_t)(r / ((int64_t)kTreeSlots * a.nsplit)),
                              (int32_t)((r / a.nsplit) % kTreeSlots), (int32_t)(r % a.nsplit), &s_w);
    return;
  }
  k -= per_layer * a.max_depth;
  tree_race_block<Elem>(a, (int32_t)(k / a.race_chunks), (int32_t)(k % a.race_chunks), &s_w);
}

}  // namespace rsv
