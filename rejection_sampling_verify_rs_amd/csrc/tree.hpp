// Tree verify: one workgroup of NT threads per request walks its draft tree.
//
// The drafts of a request form a tree -- each node one draft token, its parent
// earlier in the node order or -1 for a child of the last prefix position --
// and the target scored the prefix position (row 0) and every node (row
// 1 + i), row r predicting the children of its node [投机解码深度实战 §四: one
// target forward over the whole tree].  The walk goes one depth at a time
// from the root: it streams the current node's row, looks for an accepted
// child among the current layer's siblings, descends into it, and stops at
// the first depth where none is accepted; one extra token then comes from the
// stop node's row [投机解码（Speculative Decoding）端到端深挖 §6.2].
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
// random numbers.  Only the rows on the accepted path (and the stop row) are
// read: a few rows of the tree's dozens.  The walk runs one workgroup per
// request; the final race of random requests is spread over (request, chunk)
// workgroups and reduced by an emit kernel, as on the chain paths.
#pragma once

#include "common.hpp"
#include "philox.hpp"
#include "race.hpp"
#include "row_pass.hpp"

namespace rsv {

constexpr int kTreeMaxNodes = 64;  // one wavefront lane per node

constexpr int kTreeRaceTPT = 32;  // tokens per thread of a race workgroup (8192 tokens per chunk)

// The walk, one workgroup per request.  A greedy request's output is written
// here; a random request leaves a race record (stop row, statistics, stop
// node) for tree_race_kernel and tree_emit_kernel, which spread the final
// race over the whole GPU.
template <typename Elem, int NT>
__global__ __launch_bounds__(NT) void tree_kernel(
    const Elem* __restrict__ logits, const int32_t* __restrict__ tokens, const int32_t* __restrict__ parents,
    const int32_t* __restrict__ cu, const float* __restrict__ temperature, int32_t N, int32_t max_nodes,
    int32_t max_depth, int32_t V, uint64_t seed, int32_t* __restrict__ out, int32_t* __restrict__ path,
    int32_t* __restrict__ num_accepted, ReqRecord* __restrict__ records) {
  constexpr int NW = NT / 64;
  // 16-byte vectors per thread per statistics pass (the most without spills)
  constexpr int NVP = NT >= 1024 ? 4 : (NT >= 512 ? 8 : 16);
  __shared__ float s_f[NW];
  __shared__ int s_i[NW];
  __shared__ double s_d[NW];
  __shared__ int32_t s_tok[kTreeMaxNodes], s_par[kTreeMaxNodes];
  __shared__ int s_valid, s_next;
  const int32_t b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int32_t s = cu[b], e = cu[b + 1];
  const int32_t n = e - s;
  int32_t* ob = out + (int64_t)b * (max_depth + 1);
  int32_t* pb = path + (int64_t)b * max_depth;

  // Validate the tree (wavefront 0): sizes, parents before children, tokens in
  // range, every node shallower than max_depth.
  if (tid < 64) {
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
    if (lane < kTreeMaxNodes) {
      s_tok[lane] = tk;
      s_par[lane] = pr;
    }
    if (lane == 0) s_valid = ok;
  }
  __syncthreads();
  if (!s_valid) {
    if (tid <= max_depth) ob[tid] = -1;
    if (tid < max_depth) pb[tid] = -1;
    if (tid == 0) {
      num_accepted[b] = -1;
      records[b].mode = kModeDone;
    }
    return;
  }
  const float T = temperature[b];
  const bool greedy = !(T > 0.f);
  const float cs = greedy ? 0.f : scale_of(T);
  const int64_t row0 = (int64_t)s + b;

  int32_t cur = -1, d = 0;
  RowStats st;
  for (;;) {
    const Elem* prow = logits + (row0 + 1 + cur) * (int64_t)V;
    const bool child = lane < n && s_par[lane] == cur;
    // the children's logits, issued before the row pass (random requests)
    float lt = -INFINITY;
    if (!greedy && tid < 64 && child) lt = to_f32(prow[s_tok[lane]]);
    st = row_stats<Elem, NT, NVP>(prow, V, greedy, cs, s_f, s_i, s_d);
    if (tid < 64) {
      const unsigned long long kids = __ballot(child);
      int32_t next = -1;
      if (greedy) {
        const unsigned long long m = __ballot(child && s_tok[lane] == st.argmax);
        next = m ? __ffsll((long long)m) - 1 : -1;
      } else {
        bool dup = false;  // a repeat of an earlier sibling's token
        if (child) {
          for (int k = 0; k < lane; ++k)
            if (((kids >> k) & 1ull) && s_tok[k] == s_tok[lane]) dup = true;
        }
        const bool take = child && !dup;
        double cum = take ? exp2((double)lt * (double)cs - (double)st.shift) / st.sum : 0.0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {  // inclusive prefix sum in node order
          const double v = __shfl_up(cum, o);
          if (lane >= o) cum += v;
        }
        const double u = accept_uniform(seed, b, d);
        const unsigned long long m = __ballot(take && u < cum);
        next = m ? __ffsll((long long)m) - 1 : -1;
      }
      if (lane == 0) {
        s_next = next;
        if (next >= 0) {
          ob[d] = s_tok[next];
          pb[d] = next;
        }
      }
    }
    __syncthreads();
    const int32_t next = s_next;
    __syncthreads();  // s_next is rewritten at the next depth
    if (next < 0) break;
    cur = next;
    ++d;
  }

  if (tid >= d && tid < max_depth) pb[tid] = -1;
  if (greedy) {
    if (tid == 0) {
      ob[d] = st.argmax;
      num_accepted[b] = d;
      records[b].mode = kModeDone;
    }
    if (tid > d && tid <= max_depth) ob[tid] = -1;
    return;
  }
  if (tid == 0) {  // the race over p without the stop node's children
    ReqRecord r;
    r.mode = kModeBonus;
    r.phase = 0;
    r.n = d;
    r.row = (int32_t)(row0 + 1 + cur);
    r.slot0 = s;
    r.exclude = cur;  // the stop node (-1: the root); its children leave the race
    r.c = cs;
    r.shift = st.shift;
    r.inv_sum = (float)(1.0 / st.sum);
    r.tau = -INFINITY;
    r.pad[0] = n;
    r.pad[1] = 0;
    records[b] = r;
  }
}

// The stop row's race, chunk c (kRaceThreads * kTreeRaceTPT tokens) of
// request b: the stop node's children (those with a token in the chunk) are
// marked in an LDS bitmap and get weight 0.  cand[b * nchunks + c] receives
// the packed winner of the chunk (0: none).
template <typename Elem>
__global__ __launch_bounds__(kRaceThreads) void tree_race_kernel(
    const Elem* __restrict__ logits, const int32_t* __restrict__ tokens, const int32_t* __restrict__ parents,
    int32_t V, uint64_t seed, int32_t nchunks, const ReqRecord* __restrict__ records,
    unsigned long long* __restrict__ cand) {
  constexpr int NG = kTreeRaceTPT / 4;   // groups of four tokens per thread
  constexpr int kChunk = kRaceThreads * kTreeRaceTPT;
  using R4 = Raw4<Elem>;
  __shared__ uint32_t bits[kChunk / 32];
  __shared__ unsigned long long lds_u[kRaceThreads / 64];
  const int32_t b = (int32_t)(blockIdx.x / nchunks), c = (int32_t)(blockIdx.x % nchunks);
  const ReqRecord rec = records[b];
  if (rec.mode != kModeBonus) return;
  const int tid = threadIdx.x;
  const int32_t x0 = c * kChunk;
  for (int w = tid; w < kChunk / 32; w += kRaceThreads) bits[w] = 0u;
  __syncthreads();
  if (tid < rec.pad[0] && parents[rec.slot0 + tid] == rec.exclude) {
    const int32_t x = tokens[rec.slot0 + tid] - x0;
    if (x >= 0 && x < kChunk) atomicOr(bits + (x >> 5), 1u << (x & 31));
  }
  __syncthreads();
  const Elem* lrow = logits + (int64_t)rec.row * V;
  const bool fast = ((uintptr_t)lrow % sizeof(typename R4::T)) == 0;
  const int32_t Gend = (V + 3) / 4, Gfull = fast ? V / 4 : 0;
  const int32_t G0 = c * (kRaceThreads * NG);
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  typename R4::T lw[NG];
  if (Gfull > 0) {  // unconditional loads (index clamped into the vector part): all in flight together
#pragma unroll
    for (int i = 0; i < NG; ++i)
      lw[i] = stream_load(reinterpret_cast<const typename R4::T*>(lrow) + min(G0 + tid + i * kRaceThreads, Gfull - 1));
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
      load_group_scalar(lrow, (const float*)nullptr, G, V, l, qd);
    }
    const int32_t xl = 4 * G - x0;  // the group's offset in the chunk: bits 4 (G - G0) .. + 3
    const uint32_t w = bits[xl >> 5] >> (xl & 31);
#pragma unroll
    for (int k = 0; k < 4; ++k) l[k] = ((w >> k) & 1u) ? -INFINITY : l[k];
    race_group_m<kModeBonus, false>(l, qz, -1, rec.c, rec.shift, rec.inv_sum, -INFINITY, k0, k1, (uint32_t)rec.n,
                                    (uint32_t)b, G, best_key, best_x);
  }
  const unsigned long long win = block_reduce<kRaceThreads>(pack_key(best_key, best_x), lds_u, MaxOp());
  if (tid == 0) cand[(int64_t)b * nchunks + c] = win;
}

// One wavefront per random request: the race winner -> output row.  If every
// token with mass was a child of the stop node, race over p instead.
template <typename Elem>
__global__ __launch_bounds__(64) void tree_emit_kernel(const Elem* __restrict__ logits, int32_t max_depth, int32_t V,
                                                       uint64_t seed, int32_t nchunks,
                                                       const ReqRecord* __restrict__ records,
                                                       const unsigned long long* __restrict__ cand,
                                                       int32_t* __restrict__ out, int32_t* __restrict__ num_accepted) {
  const int32_t b = blockIdx.x;
  const int lane = threadIdx.x;
  const ReqRecord rec = records[b];
  if (rec.mode != kModeBonus) return;
  unsigned long long win = 0ull;
  for (int32_t c = lane; c < nchunks; c += 64) {
    const unsigned long long v = cand[(int64_t)b * nchunks + c];
    win = v > win ? v : win;
  }
  win = wave_max(win);
  if (win == 0ull) {
    const Elem* lrow = logits + (int64_t)rec.row * V;
    float bk = 0.f;
    int32_t bx = INT_MAX;
    for (int32_t G = lane; G < (V + 3) / 4; G += 64) {
      float l[4], qz[4];
      load_group_scalar(lrow, (const float*)nullptr, G, V, l, qz);
      race_group(l, qz, kModeBonus, -1, rec.c, rec.shift, rec.inv_sum, -INFINITY, (uint32_t)seed,
                 (uint32_t)(seed >> 32), (uint32_t)rec.n, (uint32_t)b, G, bk, bx);
    }
    win = wave_max(pack_key(bk, bx));
  }
  int32_t* ob = out + (int64_t)b * (max_depth + 1);
  if (lane == 0) {
    ob[rec.n] = unpack_token(win);
    num_accepted[b] = rec.n;
  }
  for (int32_t i = rec.n + 1 + lane; i <= max_depth; i += 64) ob[i] = -1;
}

}  // namespace rsv
