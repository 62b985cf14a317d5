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
// read: a few rows of the tree's dozens.
#pragma once

#include "common.hpp"
#include "philox.hpp"
#include "race.hpp"
#include "request_path.hpp"
#include "row_pass.hpp"

namespace rsv {

constexpr int kTreeMaxNodes = 64;  // one wavefront lane per node

template <typename Elem, int NT>
__global__ __launch_bounds__(NT) void tree_kernel(
    const Elem* __restrict__ logits, const int32_t* __restrict__ tokens, const int32_t* __restrict__ parents,
    const int32_t* __restrict__ cu, const float* __restrict__ temperature, int32_t N, int32_t max_nodes,
    int32_t max_depth, int32_t V, uint64_t seed, int32_t* __restrict__ out, int32_t* __restrict__ path,
    int32_t* __restrict__ num_accepted) {
  constexpr int NW = NT / 64;
  constexpr int NVP = 8;  // 16-byte vectors per thread per statistics pass
  extern __shared__ uint32_t excl_bits[];  // (V + 31) / 32 words: tokens out of the final race
  __shared__ float s_f[NW];
  __shared__ int s_i[NW];
  __shared__ double s_d[NW];
  __shared__ unsigned long long s_u[NW];
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
    if (tid == 0) num_accepted[b] = -1;
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

  int32_t token;
  if (greedy) {
    token = st.argmax;
  } else {
    // race over p without the stop node's children (none: the bonus)
    const int nwords = (V + 31) / 32;
    for (int w = tid; w < nwords; w += NT) excl_bits[w] = 0u;
    __syncthreads();
    if (tid < 64 && lane < n && s_par[lane] == cur) atomicOr(excl_bits + (s_tok[lane] >> 5), 1u << (s_tok[lane] & 31));
    __syncthreads();
    const Elem* lrow = logits + (row0 + 1 + cur) * (int64_t)V;
    const float inv_sum = (float)(1.0 / st.sum);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    unsigned long long win = race_row<Elem, NT>(lrow, nullptr, kModeBonus, -1, cs, st.shift, inv_sum, k0, k1,
                                                (uint32_t)d, (uint32_t)b, V, s_u, excl_bits);
    if (win == 0ull)  // every token with mass was drafted: race over p
      win = race_row<Elem, NT>(lrow, nullptr, kModeBonus, -1, cs, st.shift, inv_sum, k0, k1, (uint32_t)d,
                               (uint32_t)b, V, s_u);
    token = unpack_token(win);
  }
  if (tid == 0) {
    ob[d] = token;
    num_accepted[b] = d;
  }
  if (tid > d && tid <= max_depth) ob[tid] = -1;
  if (tid >= d && tid < max_depth) pb[tid] = -1;
}

}  // namespace rsv
