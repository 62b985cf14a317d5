// Per-request path: one workgroup of NT threads owns one request.
//
// It walks the request's rows in order -- a statistics pass over row j
// (block-wide max and exp-sum, or argmax for a greedy request), then the
// accept test of draft j -- and stops at the first rejection: rows after it
// cannot change the output, because the drafts behind a rejected one are
// discarded [第12章 投机解码：以小博大 §12.9; vllm v1 源码精读（五） §7].  It then
// races the sampled row (just streamed, so mostly served from the Infinity
// Cache) and writes the output row.  Nothing crosses workgroups, so there are
// no atomics, fences or further launches.  Its critical path is the longest
// request's serial row walk on one CU.
#pragma once

#include "common.hpp"
#include "philox.hpp"
#include "race.hpp"
#include "row_pass.hpp"
#include "rs_verify.h"

namespace rsv {

// Block-wide exponential race over one row (see race_group); returns the
// packed winner (key bits, ~x) or 0 when no residual value is positive.
template <typename Elem, int NT>
__device__ __forceinline__ unsigned long long race_row(const Elem* __restrict__ lrow, const float* __restrict__ qrow,
                                                       int mode, int32_t exclude, float cs, float shift,
                                                       float inv_sum, uint32_t k0, uint32_t k1, uint32_t j,
                                                       uint32_t b, int32_t V, unsigned long long* s_u) {
  constexpr int NB = 4;  // groups of four tokens per thread per batch, double-buffered
  using R4 = Raw4<Elem>;
  const int tid = threadIdx.x;
  const bool has_q = qrow != nullptr;
  const bool fast = ((uintptr_t)lrow % sizeof(typename R4::T)) == 0 && ((uintptr_t)qrow % 16) == 0;
  const int32_t Gend = (V + 3) / 4;
  const int32_t Gfull = fast ? V / 4 : 0;
  float best_key = 0.f;
  int32_t best_x = INT_MAX;

  typename R4::T lw[2][NB];
  float4 qw[2][NB];
  auto load = [&](int buf, int32_t Gb) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int32_t G = Gb + tid + i * NT;
      if (G < Gfull) {
        lw[buf][i] = reinterpret_cast<const typename R4::T*>(lrow)[G];
        if (has_q) qw[buf][i] = reinterpret_cast<const float4*>(qrow)[G];
      }
    }
  };
  auto compute = [&](int buf, int32_t Gb) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int32_t G = Gb + tid + i * NT;
      if (G < Gend) {
        float l[4], qv[4];
        if (G < Gfull) {
          R4::unpack(lw[buf][i], l);
          qv[0] = has_q ? qw[buf][i].x : 0.f;
          qv[1] = has_q ? qw[buf][i].y : 0.f;
          qv[2] = has_q ? qw[buf][i].z : 0.f;
          qv[3] = has_q ? qw[buf][i].w : 0.f;
        } else {
          load_group_scalar(lrow, qrow, G, V, l, qv);
        }
        race_group(l, qv, mode, exclude, cs, shift, inv_sum, -INFINITY, k0, k1, j, b, G, best_key, best_x);
      }
    }
  };
  constexpr int32_t step = NB * NT;
  load(0, 0);
  for (int32_t Gb = 0; Gb < Gend; Gb += 2 * step) {
    if (Gb + step < Gend) load(1, Gb + step);
    compute(0, Gb);
    if (Gb + step >= Gend) break;
    if (Gb + 2 * step < Gend) load(0, Gb + 2 * step);
    compute(1, Gb + step);
  }
  return block_reduce<NT>(pack_key(best_key, best_x), s_u, MaxOp());
}

constexpr int kRequestNVP = 8;  // 16-byte vectors per thread per statistics pass

template <typename Elem, int NT>
__global__ __launch_bounds__(NT) void request_kernel(
    const Elem* __restrict__ logits, const float* __restrict__ q, const int32_t* __restrict__ draft,
    const int32_t* __restrict__ cu, const float* __restrict__ temperature, int32_t greedy_all, int32_t D,
    int32_t max_k, int32_t V, uint64_t seed, int32_t* __restrict__ out, int32_t* __restrict__ num_accepted,
    double* __restrict__ dbg_p) {
  constexpr int NW = NT / 64;
  constexpr int NVP = kRequestNVP;
  __shared__ float s_f[NW];
  __shared__ int s_i[NW];
  __shared__ double s_d[NW];
  __shared__ unsigned long long s_u[NW];
  __shared__ int32_t s_draft[RS_MAX_SPEC_LEN];
  __shared__ int s_valid, s_accept;
  const int32_t b = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t s = cu[b], e = cu[b + 1];
  const int32_t K = e - s;
  int32_t* ob = out + (int64_t)b * (max_k + 1);
  bool valid = request_valid(s, e, D, max_k);
  if (tid == 0) s_valid = valid;
  __syncthreads();
  if (valid && tid < K) {
    const int32_t x = draft[s + tid];
    s_draft[tid] = x;
    if (x < 0 || x >= V) s_valid = 0;
  }
  __syncthreads();
  if (!s_valid) {
    if (tid <= max_k) ob[tid] = -1;
    if (tid == 0) num_accepted[b] = -1;
    return;
  }
  const float T = greedy_all ? 0.f : temperature[b];
  const bool greedy = !(T > 0.f);
  const float cs = greedy ? 0.f : scale_of(T);

  // Walk rows 0..K until the first rejection.
  int32_t n = K;
  RowStats st;
  for (int32_t j = 0; j <= K; ++j) {
    const int64_t row = (int64_t)s + b + j;
    const Elem* prow = logits + row * V;
    // issue the accept-test gathers early; they are used after the reductions
    float lstar = 0.f, qstar = 1.f;
    if (!greedy && tid == 0 && j < K) {
      const int32_t x = s_draft[j];
      lstar = to_f32(prow[x]);
      if (q) qstar = q[((int64_t)s + j) * V + x];
    }
    st = row_stats<Elem, NT, NVP>(prow, V, greedy, cs, s_f, s_i, s_d);
    if (j == K) break;  // bonus row: all drafts accepted
    if (greedy) {
      if (s_draft[j] != st.argmax) {
        n = j;
        break;
      }
    } else {
      if (tid == 0) {
        const double ps = exp2((double)lstar * (double)cs - (double)st.shift) / st.sum;
        const double u = accept_uniform(seed, b, j);
        s_accept = (u * (double)qstar < ps);
        if (dbg_p) dbg_p[s + j] = ps;
      }
      __syncthreads();
      const bool acc = s_accept;
      __syncthreads();  // s_accept is rewritten at the next position
      if (!acc) {
        n = j;
        break;
      }
    }
  }

  int32_t token;
  if (greedy) {
    token = st.argmax;
    if (dbg_p && tid < K) dbg_p[s + tid] = __builtin_nan("");
  } else {
    const int mode = n < K ? (q ? kModeResampleQ : kModeResampleOneHot) : kModeBonus;
    const Elem* lrow = logits + ((int64_t)s + b + n) * V;
    const float* qrow = mode == kModeResampleQ ? q + ((int64_t)s + n) * V : nullptr;
    const int32_t exclude = mode == kModeResampleOneHot ? s_draft[n] : -1;
    const float inv_sum = (float)(1.0 / st.sum);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    unsigned long long win =
        race_row<Elem, NT>(lrow, qrow, mode, exclude, cs, st.shift, inv_sum, k0, k1, (uint32_t)n, (uint32_t)b, V, s_u);
    if (win == 0ull)  // every residual value rounded to zero: race over p at the same row
      win = race_row<Elem, NT>(lrow, nullptr, kModeBonus, -1, cs, st.shift, inv_sum, k0, k1, (uint32_t)n,
                               (uint32_t)b, V, s_u);
    token = unpack_token(win);
  }
  if (tid <= max_k) ob[tid] = tid < n ? s_draft[tid] : (tid == n ? token : -1);
  if (tid == 0) num_accepted[b] = n;
}

}  // namespace rsv
