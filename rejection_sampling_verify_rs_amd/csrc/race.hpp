// Exponential race over one row: argmax_x r(x) / E_x with E_x ~ Exp(1) from
// Philox, which samples r / sum(r) without normalising r
// [第12章 投机解码：以小博大 §12.9, last bullet].
//   resample with q:  r = max(0, p - q)             [§12.2.1 step 3]
//   resample, no q:   r = p, except r(x*) = 0       [§12.9, last bullet]
//   bonus:            r = p                         [§12.3.2]
// with p = exp2(l c - shift) / sum in fp32.  E_x = -ln U_x and the key is
// r / E'_x with E' = -log2 U = E / ln 2 (a common factor, so the argmax is the
// same).  Ties go to the lowest token index.
#pragma once

#include "common.hpp"
#include "philox.hpp"

namespace rsv {

// Keys of the four tokens 4G .. 4G+3 of one group from preloaded logits l[]
// and draft probabilities qv[] (tokens at or beyond V carry l = -inf, so
// r = 0).  Keeps the thread's best (key, x); tokens are visited in increasing
// x, so '>' keeps the lowest index among equal keys.
__device__ __forceinline__ void race_group(const float (&l)[4], const float (&qv)[4], int mode, int32_t exclude,
                                           float cs, float shift, float inv_sum, uint32_t k0, uint32_t k1,
                                           uint32_t j, uint32_t b, int32_t G, float& best_key,
                                           int32_t& best_x) {
  const PhiloxOut o = philox4x32_10((uint32_t)G, j, b, 1u, k0, k1);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int32_t x = 4 * G + k;
    const float ex = exp2_hw(fmaf(l[k], cs, -shift));
    float r;
    if (mode == kModeResampleQ)
      r = fmaxf(ex * inv_sum - qv[k], 0.f);
    else if (mode == kModeResampleOneHot)
      r = (x == exclude) ? 0.f : ex;
    else
      r = ex;
    if (r > 0.f) {
      const float ep = -__builtin_amdgcn_logf(race_uniform_f32(o.w[k]));
      const float key = r * __builtin_amdgcn_rcpf(ep);
      if (key > best_key) {
        best_key = key;
        best_x = x;
      }
    }
  }
}

// Element-wise load of group G (tokens at or beyond V get l = -inf, q = 0).
template <typename Elem>
__device__ __forceinline__ void load_group_scalar(const Elem* __restrict__ lrow, const float* __restrict__ qrow,
                                                  int32_t G, int32_t V, float (&l)[4], float (&qv)[4]) {
  const int32_t x0 = 4 * G;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    l[k] = (x0 + k < V) ? to_f32(lrow[x0 + k]) : -INFINITY;
    qv[k] = (qrow && x0 + k < V) ? qrow[x0 + k] : 0.f;
  }
}

// One workgroup races chunk c (kRaceThreads * TPT tokens) of request b's
// sampled row described by `rec` and returns the packed best of the chunk
// (0 = no positive key) in every thread.
template <typename Elem, int TPT>
__device__ __forceinline__ unsigned long long race_chunk(const Elem* __restrict__ logits, const float* __restrict__ q,
                                                         int32_t V, uint64_t seed, const ReqRecord& rec, int32_t b,
                                                         int32_t c) {
  constexpr int NG = TPT / 4;  // groups of four tokens per thread
  using R4 = Raw4<Elem>;
  __shared__ unsigned long long lds_u[kRaceThreads / 64];
  const int tid = threadIdx.x;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const Elem* lrow = logits + (int64_t)rec.row * V;
  const bool has_q = rec.mode == kModeResampleQ;
  const float* qrow = has_q ? q + ((int64_t)rec.slot0 + rec.n) * V : nullptr;
  // Vector loads need 8 / 16-byte aligned rows; otherwise every group goes element-wise.
  const bool fast = ((uintptr_t)lrow % sizeof(typename R4::T)) == 0 && ((uintptr_t)qrow % 16) == 0;
  const int32_t G0 = c * (kRaceThreads * NG);
  const int32_t Gend = (V + 3) / 4;
  const int32_t Gfull = fast ? V / 4 : 0;  // groups loaded as vectors

  // Issue every vector load of this thread before any arithmetic.
  typename R4::T lw[NG];
  float4 qw[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int32_t G = G0 + tid + i * kRaceThreads;
    if (G < Gfull) {
      lw[i] = reinterpret_cast<const typename R4::T*>(lrow)[G];
      if (has_q) qw[i] = reinterpret_cast<const float4*>(qrow)[G];
    }
  }
  float best_key = 0.f;
  int32_t best_x = INT_MAX;
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int32_t G = G0 + tid + i * kRaceThreads;
    if (G < Gend) {
      float l[4], qv[4];
      if (G < Gfull) {
        R4::unpack(lw[i], l);
        qv[0] = has_q ? qw[i].x : 0.f;
        qv[1] = has_q ? qw[i].y : 0.f;
        qv[2] = has_q ? qw[i].z : 0.f;
        qv[3] = has_q ? qw[i].w : 0.f;
      } else {
        load_group_scalar(lrow, qrow, G, V, l, qv);
      }
      race_group(l, qv, rec.mode, rec.exclude, rec.c, rec.shift, rec.inv_sum, k0, k1, (uint32_t)rec.n,
                 (uint32_t)b, G, best_key, best_x);
    }
  }
  return block_reduce<kRaceThreads>(pack_key(best_key, best_x), lds_u, MaxOp());
}

}  // namespace rsv
