// Exponential race over one row: argmax_x r(x) / E_x with E_x ~ Exp(1) from
// Philox, which samples r / sum(r) without normalising r
// [第12章 投机解码：以小博大 §12.9, last bullet].
//   resample with q:  r = max(0, p - q)             [§12.2.1 step 3]
//   resample, no q:   r = p, except r(x*) = 0       [§12.9, last bullet]
//   bonus:            r = p                         [§12.3.2]
// with p = exp2(l c - shift) / sum in fp32; without q the factor 1 / sum is
// common to every token and left out.  E_x = -ln U_x and the key is r / E'_x
// with E' = -log2 U = E / ln 2 (a common factor, so the argmax is the same).
// Ties go to the lowest token index.
//
// Per token the work is one exp2, one log2 and one reciprocal (each a
// half-rate transcendental on gfx950) and a handful of full-rate ops; one
// Philox4x32-10 evaluation (18 v_mad_u64_u32 + XORs) serves four tokens.  The
// loop body is branch-free: r = 0 gives key 0, which never beats the initial
// best of 0.
#pragma once

#include "common.hpp"
#include "philox.hpp"

namespace rsv {

// r(x) for one token, ex = exp2(l c - shift).
template <int MODE>
__device__ __forceinline__ float race_weight(float ex, float qv, int32_t x, int32_t exclude, float inv_sum) {
  if constexpr (MODE == kModeResampleQ) {
    return fmaxf(fmaf(ex, inv_sum, -qv), 0.f);
  } else if constexpr (MODE == kModeResampleOneHot) {
    return x == exclude ? 0.f : ex;
  } else {
    return ex;
  }
}

// Keys of the four tokens 4G .. 4G+3 from their logits l[] and draft
// probabilities qv[] (tokens at or beyond V carry l = -inf, so r = 0).  Keeps
// the thread's best (key, x); tokens arrive in increasing x, so '>' keeps the
// lowest index among equal keys.
template <int MODE, bool FILT>
__device__ __forceinline__ void race_group_m(const float (&l)[4], const float (&qv)[4], int32_t exclude, float cs,
                                             float shift, float inv_sum, float tau, uint32_t k0, uint32_t k1,
                                             uint32_t j, uint32_t b, int32_t G, float& best_key, int32_t& best_x) {
  const PhiloxOut o = philox4x32_10((uint32_t)G, j, b, 1u, k0, k1);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int32_t x = 4 * G + k;
    // a token below the filter threshold has p' = 0 (exp2(-inf) = 0)
    const float lk = FILT ? (l[k] >= tau ? l[k] : -INFINITY) : l[k];
    const float r = race_weight<MODE>(exp2_hw(fmaf(lk, cs, -shift)), qv[k], x, exclude, inv_sum);
    const float key = r * __builtin_amdgcn_rcpf(-__builtin_amdgcn_logf(race_uniform_f32(o.w[k])));
    const bool up = key > best_key;
    best_key = up ? key : best_key;
    best_x = up ? x : best_x;
  }
}

// The same with the mode and the filter chosen at run time (per-request path,
// output fallback); tau = -inf means no filter.
__device__ __forceinline__ void race_group(const float (&l)[4], const float (&qv)[4], int mode, int32_t exclude,
                                           float cs, float shift, float inv_sum, float tau, uint32_t k0, uint32_t k1,
                                           uint32_t j, uint32_t b, int32_t G, float& best_key, int32_t& best_x) {
  if (tau > -INFINITY) {
    if (mode == kModeResampleQ)
      race_group_m<kModeResampleQ, true>(l, qv, exclude, cs, shift, inv_sum, tau, k0, k1, j, b, G, best_key, best_x);
    else if (mode == kModeResampleOneHot)
      race_group_m<kModeResampleOneHot, true>(l, qv, exclude, cs, shift, inv_sum, tau, k0, k1, j, b, G, best_key,
                                              best_x);
    else
      race_group_m<kModeBonus, true>(l, qv, exclude, cs, shift, inv_sum, tau, k0, k1, j, b, G, best_key, best_x);
  } else if (mode == kModeResampleQ) {
    race_group_m<kModeResampleQ, false>(l, qv, exclude, cs, shift, inv_sum, tau, k0, k1, j, b, G, best_key, best_x);
  } else if (mode == kModeResampleOneHot) {
    race_group_m<kModeResampleOneHot, false>(l, qv, exclude, cs, shift, inv_sum, tau, k0, k1, j, b, G, best_key,
                                             best_x);
  } else {
    race_group_m<kModeBonus, false>(l, qv, exclude, cs, shift, inv_sum, tau, k0, k1, j, b, G, best_key, best_x);
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

// Groups G0 + tid + i * kRaceThreads (i < TPT / 4) of one row.  FULL: every
// group lies below Gfull (vector-loadable), so loads and arithmetic run
// unguarded and the loads can be waited on one at a time.
template <typename Elem, int TPT, int MODE, bool FILT, bool FULL, bool PRIO>
__device__ __forceinline__ void race_span(const Elem* __restrict__ lrow, const float* __restrict__ qrow, int32_t V,
                                          int32_t G0, int32_t Gfull, int32_t Gend, int32_t exclude, float cs,
                                          float shift, float inv_sum, float tau, uint32_t k0, uint32_t k1, uint32_t j,
                                          uint32_t b, float& best_key, int32_t& best_x) {
  constexpr int NG = TPT / 4;
  constexpr bool kQ = MODE == kModeResampleQ;
  using R4 = Raw4<Elem>;
  const int tid = threadIdx.x;
  typename R4::T lw[NG];
  float4 qw[NG];
  // Issue every load of this thread before any arithmetic (PRIO: at raised
  // issue priority, back to the default for the arithmetic).
  if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int32_t G = G0 + tid + i * kRaceThreads;
    if (FULL || G < Gfull) {
      lw[i] = stream_load(reinterpret_cast<const typename R4::T*>(lrow) + G);
      if (kQ) qw[i] = stream_load(reinterpret_cast<const float4*>(qrow) + G);
    }
  }
  if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int32_t G = G0 + tid + i * kRaceThreads;
    float l[4], qv[4] = {0.f, 0.f, 0.f, 0.f};
    if (FULL || G < Gfull) {
      R4::unpack(lw[i], l);
      if (kQ) {
        qv[0] = qw[i].x;
        qv[1] = qw[i].y;
        qv[2] = qw[i].z;
        qv[3] = qw[i].w;
      }
    } else if (G < Gend) {
      load_group_scalar(lrow, kQ ? qrow : nullptr, G, V, l, qv);
    } else {
      continue;
    }
    race_group_m<MODE, FILT>(l, qv, exclude, cs, shift, inv_sum, tau, k0, k1, j, b, G, best_key, best_x);
  }
}

template <typename Elem, int TPT, int MODE, bool FILT, bool PRIO>
__device__ __forceinline__ unsigned long long race_chunk_m(const Elem* __restrict__ logits,
                                                           const float* __restrict__ q, int32_t V, uint64_t seed,
                                                           const ReqRecord& rec, int32_t b, int32_t c) {
  constexpr int NG = TPT / 4;  // groups of four tokens per thread
  using R4 = Raw4<Elem>;
  __shared__ unsigned long long lds_u[kRaceThreads / 64];
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const Elem* lrow = logits + (int64_t)rec.row * V;
  const float* qrow = MODE == kModeResampleQ ? q + ((int64_t)rec.slot0 + rec.n) * V : nullptr;
  // Vector loads need 8 / 16-byte aligned rows; otherwise every group goes element-wise.
  const bool fast = ((uintptr_t)lrow % sizeof(typename R4::T)) == 0 && ((uintptr_t)qrow % 16) == 0;
  const int32_t G0 = c * (kRaceThreads * NG);
  const int32_t Gend = (V + 3) / 4;
  const int32_t Gfull = fast ? V / 4 : 0;  // groups loaded as vectors
  float best_key = 0.f;
  int32_t best_x = INT_MAX;
  if (G0 + kRaceThreads * NG <= Gfull)
    race_span<Elem, TPT, MODE, FILT, true, PRIO>(lrow, qrow, V, G0, Gfull, Gend, rec.exclude, rec.c, rec.shift,
                                           rec.inv_sum, rec.tau, k0, k1, (uint32_t)rec.n, (uint32_t)b, best_key,
                                           best_x);
  else
    race_span<Elem, TPT, MODE, FILT, false, PRIO>(lrow, qrow, V, G0, Gfull, Gend, rec.exclude, rec.c, rec.shift,
                                            rec.inv_sum, rec.tau, k0, k1, (uint32_t)rec.n, (uint32_t)b, best_key,
                                            best_x);
  return block_reduce<kRaceThreads>(pack_key(best_key, best_x), lds_u, MaxOp());
}

// One workgroup races chunk c (kRaceThreads * TPT tokens) of request b's
// sampled row described by `rec` and returns the packed best of the chunk
// (0 = no positive key) in every thread.
template <typename Elem, int TPT, bool PRIO = false>
__device__ __forceinline__ unsigned long long race_chunk(const Elem* __restrict__ logits, const float* __restrict__ q,
                                                         int32_t V, uint64_t seed, const ReqRecord& rec, int32_t b,
                                                         int32_t c) {
  if (rec.tau > -INFINITY) {  // filtered target distribution (top-k / top-p)
    if (rec.mode == kModeResampleQ)
      return race_chunk_m<Elem, TPT, kModeResampleQ, true, PRIO>(logits, q, V, seed, rec, b, c);
    if (rec.mode == kModeResampleOneHot)
      return race_chunk_m<Elem, TPT, kModeResampleOneHot, true, PRIO>(logits, q, V, seed, rec, b, c);
    return race_chunk_m<Elem, TPT, kModeBonus, true, PRIO>(logits, q, V, seed, rec, b, c);
  }
  if (rec.mode == kModeResampleQ) return race_chunk_m<Elem, TPT, kModeResampleQ, false, PRIO>(logits, q, V, seed, rec, b, c);
  if (rec.mode == kModeResampleOneHot)
    return race_chunk_m<Elem, TPT, kModeResampleOneHot, false, PRIO>(logits, q, V, seed, rec, b, c);
  return race_chunk_m<Elem, TPT, kModeBonus, false, PRIO>(logits, q, V, seed, rec, b, c);
}

// Output of one request, by wavefront 0 of the workgroup that raced its last
// chunk (stream path): reduce the chunk winners, read through coherent loads,
// and write the output row.  If every residual value rounded to zero
// (possible only through rounding), race over p at the same row instead.
template <typename Elem>
__device__ __forceinline__ void finish_request(const Elem* __restrict__ logits, const int32_t* __restrict__ draft,
                                               int32_t max_k, int32_t V, int32_t nchunks, uint64_t seed,
                                               const ReqRecord& rec, int32_t b,
                                               const unsigned long long* __restrict__ cand,
                                               int32_t* __restrict__ out, int32_t* __restrict__ num_accepted) {
  const int lane = threadIdx.x & 63;
  unsigned long long win = 0ull;
  for (int32_t c = lane; c < nchunks; c += 64) {
    const unsigned long long v = load_coherent(cand + (int64_t)b * nchunks + c);
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
      race_group(l, qz, kModeBonus, -1, rec.c, rec.shift, rec.inv_sum, rec.tau, (uint32_t)seed, (uint32_t)(seed >> 32),
                 (uint32_t)rec.n, (uint32_t)b, G, bk, bx);
    }
    win = wave_max(pack_key(bk, bx));
  }
  const int32_t token = unpack_token(win);
  int32_t* ob = out + (int64_t)b * (max_k + 1);
  if (lane <= max_k) ob[lane] = lane < rec.n ? draft[rec.slot0 + lane] : (lane == rec.n ? token : -1);
  if (lane == 0) num_accepted[b] = rec.n;
}


}  // namespace rsv
