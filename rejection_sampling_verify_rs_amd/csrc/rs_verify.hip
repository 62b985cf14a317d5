// rs_verify.hip -- gfx950 kernels and C ABI of the batched speculative-
// sampling verify step (see include/rs_verify.h for the contract).
//
// One call runs three kernels on the caller's stream:
//
//  1. row pass   one workgroup per (request, position, V-chunk).  Streams the
//                chunk of target logits with 16-byte loads into registers,
//                takes the chunk maximum, then (random requests) the sum of
//                exp2(l * c - shift) with c = log2(e) / T and shift = fl(m * c),
//                accumulated per 16-byte vector in fp32 and across vectors in
//                fp64; greedy requests take the lowest-index argmax instead.
//                Writes a 16-byte partial per chunk.
//                [p = softmax(l / T): 第12章 投机解码：以小博大 §12.2.3, §12.9]
//  2. scan       one wavefront per request, one lane per position.  Merges
//                the chunk partials, gathers l(x*) and q(x*), evaluates the
//                accept test u * q(x*) < p(x*) in fp64 (greedy: x* == argmax),
//                takes the first rejection with a ballot and writes either
//                the final output (greedy) or a sampling record.
//                [§12.2.1; 投机解码（Speculative Decoding）端到端深挖 §7.3, §7.1;
//                 vllm v1 源码精读（五） §7]
//  3. race       one workgroup per (request, V-chunk) on the single row each
//                random request samples from: the exponential race
//                argmax_x r(x) / E_x with r = max(0, p - q) (one-hot q: p
//                without x*) at the first rejection, r = p at the bonus row.
//                Chunk winners merge through a 64-bit atomicMax on
//                (key bits, ~x); the last workgroup of a request writes its
//                output row.  [§12.2.1 step 3; §12.3.2; §12.9 last bullet]
//
// All accesses are bounded by the host-checked sizes; requests with
// out-of-range metadata are written as invalid instead of being read.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <climits>

#include "philox.hpp"
#include "rs_verify.h"

namespace rsv {

constexpr int kRowThreads = 256;
constexpr int kScanThreads = 64;
constexpr int kRaceThreads = 256;
constexpr size_t kRegionAlign = 256;
constexpr int kTargetBlocks = 2048;  // enough workgroups to fill 256 CUs several times

enum Mode : int32_t { kModeDone = 0, kModeResampleQ = 1, kModeResampleOneHot = 2, kModeBonus = 3 };

// Per (row, chunk) statistics.  Random rows: shift = fl32(m * c) and
// sum = sum_x exp2(fl32(l_x * c - shift)).  Greedy rows: shift = chunk max of
// the raw logits and argmax = lowest index holding it (-1 for an empty chunk).
struct RowPartial {
  float shift;
  int32_t argmax;
  double sum;
};
static_assert(sizeof(RowPartial) == 16, "RowPartial layout");

// What the race needs for one random request.
struct ReqRecord {
  int32_t mode;
  int32_t n;       // accepted drafts
  int32_t row;     // logits row sampled from
  int32_t slot0;   // cu[b]
  float c;         // log2(e) / T
  float shift;     // merged shift of that row
  float inv_sum;   // 1 / sum, rounded to fp32
  int32_t exclude; // draft id excluded from a one-hot residual, else -1
};
static_assert(sizeof(ReqRecord) == 32, "ReqRecord layout");

// ------------------------------------------------------------------ helpers
__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ float to_f32(float v) { return v; }

// The W values of one 16-byte vector.
template <typename Elem>
struct Vec;
template <>
struct Vec<uint16_t> {
  static constexpr int W = 8;
  static __device__ __forceinline__ float get(const uint4& v, int k) {
    const uint32_t w = (k < 2) ? v.x : (k < 4) ? v.y : (k < 6) ? v.z : v.w;
    return (k & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
  }
};
template <>
struct Vec<float> {
  static constexpr int W = 4;
  static __device__ __forceinline__ float get(const uint4& v, int k) {
    const uint32_t w = (k == 0) ? v.x : (k == 1) ? v.y : (k == 2) ? v.z : v.w;
    return __uint_as_float(w);
  }
};

// c = log2(e) / T, rounded once to fp32.  Shared by every kernel so the row
// pass, the accept test and the race use the same scale.
__device__ __forceinline__ float scale_of(float T) { return (float)(1.4426950408889634 / (double)T); }

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const T w = __shfl_xor(v, o);
    v = w > v ? w : v;
  }
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_min(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const T w = __shfl_xor(v, o);
    v = w < v ? w : v;
  }
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Block-wide reductions for NT threads (NT / 64 waves), result in every thread.
template <int NT, typename T, typename Op>
__device__ __forceinline__ T block_reduce(T v, T* lds, Op op) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = op(v);
  if (NW == 1) return v;
  __syncthreads();
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  T r = lds[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    const T w = lds[i];
    r = op.combine(r, w);
  }
  return r;
}
struct MaxOp {
  template <typename T>
  __device__ T operator()(T v) const { return wave_max(v); }
  template <typename T>
  __device__ T combine(T a, T b) const { return b > a ? b : a; }
};
struct MinOp {
  template <typename T>
  __device__ T operator()(T v) const { return wave_min(v); }
  template <typename T>
  __device__ T combine(T a, T b) const { return b < a ? b : a; }
};
struct SumOp {
  template <typename T>
  __device__ T operator()(T v) const { return wave_sum(v); }
  template <typename T>
  __device__ T combine(T a, T b) const { return a + b; }
};

__device__ __forceinline__ bool request_valid(int32_t s, int32_t e, int32_t D, int32_t max_k) {
  return s >= 0 && s <= e && e <= D && e - s <= max_k;
}

// ------------------------------------------------------------- 1. row pass
// Statistics of the NV vectors a thread holds: chunk max (phase 1), then the
// exp-sum (random) or the lowest index of the block max (greedy).  FULL
// instantiations (every vector in range) carry no per-vector guards.
template <typename Elem, int NV, bool FULL>
__device__ __forceinline__ float chunk_max(const uint4 (&data)[NV], int v0, int tid, int nvec, float m) {
  using VT = Vec<Elem>;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (FULL || v0 + tid + i * kRowThreads < nvec) {
#pragma unroll
      for (int k = 0; k < VT::W; ++k) m = fmaxf(m, VT::get(data[i], k));
    }
  }
  return m;
}

template <typename Elem, int NV, bool FULL>
__device__ __forceinline__ double chunk_expsum(const uint4 (&data)[NV], int v0, int tid, int nvec, float cs,
                                               float shift) {
  using VT = Vec<Elem>;
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (FULL || v0 + tid + i * kRowThreads < nvec) {
      float sv = exp2_hw(fmaf(VT::get(data[i], 0), cs, -shift));
#pragma unroll
      for (int k = 1; k < VT::W; ++k) sv += exp2_hw(fmaf(VT::get(data[i], k), cs, -shift));
      acc += (double)sv;
    }
  }
  return acc;
}

template <typename Elem, int NV, bool FULL>
__device__ __forceinline__ int chunk_argmax(const uint4 (&data)[NV], int v0, int tid, int nvec, int head, float m) {
  using VT = Vec<Elem>;
  int idx = INT_MAX;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = v0 + tid + i * kRowThreads;
    if (FULL || v < nvec) {
#pragma unroll
      for (int k = 0; k < VT::W; ++k)
        if (VT::get(data[i], k) == m) idx = min(idx, head + v * VT::W + k);
    }
  }
  return idx;
}

// Grid: nsplit * (max_k + 1) * B workgroups, chunk fastest, then position,
// then request, so consecutive workgroups stream consecutive memory.
template <typename Elem, int NV>
__global__ __launch_bounds__(kRowThreads) void row_pass_kernel(
    const Elem* __restrict__ logits, const int32_t* __restrict__ cu, const float* __restrict__ temperature,
    int32_t greedy_all, int32_t D, int32_t max_k, int32_t V, int32_t nsplit, RowPartial* __restrict__ partials) {
  using VT = Vec<Elem>;
  constexpr int W = VT::W;
  __shared__ float lds_f[kRowThreads / 64];
  __shared__ int lds_i[kRowThreads / 64];
  __shared__ double lds_d[kRowThreads / 64];

  const int32_t bid = blockIdx.x;
  const int32_t c = bid % nsplit;
  const int32_t rest = bid / nsplit;
  const int32_t j = rest % (max_k + 1);
  const int32_t b = rest / (max_k + 1);
  const int32_t s = cu[b], e = cu[b + 1];
  if (!request_valid(s, e, D, max_k) || j > e - s) return;
  const int64_t row = (int64_t)s + b + j;
  const float T = greedy_all ? 0.f : temperature[b];
  const bool greedy = !(T > 0.f);
  const float cs = greedy ? 0.f : scale_of(T);

  // Split the row into an unaligned head, 16-byte vectors and a tail.
  const Elem* prow = logits + row * (int64_t)V;
  int head = (int)(((16u - ((uint32_t)(uintptr_t)prow & 15u)) & 15u) / sizeof(Elem));
  if (head > V) head = V;
  const int nvec = (V - head) / W;
  const int tail = V - head - nvec * W;
  const uint4* pv = reinterpret_cast<const uint4*>(prow + head);
  const int v0 = c * NV * kRowThreads;
  const int tid = threadIdx.x;
  // Full chunks (all but a row's last) run the unguarded instantiations.
  const bool full = v0 + NV * kRowThreads <= nvec;

  uint4 data[NV];
  if (full) {
#pragma unroll
    for (int i = 0; i < NV; ++i) data[i] = pv[v0 + tid + i * kRowThreads];
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = v0 + tid + i * kRowThreads;
      if (v < nvec) data[i] = pv[v];
    }
  }
  float extra = -INFINITY;
  int extra_idx = INT_MAX;
  if (c == 0) {
    if (tid < head) {
      extra = to_f32(prow[tid]);
      extra_idx = tid;
    } else if (tid >= 8 && tid - 8 < tail) {
      extra_idx = head + nvec * W + (tid - 8);
      extra = to_f32(prow[extra_idx]);
    }
  }

  // Phase 1: chunk maximum.
  float m = full ? chunk_max<Elem, NV, true>(data, v0, tid, nvec, extra)
                 : chunk_max<Elem, NV, false>(data, v0, tid, nvec, extra);
  m = block_reduce<kRowThreads>(m, lds_f, MaxOp());

  RowPartial* out = partials + row * nsplit + c;
  if (greedy) {
    int idx = INT_MAX;
    if (m > -INFINITY) {
      idx = full ? chunk_argmax<Elem, NV, true>(data, v0, tid, nvec, head, m)
                 : chunk_argmax<Elem, NV, false>(data, v0, tid, nvec, head, m);
      if (extra == m) idx = min(idx, extra_idx);
    }
    idx = block_reduce<kRowThreads>(idx, lds_i, MinOp());
    if (tid == 0) {
      RowPartial p;
      p.shift = m;
      p.argmax = (idx == INT_MAX) ? -1 : idx;
      p.sum = 0.0;
      *out = p;
    }
    return;
  }

  // Phase 2: sum of exp2(l * c - shift) with shift = fl32(m * c).
  const float shift = (m > -INFINITY) ? m * cs : -INFINITY;
  double acc = 0.0;
  if (m > -INFINITY) {
    acc = full ? chunk_expsum<Elem, NV, true>(data, v0, tid, nvec, cs, shift)
               : chunk_expsum<Elem, NV, false>(data, v0, tid, nvec, cs, shift);
    if (extra_idx != INT_MAX) acc += (double)exp2_hw(fmaf(extra, cs, -shift));
  }
  acc = block_reduce<kRowThreads>(acc, lds_d, SumOp());
  if (tid == 0) {
    RowPartial p;
    p.shift = shift;
    p.argmax = -1;
    p.sum = acc;
    *out = p;
  }
}

// Merge the nsplit partials of one random row: common shift and fp64 sum.
__device__ __forceinline__ void merge_random(const RowPartial* P, int nsplit, float& shift, double& S) {
  float sh = -INFINITY;
  for (int c = 0; c < nsplit; ++c) sh = fmaxf(sh, P[c].shift);
  double acc = 0.0;
  for (int c = 0; c < nsplit; ++c)
    if (P[c].sum > 0.0) acc += P[c].sum * exp2((double)P[c].shift - (double)sh);
  shift = sh;
  S = acc;
}

// Merge the partials of one greedy row: global max, lowest index holding it.
__device__ __forceinline__ int32_t merge_greedy(const RowPartial* P, int nsplit) {
  float m = -INFINITY;
  int32_t idx = INT_MAX;
  for (int c = 0; c < nsplit; ++c) {
    const float v = P[c].shift;
    const int32_t a = P[c].argmax;
    if (a < 0) continue;
    if (v > m || (v == m && a < idx)) {
      if (v > m) m = v;
      idx = a;
    }
  }
  return idx == INT_MAX ? -1 : idx;
}

// ------------------------------------------------------------------ 2. scan
// Decide one request with one wavefront; lane j handles draft position j
// (K_b <= 32 < 64).  Merges the chunk partials, gathers l(x*) and q(x*), runs
// the accept test in fp64 (greedy: x* == argmax) and takes the first rejection
// with a ballot.  Greedy and invalid requests get their output row written
// here and mode kModeDone; random requests get the record the race needs.
// Every lane returns the same record.
template <typename Elem>
__device__ __forceinline__ ReqRecord scan_request(
    int32_t b, const Elem* __restrict__ logits, const float* __restrict__ q, const int32_t* __restrict__ draft,
    const int32_t* __restrict__ cu, const float* __restrict__ temperature, int32_t greedy_all, int32_t D,
    int32_t max_k, int32_t V, int32_t nsplit, uint64_t seed, const RowPartial* __restrict__ partials,
    int32_t* __restrict__ out, int32_t* __restrict__ num_accepted, double* __restrict__ dbg_p) {
  const int lane = threadIdx.x & 63;
  const int32_t s = cu[b], e = cu[b + 1];
  const int32_t K = e - s;
  int32_t* ob = out + (int64_t)b * (max_k + 1);
  ReqRecord r;
  r.mode = kModeDone;
  bool valid = request_valid(s, e, D, max_k);
  int32_t x = -1;
  if (valid && lane < K) x = draft[s + lane];
  valid = valid && (__ballot(valid && lane < K && (x < 0 || x >= V)) == 0ull);
  if (!valid) {
    if (lane <= max_k) ob[lane] = -1;
    if (lane == 0) num_accepted[b] = -1;
    return r;
  }
  const float T = greedy_all ? 0.f : temperature[b];
  const bool greedy = !(T > 0.f);
  const float cs = greedy ? 0.f : scale_of(T);

  float shift = -INFINITY;
  double S = 0.0;
  int32_t amax = -1;
  bool accept = false;
  if (lane <= K) {
    const int64_t row = (int64_t)s + b + lane;
    const RowPartial* P = partials + row * nsplit;
    if (greedy) {
      amax = merge_greedy(P, nsplit);
      accept = (lane < K) && (x == amax);
      if (dbg_p && lane < K) dbg_p[s + lane] = __builtin_nan("");
    } else {
      merge_random(P, nsplit, shift, S);
      if (lane < K) {
        const double ls = (double)to_f32(logits[row * (int64_t)V + x]);
        const double ps = exp2(ls * (double)cs - (double)shift) / S;
        const double qs = q ? (double)q[((int64_t)s + lane) * (int64_t)V + x] : 1.0;
        const double u = accept_uniform(seed, b, lane);
        accept = u * qs < ps;
        if (dbg_p) dbg_p[s + lane] = ps;
      }
    }
  }
  const unsigned long long rej = __ballot(lane < K && !accept);
  const int n = rej ? (__ffsll((long long)rej) - 1) : K;
  const float shift_n = __shfl(shift, n);
  const double S_n = __shfl(S, n);
  const int32_t amax_n = __shfl(amax, n);
  const int32_t x_n = __shfl(x, n);

  if (greedy) {
    if (lane <= max_k) ob[lane] = lane < n ? x : (lane == n ? amax_n : -1);
    if (lane == 0) num_accepted[b] = n;
    return r;
  }
  r.mode = n < K ? (q ? kModeResampleQ : kModeResampleOneHot) : kModeBonus;
  r.n = n;
  r.row = s + b + n;
  r.slot0 = s;
  r.c = cs;
  r.shift = shift_n;
  r.inv_sum = (float)(1.0 / S_n);
  r.exclude = (n < K && !q) ? x_n : -1;
  return r;
}

// Split path, step 2: one wavefront per request writes the sampling record.
template <typename Elem>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    const Elem* __restrict__ logits, const float* __restrict__ q, const int32_t* __restrict__ draft,
    const int32_t* __restrict__ cu, const float* __restrict__ temperature, int32_t greedy_all, int32_t D,
    int32_t max_k, int32_t V, int32_t nsplit, uint64_t seed, const RowPartial* __restrict__ partials,
    ReqRecord* __restrict__ records, int32_t* __restrict__ out, int32_t* __restrict__ num_accepted,
    double* __restrict__ dbg_p) {
  const int32_t b = blockIdx.x;
  const ReqRecord r = scan_request(b, logits, q, draft, cu, temperature, greedy_all, D, max_k, V, nsplit, seed,
                                   partials, out, num_accepted, dbg_p);
  if (threadIdx.x == 0) records[b] = r;
}

// ------------------------------------------------------------------ 3. race
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
      // E' = -log2(U) = E / ln 2: the common factor does not move the argmax.
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

// Raw 4-token logits vector: 8 bytes of bf16 or 16 bytes of fp32.
template <typename Elem>
struct Raw4;
template <>
struct Raw4<uint16_t> {
  using T = uint2;
  static __device__ __forceinline__ void unpack(const uint2& v, float (&l)[4]) {
    l[0] = __uint_as_float(v.x << 16);
    l[1] = __uint_as_float(v.x & 0xFFFF0000u);
    l[2] = __uint_as_float(v.y << 16);
    l[3] = __uint_as_float(v.y & 0xFFFF0000u);
  }
};
template <>
struct Raw4<float> {
  using T = float4;
  static __device__ __forceinline__ void unpack(const float4& v, float (&l)[4]) {
    l[0] = v.x;
    l[1] = v.y;
    l[2] = v.z;
    l[3] = v.w;
  }
};

__device__ __forceinline__ unsigned long long pack_key(float key, int32_t x) {
  return key > 0.f ? (((unsigned long long)__float_as_uint(key) << 32) | (0xFFFFFFFFu - (uint32_t)x)) : 0ull;
}

// One workgroup per (request, chunk of 256 * TPT tokens).  Writes the chunk's
// packed best (key bits, ~x) to cand[b * nchunks + c]; 0 = no positive key.
template <typename Elem, int TPT>
__global__ __launch_bounds__(kRaceThreads) void race_kernel(const Elem* __restrict__ logits,
                                                            const float* __restrict__ q, int32_t V, int32_t nchunks,
                                                            uint64_t seed, const ReqRecord* __restrict__ records,
                                                            unsigned long long* __restrict__ cand) {
  constexpr int NG = TPT / 4;  // groups of four tokens per thread
  using R4 = Raw4<Elem>;
  __shared__ unsigned long long lds_u[kRaceThreads / 64];
  const int32_t c = blockIdx.x % nchunks;
  const int32_t b = blockIdx.x / nchunks;
  const ReqRecord rec = records[b];
  if (rec.mode == kModeDone) return;
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
  const unsigned long long packed = block_reduce<kRaceThreads>(pack_key(best_key, best_x), lds_u, MaxOp());
  if (tid == 0) cand[(int64_t)b * nchunks + c] = packed;
}

// ------------------------------------------------------------------ 4. emit
// One wavefront per random request: reduce the chunk winners and write the
// output row.  If every residual value rounded to zero (possible only through
// rounding), race over p at the same row instead.
template <typename Elem>
__global__ __launch_bounds__(64) void emit_kernel(const Elem* __restrict__ logits, const int32_t* __restrict__ draft,
                                                  int32_t max_k, int32_t V, int32_t nchunks, uint64_t seed,
                                                  const ReqRecord* __restrict__ records,
                                                  const unsigned long long* __restrict__ cand,
                                                  int32_t* __restrict__ out, int32_t* __restrict__ num_accepted) {
  const int32_t b = blockIdx.x;
  const int lane = threadIdx.x;
  const ReqRecord rec = records[b];
  if (rec.mode == kModeDone) return;
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
      race_group(l, qz, kModeBonus, -1, rec.c, rec.shift, rec.inv_sum, (uint32_t)seed, (uint32_t)(seed >> 32),
                 (uint32_t)rec.n, (uint32_t)b, G, bk, bx);
    }
    win = wave_max(pack_key(bk, bx));
  }
  const int32_t token = win ? (int32_t)(0xFFFFFFFFu - (uint32_t)(win & 0xFFFFFFFFull)) : -1;
  int32_t* ob = out + (int64_t)b * (max_k + 1);
  if (lane <= max_k) ob[lane] = lane < rec.n ? draft[rec.slot0 + lane] : (lane == rec.n ? token : -1);
  if (lane == 0) num_accepted[b] = rec.n;
}

// ------------------------------------------ per-request path (early exit)
// One workgroup of NT threads owns one request.  It walks the request's rows
// in order: a statistics pass over row j (block-wide max and exp-sum, or
// argmax for greedy requests), then the accept test of draft j; it stops at
// the first rejection, because rows after it cannot change the output (the
// drafts behind a rejected one are discarded).  It then races the sampled row
// (just streamed, so mostly served from the Infinity Cache) and writes the
// output row.  No state crosses workgroups, so no atomics, fences or extra
// launches are needed.
struct RowStats {
  float shift;     // fl32(max * c) (random) or max (greedy)
  int32_t argmax;  // greedy: lowest index of the max
  double sum;      // random: sum_x exp2(fl32(l_x * c - shift))
};

// Block-wide statistics of one row.  Each thread keeps its own running max,
// shift and fp64 sum across passes of NVP 16-byte vectors (rescaling its sum
// exactly when its max grows), then the workgroup merges them.
template <typename Elem, int NT, int NVP>
__device__ __forceinline__ RowStats row_stats(const Elem* __restrict__ prow, int32_t V, bool greedy, float cs,
                                              float* s_f, int* s_i, double* s_d) {
  using VT = Vec<Elem>;
  constexpr int W = VT::W;
  const int tid = threadIdx.x;
  int head = (int)(((16u - ((uint32_t)(uintptr_t)prow & 15u)) & 15u) / sizeof(Elem));
  if (head > V) head = V;
  const int nvec = (V - head) / W;
  const int tail = V - head - nvec * W;
  const uint4* pv = reinterpret_cast<const uint4*>(prow + head);

  float m = -INFINITY, sh = -INFINITY;
  double S = 0.0;
  int am = INT_MAX;
  for (int v0 = 0; v0 < nvec; v0 += NVP * NT) {
    uint4 d[NVP];
#pragma unroll
    for (int i = 0; i < NVP; ++i) {
      const int v = v0 + tid + i * NT;
      if (v < nvec) d[i] = pv[v];
    }
    float pm = -INFINITY;
#pragma unroll
    for (int i = 0; i < NVP; ++i) {
      if (v0 + tid + i * NT < nvec) {
#pragma unroll
        for (int k = 0; k < W; ++k) pm = fmaxf(pm, VT::get(d[i], k));
      }
    }
    if (greedy) {
      if (pm > m) {  // an equal max from an earlier pass has the lower index
        m = pm;
        am = INT_MAX;
#pragma unroll
        for (int i = 0; i < NVP; ++i) {
          const int v = v0 + tid + i * NT;
          if (v < nvec) {
#pragma unroll
            for (int k = 0; k < W; ++k)
              if (VT::get(d[i], k) == pm) am = min(am, head + v * W + k);
          }
        }
      }
    } else if (pm > -INFINITY) {
      if (pm > m) {
        const float nsh = pm * cs;
        if (S > 0.0) S *= exp2((double)sh - (double)nsh);
        sh = nsh;
        m = pm;
      }
#pragma unroll
      for (int i = 0; i < NVP; ++i) {
        if (v0 + tid + i * NT < nvec) {
          float sv = 0.f;
#pragma unroll
          for (int k = 0; k < W; ++k) sv += exp2_hw(fmaf(VT::get(d[i], k), cs, -sh));
          S += (double)sv;
        }
      }
    }
  }
  // unaligned head and tail elements
  int xi = -1;
  if (tid < head) xi = tid;
  else if (tid >= 8 && tid - 8 < tail) xi = head + nvec * W + (tid - 8);
  if (xi >= 0) {
    const float v = to_f32(prow[xi]);
    if (greedy) {
      if (v > m || (v == m && xi < am)) {
        m = v;
        am = xi;
      }
    } else if (v > -INFINITY) {
      if (v > m) {
        const float nsh = v * cs;
        if (S > 0.0) S *= exp2((double)sh - (double)nsh);
        sh = nsh;
        m = v;
      }
      S += (double)exp2_hw(fmaf(v, cs, -sh));
    }
  }
  RowStats r;
  if (greedy) {
    const float M = block_reduce<NT>(m, s_f, MaxOp());
    r.shift = M;
    const int idx = block_reduce<NT>((m == M && am != INT_MAX) ? am : INT_MAX, s_i, MinOp());
    r.argmax = idx == INT_MAX ? -1 : idx;
    r.sum = 0.0;
  } else {
    const float SH = block_reduce<NT>(sh, s_f, MaxOp());
    const double part = S > 0.0 ? S * exp2((double)sh - (double)SH) : 0.0;
    r.shift = SH;
    r.sum = block_reduce<NT>(part, s_d, SumOp());
    r.argmax = -1;
  }
  return r;
}

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
        race_group(l, qv, mode, exclude, cs, shift, inv_sum, k0, k1, j, b, G, best_key, best_x);
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

template <typename Elem, int NT>
__global__ __launch_bounds__(NT) void request_kernel(
    const Elem* __restrict__ logits, const float* __restrict__ q, const int32_t* __restrict__ draft,
    const int32_t* __restrict__ cu, const float* __restrict__ temperature, int32_t greedy_all, int32_t D,
    int32_t max_k, int32_t V, uint64_t seed, int32_t* __restrict__ out, int32_t* __restrict__ num_accepted,
    double* __restrict__ dbg_p) {
  constexpr int NW = NT / 64;
  constexpr int NVP = 8;  // 16-byte vectors per thread per statistics pass
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
    token = win ? (int32_t)(0xFFFFFFFFu - (uint32_t)(win & 0xFFFFFFFFull)) : -1;
  }
  if (tid <= max_k) ob[tid] = tid < n ? s_draft[tid] : (tid == n ? token : -1);
  if (tid == 0) num_accepted[b] = n;
}

// -------------------------------------------------- debug: full p per row
template <typename Elem>
__global__ __launch_bounds__(256) void probs_kernel(const Elem* __restrict__ logits, const int32_t* __restrict__ cu,
                                                    const float* __restrict__ temperature, int32_t D, int32_t max_k,
                                                    int32_t V, int32_t nsplit, const RowPartial* __restrict__ partials,
                                                    float* __restrict__ probs) {
  const int32_t j = blockIdx.x % (max_k + 1);
  const int32_t b = blockIdx.x / (max_k + 1);
  const int32_t s = cu[b], e = cu[b + 1];
  if (!request_valid(s, e, D, max_k) || j > e - s) return;
  const float T = temperature[b];
  if (!(T > 0.f)) return;
  const float cs = scale_of(T);
  const int64_t row = (int64_t)s + b + j;
  float shift;
  double S;
  merge_random(partials + row * nsplit, nsplit, shift, S);
  const float inv = (float)(1.0 / S);
  for (int32_t x = threadIdx.x; x < V; x += 256)
    probs[row * V + x] = exp2_hw(fmaf(to_f32(logits[row * V + x]), cs, -shift)) * inv;
}

// ---------------------------------------------------------------- host side
struct Plan {
  int esize, W, nvec_max;
  int nsplit_max;       // partial slots per row in the workspace
  int row_nv, nsplit;   // this launch
  int race_tpt, race_chunks;
  int race_chunks_max;  // candidate slots per request in the workspace
  bool per_request;     // one workgroup per request (early exit) instead of row pass + scan + race + emit
  int request_nt;       // threads per per-request workgroup
  size_t off_partials, off_records, off_cand, total;
};

static size_t align_up(size_t v) { return (v + kRegionAlign - 1) / kRegionAlign * kRegionAlign; }

static int nsplit_for(int nvec_max, int nv) {
  const int cv = nv * kRowThreads;
  const int n = (nvec_max + cv - 1) / cv;
  return n < 1 ? 1 : n;
}

// Sizes are assumed validated (B >= 1, V >= 1, 0 <= max_k <= 32, 0 <= D <= B * max_k).
static bool make_plan(int32_t B, int32_t D, int32_t max_k, int32_t V, rs_dtype dt, int force_nv, int force_tpt,
                      int force_path, Plan& p) {
  p.esize = dt == RS_BF16 ? 2 : 4;
  p.W = 16 / p.esize;
  p.nvec_max = V / p.W;
  p.nsplit_max = nsplit_for(p.nvec_max, 1);
  const int64_t R = (int64_t)D + B;
  if (force_nv) {
    p.row_nv = force_nv;
  } else {
    p.row_nv = 1;
    for (int nv : {16, 8, 4, 2}) {
      if (R * nsplit_for(p.nvec_max, nv) >= kTargetBlocks) {
        p.row_nv = nv;
        break;
      }
    }
  }
  p.nsplit = nsplit_for(p.nvec_max, p.row_nv);
  if (force_tpt) {
    p.race_tpt = force_tpt;
  } else {
    p.race_tpt = 4;
    for (int t : {32, 16, 8}) {
      const int64_t chunks = ((int64_t)V + kRaceThreads * t - 1) / (kRaceThreads * t);
      if ((int64_t)B * chunks >= kTargetBlocks) {
        p.race_tpt = t;
        break;
      }
    }
  }
  p.race_chunks = (int)(((int64_t)V + kRaceThreads * p.race_tpt - 1) / (kRaceThreads * p.race_tpt));
  p.race_chunks_max = (int)(((int64_t)V + kRaceThreads * 4 - 1) / (kRaceThreads * 4));
  // The split path is the default: it spreads every row across the whole GPU.
  // The per-request path (early exit inside one workgroup) is available on
  // request; it is limited by the serial row walk of the longest request.
  p.per_request = force_path == 1;
  p.request_nt = V >= 65536 ? 1024 : 256;
  p.off_partials = 0;
  p.off_records = align_up((size_t)R * p.nsplit_max * sizeof(RowPartial));
  p.off_cand = p.off_records + align_up((size_t)B * sizeof(ReqRecord));
  p.total = p.off_cand + align_up((size_t)B * p.race_chunks_max * sizeof(unsigned long long));
  // 1-D grids must stay below 2^31 workgroups.
  const int64_t row_blocks = (int64_t)p.nsplit * (max_k + 1) * B;
  const int64_t race_blocks = (int64_t)p.race_chunks * B;
  return row_blocks < INT32_MAX && race_blocks < INT32_MAX;
}

static bool sizes_ok(int32_t B, int32_t D, int32_t max_k, int32_t V) {
  return B >= 1 && V >= 1 && max_k >= 0 && max_k <= RS_MAX_SPEC_LEN && D >= 0 && (int64_t)D <= (int64_t)B * max_k;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

template <typename Elem>
static rs_status launch(const void* logits_v, const float* q, const int32_t* draft, const int32_t* cu,
                        const float* temperature, int greedy_all, int32_t B, int32_t D, int32_t max_k, int32_t V,
                        uint64_t seed, int32_t* out, int32_t* nacc, void* ws, const Plan& p, const rs_debug* dbg,
                        hipStream_t stream) {
  const Elem* logits = static_cast<const Elem*>(logits_v);
  char* w = static_cast<char*>(ws);
  RowPartial* partials = reinterpret_cast<RowPartial*>(w + p.off_partials);
  ReqRecord* records = reinterpret_cast<ReqRecord*>(w + p.off_records);
  unsigned long long* cand = reinterpret_cast<unsigned long long*>(w + p.off_cand);
  hipEvent_t* ev = dbg ? dbg->events : nullptr;

  double* dbg_p = dbg ? dbg->draft_target_prob : nullptr;
  if (ev && hipEventRecord(ev[0], stream) != hipSuccess) return RS_ERR_HIP;

  if (p.per_request && !(dbg && dbg->probs)) {
    // One workgroup per request: early-exit statistics, accept tests, race, output.
    if (p.request_nt == 1024)
      request_kernel<Elem, 1024><<<(unsigned)B, 1024, 0, stream>>>(logits, q, draft, cu, temperature, greedy_all, D,
                                                                  max_k, V, seed, out, nacc, dbg_p);
    else
      request_kernel<Elem, 256><<<(unsigned)B, 256, 0, stream>>>(logits, q, draft, cu, temperature, greedy_all, D,
                                                                max_k, V, seed, out, nacc, dbg_p);
    if (hipGetLastError() != hipSuccess) return RS_ERR_HIP;
    if (ev && (hipEventRecord(ev[1], stream) != hipSuccess || hipEventRecord(ev[2], stream) != hipSuccess))
      return RS_ERR_HIP;
  } else {
    // Split: row pass over every row, scan, chunked race, emit.
    const unsigned row_blocks = (unsigned)(p.nsplit * (max_k + 1) * B);
#define RS_ROW(NV)                                                                                        \
  case NV:                                                                                                \
    row_pass_kernel<Elem, NV><<<row_blocks, kRowThreads, 0, stream>>>(logits, cu, temperature, greedy_all, \
                                                                      D, max_k, V, p.nsplit, partials);   \
    break;
    switch (p.row_nv) {
      RS_ROW(1)
      RS_ROW(2)
      RS_ROW(4)
      RS_ROW(8)
      RS_ROW(16)
      default:
        return RS_ERR_INVALID_ARG;
    }
#undef RS_ROW
    if (hipGetLastError() != hipSuccess) return RS_ERR_HIP;
    if (ev && hipEventRecord(ev[1], stream) != hipSuccess) return RS_ERR_HIP;
    if (dbg && dbg->probs && !greedy_all) {
      probs_kernel<Elem><<<(unsigned)((max_k + 1) * B), 256, 0, stream>>>(logits, cu, temperature, D, max_k, V,
                                                                            p.nsplit, partials, dbg->probs);
      if (hipGetLastError() != hipSuccess) return RS_ERR_HIP;
    }
    scan_kernel<Elem><<<(unsigned)B, kScanThreads, 0, stream>>>(logits, q, draft, cu, temperature, greedy_all, D,
                                                                max_k, V, p.nsplit, seed, partials, records, out,
                                                                nacc, dbg_p);
    if (hipGetLastError() != hipSuccess) return RS_ERR_HIP;
    if (ev && hipEventRecord(ev[2], stream) != hipSuccess) return RS_ERR_HIP;
    if (!greedy_all) {
      const unsigned race_blocks = (unsigned)(p.race_chunks * B);
#define RS_RACE(TPT)                                                                                     \
  case TPT:                                                                                              \
    race_kernel<Elem, TPT><<<race_blocks, kRaceThreads, 0, stream>>>(logits, q, V, p.race_chunks, seed, records, \
                                                                     cand);                              \
    break;
      switch (p.race_tpt) {
        RS_RACE(4)
        RS_RACE(8)
        RS_RACE(16)
        RS_RACE(32)
        default:
          return RS_ERR_INVALID_ARG;
      }
#undef RS_RACE
      if (hipGetLastError() != hipSuccess) return RS_ERR_HIP;
      emit_kernel<Elem><<<(unsigned)B, 64, 0, stream>>>(logits, draft, max_k, V, p.race_chunks, seed, records, cand,
                                                        out, nacc);
      if (hipGetLastError() != hipSuccess) return RS_ERR_HIP;
    }
  }
  if (ev && hipEventRecord(ev[3], stream) != hipSuccess) return RS_ERR_HIP;
  return RS_OK;
}

static rs_status verify_impl(const void* logits, rs_dtype dt, const float* q, const int32_t* draft, const int32_t* cu,
                             const float* temperature, int greedy_all, int32_t B, int32_t D, int32_t max_k, int32_t V,
                             uint64_t seed, int32_t* out, int32_t* nacc, void* ws, size_t ws_bytes,
                             const rs_debug* dbg, hipStream_t stream) {
  // Every check below runs before the first HIP call.
  if (B < 0 || D < 0 || V < 1 || max_k < 0) return RS_ERR_INVALID_ARG;
  if (dt != RS_F32 && dt != RS_BF16) return RS_ERR_UNSUPPORTED;
  if (B == 0) return RS_OK;
  if (!sizes_ok(B, D, max_k, V)) return RS_ERR_INVALID_ARG;
  if (!logits || !cu || !out || !nacc || (D > 0 && !draft) || (!greedy_all && !temperature))
    return RS_ERR_INVALID_ARG;
  const size_t es = dt == RS_BF16 ? 2 : 4;
  if (!aligned(logits, es) || (q && !aligned(q, 4)) || !aligned(cu, 4) || !aligned(out, 4) || !aligned(nacc, 4) ||
      (draft && !aligned(draft, 4)) || (temperature && !aligned(temperature, 4)))
    return RS_ERR_UNSUPPORTED;
  if (dbg) {
    const int nv = dbg->row_vectors_per_thread, tpt = dbg->race_tokens_per_thread;
    if (!(nv == 0 || nv == 1 || nv == 2 || nv == 4 || nv == 8 || nv == 16)) return RS_ERR_INVALID_ARG;
    if (!(tpt == 0 || tpt == 4 || tpt == 8 || tpt == 16 || tpt == 32)) return RS_ERR_INVALID_ARG;
    if (dbg->sampling_path < 0 || dbg->sampling_path > 2) return RS_ERR_INVALID_ARG;
    if ((dbg->draft_target_prob && !aligned(dbg->draft_target_prob, 8)) || (dbg->probs && !aligned(dbg->probs, 4)))
      return RS_ERR_UNSUPPORTED;
  }
  Plan p;
  if (!make_plan(B, D, max_k, V, dt, dbg ? dbg->row_vectors_per_thread : 0, dbg ? dbg->race_tokens_per_thread : 0,
                 dbg ? dbg->sampling_path : 0, p))
    return RS_ERR_UNSUPPORTED;
  if (!ws || !aligned(ws, 16) || ws_bytes < p.total) return RS_ERR_WORKSPACE;
  if (dt == RS_BF16)
    return launch<uint16_t>(logits, q, draft, cu, temperature, greedy_all, B, D, max_k, V, seed, out, nacc, ws, p, dbg,
                            stream);
  return launch<float>(logits, q, draft, cu, temperature, greedy_all, B, D, max_k, V, seed, out, nacc, ws, p, dbg,
                       stream);
}

}  // namespace rsv

extern "C" {

size_t rs_verify_workspace_size(int32_t batch, int32_t total_draft_tokens, int32_t max_k, int32_t vocab,
                                rs_dtype logits_dtype) {
  if (logits_dtype != RS_F32 && logits_dtype != RS_BF16) return 0;
  if (batch == 0 && total_draft_tokens == 0 && vocab >= 1 && max_k >= 0 && max_k <= RS_MAX_SPEC_LEN) return 0;
  if (!rsv::sizes_ok(batch, total_draft_tokens, max_k, vocab)) return 0;
  rsv::Plan p;
  if (!rsv::make_plan(batch, total_draft_tokens, max_k, vocab, logits_dtype, 0, 0, 0, p)) return 0;
  return p.total;
}

rs_status rs_verify(const void* target_logits, rs_dtype logits_dtype, const float* draft_probs,
                    const int32_t* draft_token_ids, const int32_t* cu_num_draft_tokens, const float* temperature,
                    int32_t batch, int32_t total_draft_tokens, int32_t max_k, int32_t vocab, uint64_t seed,
                    int32_t* output_token_ids, int32_t* num_accepted, void* workspace, size_t workspace_bytes,
                    const rs_debug* debug, hipStream_t stream) {
  return rsv::verify_impl(target_logits, logits_dtype, draft_probs, draft_token_ids, cu_num_draft_tokens, temperature,
                          0, batch, total_draft_tokens, max_k, vocab, seed, output_token_ids, num_accepted, workspace,
                          workspace_bytes, debug, stream);
}

rs_status rs_verify_greedy(const void* target_logits, rs_dtype logits_dtype, const int32_t* draft_token_ids,
                           const int32_t* cu_num_draft_tokens, int32_t batch, int32_t total_draft_tokens,
                           int32_t max_k, int32_t vocab, int32_t* output_token_ids, int32_t* num_accepted,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return rsv::verify_impl(target_logits, logits_dtype, nullptr, draft_token_ids, cu_num_draft_tokens, nullptr, 1,
                          batch, total_draft_tokens, max_k, vocab, 0, output_token_ids, num_accepted, workspace,
                          workspace_bytes, nullptr, stream);
}

const char* rs_status_string(rs_status status) {
  switch (status) {
    case RS_OK:
      return "RS_OK";
    case RS_ERR_INVALID_ARG:
      return "RS_ERR_INVALID_ARG: invalid argument (NULL pointer, bad size or max_k)";
    case RS_ERR_UNSUPPORTED:
      return "RS_ERR_UNSUPPORTED: unsupported dtype, alignment or size";
    case RS_ERR_WORKSPACE:
      return "RS_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case RS_ERR_HIP:
      return "RS_ERR_HIP: a HIP launch or event call failed";
  }
  return "unknown rs_status";
}

int32_t rs_abi_version(void) { return RS_VERIFY_ABI_VERSION; }

}  // extern "C"
