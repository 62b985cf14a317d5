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

  uint4 data[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = v0 + tid + i * kRowThreads;
    if (v < nvec) data[i] = pv[v];
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
  float m = extra;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (v0 + tid + i * kRowThreads < nvec) {
#pragma unroll
      for (int k = 0; k < W; ++k) m = fmaxf(m, VT::get(data[i], k));
    }
  }
  m = block_reduce<kRowThreads>(m, lds_f, MaxOp());

  RowPartial* out = partials + row * nsplit + c;
  if (greedy) {
    int idx = INT_MAX;
    if (m > -INFINITY) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int v = v0 + tid + i * kRowThreads;
        if (v < nvec) {
#pragma unroll
          for (int k = 0; k < W; ++k)
            if (VT::get(data[i], k) == m) idx = min(idx, head + v * W + k);
        }
      }
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
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (v0 + tid + i * kRowThreads < nvec) {
        float sv = 0.f;
#pragma unroll
        for (int k = 0; k < W; ++k) sv += exp2_hw(fmaf(VT::get(data[i], k), cs, -shift));
        acc += (double)sv;
      }
    }
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
// One wavefront per request; lane j handles draft position j (K_b <= 32).
template <typename Elem>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    const Elem* __restrict__ logits, const float* __restrict__ q, const int32_t* __restrict__ draft,
    const int32_t* __restrict__ cu, const float* __restrict__ temperature, int32_t greedy_all, int32_t D,
    int32_t max_k, int32_t V, int32_t nsplit, uint64_t seed, const RowPartial* __restrict__ partials,
    ReqRecord* __restrict__ records, unsigned long long* __restrict__ slots, uint32_t* __restrict__ counters,
    int32_t* __restrict__ out, int32_t* __restrict__ num_accepted, double* __restrict__ dbg_p) {
  const int32_t b = blockIdx.x;
  const int lane = threadIdx.x;
  const int32_t s = cu[b], e = cu[b + 1];
  const int32_t K = e - s;
  int32_t* ob = out + (int64_t)b * (max_k + 1);
  bool valid = request_valid(s, e, D, max_k);
  int32_t x = -1;
  if (valid && lane < K) x = draft[s + lane];
  valid = valid && (__ballot(valid && lane < K && (x < 0 || x >= V)) == 0ull);
  if (!valid) {
    if (lane <= max_k) ob[lane] = -1;
    if (lane == 0) {
      num_accepted[b] = -1;
      records[b].mode = kModeDone;
    }
    return;
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
    if (lane == 0) {
      num_accepted[b] = n;
      records[b].mode = kModeDone;
    }
    return;
  }
  if (lane == 0) {
    ReqRecord r;
    r.mode = n < K ? (q ? kModeResampleQ : kModeResampleOneHot) : kModeBonus;
    r.n = n;
    r.row = s + b + n;
    r.slot0 = s;
    r.c = cs;
    r.shift = shift_n;
    r.inv_sum = (float)(1.0 / S_n);
    r.exclude = (n < K && !q) ? x_n : -1;
    records[b] = r;
    slots[b] = 0ull;
    counters[b] = 0u;
  }
}

// ------------------------------------------------------------------ 3. race
// Race over the four tokens 4G .. 4G+3 (those below V) of one group, keeping
// the thread's best (key, x).  Tokens are visited in increasing x, so '>'
// keeps the lowest index among equal keys.
template <typename Elem>
__device__ __forceinline__ void race_group(const Elem* __restrict__ lrow, const float* __restrict__ qrow,
                                           int mode, int32_t exclude, float cs, float shift, float inv_sum,
                                           uint32_t k0, uint32_t k1, uint32_t j, uint32_t b, int32_t G,
                                           int32_t V, float& best_key, int32_t& best_x) {
  const PhiloxOut o = philox4x32_10((uint32_t)G, j, b, 1u, k0, k1);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int32_t x = 4 * G + k;
    if (x < V) {
      const float ex = exp2_hw(fmaf(to_f32(lrow[x]), cs, -shift));
      float r;
      if (mode == kModeResampleQ)
        r = fmaxf(ex * inv_sum - qrow[x], 0.f);
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
}

__device__ __forceinline__ unsigned long long pack_key(float key, int32_t x) {
  return key > 0.f ? (((unsigned long long)__float_as_uint(key) << 32) | (0xFFFFFFFFu - (uint32_t)x)) : 0ull;
}

template <typename Elem, int TPT>
__global__ __launch_bounds__(kRaceThreads) void race_kernel(
    const Elem* __restrict__ logits, const float* __restrict__ q, const int32_t* __restrict__ draft,
    int32_t max_k, int32_t V, int32_t nchunks, uint64_t seed, const ReqRecord* __restrict__ records,
    unsigned long long* __restrict__ slots, uint32_t* __restrict__ counters, int32_t* __restrict__ out,
    int32_t* __restrict__ num_accepted) {
  __shared__ unsigned long long lds_u[kRaceThreads / 64];
  __shared__ int lds_last;
  const int32_t c = blockIdx.x % nchunks;
  const int32_t b = blockIdx.x / nchunks;
  const ReqRecord rec = records[b];
  if (rec.mode == kModeDone) return;
  const int tid = threadIdx.x;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const Elem* lrow = logits + (int64_t)rec.row * V;
  const float* qrow = (rec.mode == kModeResampleQ) ? q + ((int64_t)rec.slot0 + rec.n) * V : nullptr;
  const int32_t G0 = c * (kRaceThreads * TPT / 4);
  const int32_t Gend = (V + 3) / 4;

  float best_key = 0.f;
  int32_t best_x = INT_MAX;
#pragma unroll
  for (int i = 0; i < TPT / 4; ++i) {
    const int32_t G = G0 + tid + i * kRaceThreads;
    if (G < Gend)
      race_group(lrow, qrow, rec.mode, rec.exclude, rec.c, rec.shift, rec.inv_sum, k0, k1, (uint32_t)rec.n,
                 (uint32_t)b, G, V, best_key, best_x);
  }
  const unsigned long long packed = block_reduce<kRaceThreads>(pack_key(best_key, best_x), lds_u, MaxOp());
  if (tid == 0) {
    if (packed) atomicMax(&slots[b], packed);
    __threadfence();
    const uint32_t done = atomicAdd(&counters[b], 1u);
    lds_last = (done == (uint32_t)nchunks - 1u);
  }
  __syncthreads();
  if (!lds_last) return;

  // Last workgroup of this request: read the winner and write the output row.
  __threadfence();
  unsigned long long win = __hip_atomic_load(&slots[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (win == 0ull) {
    // Every residual value rounded to zero: race over p at the same row.
    float bk = 0.f;
    int32_t bx = INT_MAX;
    for (int32_t G = tid; G < Gend; G += kRaceThreads)
      race_group(lrow, nullptr, kModeBonus, -1, rec.c, rec.shift, rec.inv_sum, k0, k1, (uint32_t)rec.n,
                 (uint32_t)b, G, V, bk, bx);
    win = block_reduce<kRaceThreads>(pack_key(bk, bx), lds_u, MaxOp());
  }
  const int32_t token = win ? (int32_t)(0xFFFFFFFFu - (uint32_t)(win & 0xFFFFFFFFull)) : -1;
  int32_t* ob = out + (int64_t)b * (max_k + 1);
  for (int i = tid; i <= max_k; i += kRaceThreads)
    ob[i] = i < rec.n ? draft[rec.slot0 + i] : (i == rec.n ? token : -1);
  if (tid == 0) num_accepted[b] = rec.n;
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
  size_t off_partials, off_records, off_slots, off_counters, total;
};

static size_t align_up(size_t v) { return (v + kRegionAlign - 1) / kRegionAlign * kRegionAlign; }

static int nsplit_for(int nvec_max, int nv) {
  const int cv = nv * kRowThreads;
  const int n = (nvec_max + cv - 1) / cv;
  return n < 1 ? 1 : n;
}

// Sizes are assumed validated (B >= 1, V >= 1, 0 <= max_k <= 32, 0 <= D <= B * max_k).
static bool make_plan(int32_t B, int32_t D, int32_t max_k, int32_t V, rs_dtype dt, int force_nv, int force_tpt,
                      Plan& p) {
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
  p.off_partials = 0;
  p.off_records = align_up((size_t)R * p.nsplit_max * sizeof(RowPartial));
  p.off_slots = p.off_records + align_up((size_t)B * sizeof(ReqRecord));
  p.off_counters = p.off_slots + align_up((size_t)B * sizeof(unsigned long long));
  p.total = p.off_counters + align_up((size_t)B * sizeof(uint32_t));
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
  unsigned long long* slots = reinterpret_cast<unsigned long long*>(w + p.off_slots);
  uint32_t* counters = reinterpret_cast<uint32_t*>(w + p.off_counters);
  hipEvent_t* ev = dbg ? dbg->events : nullptr;

  if (ev && hipEventRecord(ev[0], stream) != hipSuccess) return RS_ERR_HIP;
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

  scan_kernel<Elem><<<(unsigned)B, kScanThreads, 0, stream>>>(
      logits, q, draft, cu, temperature, greedy_all, D, max_k, V, p.nsplit, seed, partials, records, slots, counters,
      out, nacc, dbg ? dbg->draft_target_prob : nullptr);
  if (hipGetLastError() != hipSuccess) return RS_ERR_HIP;
  if (ev && hipEventRecord(ev[2], stream) != hipSuccess) return RS_ERR_HIP;

  if (!greedy_all) {
    const unsigned race_blocks = (unsigned)(p.race_chunks * B);
#define RS_RACE(TPT)                                                                                          \
  case TPT:                                                                                                   \
    race_kernel<Elem, TPT><<<race_blocks, kRaceThreads, 0, stream>>>(logits, q, draft, max_k, V, p.race_chunks, \
                                                                     seed, records, slots, counters, out, nacc); \
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
    if ((dbg->draft_target_prob && !aligned(dbg->draft_target_prob, 8)) || (dbg->probs && !aligned(dbg->probs, 4)))
      return RS_ERR_UNSUPPORTED;
  }
  Plan p;
  if (!make_plan(B, D, max_k, V, dt, dbg ? dbg->row_vectors_per_thread : 0, dbg ? dbg->race_tokens_per_thread : 0, p))
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
  if (!rsv::make_plan(batch, total_draft_tokens, max_k, vocab, logits_dtype, 0, 0, p)) return 0;
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
