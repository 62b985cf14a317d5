// Shared types and wavefront / workgroup helpers of the verify kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <climits>

namespace rsv {

constexpr int kRowThreads = 256;   // row-pass and race workgroups
constexpr int kRaceThreads = 256;
static_assert(kRowThreads == kRaceThreads, "phase kernels mix row and race tasks in one grid");
constexpr int kScanThreads = 64;  // one wavefront per request

// Per-request state between kernels.
enum Mode : int32_t {
  kModeDone = 0,            // output row already written (greedy, invalid)
  kModeResampleQ = 1,       // race over max(0, p - q) at the first rejection
  kModeResampleOneHot = 2,  // race over p without the rejected draft (no q)
  kModeBonus = 3,           // race over p at the bonus row (all accepted)
  kModeActive = 4           // every position so far accepted; later rows still needed
};

// Per (row, V-chunk) statistics.  Random rows: shift = fl32(m * c) and
// sum = sum_x exp2(fl32(l_x * c - shift)).  Greedy rows: shift = chunk max of
// the raw logits and argmax = lowest index holding it (-1 for an empty chunk).
struct RowPartial {
  float shift;
  int32_t argmax;
  double sum;
};
static_assert(sizeof(RowPartial) == 16, "RowPartial layout");

// Per draft slot: l(x*) and q(x*), gathered by chunk 0 of the slot's row so
// the scan does not wait on them.
struct Gathered {
  float lstar;
  float qstar;
};

// What the race and the emit step need for one request.
struct ReqRecord {
  int32_t mode;     // Mode
  int32_t phase;    // phase in which the request was decided
  int32_t n;        // accepted drafts
  int32_t row;      // logits row sampled from
  int32_t slot0;    // cu[b]
  int32_t exclude;  // draft id excluded from a one-hot residual, else -1
  float c;          // log2(e) / T
  float shift;      // merged shift of the sampled row
  float inv_sum;    // 1 / sum of the sampled row, rounded to fp32
  float tau;        // tokens with logit < tau are filtered out (-inf: none)
  int32_t pad[2];
};
static_assert(sizeof(ReqRecord) == 48, "ReqRecord layout");

__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ float to_f32(float v) { return v; }

// The W values of one 16-byte vector of logits.
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

// Four consecutive logits as one load: 8 bytes of bf16 or 16 bytes of fp32.
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

// Streaming loads for data read once per call (logits rows, q rows): the
// non-temporal hint keeps them from displacing reused lines in the caches
// (measured on the verify stream: 127 -> 122 us per call at B=256 K=8
// V=151936).  Clang's builtin takes native vector types only.
typedef unsigned int stream_u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int stream_u32x4 __attribute__((ext_vector_type(4)));
typedef float stream_f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  const stream_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const stream_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 stream_load(const uint2* p) {
  const stream_u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const stream_u32x2*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ float4 stream_load(const float4* p) {
  const stream_f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const stream_f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// c = log2(e) / T, rounded once to fp32.  Every kernel uses this same scale
// so the statistics, the accept test and the race agree.
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

// Workgroup-wide reduction over NT threads (NT / 64 wavefronts) through
// NT / 64 LDS slots; every thread gets the result.  The leading barrier lets
// consecutive reductions reuse the same slots.
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
  for (int i = 1; i < NW; ++i) r = op.combine(r, lds[i]);
  return r;
}

__device__ __forceinline__ bool request_valid(int32_t s, int32_t e, int32_t D, int32_t max_k) {
  return s >= 0 && s <= e && e <= D && e - s <= max_k;
}

// Hand-off between workgroups of one kernel (the stream path).  Data is
// written with agent-scope atomic stores, which write through the XCD's L2 to
// the device-coherent level, and read back with agent-scope atomic loads,
// which do not hit a stale L2 line.  A producer waits until its stores have
// been acknowledged (s_waitcnt) before it bumps an arrival counter, and a
// consumer reads only after observing the counter or flag.  No L2 writeback
// or invalidate (a device fence) is needed, because nothing handed over this
// way sits in an L2 as a dirty or stale line.
__device__ __forceinline__ void store_coherent(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long load_coherent(const unsigned long long* p) {
  return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent32(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_coherent32(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long atomic_or64(unsigned long long* p, unsigned long long v) {
  return __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Compare-and-swap; true if *p held `expected` and now holds `desired`.
__device__ __forceinline__ bool atomic_cas32(int32_t* p, int32_t expected, int32_t desired) {
  return __hip_atomic_compare_exchange_strong(p, &expected, desired, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
}
// Wait for every memory access this wavefront has issued (stores included).
__device__ __forceinline__ void wait_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Arrival counter: true in exactly one caller, the last of `total`.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t total) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == total - 1u;
}

// Race keys order as unsigned integers: (fp32 bits of the positive key) << 32
// | ~x, so the maximum is the largest key and, among equal keys, the lowest x.
// 0 means "no positive key".
__device__ __forceinline__ unsigned long long pack_key(float key, int32_t x) {
  return key > 0.f ? (((unsigned long long)__float_as_uint(key) << 32) | (0xFFFFFFFFu - (uint32_t)x)) : 0ull;
}
__device__ __forceinline__ int32_t unpack_token(unsigned long long packed) {
  return packed ? (int32_t)(0xFFFFFFFFu - (uint32_t)(packed & 0xFFFFFFFFull)) : -1;
}

}  // namespace rsv
