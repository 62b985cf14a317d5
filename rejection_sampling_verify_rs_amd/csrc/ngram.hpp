// Batched n-gram (prompt lookup) draft proposer: one workgroup per request.
//
// For n = max_n down to min_n, the pattern is the context's last n tokens;
// the proposal is the k tokens after the leftmost earlier occurrence of the
// pattern (an occurrence ending before the pattern begins), fewer if the
// context ends first; k is capped by max_model_len - len(context); the first
// n that matches wins [第12章 投机解码：以小博大 §12.4.4].  The pages search with
// KMP on the CPU; here every start position is tested at once: thread by
// thread, end position e gets SL(e), the number of tokens ending at e that
// agree with the context's tail (capped at max_n), and an occurrence of the
// n-gram ends at e iff SL(e) >= n.  The smallest such e per n is an LDS
// atomic minimum, so the result is the leftmost occurrence, as with KMP.
// The first kernel writes padded proposals and counts; the second packs them
// into the flat, prefix-summed layout rs_verify takes.
#pragma once

#include "common.hpp"

namespace rsv {

constexpr int kNgramThreads = 256;
constexpr int kNgramMaxN = 64;
constexpr int kNgramBatch = 16;  // context positions per thread whose tokens are loaded together

__global__ __launch_bounds__(kNgramThreads) void ngram_kernel(const int32_t* __restrict__ ctx,
                                                             const int32_t* __restrict__ cu, int32_t total,
                                                             int32_t min_n, int32_t max_n, int32_t k,
                                                             int64_t max_model_len, int32_t* __restrict__ padded,
                                                             int32_t* __restrict__ count) {
  __shared__ int32_t s_tail[kNgramMaxN];  // s_tail[t] = context[N - 1 - t]
  __shared__ int32_t s_best[kNgramMaxN + 1];
  const int32_t b = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t s = cu[b], e = cu[b + 1];
  int32_t* pb = padded + (int64_t)b * k;
  const bool valid = s >= 0 && s <= e && e <= total;
  const int32_t N = valid ? e - s : 0;
  const int64_t keff64 = (int64_t)k < max_model_len - N ? (int64_t)k : max_model_len - N;
  const int32_t keff = keff64 > 0 ? (int32_t)keff64 : 0;
  if (tid < k) pb[tid] = -1;
  if (keff == 0 || N < 2 * min_n) {
    if (tid == 0) count[b] = 0;
    return;
  }
  const int32_t* c = ctx + s;
  if (tid < max_n) s_tail[tid] = tid < N ? c[N - 1 - tid] : -1;
  if (tid <= max_n) s_best[tid] = INT_MAX;
  __syncthreads();
  // End positions e in [min_n - 1, N - min_n - 1].  The token at each of a
  // thread's kNgramBatch positions is loaded first, all in flight together;
  // only a position whose token equals the context's last one reads further
  // back (a chain of dependent loads per position was the kernel's latency).
  const int32_t last_pos = N - min_n - 1;
  const int32_t t0 = s_tail[0];
  for (int32_t base = min_n - 1 + tid; base <= last_pos; base += kNgramThreads * kNgramBatch) {
    int32_t tok[kNgramBatch];
#pragma unroll
    for (int i = 0; i < kNgramBatch; ++i) {
      const int32_t pos = base + i * kNgramThreads;
      tok[i] = pos <= last_pos ? c[pos] : ~t0;
    }
#pragma unroll
    for (int i = 0; i < kNgramBatch; ++i) {
      const int32_t pos = base + i * kNgramThreads;
      if (pos > last_pos || tok[i] != t0) continue;
      int32_t sl = 1;
      while (sl < max_n && pos - sl >= 0 && c[pos - sl] == s_tail[sl]) ++sl;
      // n-grams of every length n <= sl end at pos; each also needs pos <= N - n - 1
      const int32_t top = min(sl, N - 1 - pos);
      for (int32_t n = min_n; n <= top; ++n) atomicMin(s_best + n, pos);
    }
  }
  __syncthreads();
  if (tid == 0) {
    int32_t end = -1;
    for (int32_t n = max_n; n >= min_n && end < 0; --n)
      if (s_best[n] != INT_MAX) end = s_best[n];
    const int32_t cnt = end < 0 ? 0 : min(keff, N - 1 - end);
    s_best[0] = end;
    count[b] = cnt;
    s_tail[0] = cnt;  // reuse: broadcast the count
  }
  __syncthreads();
  const int32_t end = s_best[0], cnt = s_tail[0];
  if (tid < cnt) pb[tid] = c[end + 1 + tid];
}

// One workgroup: cu_out = prefix sums of count, then flat[cu_out[b] + i] =
// padded[b, i] for i < count[b].
__global__ __launch_bounds__(1024) void ngram_pack_kernel(const int32_t* __restrict__ padded,
                                                         const int32_t* __restrict__ count, int32_t B, int32_t k,
                                                         int32_t* __restrict__ flat, int32_t* __restrict__ cu_out) {
  __shared__ int32_t s_part[16];
  __shared__ int32_t s_carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    s_carry = 0;
    cu_out[0] = 0;
  }
  __syncthreads();
  for (int32_t b0 = 0; b0 < B; b0 += 1024) {
    const int32_t b = b0 + tid;
    const int32_t v = b < B ? count[b] : 0;
    int32_t inc = v;  // inclusive scan over the wave, then over the waves
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t t = __shfl_up(inc, o);
      if (lane >= o) inc += t;
    }
    if (lane == 63) s_part[wave] = inc;
    __syncthreads();
    int32_t base = s_carry;
    for (int w = 0; w < wave; ++w) base += s_part[w];
    const int32_t start = base + inc - v;
    if (b < B) {
      cu_out[b + 1] = start + v;
      for (int32_t i = 0; i < v; ++i) flat[start + i] = padded[(int64_t)b * k + i];
    }
    __syncthreads();
    if (tid == 1023) s_carry = start + v;
    __syncthreads();
  }
}

}  // namespace rsv
