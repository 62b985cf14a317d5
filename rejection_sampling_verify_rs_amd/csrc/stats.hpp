// Running acceptance counters of verify steps.
//
// A serving engine exports, per verify step, the number of draft proposals
// (requests that proposed at least one draft -- a count of proposals, not of
// tokens), the draft tokens proposed, the draft tokens accepted and the
// accepted tokens per draft position [第12章 投机解码：以小博大 §12.7.5].  The
// acceptance rate is accepted / proposed (bonus excluded) and the acceptance
// length emitted tokens / verifies, every verify emitting its accepted drafts
// plus one extra token [投机解码（Speculative Decoding）端到端深挖 §13].  One
// verify is one request in one step; requests whose output is invalid
// (num_accepted = -1) are not counted.
//
// Layout of the int64 counters (kStatsScalars + RS_MAX_SPEC_LEN entries):
//   [0] draft proposals  [1] proposed draft tokens  [2] accepted draft tokens
//   [3] emitted tokens   [4] verifies               [5 + j] accepted at position j
#pragma once

#include "common.hpp"

namespace rsv {

constexpr int kStatsScalars = 5;
constexpr int kStatsThreads = 256;
constexpr int kStatsPositions = 32;

// One thread per request; per-position counts in LDS, scalars by workgroup
// reduction; one global atomic add per counter and workgroup.
__global__ __launch_bounds__(kStatsThreads) void stats_kernel(const int32_t* __restrict__ num_accepted,
                                                             const int32_t* __restrict__ cu, int32_t B,
                                                             unsigned long long* __restrict__ counters) {
  __shared__ unsigned int pos[kStatsPositions];
  __shared__ unsigned long long lds[kStatsThreads / 64];
  const int tid = threadIdx.x;
  const int32_t b = (int32_t)blockIdx.x * kStatsThreads + tid;
  if (tid < kStatsPositions) pos[tid] = 0u;
  __syncthreads();
  unsigned long long v[kStatsScalars] = {0ull, 0ull, 0ull, 0ull, 0ull};
  if (b < B) {
    const int32_t n = num_accepted[b];
    const int32_t K = cu[b + 1] - cu[b];
    if (n >= 0) {
      v[0] = K > 0 ? 1ull : 0ull;
      v[1] = (unsigned long long)(K > 0 ? K : 0);
      v[2] = (unsigned long long)n;
      v[3] = (unsigned long long)n + 1ull;
      v[4] = 1ull;
      for (int j = 0; j < n && j < kStatsPositions; ++j) atomicAdd(pos + j, 1u);
    }
  }
#pragma unroll
  for (int i = 0; i < kStatsScalars; ++i) v[i] = block_reduce<kStatsThreads>(v[i], lds, SumOp());
  __syncthreads();
  if (tid < kStatsScalars) {
    unsigned long long x = 0ull;
#pragma unroll
    for (int i = 0; i < kStatsScalars; ++i) x = (tid == i) ? v[i] : x;
    if (x) atomicAdd(counters + tid, x);
  } else if (tid >= 64 && tid < 64 + kStatsPositions) {
    const unsigned int c = pos[tid - 64];
    if (c) atomicAdd(counters + kStatsScalars + (tid - 64), (unsigned long long)c);
  }
}

}  // namespace rsv
