// Top-k / top-p filtering of the target distribution, one workgroup per row.
//
// Rejection sampling constrains the target distribution with the temperature,
// top-k and top-p before the accept test, the residual and the bonus
// [第12章 投机解码：以小博大 §12.2.3; §12.9 (compute_probs applies top-k / top-p
// per token)].  Reading of the tie rules (the pages name the step only):
//   top-k keeps x iff fewer than k tokens have a strictly larger logit;
//   top-p then keeps x iff the mass, under the top-k-filtered softmax, of the
//   tokens with a strictly larger logit is below top_p;
// so the kept set is {x : l_x >= tau} for one threshold logit tau per row, and
// p' = exp2(l c - shift) / S' on it, S' the kept mass.
//
// The kernel finds tau exactly by radix selection on order-preserving 32-bit
// keys of the logits (bf16 logits only use the upper 16 bits): a 4096-bin
// histogram of the top 12 key bits, then of the next 12 (then of the last 8
// for fp32), each time narrowing to the bin where the cumulative count (top-k)
// or mass (top-p) from the top reaches the target.  Histograms live in LDS;
// masses are fixed point (exp2 value scaled by 2^44, truncated, u64), so the
// selection is deterministic.  The row stays in registers between passes when
// it fits (1024 threads x kFilterResident 16-byte vectors), otherwise later
// passes re-read it.  The workgroup also gathers l(x*) and q(x*) for the
// accept test, so the row statistics pass skips filtered rows entirely.
#pragma once

#include "common.hpp"
#include "row_pass.hpp"

namespace rsv {

constexpr int kFilterThreads = 1024;
constexpr int kFilterBinBits = 12;
constexpr int kFilterBins = 1 << kFilterBinBits;  // 4 per thread
constexpr int kFilterResident = 16;               // 16-byte vectors per thread kept in registers

// Per-row result: keep l >= tau; shift = fl32(max * c); sum = S' (fp64).
struct FilterRec {
  float tau;
  float shift;
  double sum;
};
static_assert(sizeof(FilterRec) == 16, "FilterRec layout");

// Does request b filter its target distribution?  (Greedy requests ignore it.)
__device__ __forceinline__ bool filter_on(const int32_t* __restrict__ top_k, const float* __restrict__ top_p,
                                          int32_t b, int32_t V) {
  if (top_k) {
    const int32_t k = top_k[b];
    if (k > 0 && k < V) return true;
  }
  if (top_p) {
    const float p = top_p[b];
    if (p > 0.f && p < 1.f) return true;
  }
  return false;
}

// Order-preserving key: key(a) < key(b) iff a < b for non-NaN floats.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// The elements of one row as seen by one thread: resident vectors, vectors
// beyond them (re-read), and at most one unaligned head / tail element.
template <typename Elem>
struct FilterRow {
  const uint4* pv;
  int nvec;
  float extra;  // -inf when the thread has none (harmless for every pass below)
  bool has_extra;
  uint4 res[kFilterResident];

  template <typename F>
  __device__ __forceinline__ void visit(F&& f) const {
    using VT = Vec<Elem>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kFilterResident; ++i) {
      if (tid + i * kFilterThreads < nvec) {
#pragma unroll
        for (int k = 0; k < VT::W; ++k) f(VT::get(res[i], k));
      }
    }
    for (int v = tid + kFilterResident * kFilterThreads; v < nvec; v += kFilterThreads) {
      const uint4 x = pv[v];
#pragma unroll
      for (int k = 0; k < VT::W; ++k) f(VT::get(x, k));
    }
    if (has_extra) f(extra);
  }
};

// Fixed-point mass of one element: floor(e * 2^44), e = exp2(l c - shift) in
// [0, 1 + 2^-23]; a row of V < 2^19 such values sums below 2^63.
__device__ __forceinline__ unsigned long long fixed_mass(float e) {
  const float x = e * 0x1p+12f;  // integer part < 2^12 + 1, fraction on a 2^-32 grid or finer (truncated)
  const uint32_t hi = (uint32_t)x;
  const uint32_t lo = (uint32_t)((x - (float)hi) * 0x1p+32f);
  return ((unsigned long long)hi << 32) | lo;
}

// Find the bin B of hist[] (kFilterBins u64 weights) where, counting from the
// top bin down, base + (weight of the bins above B) < target <= base + (weight
// of the bins from B up).  Returns B and adds the weight above B to *base;
// -1 if the target exceeds the total.  Whole workgroup; thread t owns bins
// 4t .. 4t+3.  s_u64 needs kFilterThreads / 64 + 2 slots.
__device__ __forceinline__ int find_bin(const unsigned long long* hist, double target, unsigned long long& base,
                                        unsigned long long* s_u64, int* s_bin) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NW = kFilterThreads / 64;
  __syncthreads();  // earlier readers of s_u64 / s_bin are done
  unsigned long long h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = hist[4 * tid + i];
  const unsigned long long tot = h[0] + h[1] + h[2] + h[3];
  // suffix sums over the lanes of the wave, then over the waves
  unsigned long long suf = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long v = __shfl_down(suf, o);
    if (lane + o < 64) suf += v;
  }
  if (tid == 0) *s_bin = -1;
  if (lane == 0) s_u64[wave] = suf;
  __syncthreads();
  unsigned long long above = base + (suf - tot);
  for (int w = wave + 1; w < NW; ++w) above += s_u64[w];
#pragma unroll
  for (int i = 3; i >= 0; --i) {
    if ((double)above < target && (double)(above + h[i]) >= target) {
      *s_bin = 4 * tid + i;
      s_u64[NW] = above;
    }
    above += h[i];
  }
  __syncthreads();
  const int bin = *s_bin;
  if (bin >= 0) base = s_u64[NW];
  __syncthreads();  // s_u64 and s_bin are reused
  return bin;
}

// Total of hist[] (whole workgroup).
__device__ __forceinline__ unsigned long long hist_total(const unsigned long long* hist, unsigned long long* s_u64) {
  const int tid = threadIdx.x;
  unsigned long long t = hist[4 * tid] + hist[4 * tid + 1] + hist[4 * tid + 2] + hist[4 * tid + 3];
  return block_reduce<kFilterThreads>(t, s_u64, SumOp());
}

// Radix selection: the key kappa such that, over the elements with key >=
// kmin, weight(key > kappa) < target <= weight(key >= kappa), weights being 1
// (MASS = false) or the fixed-point mass.  With MASS and top_p > 0 the target
// is top_p times the total weight (taken from the first histogram).
template <typename Elem, bool MASS>
__device__ __forceinline__ uint32_t radix_select(const FilterRow<Elem>& row, uint32_t kmin, double target,
                                                 float top_p, float cs, float shift, unsigned long long* hist,
                                                 unsigned long long* s_u64, int* s_bin) {
  const int tid = threadIdx.x;
  constexpr int levels = sizeof(Elem) == 2 ? 2 : 3;  // bf16 keys end in 16 constant bits
  uint32_t prefix = 0, pmask = 0;
  unsigned long long base = 0;
#pragma unroll
  for (int lv = 0; lv < levels; ++lv) {
    const int sh = lv == 0 ? 20 : (lv == 1 ? 8 : 0);
    const uint32_t bmask = lv == 2 ? 0xFFu : (uint32_t)(kFilterBins - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[4 * tid + i] = 0ull;
    __syncthreads();
    row.visit([&](float l) {
      const uint32_t key = order_key(l);
      if (key >= kmin && (key & pmask) == prefix) {
        const unsigned long long w = MASS ? fixed_mass(exp2_hw(fmaf(l, cs, -shift))) : 1ull;
        if (w) atomicAdd(hist + ((key >> sh) & bmask), w);
      }
    });
    __syncthreads();
    if (MASS && lv == 0) target = (double)top_p * (double)hist_total(hist, s_u64);
    const int bin = find_bin(hist, target, base, s_u64, s_bin);
    if (bin < 0) return kmin;  // cannot happen for a target within the total; keep everything
    prefix |= (uint32_t)bin << sh;
    pmask |= bmask << sh;
  }
  if (levels == 2) prefix |= (prefix & 0x80000000u) ? 0u : 0xFFu;  // bf16: low bits follow the sign
  return prefix;
}

// One workgroup per (request, position) row of the positions [j_begin,
// j_begin + j_count) of every random request with a filter (and, after the
// first phase, still active): writes frec[row] and, for a draft position, the
// gathers l(x*), q(x*).
template <typename Elem>
__global__ __launch_bounds__(kFilterThreads) void filter_kernel(
    const Elem* __restrict__ logits, const float* __restrict__ q, const int32_t* __restrict__ draft,
    const int32_t* __restrict__ cu, const float* __restrict__ temperature, const int32_t* __restrict__ top_k,
    const float* __restrict__ top_p, int32_t D, int32_t max_k, int32_t V, int32_t j_begin, int32_t j_count,
    const ReqRecord* __restrict__ records, FilterRec* __restrict__ frec, Gathered* __restrict__ gath) {
  using VT = Vec<Elem>;
  constexpr int W = VT::W;
  __shared__ unsigned long long hist[kFilterBins];
  __shared__ unsigned long long s_u64[kFilterThreads / 64 + 2];
  __shared__ float s_f[kFilterThreads / 64];
  __shared__ double s_d[kFilterThreads / 64];
  __shared__ int s_bin;
  const int tid = threadIdx.x;
  const int32_t j = j_begin + (int32_t)(blockIdx.x % j_count);
  const int32_t b = (int32_t)(blockIdx.x / j_count);
  const int32_t s = cu[b], e = cu[b + 1];
  if (!request_valid(s, e, D, max_k) || j > e - s) return;
  const float T = temperature[b];
  if (!(T > 0.f) || !filter_on(top_k, top_p, b, V)) return;
  if (j_begin > 0 && records[b].mode != kModeActive) return;
  const int32_t K = e - s;
  const float cs = scale_of(T);
  const int64_t row = (int64_t)s + b + j;
  const Elem* prow = logits + row * (int64_t)V;

  if (j < K && tid == 64) {  // accept-test gathers
    const int32_t xs = draft[s + j];
    if (xs >= 0 && xs < V) {
      Gathered g;
      g.lstar = to_f32(prow[xs]);
      g.qstar = q ? q[((int64_t)s + j) * V + xs] : 1.f;
      gath[s + j] = g;
    }
  }

  FilterRow<Elem> r;
  int head = (int)(((16u - ((uint32_t)(uintptr_t)prow & 15u)) & 15u) / sizeof(Elem));
  if (head > V) head = V;
  r.nvec = (V - head) / W;
  const int tail = V - head - r.nvec * W;
  r.pv = reinterpret_cast<const uint4*>(prow + head);
#pragma unroll
  for (int i = 0; i < kFilterResident; ++i) {
    const int v = tid + i * kFilterThreads;
    if (v < r.nvec) r.res[i] = r.pv[v];
  }
  r.has_extra = false;
  r.extra = -INFINITY;
  if (tid < head) {
    r.extra = to_f32(prow[tid]);
    r.has_extra = true;
  } else if (tid >= 8 && tid - 8 < tail) {
    r.extra = to_f32(prow[head + r.nvec * W + (tid - 8)]);
    r.has_extra = true;
  }

  // maximum -> shift, exactly as the row statistics compute it
  float m = -INFINITY;
  r.visit([&](float l) { m = fmaxf(m, l); });
  m = block_reduce<kFilterThreads>(m, s_f, MaxOp());
  const float shift = m * cs;

  uint32_t kappa = 0u;  // keep key >= kappa
  const int32_t kb = top_k ? top_k[b] : 0;
  if (kb > 0 && kb < V) kappa = radix_select<Elem, false>(r, 0u, (double)kb, 0.f, cs, shift, hist, s_u64, &s_bin);
  const float pb = top_p ? top_p[b] : 1.f;
  if (pb > 0.f && pb < 1.f) kappa = radix_select<Elem, true>(r, kappa, 0.0, pb, cs, shift, hist, s_u64, &s_bin);
  const float tau = kappa ? key_value(kappa) : -INFINITY;  // key 0 is no float: nothing filtered

  // kept mass S' = sum over l >= tau of exp2(l c - shift), fp64
  double acc = 0.0;
  r.visit([&](float l) {
    if (l >= tau) acc += (double)exp2_hw(fmaf(l, cs, -shift));
  });
  acc = block_reduce<kFilterThreads>(acc, s_d, SumOp());
  if (tid == 0) {
    FilterRec f;
    f.tau = tau;
    f.shift = shift;
    f.sum = acc;
    frec[row] = f;
  }
}

}  // namespace rsv
