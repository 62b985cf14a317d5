// Top-k / top-p filtering of the target distribution.
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
// A filtered row is first streamed by the ordinary row-statistics task, which
// also stores every thread's maximum of its 16 x 16-byte "segment" of the row
// (chunk_task's tmax).  filter_row then works per row from those maxima:
//   * the k-th largest segment maximum bounds the k-th largest logit from
//     below (k segments hold an element at least that large); the segment
//     maxima, taken from the top until their mass reaches the top-p target,
//     likewise bound the top-p threshold;
//   * only the segments whose maximum reaches the bound can hold a kept
//     token: they are re-read (a few KB per row) and their elements at or
//     above the bound copied to an LDS list;
//   * tau is found exactly on that list: by ranking (each value against all
//     others) for lists of up to 256 values, else by radix selection on
//     order-preserving 32-bit keys of the logits (bf16 logits use the upper
//     16 bits) with 8-bit digits -- a 256-bin LDS histogram per digit, each
//     time narrowing to the bin where the cumulative count (top-k) or mass
//     (top-p) from the top reaches the target.  Masses are fixed point (exp2
//     value scaled by 2^44, truncated, u64), so the selection is
//     deterministic;
//   * S' is summed over the list.
// When no bound can be formed (k above the number of segments, segment maxima
// lighter than the top-p target), the bound admits too many segments (with
// bf16 logits: more than kGatherMaxSegsBf16) or the list overflows, the selection runs
// over the whole row, re-read from memory: for bf16 logits by exact value
// (select_value_bins), else -- or when the threshold lies below the values
// that method counts -- by distance bins (select_row).
#pragma once

#include "common.hpp"
#include "row_pass.hpp"

namespace rsv {

constexpr int kFilterThreads = 256;  // a workgroup per row
constexpr int kFilterBins = 256;      // one radix digit of 8 bits: bin t owned by thread t of the first 256
constexpr int kRankMax = 256;         // lists ranked directly (larger ones by radix selection)
constexpr int kRankParts = kFilterThreads / kRankMax;  // threads sharing one value's ranking
// Histogram copies, chosen by lane & 3, so fewer lanes of one wavefront
// instruction add to the same LDS word (same-address atomics serialise); copy
// c starts at c * kHistStride words so equal bins of different copies sit in
// different banks.
constexpr int kHistCopies = 4;
constexpr int kHistStride = kFilterBins + 1;
constexpr int kFilterCand = 4096;     // candidate list entries in LDS
constexpr int kStashW = 1024;         // per-wavefront LDS queue of window elements (select_row)
constexpr int kFilterSegList = 1024;  // segments re-read per row at most
// With bf16 logits a bound that admits more segments than this skips the
// gather for the one-pass value-bin selection over the row: ~1000 listed
// segments took ~55 us to gather against ~28 us for the value bins.
constexpr int kGatherMaxSegsBf16 = 384;
constexpr int kSegVectors = 16;       // 16-byte vectors per segment: the row task's vectors per thread

// Per-row result: keep l >= tau; shift = fl32(max * c); sum = S' (fp64).
struct FilterRec {
  float tau;
  float shift;
  double sum;
};
static_assert(sizeof(FilterRec) == 16, "FilterRec layout");

// A filter record crosses workgroups inside one kernel (the request's last
// filter workgroup scans it): agent-scope 64-bit stores and loads, as the
// other hand-offs, with an s_waitcnt before the arrival is counted.
__device__ __forceinline__ void store_frec_coherent(FilterRec* p, const FilterRec& f) {
  unsigned long long* w = reinterpret_cast<unsigned long long*>(p);
  store_coherent(w, ((unsigned long long)__float_as_uint(f.shift) << 32) | __float_as_uint(f.tau));
  store_coherent(w + 1, (unsigned long long)__double_as_longlong(f.sum));
}
template <bool COH>
__device__ __forceinline__ FilterRec load_frec(const FilterRec* p) {
  if (!COH) return *p;
  const unsigned long long* w = reinterpret_cast<const unsigned long long*>(p);
  const unsigned long long a = load_coherent(w), b = load_coherent(w + 1);
  FilterRec f;
  f.tau = __uint_as_float((uint32_t)a);
  f.shift = __uint_as_float((uint32_t)(a >> 32));
  f.sum = __longlong_as_double((long long)b);
  return f;
}

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

// Order-preserving key: key(a) < key(b) iff a < b, and key(a) == key(b) iff
// a == b, for non-NaN floats.  -0 and +0 are one value and get one key (that
// of +0): the kept set is decided by comparing values, and the selections and
// sums by comparing keys, so the two must agree on ties.
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  u = u == 0x80000000u ? 0u : u;
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Fixed-point mass of one element: floor(e * 2^44), e = exp2(l c - shift) in
// [0, 1 + 2^-23]; a row of V < 2^20 such values sums below 2^64.
__device__ __forceinline__ unsigned long long fixed_mass(float e) {
  const float x = e * 0x1p+12f;  // integer part < 2^12 + 1, fraction on a 2^-32 grid or finer (truncated)
  const uint32_t hi = (uint32_t)x;
  const uint32_t lo = (uint32_t)((x - (float)hi) * 0x1p+32f);
  return ((unsigned long long)hi << 32) | lo;
}

// One row split into an unaligned head, 16-byte vectors and a tail, exactly as
// the row-statistics task splits it.
template <typename Elem>
struct RowView {
  const Elem* prow;
  const uint4* pv;
  int head, nvec, tail;
  __device__ __forceinline__ RowView(const Elem* p, int32_t V) : prow(p) {
    constexpr int W = Vec<Elem>::W;
    head = (int)(((16u - ((uint32_t)(uintptr_t)p & 15u)) & 15u) / sizeof(Elem));
    if (head > V) head = V;
    nvec = (V - head) / W;
    tail = V - head - nvec * W;
    pv = reinterpret_cast<const uint4*>(p + head);
  }
  // The head / tail element held by thread t of chunk 0 in the row task (a
  // row task thread t < head holds prow[t]; 8 <= t < 8 + tail a tail element).
  __device__ __forceinline__ bool extra(int t, float& v) const {
    constexpr int W = Vec<Elem>::W;
    if (t < head) {
      v = to_f32(prow[t]);
      return true;
    }
    if (t >= 8 && t - 8 < tail) {
      v = to_f32(prow[head + nvec * W + (t - 8)]);
      return true;
    }
    return false;
  }
};

// Element visitors for the selection: each calls f(value) for the elements
// the calling thread holds.
template <typename Elem>
struct RowVisitor {  // the whole row, read from memory kRowBatch vectors per thread at a time
  static constexpr int kRowBatch = 4096 / kFilterThreads;
  RowView<Elem> rv;
  template <typename F>
  __device__ __forceinline__ void operator()(F&& f) const {
    using VT = Vec<Elem>;
    for (int v0 = threadIdx.x; v0 < rv.nvec; v0 += kRowBatch * kFilterThreads) {
      // unconditional loads (clamped index), so all kRowBatch are in flight together
      uint4 x[kRowBatch];
#pragma unroll
      for (int i = 0; i < kRowBatch; ++i) x[i] = rv.pv[min(v0 + i * kFilterThreads, rv.nvec - 1)];
#pragma unroll
      for (int i = 0; i < kRowBatch; ++i) {
        if (v0 + i * kFilterThreads < rv.nvec) {
#pragma unroll
          for (int k = 0; k < VT::W; ++k) f(VT::get(x[i], k));
        }
      }
    }
    float e;
    if (threadIdx.x < 16 && rv.extra(threadIdx.x, e)) f(e);
  }
  // The same elements, but f runs on every lane at every step (-inf where the
  // lane holds no element), so that f may use wavefront-wide operations.
  template <typename F>
  __device__ __forceinline__ void uniform(F&& f) const {
    using VT = Vec<Elem>;
    for (int base = 0; base < rv.nvec; base += kRowBatch * kFilterThreads) {
      const int v0 = base + (int)threadIdx.x;
      uint4 x[kRowBatch];
#pragma unroll
      for (int i = 0; i < kRowBatch; ++i) x[i] = rv.pv[min(v0 + i * kFilterThreads, rv.nvec - 1)];
#pragma unroll
      for (int i = 0; i < kRowBatch; ++i) {
        const bool ok = v0 + i * kFilterThreads < rv.nvec;
#pragma unroll
        for (int k = 0; k < VT::W; ++k) f(ok ? VT::get(x[i], k) : -INFINITY);
      }
    }
    float e = -INFINITY, t;
    if (threadIdx.x < 16 && rv.extra(threadIdx.x, t)) e = t;
    f(e);
  }
};
constexpr int kSegPerThread = 4096 / kFilterThreads;  // segment maxima a thread keeps in registers (rows of up
                                                      // to 4096 segments)

struct MaxVisitor {  // the segment maxima, kSegPerThread per thread in registers
  const float (&mx)[kSegPerThread];
  template <typename F>
  __device__ __forceinline__ void operator()(F&& f) const {
#pragma unroll
    for (int i = 0; i < kSegPerThread; ++i)
      if (mx[i] > -INFINITY) f(mx[i]);
  }
};
struct ListVisitor {  // a candidate list in LDS
  const float* vals;
  int n;
  template <typename F>
  __device__ __forceinline__ void operator()(F&& f) const {
    for (int i = threadIdx.x; i < n; i += kFilterThreads) {
      const float v = vals[i];
      if (v > -INFINITY) f(v);
    }
  }
};

__device__ __forceinline__ void hist_clear(unsigned long long* hist) {
  for (int i = threadIdx.x; i < kHistCopies * kHistStride; i += kFilterThreads) hist[i] = 0ull;
}
__device__ __forceinline__ void hist_add(unsigned long long* hist, int bin, unsigned long long w) {
  atomicAdd(hist + (threadIdx.x & (kHistCopies - 1)) * kHistStride + bin, w);
}

// Find the bin B of hist[] (kFilterBins u64 weights, thread t < kFilterBins
// owning bin t) where, counting from the top bin down, base + (weight of the
// bins above B) < target <= base + (weight of the bins from B up).  Returns B
// and adds the weight above B to base; -1 if the target exceeds the total.
// Whole workgroup.  s_u64 needs kFilterBins / 64 + 1 slots.
__device__ __forceinline__ int find_bin(const unsigned long long* hist, double target, unsigned long long& base,
                                        unsigned long long* s_u64, int* s_bin) {
  constexpr int NWB = kFilterBins / 64;  // the wavefronts that own bins
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool owner = tid < kFilterBins;  // whole wavefronts
  __syncthreads();  // the histogram is complete; earlier readers of s_u64 / s_bin are done
  unsigned long long h = 0ull, suf = 0ull;
  if (owner) {
#pragma unroll
    for (int c = 0; c < kHistCopies; ++c) h += hist[c * kHistStride + tid];
    suf = h;  // suffix sums over the lanes of the wave, then over the waves
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned long long v = __shfl_down(suf, o);
      if (lane + o < 64) suf += v;
    }
    if (lane == 0) s_u64[wave] = suf;
  }
  if (tid == 0) *s_bin = -1;
  __syncthreads();
  if (owner) {
    unsigned long long above = base + (suf - h);
    for (int w = wave + 1; w < NWB; ++w) above += s_u64[w];
    if ((double)above < target && (double)(above + h) >= target) {
      *s_bin = tid;
      s_u64[NWB] = above;
    }
  }
  __syncthreads();
  const int bin = *s_bin;
  if (bin >= 0) base = s_u64[NWB];
  __syncthreads();  // s_u64, s_bin and hist are reused
  return bin;
}

// Radix selection with 8-bit digits: the key kappa such that, over the
// visited elements with key >= kmin, weight(key > kappa) < target <=
// weight(key >= kappa), weights being 1 (MASS = false) or the fixed-point
// mass.  With fewer than all levels (nlev) it returns the smallest key of the
// group that holds kappa -- a lower bound of it.  Returns 0 (no float has key
// 0) when the target exceeds the total weight.
template <typename Elem, bool MASS, typename Vis>
__device__ __forceinline__ uint32_t radix_select(const Vis& vis, uint32_t kmin, double target, float cs, float shift,
                                                 int nlev, unsigned long long* hist, unsigned long long* s_u64,
                                                 int* s_bin) {
  constexpr int kLevels = sizeof(Elem) == 2 ? 2 : 4;  // bf16 keys end in 16 constant bits
  uint32_t prefix = 0, pmask = 0;
  unsigned long long base = 0;
  for (int lv = 0; lv < kLevels && lv < nlev; ++lv) {
    const int sh = 24 - 8 * lv;
    hist_clear(hist);
    __syncthreads();
    vis([&](float l) {
      const uint32_t key = order_key(l);
      if (key >= kmin && (key & pmask) == prefix) {
        const unsigned long long w = MASS ? fixed_mass(exp2_hw(fmaf(l, cs, -shift))) : 1ull;
        if (w) hist_add(hist, (int)((key >> sh) & 0xFFu), w);
      }
    });
    const int bin = find_bin(hist, target, base, s_u64, s_bin);
    if (bin < 0) return 0u;
    prefix |= (uint32_t)bin << sh;
    pmask |= 0xFFu << sh;
  }
  return prefix;  // bf16: the low 16 bits stay 0, below every key of the selected value and above the next
}

// The same selection over a list of at most kRankMax values in LDS by
// ranking: value v_i is the answer iff the weight of the values > v_i is
// below the target and the weight of those >= v_i reaches it.  Value i is
// ranked by the kRankParts adjacent lanes kRankParts i .. + kRankParts - 1,
// each over every kRankParts-th value, and their sums combined by shuffles.
template <bool MASS>
__device__ __forceinline__ uint32_t rank_select(const float* vals, int n, uint32_t kmin, double target, float cs,
                                                float shift, unsigned long long* wts, uint32_t* s_key) {
  const int tid = threadIdx.x;
  const int i = tid / kRankParts, part = tid % kRankParts;
  __syncthreads();
  if (tid < n) {
    const float v = vals[tid];
    wts[tid] = (order_key(v) >= kmin) ? (MASS ? fixed_mass(exp2_hw(fmaf(v, cs, -shift))) : 1ull) : 0ull;
  }
  if (tid == 0) *s_key = 0u;
  __syncthreads();
  float v = -INFINITY;
  uint32_t kv = 0u;
  if (i < n) {
    v = vals[i];
    kv = order_key(v);
  }
  const bool mine = i < n && kv >= kmin;
  unsigned long long gt = 0ull, eq = 0ull;
  if (mine) {
    for (int k = part; k < n; k += kRankParts) {
      const float u = vals[k];
      const unsigned long long w = wts[k];
      gt += u > v ? w : 0ull;
      eq += u == v ? w : 0ull;
    }
  }
#pragma unroll
  for (int o = 1; o < kRankParts; o <<= 1) {  // every lane takes part
    gt += __shfl_xor(gt, o);
    eq += __shfl_xor(eq, o);
  }
  if (mine && part == 0 && (double)gt < target && (double)(gt + eq) >= target)
    *s_key = kv;  // equal values write the same key
  __syncthreads();
  const uint32_t k = *s_key;
  __syncthreads();
  return k;
}

// Sum over the visited elements with key >= kmin of the fixed-point mass
// (whole workgroup).
template <typename Vis>
__device__ __forceinline__ unsigned long long fixed_total(const Vis& vis, uint32_t kmin, float cs, float shift,
                                                          unsigned long long* s_u64) {
  unsigned long long t = 0ull;
  vis([&](float l) {
    if (order_key(l) >= kmin) t += fixed_mass(exp2_hw(fmaf(l, cs, -shift)));
  });
  return block_reduce<kFilterThreads>(t, s_u64, SumOp());
}

// Copy into cand[] every element >= t of the segments whose maximum is >= t
// (segment sg = threadIdx.x + i * kFilterThreads has maximum mx[i]: row-task
// chunk sg / 256, thread sg % 256, holding vectors chunk * 4096 + thread +
// u * 256 for u < 16, plus a head / tail element in chunk 0).  The segments
// are listed first, then all threads share their (segment, vector) loads.
// Returns the element count, or -1 if more than max_segs segments qualify or
// the elements overflow their list.
template <typename Elem>
__device__ __forceinline__ int gather_segments(const RowView<Elem>& rv, const float (&mx)[kSegPerThread], float t,
                                               float* cand, int* qseg, int* s_cnt, int* s_nq,
                                               int max_segs = kFilterSegList) {
  using VT = Vec<Elem>;
  constexpr int kItems = kSegVectors + 1;  // 16 vectors and the head / tail element
  constexpr int kBatch = 4;
  const int tid = threadIdx.x;
  __syncthreads();
  if (tid == 0) {
    *s_cnt = 0;
    *s_nq = 0;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kSegPerThread; ++i) {
    if (mx[i] >= t) {
      const int slot = atomicAdd(s_nq, 1);
      if (slot < kFilterSegList) qseg[slot] = tid + i * kFilterThreads;
    }
  }
  __syncthreads();
  const int nq = *s_nq;
  if (nq > max_segs || rv.nvec == 0) return -1;  // (rows shorter than one vector: whole-row selection)
  auto put = [&](float l) {
    if (l >= t) {
      const int slot = atomicAdd(s_cnt, 1);
      if (slot < kFilterCand) cand[slot] = l;
    }
  };
  const int nitems = nq * kItems;
  for (int it0 = tid; it0 < nitems; it0 += kBatch * kFilterThreads) {
    uint4 x[kBatch];
    float ex[kBatch];
    int kind[kBatch];  // 0 none, 1 vector, 2 extra element
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {  // vector loads unconditional (clamped index): all in flight together
      const int it = it0 + r * kFilterThreads;
      const int sg = qseg[min(it, nitems - 1) / kItems], u = it % kItems;
      const int c = sg / kRowThreads, th = sg % kRowThreads;
      const int v = c * kSegVectors * kRowThreads + th + u * kRowThreads;
      x[r] = rv.pv[min(v, rv.nvec - 1)];
      kind[r] = 0;
      if (it < nitems) {
        if (u < kSegVectors) {
          if (v < rv.nvec) kind[r] = 1;
        } else if (c == 0 && rv.extra(th, ex[r])) {
          kind[r] = 2;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      if (kind[r] == 1) {
#pragma unroll
        for (int k = 0; k < VT::W; ++k) put(VT::get(x[r], k));
      } else if (kind[r] == 2) {
        put(ex[r]);
      }
    }
  }
  __syncthreads();
  const int n = *s_cnt;
  return n <= kFilterCand ? n : -1;
}

// Selection over the whole row (no usable bound).  Elements are binned by
// their distance below the row maximum in log2(e) units, d = shift - l c:
// first only those within win bits of the maximum, 256 / win bins per bit
// (the others are skipped at the cost of a compare); if that window holds
// less than the target weight, then the whole row with 4 bins per bit and
// everything beyond 64 bits in the lowest bin (directly when win >= 64).
// For a mass target the caller derives win from a bound: the elements more
// than D bits below the maximum weigh under V 2^-D together, so the threshold
// lies within D bits once that is at most the mass the target leaves out.
// Larger logits go to higher bins.  The bin where the cumulative weight
// from the top reaches the target is gathered and selected exactly, with the
// target less the weight above it.  If that bin overflows the candidate list,
// radix selection runs on the keys of the whole row.  The candidate list is
// left holding only that bin.
//
// In the window pass each wavefront appends the elements that pass the
// window's pre-test to its queue in LDS (ballot and lane prefix count), and
// bins them 64 at a time with every lane busy: a lane rarely holds a window
// element, but nearly every step of the wavefront has one.  When no queue
// overflowed, the queues still hold every window element, and the selected
// bin is gathered from them instead of from the row.
//
// On return n_out is the number of candidates (the elements of the selected
// bin) and base_out the weight above that bin, or n_out = -1 when the radix
// selection over the row's keys ran instead.
template <typename Elem, bool MASS>
__device__ __forceinline__ uint32_t select_row(const RowVisitor<Elem>& all, uint32_t kmin, double target, float win,
                                               float cs, float shift, float* cand, unsigned long long* hist,
                                               unsigned long long* wts, unsigned long long* s_u64, int* s_bin,
                                               uint32_t* s_key, int* s_cnt, int* s_over, float* stash,
                                               int& n_out, unsigned long long& base_out) {
  n_out = -1;
  const int lane = threadIdx.x & 63;
  float* sw = stash + (threadIdx.x >> 6) * kStashW;  // this wavefront's queue
#pragma unroll 1
  for (int wide = win < 64.f ? 0 : 1; wide < 2; ++wide) {
    const float per_bit = wide ? 4.f : 256.f / win;
    auto dbin = [&](float l) -> int {  // -1: outside the window
      const float d = -fmaf(l, cs, -shift) * per_bit;  // >= about 0; +inf for l = -inf
      if (!wide && !(d < 256.f)) return -1;
      return 255 - (int)fminf(fmaxf(d, 0.f), 255.f);
    };
    // Cheap pre-tests on the logit itself (one compare per element) with a
    // margin of 1/16 bit; the exact bin test follows for the few that pass.
    const float lo_win = wide ? -INFINITY : (shift - (win + 0.0625f)) / cs;
    hist_clear(hist);
    if (threadIdx.x == 0) *s_over = 0;
    auto process = [&](float l) {
      const int bin = dbin(l);
      if (bin >= 0 && order_key(l) >= kmin) {
        const unsigned long long w = MASS ? fixed_mass(exp2_hw(fmaf(l, cs, -shift))) : 1ull;
        if (w) hist_add(hist, bin, w);
      }
    };
    __syncthreads();
    int qn = 0;  // elements queued by this wavefront (the same in all its lanes)
    if (wide) {
      all([&](float l) { process(l); });
    } else {
      int qd = 0;  // of which binned
      all.uniform([&](float l) {
        const bool in = l >= lo_win;
        const unsigned long long m = __ballot(in);
        if (m) {
          const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          if (in) sw[(qn + rank) & (kStashW - 1)] = l;
          qn += __popcll(m);
          if (qn - qd >= 64) {  // fewer than 128 queued and unbinned: the ring never overwrites them
            process(sw[(qd + lane) & (kStashW - 1)]);
            qd += 64;
          }
        }
      });
      if (lane < qn - qd) process(sw[(qd + lane) & (kStashW - 1)]);
      if (lane == 0 && qn > kStashW) *s_over = 1;
    }
    unsigned long long base = 0ull;
    const int B = find_bin(hist, target, base, s_u64, s_bin);
    if (B < 0) continue;  // the window holds less than the target
    // logits of bin B lie in ((shift - d_hi) / c, (shift - d_lo) / c]; pre-test with a margin
    const float d_lo = (float)(255 - B) / per_bit - 0.0625f, d_hi = (float)(256 - B) / per_bit + 0.0625f;
    const float lo_b = (B == 0 && wide) ? -INFINITY : (shift - d_hi) / cs, hi_b = (shift - d_lo) / cs;
    if (threadIdx.x == 0) *s_cnt = 0;
    __syncthreads();
    auto put = [&](float l) {
      if (l >= lo_b && l <= hi_b && dbin(l) == B && order_key(l) >= kmin) {
        const int slot = atomicAdd(s_cnt, 1);
        if (slot < kFilterCand) cand[slot] = l;
      }
    };
    if (!wide && !*s_over) {  // (s_over is settled: find_bin synchronised the workgroup)
      for (int i = lane; i < qn; i += 64) put(sw[i]);
    } else {
      all(put);
    }
    __syncthreads();
    const int n = *s_cnt;
    const double rest = target - (double)base;
    if (n > kFilterCand) return radix_select<Elem, MASS>(all, kmin, target, cs, shift, 4, hist, s_u64, s_bin);
    n_out = n;
    base_out = base;
    if (n <= kRankMax) return rank_select<MASS>(cand, n, kmin, rest, cs, shift, wts, s_key);
    return radix_select<Elem, MASS>(ListVisitor{cand, n}, kmin, rest, cs, shift, 4, hist, s_u64, s_bin);
  }
  return 0u;
}

// Whole-row selection for bf16 logits by exact value.  A bf16 row holds few
// distinct values near its maximum, so one pass counts the elements of each
// of the kValueBins values just below the row maximum (u32 LDS counters, no
// per-element mass); the weight of a bin is then count x (1 or the
// fixed-point mass of its value), and a scan from the top finds the value
// where the cumulative weight reaches the target.  Every element of a bin
// has that value, so the weights are exactly the per-element sums the
// selection above forms, and ties stay together; the kept mass is the
// weight above the threshold's bin plus the bin.  Elements below lo_pre
// (the top-p window's pre-test; -inf for counts) are not counted: they lie in
// no bin that can hold the threshold.  Returns the 32-bit order key of the
// threshold value, with its bin's weight and the weight above it, or 0 when
// the target is not reached within the bins (the caller then selects with
// select_row).
constexpr int kValueBins = kFilterThreads / 64 * kStashW;  // 4096: the queues' LDS, as u32 counters

// 16-bit order key of a bf16 value u (sign bit, 15-bit magnitude m):
// 0x8000 + m if positive, 0x8000 - m if negative, so both zeros get 0x8000.
__device__ __forceinline__ uint32_t bf16_key(float l) {  // l: a widened bf16 value
  const uint32_t u = __float_as_uint(l) >> 16, m = u & 0x7FFFu;
  return (u & 0x8000u) ? 0x8000u - m : 0x8000u + m;
}
__device__ __forceinline__ float bf16_value(uint32_t key) {
  const uint32_t u = key >= 0x8000u ? key - 0x8000u : 0x8000u | (0x8000u - key);
  return __uint_as_float(u << 16);
}

typedef unsigned short vb_u16x2 __attribute__((ext_vector_type(2)));
typedef short vb_i16x2 __attribute__((ext_vector_type(2)));

// The distances ktop - key of the two bf16 values packed in w, one per
// 16-bit half, in packed 16-bit integer arithmetic: with s = 0xFFFF for a
// negative half, (m ^ s) - s is +m or -m, and ktop - (0x8000 +- m) =
// (ktop - 0x8000) -+ m modulo 2^16.  top2 holds ktop - 0x8000 in both halves.
__device__ __forceinline__ uint32_t bf16_pair_dist(uint32_t w, uint32_t top2) {
  const vb_i16x2 x = __builtin_bit_cast(vb_i16x2, w);
  const vb_u16x2 s = __builtin_bit_cast(vb_u16x2, (vb_i16x2)(x >> (short)15));
  const vb_u16x2 m = __builtin_bit_cast(vb_u16x2, w & 0x7FFF7FFFu);
  const vb_u16x2 d = __builtin_bit_cast(vb_u16x2, top2) - ((m ^ s) - s);
  return __builtin_bit_cast(uint32_t, d);
}

// Adds one to cnt[d] for every element of the bf16 row at distance d < dlim
// below the key ktop, reading the row's 16-byte vectors as 32-bit words.
__device__ __forceinline__ void count_value_bins(const RowView<uint16_t>& rv, uint32_t ktop, uint32_t dlim,
                                                 uint32_t* cnt) {
  constexpr int KB = RowVisitor<uint16_t>::kRowBatch;
  const uint32_t top2 = ((ktop - 0x8000u) & 0xFFFFu) * 0x10001u;
  auto pair = [&](uint32_t w) {
    const uint32_t d = bf16_pair_dist(w, top2);
    const uint32_t lo = d & 0xFFFFu, hi = d >> 16;
    if (lo < dlim) atomicAdd(cnt + lo, 1u);
    if (hi < dlim) atomicAdd(cnt + hi, 1u);
  };
  for (int v0 = threadIdx.x; v0 < rv.nvec; v0 += KB * kFilterThreads) {
    uint4 x[KB];  // unconditional loads (clamped index), all in flight together
#pragma unroll
    for (int i = 0; i < KB; ++i) x[i] = rv.pv[min(v0 + i * kFilterThreads, rv.nvec - 1)];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      if (v0 + i * kFilterThreads < rv.nvec) {
        pair(x[i].x);
        pair(x[i].y);
        pair(x[i].z);
        pair(x[i].w);
      }
    }
  }
  float e;
  if (threadIdx.x < 16 && rv.extra(threadIdx.x, e)) {
    const uint32_t d = ktop - bf16_key(e);
    if (d < dlim) atomicAdd(cnt + d, 1u);
  }
}

template <bool MASS>
__device__ __forceinline__ uint32_t select_value_bins(const RowVisitor<uint16_t>& all, float rowmax, uint32_t kmin,
                                                      double target, float lo_pre, float cs, float shift,
                                                      uint32_t* cnt, unsigned long long* s_u64, int* s_bin,
                                                      unsigned long long* s_vb, unsigned long long& bin_out,
                                                      unsigned long long& above_out) {
  constexpr int NW = kFilterThreads / 64;
  constexpr int PER = kValueBins / kFilterThreads;  // bins per thread: thread t owns [t PER, t PER + PER)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t ktop = bf16_key(rowmax);
  // l >= lo_pre  <=>  bf16_key(l) >= klo, the key of the least bf16 value >= lo_pre
  // (bf16_key truncates lo_pre towards zero)
  uint32_t klo = 0u;
  if (lo_pre > -INFINITY) {
    klo = bf16_key(lo_pre);
    if (bf16_value(klo) < lo_pre) ++klo;
  }
  const uint32_t dlim = klo > ktop ? 0u : min(ktop - klo + 1u, (uint32_t)kValueBins);  // bin 0 = the maximum
  __syncthreads();  // earlier users of the LDS are done
  for (int i = tid; i < kValueBins; i += kFilterThreads) cnt[i] = 0u;
  if (tid == 0) *s_bin = -1;
  __syncthreads();
  // The counting pass is the slowest stage of the kernel's slowest rows and
  // is issue-bound: it runs at raised issue priority over the waves of other
  // rows' shorter stages on the same SIMDs (top-p 0.9 alone at B=256 K=8
  // V=151936: 226 -> 222 us per call).
  __builtin_amdgcn_s_setprio(1);
  count_value_bins(all.rv, ktop, dlim, cnt);
  __builtin_amdgcn_s_setprio(0);
  __syncthreads();
  unsigned long long w[PER], sum = 0ull;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t d = (uint32_t)(tid * PER + i);
    const uint32_t c = cnt[d];
    w[i] = 0ull;
    if (c && d <= ktop) {
      const float v = bf16_value(ktop - d);
      if (order_key(v) >= kmin) w[i] = MASS ? (unsigned long long)c * fixed_mass(exp2_hw(fmaf(v, cs, -shift))) : c;
    }
    sum += w[i];
  }
  // exclusive prefix of the thread sums in thread order (top bins first)
  unsigned long long incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) s_u64[wave] = incl;
  __syncthreads();
  unsigned long long above = incl - sum;
  for (int q = 0; q < wave; ++q) above += s_u64[q];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if ((double)above < target && (double)(above + w[i]) >= target) {  // one bin at most
      *s_bin = tid * PER + i;
      s_vb[0] = w[i];
      s_vb[1] = above;
    }
    above += w[i];
  }
  __syncthreads();
  const int bin = *s_bin;
  uint32_t key = 0u;
  if (bin >= 0) {
    bin_out = s_vb[0];
    above_out = s_vb[1];
    key = order_key(bf16_value(ktop - (uint32_t)bin));
  }
  __syncthreads();  // s_u64, s_bin, s_vb and the counters are reused
  (void)NW;
  return key;
}

// Select over the candidate list: ranking for short lists, radix otherwise.
template <typename Elem, bool MASS>
__device__ __forceinline__ uint32_t select_list(const float* cand, int n, uint32_t kmin, double target, float cs,
                                                float shift, unsigned long long* hist, unsigned long long* wts,
                                                unsigned long long* s_u64, int* s_bin, uint32_t* s_key) {
  if (n <= kRankMax) return rank_select<MASS>(cand, n, kmin, target, cs, shift, wts, s_key);
  return radix_select<Elem, MASS>(ListVisitor{cand, n}, kmin, target, cs, shift, 4, hist, s_u64, s_bin);
}

// One workgroup per (request, position) row of the positions [j_begin,
// j_begin + j_count) of every random request with a filter (and, after the
// first phase, still active), after the row task streamed it: writes
// frec[row] from the row's partials and segment maxima.
template <typename Elem>
__device__ __forceinline__ void filter_row(
    const Elem* __restrict__ logits, const int32_t* __restrict__ cu, const float* __restrict__ temperature,
    const int32_t* __restrict__ top_k, const float* __restrict__ top_p, int32_t D, int32_t max_k, int32_t V,
    int32_t j_begin, int32_t j_count, int32_t nsplit, const ReqRecord* __restrict__ records,
    const RowPartial* __restrict__ partials, const float* __restrict__ tmaxbuf, FilterRec* __restrict__ frec) {
  __shared__ unsigned long long hist[kHistCopies * kHistStride];
  __shared__ unsigned long long wts[kRankMax];
  __shared__ float cand[kFilterCand];
  __shared__ int qseg[kFilterSegList];
  __shared__ unsigned long long s_u64[kFilterThreads / 64 + 1];
  __shared__ double s_d[kFilterThreads / 64];
  __shared__ float stash[kFilterThreads / 64 * kStashW];
  __shared__ int s_bin, s_cnt, s_nq, s_over;
  __shared__ uint32_t s_key;
  __shared__ float s_f[kFilterThreads / 64];
  __shared__ unsigned long long s_vb[2];
  const int32_t j = j_begin + (int32_t)(blockIdx.x % j_count);
  const int32_t b = (int32_t)(blockIdx.x / j_count);
  const int32_t s = cu[b], e = cu[b + 1];
  if (!request_valid(s, e, D, max_k) || j > e - s) return;
  const float T = temperature[b];
  if (!(T > 0.f) || !filter_on(top_k, top_p, b, V)) return;
  if (j_begin > 0 && records[b].mode != kModeActive) return;
  const float cs = scale_of(T);
  const int64_t row = (int64_t)s + b + j;
  const RowView<Elem> rv(logits + row * (int64_t)V, V);
  const RowVisitor<Elem> all{rv};
  const int nseg = nsplit * kRowThreads;
  const float* tmax = tmaxbuf + row * nseg;
  // the row's segment maxima, kSegPerThread per thread (-inf past the end;
  // rows with more segments than that select over the whole row)
  const bool use_maxima = nseg <= kSegPerThread * kFilterThreads;
  float mx[kSegPerThread];
#pragma unroll
  for (int i = 0; i < kSegPerThread; ++i) {  // unconditional loads (clamped index): all in flight together
    const int sg = threadIdx.x + i * kFilterThreads;
    const float v = tmax[min(sg, nseg - 1)];
    mx[i] = (use_maxima && sg < nseg) ? v : -INFINITY;
  }
  const MaxVisitor maxima{mx};
  const int max_segs = sizeof(Elem) == 2 ? kGatherMaxSegsBf16 : kFilterSegList;  // beyond: the value bins
  constexpr int kBoundLevels = 2;  // key bits that bound a threshold from the maxima

  float shift;
  double S;
  merge_random(partials + row * nsplit, nsplit, shift, S);

  unsigned long long kept_fixed = 0ull;  // top-p by value bins: the kept mass in the fixed-point unit (0: not used)
  auto row_max = [&]() {  // the row's maximum, from the segment maxima (they cover every element)
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kSegPerThread; ++i) m = fmaxf(m, mx[i]);
    return block_reduce<kFilterThreads>(m, s_f, MaxOp());
  };
  int nbin = -1;                 // top-p over the row: elements of the threshold's bin in cand[0 .. nbin)
  unsigned long long above_bin = 0ull;  // and the fixed-point mass above that bin
  int ncand = -1;       // candidate list: every element >= its bound is in cand[0 .. ncand) (-1: none)
  uint32_t kappa = 0u;  // keep key >= kappa (0: everything)
  const int32_t kb = top_k ? top_k[b] : 0;
  if (kb > 0 && kb < V) {
    const uint32_t bound =
        use_maxima
            ? radix_select<Elem, false>(maxima, 0u, (double)kb, cs, shift, kBoundLevels, hist, s_u64, &s_bin)
            : 0u;
    if (bound) ncand = gather_segments(rv, mx, key_value(bound), cand, qseg, &s_cnt, &s_nq, max_segs);
    if (ncand >= 0) {
      kappa = select_list<Elem, false>(cand, ncand, 0u, (double)kb, cs, shift, hist, wts, s_u64, &s_bin, &s_key);
    } else {
      int nb;
      unsigned long long cb, ab;
      kappa = 0u;
      if constexpr (sizeof(Elem) == 2) {
        if (use_maxima)
          kappa = select_value_bins<false>(all, row_max(), 0u, (double)kb, -INFINITY, cs, shift,
                                           reinterpret_cast<uint32_t*>(stash), s_u64, &s_bin, s_vb, cb, ab);
      }
      if (!kappa)
        kappa = select_row<Elem, false>(all, 0u, (double)kb, 16.f, cs, shift, cand, hist, wts, s_u64, &s_bin, &s_key,
                                        &s_cnt, &s_over, stash, nb, cb);
    }
  }
  const float pb = top_p ? top_p[b] : 1.f;
  if (pb > 0.f && pb < 1.f) {
    // target: top_p times the mass kept by top-k (all of it without top-k)
    const double total = kappa == 0u ? S * 0x1p+44  // the row's sum in the fixed-point unit
                                     : (double)(ncand >= 0 ? fixed_total(ListVisitor{cand, ncand}, kappa, cs, shift,
                                                                         s_u64)
                                                           : fixed_total(all, kappa, cs, shift, s_u64));
    const double P = (double)pb * total;
    if (ncand < 0) {
      const uint32_t bound =
          use_maxima ? radix_select<Elem, true>(maxima, kappa, P, cs, shift, kBoundLevels, hist, s_u64, &s_bin)
                     : 0u;
      if (bound) ncand = gather_segments(rv, mx, key_value(bound), cand, qseg, &s_cnt, &s_nq, max_segs);
    }
    uint32_t kp;
    if (ncand >= 0) {
      kp = select_list<Elem, true>(cand, ncand, kappa, P, cs, shift, hist, wts, s_u64, &s_bin, &s_key);
    } else {
      // window: D >= log2(2 V 2^44 / (total - P)) bits, so that V 2^-D (plus the
      // truncation of up to V fixed-point units) stays within the left-out mass
      // (capped at 16 bits: a wider bound comes from a peaked row, whose
      // threshold normally lies within 16 bits of its maximum; if it does not,
      // the pass over the whole row follows)
      const double wb = log2(2.0 * (double)V * 0x1p+44 / (total - P)) + 0.0625;
      const float win = (float)fmin(fmax(wb, 1.0), 16.0);
      kp = 0u;
      if constexpr (sizeof(Elem) == 2) {
        if (use_maxima) {
          unsigned long long bw, ab;
          kp = select_value_bins<true>(all, row_max(), kappa, P, (shift - (win + 0.0625f)) / cs, cs, shift,
                                       reinterpret_cast<uint32_t*>(stash), s_u64, &s_bin, s_vb, bw, ab);
          if (kp) kept_fixed = ab + bw;
        }
      }
      if (!kp)
        kp = select_row<Elem, true>(all, kappa, P, win, cs, shift, cand, hist, wts, s_u64, &s_bin, &s_key, &s_cnt,
                                    &s_over, stash, nbin, above_bin);
    }
    if (kp) kappa = kp;
  }
  const float tau = kappa ? key_value(kappa) : -INFINITY;  // key 0 is no float: nothing filtered

  // kept mass S' = sum over l >= tau of exp2(l c - shift): in fp64 over the
  // candidate list when it holds every kept element (tau >= its bound); from
  // the fixed-point masses when the selection over the row left the weight
  // above the threshold's bin and that bin's elements; else over the row
  double acc = 0.0;
  auto add = [&](float l) {
    if (l >= tau) acc += (double)exp2_hw(fmaf(l, cs, -shift));
  };
  if (ncand >= 0) {
    ListVisitor{cand, ncand}(add);
    acc = block_reduce<kFilterThreads>(acc, s_d, SumOp());
  } else if (kept_fixed) {
    acc = (double)kept_fixed * 0x1p-44;
  } else if (nbin >= 0 && kappa) {
    acc = (double)(above_bin + fixed_total(ListVisitor{cand, nbin}, kappa, cs, shift, s_u64)) * 0x1p-44;
  } else {
    all(add);
    acc = block_reduce<kFilterThreads>(acc, s_d, SumOp());
  }
  if (threadIdx.x == 0) {
    FilterRec f;
    f.tau = tau;
    f.shift = shift;
    f.sum = acc;
    store_frec_coherent(frec + row, f);
    wait_memory();  // acknowledged before thread 0 counts the workgroup's arrival
  }
}

}  // namespace rsv
