// Row statistics.
//
// p = softmax(l / T) on the target only [第12章 投机解码：以小博大 §12.2.3;
// §12.9 (compute_probs)].  Logits are streamed with coalesced 16-byte loads
// into registers; for a random row the statistics are m = max l,
// shift = fl32(m * c) with c = log2(e) / T, and
// sum = sum_x exp2(fl32(l_x * c - shift)), accumulated per 16-byte vector in
// fp32 and across vectors in fp64.  Greedy rows (T <= 0) keep the lowest
// index of the max instead [§12.2.4].
//
//   chunk_task  one workgroup, one (row, V-chunk): the default path's unit of
//               work (fine-grained, so the grid load-balances).  Chunk 0 also
//               gathers l(x*) and q(x*) for the accept test.
//   row_stats   one workgroup, a whole row in passes, each thread rescaling
//               its own fp64 sum exactly when its max grows (per-request path).
#pragma once

#include "common.hpp"

namespace rsv {

struct RowStats {
  float shift;     // random: fl32(max * c); greedy: max
  int32_t argmax;  // greedy: lowest index of the max
  double sum;      // random: sum_x exp2(fl32(l_x * c - shift))
};

// Partials and gathers, plain or through coherent 64-bit accesses (COH: they
// cross workgroups inside one kernel).
template <bool COH>
__device__ __forceinline__ void store_partial(RowPartial* p, float shift, int32_t argmax, double sum) {
  if (COH) {
    unsigned long long* w = reinterpret_cast<unsigned long long*>(p);
    store_coherent(w, ((unsigned long long)(uint32_t)argmax << 32) | __float_as_uint(shift));
    store_coherent(w + 1, (unsigned long long)__double_as_longlong(sum));
  } else {
    RowPartial r;
    r.shift = shift;
    r.argmax = argmax;
    r.sum = sum;
    *p = r;
  }
}
template <bool COH>
__device__ __forceinline__ RowPartial load_partial(const RowPartial* p) {
  if (!COH) return *p;
  const unsigned long long* w = reinterpret_cast<const unsigned long long*>(p);
  const unsigned long long a = load_coherent(w), b = load_coherent(w + 1);
  RowPartial r;
  r.shift = __uint_as_float((uint32_t)a);
  r.argmax = (int32_t)(a >> 32);
  r.sum = __longlong_as_double((long long)b);
  return r;
}
template <bool COH>
__device__ __forceinline__ void store_gathered(Gathered* g, float lstar, float qstar) {
  if (COH) {
    store_coherent(reinterpret_cast<unsigned long long*>(g),
                   ((unsigned long long)__float_as_uint(qstar) << 32) | __float_as_uint(lstar));
  } else {
    g->lstar = lstar;
    g->qstar = qstar;
  }
}
template <bool COH>
__device__ __forceinline__ Gathered load_gathered(const Gathered* g) {
  if (!COH) return *g;
  const unsigned long long a = load_coherent(reinterpret_cast<const unsigned long long*>(g));
  Gathered r;
  r.lstar = __uint_as_float((uint32_t)a);
  r.qstar = __uint_as_float((uint32_t)(a >> 32));
  return r;
}

// Chunk helpers: NV vectors a thread holds (FULL: every vector in range).
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

// One pass over NVP vectors per thread starting at vector v0 (FULL: every
// vector in range, no guards).
template <typename Elem, int NT, int NVP, bool FULL>
__device__ __forceinline__ void stats_pass(const uint4* __restrict__ pv, int v0, int nvec, int head, bool greedy,
                                           float cs, float& m, float& sh, double& S, int& am) {
  using VT = Vec<Elem>;
  constexpr int W = VT::W;
  const int tid = threadIdx.x;
  uint4 d[NVP];
#pragma unroll
  for (int i = 0; i < NVP; ++i) {
    const int v = v0 + tid + i * NT;
    if (FULL || v < nvec) d[i] = pv[v];
  }
  float pm = -INFINITY;
#pragma unroll
  for (int i = 0; i < NVP; ++i) {
    if (FULL || v0 + tid + i * NT < nvec) {
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
        if (FULL || v < nvec) {
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
      if (FULL || v0 + tid + i * NT < nvec) {
        float sv = exp2_hw(fmaf(VT::get(d[i], 0), cs, -sh));
#pragma unroll
        for (int k = 1; k < W; ++k) sv += exp2_hw(fmaf(VT::get(d[i], k), cs, -sh));
        S += (double)sv;
      }
    }
  }
}

// Block-wide statistics of one row of V logits (NT threads).
template <typename Elem, int NT, int NVP>
__device__ __forceinline__ RowStats row_stats(const Elem* __restrict__ prow, int32_t V, bool greedy, float cs,
                                              float* s_f, int* s_i, double* s_d) {
  using VT = Vec<Elem>;
  constexpr int W = VT::W;
  const int tid = threadIdx.x;
  // Split the row into an unaligned head, 16-byte vectors and a tail.
  int head = (int)(((16u - ((uint32_t)(uintptr_t)prow & 15u)) & 15u) / sizeof(Elem));
  if (head > V) head = V;
  const int nvec = (V - head) / W;
  const int tail = V - head - nvec * W;
  const uint4* pv = reinterpret_cast<const uint4*>(prow + head);

  float m = -INFINITY, sh = -INFINITY;
  double S = 0.0;
  int am = INT_MAX;
  int v0 = 0;
  for (; v0 + NVP * NT <= nvec; v0 += NVP * NT)
    stats_pass<Elem, NT, NVP, true>(pv, v0, nvec, head, greedy, cs, m, sh, S, am);
  if (v0 < nvec) stats_pass<Elem, NT, NVP, false>(pv, v0, nvec, head, greedy, cs, m, sh, S, am);

  // unaligned head and tail elements
  int xi = -1;
  if (tid < head)
    xi = tid;
  else if (tid >= 8 && tid - 8 < tail)
    xi = head + nvec * W + (tid - 8);
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

// Statistics of chunk c (NV vectors per thread) of logits row `row`,
// written to row_partials[c] (the row's nsplit partial slots).  Chunk 0 of a
// draft position's row also stores l(x*) and q(x*) in *gath (x* = xstar,
// checked by the caller).
//
// tmax (NULL: not wanted) receives every thread's own maximum of the chunk
// (kRowThreads floats, -inf for a thread with no element): the top-k / top-p
// selection uses them to bound its threshold.
template <typename Elem, int NV, bool COH = false, bool PRIO_DROP = false>
__device__ __forceinline__ void chunk_task(const Elem* __restrict__ logits, const float* __restrict__ q, int64_t row,
                                           float T, int32_t V, int32_t nsplit, int32_t c, int32_t xstar,
                                           int64_t slot, RowPartial* __restrict__ row_partials,
                                           Gathered* __restrict__ gath, float* __restrict__ tmax = nullptr) {
  using VT = Vec<Elem>;
  constexpr int W = VT::W;
  __shared__ float lds_f[kRowThreads / 64];
  __shared__ int lds_i[kRowThreads / 64];
  __shared__ double lds_d[kRowThreads / 64];
  const bool greedy = !(T > 0.f);
  const float cs = greedy ? 0.f : scale_of(T);
  const int tid = threadIdx.x;

  // Split the row into an unaligned head, 16-byte vectors and a tail.
  const Elem* prow = logits + row * (int64_t)V;
  int head = (int)(((16u - ((uint32_t)(uintptr_t)prow & 15u)) & 15u) / sizeof(Elem));
  if (head > V) head = V;
  const int nvec = (V - head) / W;
  const int tail = V - head - nvec * W;
  const uint4* pv = reinterpret_cast<const uint4*>(prow + head);
  const int v0 = c * NV * kRowThreads;
  // Full chunks (all but a row's last) run the unguarded instantiations.
  const bool full = v0 + NV * kRowThreads <= nvec;

  uint4 data[NV];
  if (full) {
#pragma unroll
    for (int i = 0; i < NV; ++i) data[i] = stream_load(pv + v0 + tid + i * kRowThreads);
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = v0 + tid + i * kRowThreads;
      if (v < nvec) data[i] = pv[v];
    }
  }
  // PRIO_DROP: the caller raised this wave's issue priority for its loads;
  // the arithmetic runs at the default.
  if constexpr (PRIO_DROP) __builtin_amdgcn_s_setprio(0);
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
    if (xstar >= 0 && tid == 64)  // accept-test gathers, off the critical path of the scan
      store_gathered<COH>(gath + slot, to_f32(prow[xstar]), q ? q[slot * V + xstar] : 1.f);
  }

  // Phase 1: chunk maximum.
  float m = full ? chunk_max<Elem, NV, true>(data, v0, tid, nvec, extra)
                 : chunk_max<Elem, NV, false>(data, v0, tid, nvec, extra);
  if (tmax) tmax[tid] = m;
  m = block_reduce<kRowThreads>(m, lds_f, MaxOp());

  RowPartial* out = row_partials + c;
  if (greedy) {
    int idx = INT_MAX;
    if (m > -INFINITY) {
      idx = full ? chunk_argmax<Elem, NV, true>(data, v0, tid, nvec, head, m)
                 : chunk_argmax<Elem, NV, false>(data, v0, tid, nvec, head, m);
      if (extra == m) idx = min(idx, extra_idx);
    }
    idx = block_reduce<kRowThreads>(idx, lds_i, MinOp());
    if (tid == 0) store_partial<COH>(out, m, (idx == INT_MAX) ? -1 : idx, 0.0);
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
  // A coherent gather store (issued long ago) is acknowledged before the
  // workgroup can report its chunk done, which happens after this reduction.
  if (COH && c == 0 && xstar >= 0 && tid == 64) wait_memory();
  acc = block_reduce<kRowThreads>(acc, lds_d, SumOp());
  if (tid == 0) store_partial<COH>(out, shift, -1, acc);
}

// Partials merged per batch of independent loads (a row has at most this
// many chunks up to V = 262144 bf16 logits at 16 vectors per thread).
constexpr int kMergeBatch = 8;

// Merge the nsplit partials of one random row: common shift and fp64 sum.
// Up to kMergeBatch partials are loaded before any is used, so their
// latencies overlap.
template <bool COH = false>
__device__ __forceinline__ void merge_random(const RowPartial* P, int nsplit, float& shift, double& S) {
  if (nsplit <= kMergeBatch) {
    RowPartial r[kMergeBatch];
#pragma unroll
    for (int c = 0; c < kMergeBatch; ++c)
      if (c < nsplit) r[c] = load_partial<COH>(P + c);
    float sh = -INFINITY;
#pragma unroll
    for (int c = 0; c < kMergeBatch; ++c)
      if (c < nsplit) sh = fmaxf(sh, r[c].shift);
    double acc = 0.0;
#pragma unroll
    for (int c = 0; c < kMergeBatch; ++c)
      if (c < nsplit && r[c].sum > 0.0) acc += r[c].sum * exp2((double)r[c].shift - (double)sh);
    shift = sh;
    S = acc;
    return;
  }
  float sh = -INFINITY;
  for (int c = 0; c < nsplit; ++c) sh = fmaxf(sh, load_partial<COH>(P + c).shift);
  double acc = 0.0;
  for (int c = 0; c < nsplit; ++c) {
    const RowPartial r = load_partial<COH>(P + c);
    if (r.sum > 0.0) acc += r.sum * exp2((double)r.shift - (double)sh);
  }
  shift = sh;
  S = acc;
}

// Merge the partials of one greedy row: global max, lowest index holding it.
template <bool COH = false>
__device__ __forceinline__ int32_t merge_greedy(const RowPartial* P, int nsplit) {
  float m = -INFINITY;
  int32_t idx = INT_MAX;
  auto take = [&](const RowPartial& r) {
    if (r.argmax < 0) return;
    if (r.shift > m || (r.shift == m && r.argmax < idx)) {
      m = r.shift;
      idx = r.argmax;
    }
  };
  if (nsplit <= kMergeBatch) {
    RowPartial r[kMergeBatch];
#pragma unroll
    for (int c = 0; c < kMergeBatch; ++c)
      if (c < nsplit) r[c] = load_partial<COH>(P + c);
#pragma unroll
    for (int c = 0; c < kMergeBatch; ++c)
      if (c < nsplit) take(r[c]);
  } else {
    for (int c = 0; c < nsplit; ++c) take(load_partial<COH>(P + c));
  }
  return idx == INT_MAX ? -1 : idx;
}

}  // namespace rsv
