// rs_verify.hip -- gfx950 kernels and C ABI of the batched speculative-
// sampling verify step (see include/rs_verify.h for the contract).
//
// Three paths compute the same outputs; make_plan picks one per call (the
// caller can force one through rs_debug):
//
//  * stream (stream_path.hpp): one kernel streams every row position-major in
//    V-chunks, takes each request's decision in the kernel as its rows
//    complete, and races decided requests' rows in the same grid; an init
//    kernel before it and a race tail kernel after it.  Chosen for large
//    batches and for calls of up to 128 MB of logits.
//  * per-request (request_path.hpp): one workgroup per request walks its rows
//    in order and races its row.  Chosen for a few short requests.
//  * phased (here): draft positions breadth-first in phases, every kernel
//    spreading its work over the whole GPU.  Chosen otherwise, and for every
//    call with top-k / top-p:
//
//   phase_kernel 1  row statistics of positions [0, P1) of every request, one
//                   workgroup per (row, V-chunk) (row_pass.hpp).
//   scan_kernel 1   one wavefront per request: accept tests, first rejection,
//                   greedy output or race record (scan.hpp).
//   phase_kernel 2  row statistics of positions [P1, K] of the requests still
//                   active, interleaved in the same grid with the exponential
//                   race of the requests decided in phase 1 (race.hpp):
//                   streaming-bound and ALU-bound work overlap on the CUs.
//   scan_kernel 2
//   phase_kernel    the race of the requests decided in the last phase.
//   emit_kernel     one wavefront per random request: chunk winners -> token,
//                   output row.
//
//   With top-k / top-p, filter_scan_kernel takes each scan_kernel's place: a
//   workgroup per row of the phase finds the row's threshold and kept mass
//   (filter.hpp), and the last one of each request runs its scan.
//
// No path reads the rows behind a request's first rejection: drafts behind a
// rejected one are discarded [第12章 投机解码：以小博大 §12.9; vllm v1 源码精读（五）
// §7], so those rows cannot change the output (one phase reads every row).
//
// All accesses are bounded by the host-checked sizes; requests with
// out-of-range metadata are written as invalid instead of being read.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "filter.hpp"
#include "philox.hpp"
#include "race.hpp"
#include "request_path.hpp"
#include "row_pass.hpp"
#include "rs_verify.h"
#include "scan.hpp"
#include "ngram.hpp"
#include "stats.hpp"
#include "stream_path.hpp"
#include "tree.hpp"

namespace rsv {

constexpr size_t kRegionAlign = 256;
constexpr int kPathRequest = 1, kPathPhased = 2, kPathStream = 3;
// Automatic path choice, from timings of every path over batch sizes 1-512,
// draft lengths 3-8 and vocabularies of 1024-151936 on one MI355X:
//  * per-request when the batch is tiny and each request's serial walk is at
//    most kRequestMaxSteps batches of loads (the others pay ~30 us of launches);
//  * stream, with rows in 16-vector chunks, when the logits total at most
//    kStreamSmallBytes (launch-bound: 3 launches against the phased path's 6)
//    or the chunks give at least kStreamMinTasksPerPosition row tasks per
//    position;
//  * phased otherwise (mid-size batches, where too few row tasks per position
//    leave the stream kernel's decisions too little work to overlap).
constexpr int64_t kStreamMinTasksPerPosition = 512;
constexpr int64_t kStreamSmallBytes = 128ll << 20;
// A filtered call (phased path) runs one phase when the logits total at most
// this: reading every row costs less than the second phase's launches and
// its filter kernel's serial tail (measured: B=8 V=32000 top-k 50 57 -> 32 us;
// B=64 K=8 V=151936 top-p 0.9 248 -> 159 us; at 700 MB two phases win).
constexpr int64_t kFilterOnePhaseBytes = 256ll << 20;
constexpr int kRequestMaxBatch = 8;
constexpr int kRequestMaxSteps = 10;
constexpr int kTargetBlocks = 2048;  // enough workgroups to fill 256 CUs several times
constexpr int kMaxPhases = 4;

// ------------------------------------------------------------ phase kernel
// Grid: n_row row tasks (chunk fastest, then position, then request, so
// consecutive workgroups stream consecutive memory) and n_race race tasks
// (chunk fastest, then request), interleaved one for one while both last.
template <typename Elem, int NV, int TPT>
__global__ __launch_bounds__(kRowThreads) void phase_kernel(
    const Elem* __restrict__ logits, const float* __restrict__ q, const int32_t* __restrict__ draft,
    const int32_t* __restrict__ cu, const float* __restrict__ temperature, int32_t greedy_all, int32_t D,
    int32_t max_k, int32_t V, uint64_t seed, int32_t j_begin, int32_t j_count, int32_t nsplit, int32_t n_row,
    int32_t race_chunks, int32_t n_race, int32_t race_phase, RowPartial* __restrict__ partials,
    Gathered* __restrict__ gath, const ReqRecord* __restrict__ records, unsigned long long* __restrict__ cand,
    const int32_t* __restrict__ top_k, const float* __restrict__ top_p, float* __restrict__ tmaxbuf,
    uint32_t* __restrict__ req_count) {
  const int32_t id = blockIdx.x;
  const int32_t both = min(n_row, n_race);
  int32_t t;
  bool is_row;
  if (id < 2 * both) {
    is_row = (id & 1) == 0;
    t = id >> 1;
  } else {
    t = both + (id - 2 * both);
    is_row = n_row > both;
  }
  if (is_row) {
    __builtin_amdgcn_s_setprio(1);  // row waves ahead of race waves on a SIMD, as in the stream kernel
    const int32_t c = t % nsplit;
    const int32_t rest = t / nsplit;
    const int32_t j = j_begin + rest % j_count;
    const int32_t b = rest / j_count;
    // the filter kernel after this one counts its workgroups per request here
    if (req_count && c == 0 && j == j_begin && threadIdx.x == 0) req_count[b] = 0u;
    const int32_t s = cu[b], e = cu[b + 1];
    if (!request_valid(s, e, D, max_k) || j > e - s) return;
    if (j_begin > 0 && records[b].mode != kModeActive) return;
    const float T = greedy_all ? 0.f : temperature[b];
    int32_t xstar = -1;
    if (c == 0 && j < e - s && T > 0.f) {
      xstar = draft[s + j];
      if (xstar >= V) xstar = -1;
    }
    const int64_t row = (int64_t)s + b + j;
    // a filtered row also leaves its segment maxima for the filter kernel
    float* tmax = (T > 0.f && filter_on(top_k, top_p, b, V)) ? tmaxbuf + (row * nsplit + c) * kRowThreads : nullptr;
    chunk_task<Elem, NV>(logits, q, row, T, V, nsplit, c, xstar, (int64_t)s + j, partials + row * nsplit, gath,
                         tmax);
  } else {
    const int32_t c = t % race_chunks;
    const int32_t b = t / race_chunks;
    const ReqRecord rec = records[b];
    if (rec.mode == kModeDone || rec.mode == kModeActive || rec.phase != race_phase) return;
    const unsigned long long packed = race_chunk<Elem, TPT>(logits, q, V, seed, rec, b, c);
    if (threadIdx.x == 0) cand[(int64_t)b * race_chunks + c] = packed;
  }
}

// ------------------------------------------------------------- scan kernel
template <typename Elem>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    const float* __restrict__ q, const int32_t* __restrict__ draft, const int32_t* __restrict__ cu,
    const float* __restrict__ temperature, int32_t greedy_all, int32_t D, int32_t max_k, int32_t V, int32_t nsplit,
    uint64_t seed, const RowPartial* __restrict__ partials, const Gathered* __restrict__ gath, int32_t j_begin,
    int32_t j_end, int32_t phase, ReqRecord* __restrict__ records, int32_t* __restrict__ out,
    int32_t* __restrict__ num_accepted, double* __restrict__ dbg_p, const int32_t* __restrict__ top_k,
    const float* __restrict__ top_p, const FilterRec* __restrict__ frec) {
  scan_phase<Elem>(blockIdx.x, q, draft, cu, temperature, greedy_all, D, max_k, V, nsplit, seed, partials, gath,
                   j_begin, j_end, phase, records, out, num_accepted, dbg_p, top_k, top_p, frec);
}

// ------------------------------------------------- filter + scan kernel
// Calls with top-k / top-p: one workgroup per (request, position) row of the
// phase computes the row's filter record; the last of a request's j_count
// workgroups to finish then runs the request's scan with its first
// wavefront (req_count[b], zeroed by the phase's row pass, counts them).
// Each record is stored agent-coherent and acknowledged before its
// workgroup arrives; the scan loads the records coherently.
template <typename Elem>
__global__ __launch_bounds__(kFilterThreads) void filter_scan_kernel(
    const Elem* __restrict__ logits, const float* __restrict__ q, const int32_t* __restrict__ draft,
    const int32_t* __restrict__ cu, const float* __restrict__ temperature, const int32_t* __restrict__ top_k,
    const float* __restrict__ top_p, int32_t D, int32_t max_k, int32_t V, int32_t j_begin, int32_t j_count,
    int32_t phase, int32_t nsplit, uint64_t seed, const RowPartial* __restrict__ partials,
    const Gathered* __restrict__ gath, const float* __restrict__ tmax, ReqRecord* __restrict__ records,
    FilterRec* __restrict__ frec, uint32_t* __restrict__ req_count, int32_t* __restrict__ out,
    int32_t* __restrict__ num_accepted, double* __restrict__ dbg_p) {
  filter_row<Elem>(logits, cu, temperature, top_k, top_p, D, max_k, V, j_begin, j_count, nsplit, records, partials,
                   tmax, frec);
  if (threadIdx.x >= 64) return;
  const int32_t b = (int32_t)(blockIdx.x / j_count);
  int last = 0;
  if (threadIdx.x == 0) last = arrive_last(req_count + b, (uint32_t)j_count) ? 1 : 0;
  if (!__shfl(last, 0)) return;
  scan_phase<Elem, true>(b, q, draft, cu, temperature, 0, D, max_k, V, nsplit, seed, partials, gath, j_begin,
                         j_begin + j_count, phase, records, out, num_accepted, dbg_p, top_k, top_p, frec);
}

// ------------------------------------------------------------- emit kernel
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
  // The chunk winners and the record only depend on b: load them together.
  unsigned long long win = 0ull;
  for (int32_t c = lane; c < nchunks; c += 64) {
    const unsigned long long v = cand[(int64_t)b * nchunks + c];
    win = v > win ? v : win;
  }
  const ReqRecord rec = records[b];
  if (rec.mode == kModeDone || rec.mode == kModeActive) return;
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

// -------------------------------------------------- debug: full p per row
// p (p' with top-k / top-p) in the fp32 form the race uses, for every row of
// every random request (every row is streamed: the call runs one phase).
template <typename Elem>
__global__ __launch_bounds__(256) void probs_kernel(const Elem* __restrict__ logits, const int32_t* __restrict__ cu,
                                                    const float* __restrict__ temperature, int32_t D, int32_t max_k,
                                                    int32_t V, int32_t nsplit, const RowPartial* __restrict__ partials,
                                                    float* __restrict__ probs, const int32_t* __restrict__ top_k,
                                                    const float* __restrict__ top_p,
                                                    const FilterRec* __restrict__ frec) {
  const int32_t j = blockIdx.x % (max_k + 1);
  const int32_t b = blockIdx.x / (max_k + 1);
  const int32_t s = cu[b], e = cu[b + 1];
  if (!request_valid(s, e, D, max_k) || j > e - s) return;
  const float T = temperature[b];
  if (!(T > 0.f)) return;
  const float cs = scale_of(T);
  const int64_t row = (int64_t)s + b + j;
  float shift, tau = -INFINITY;
  double S;
  if (filter_on(top_k, top_p, b, V)) {
    const FilterRec f = frec[row];
    shift = f.shift;
    S = f.sum;
    tau = f.tau;
  } else {
    merge_random(partials + row * nsplit, nsplit, shift, S);
  }
  const float inv = (float)(1.0 / S);
  for (int32_t x = threadIdx.x; x < V; x += 256) {
    const float l = to_f32(logits[row * V + x]);
    probs[row * V + x] = l >= tau ? exp2_hw(fmaf(l, cs, -shift)) * inv : 0.f;
  }
}

// ---------------------------------------------------------------- host side
struct Plan {
  int W, nvec_max;
  int nsplit_max;       // partial slots per row in the workspace
  int row_nv, nsplit;   // this launch
  int race_tpt, race_chunks;
  int race_chunks_max;  // candidate slots per request in the workspace
  int path;             // kPathRequest, kPathPhased or kPathStream
  int request_nt;       // threads per per-request workgroup
  int nphases;
  int bounds[kMaxPhases + 1];
  int stream_lead;      // stream path: positions streamed before races interleave
  size_t off_partials, off_gath, off_records, off_cand;
  size_t off_row_count, off_masks, off_state, off_race_ctl, off_queue, off_tail, off_frec, off_tmax, total;
};

static size_t align_up(size_t v) { return (v + kRegionAlign - 1) / kRegionAlign * kRegionAlign; }

static int nsplit_for(int nvec_max, int nv) {
  const int cv = nv * kRowThreads;
  const int n = (nvec_max + cv - 1) / cv;
  return n < 1 ? 1 : n;
}

// End of automatic phase k (1-based) for L = max_k + 1 positions; 0 = none.
// Two phases: [0, ceil(L/3)) and the rest.
static int auto_phase_end(int L, int k) {
  if (L < 3) return 0;
  return k == 1 ? (L + 2) / 3 : 0;
}

// Sizes are assumed validated (B >= 1, V >= 1, 0 <= max_k <= 32, 0 <= D <= B * max_k).
static bool make_plan(int32_t B, int32_t D, int32_t max_k, int32_t V, rs_dtype dt, const rs_debug* dbg,
                      bool filtered, Plan& p) {
  const int force_nv = dbg ? dbg->row_vectors_per_thread : 0;
  const int force_tpt = dbg ? dbg->race_tokens_per_thread : 0;
  const int force_path = dbg ? dbg->sampling_path : 0;
  p.W = dt == RS_BF16 ? 8 : 4;
  p.nvec_max = V / p.W;
  p.nsplit_max = nsplit_for(p.nvec_max, 1);
  const int64_t R = (int64_t)D + B;
  if (filtered) {
    p.row_nv = kSegVectors;  // the filter kernel reads the row tasks' segments of 16 vectors per thread
  } else if (force_nv) {
    p.row_nv = force_nv;
  } else {
    p.row_nv = 1;
    for (int nv : {16, 4}) {
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
    const int64_t chunks32 = ((int64_t)V + kRaceThreads * 32 - 1) / (kRaceThreads * 32);
    p.race_tpt = (int64_t)B * chunks32 >= kTargetBlocks ? 32 : 8;
  }
  p.race_chunks = (int)(((int64_t)V + kRaceThreads * p.race_tpt - 1) / (kRaceThreads * p.race_tpt));
  p.race_chunks_max = (int)(((int64_t)V + kRaceThreads * 8 - 1) / (kRaceThreads * 8));
  if ((dbg && dbg->probs) || filtered)
    p.path = kPathPhased;  // full probabilities need every row (one phase); filters run per phase
  else if (force_path)
    p.path = force_path == 1 ? kPathRequest : force_path == 3 ? kPathStream : kPathPhased;
  else
    p.path = kPathPhased;  // chosen below
  p.request_nt = V >= 65536 ? 1024 : 256;
  if (!force_path && !(dbg && dbg->probs) && !filtered) {
    const int64_t per_pass = (int64_t)p.request_nt * kRequestNVP;
    const int64_t steps = (int64_t)(max_k + 1) * ((p.nvec_max + per_pass - 1) / per_pass);
    const int64_t split16 = nsplit_for(p.nvec_max, kSegVectors);  // row tasks per row in 16-vector chunks
    const bool small = R * (int64_t)V * (dt == RS_BF16 ? 2 : 4) <= kStreamSmallBytes;
    if (B <= kRequestMaxBatch && steps <= kRequestMaxSteps) {
      p.path = kPathRequest;
    } else if (small || (p.row_nv == kSegVectors && (int64_t)B * split16 >= kStreamMinTasksPerPosition)) {
      p.path = kPathStream;
    } else {
      p.path = kPathPhased;
    }
  }
  if (p.path == kPathStream && !force_nv) {  // the stream path's row tasks: 16-vector chunks
    p.row_nv = kSegVectors;
    p.nsplit = nsplit_for(p.nvec_max, kSegVectors);
  }
  // Phases: position ranges [bounds[i], bounds[i+1]).  A request decided in
  // one phase never has the rows of later phases read.  Full probabilities
  // need every row, so they force one phase.
  const int L = max_k + 1;
  p.nphases = 0;
  p.bounds[0] = 0;
  const int32_t* ends = dbg ? dbg->phase_ends : nullptr;
  if (dbg && dbg->probs) {
    // one phase
  } else if (ends && ends[0] != 0) {
    for (int k = 0; k < kMaxPhases - 1 && ends[0] > 0; ++k) {
      if (ends[k] <= p.bounds[p.nphases] || ends[k] >= L) break;
      p.bounds[++p.nphases] = ends[k];
    }
  } else if (filtered && R * (int64_t)V * (dt == RS_BF16 ? 2 : 4) <= kFilterOnePhaseBytes) {
    // one phase
  } else {
    for (int k = 1; k < kMaxPhases; ++k) {  // automatic split
      const int e = auto_phase_end(L, k);
      if (e <= p.bounds[p.nphases] || e >= L) break;
      p.bounds[++p.nphases] = e;
    }
  }
  p.bounds[++p.nphases] = L;
  // Stream path: by default every row task precedes the race tasks (row
  // tasks of already-decided requests race in their place meanwhile).
  p.stream_lead = (ends && ends[0] > 0 && ends[0] < L) ? ends[0] : L;
  p.off_partials = 0;
  p.off_gath = align_up((size_t)R * p.nsplit_max * sizeof(RowPartial));
  p.off_records = p.off_gath + align_up((size_t)(D > 0 ? D : 1) * sizeof(Gathered));
  p.off_cand = p.off_records + align_up((size_t)B * sizeof(ReqRecord));
  p.off_row_count = p.off_cand + align_up((size_t)B * p.race_chunks_max * sizeof(unsigned long long));
  p.off_masks = p.off_row_count + align_up((size_t)R * sizeof(uint32_t));
  p.off_state = p.off_masks + align_up((size_t)B * 2 * sizeof(unsigned long long));
  p.off_race_ctl = p.off_state + align_up((size_t)B * sizeof(int32_t));
  p.off_queue = p.off_race_ctl + align_up((size_t)B * kRaceCtlStride * sizeof(uint32_t));
  p.off_tail = p.off_queue + align_up((size_t)B * sizeof(int32_t));
  p.off_frec = p.off_tail + kRegionAlign;
  p.off_tmax = p.off_frec + align_up((size_t)R * sizeof(FilterRec));
  p.total = p.off_tmax + (filtered ? align_up((size_t)R * p.nsplit * kRowThreads * sizeof(float)) : 0);
  // 1-D grids must stay below 2^31 workgroups.
  return (int64_t)p.nsplit * L * B + (int64_t)p.race_chunks * B < INT32_MAX;
}

static bool sizes_ok(int32_t B, int32_t D, int32_t max_k, int32_t V) {
  return B >= 1 && V >= 1 && max_k >= 0 && max_k <= RS_MAX_SPEC_LEN && D >= 0 && (int64_t)D <= (int64_t)B * max_k;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Records events[k] after the k-th kernel (events[0] before the first).
struct EventLog {
  const rs_debug* dbg;
  int launched = 0;
  bool ok = true;
  void mark(hipStream_t stream) {
    if (dbg && dbg->events && launched < dbg->num_events)
      ok = ok && hipEventRecord(dbg->events[launched], stream) == hipSuccess;
  }
  bool after_kernel(hipStream_t stream) {
    if (hipGetLastError() != hipSuccess) return false;
    ++launched;
    mark(stream);
    return ok;
  }
};

struct PhaseArgs {
  int32_t j_begin, j_count, nsplit, n_row, race_chunks, n_race, race_phase;
};

template <typename Elem, int NV, int TPT>
static void launch_phase(hipStream_t stream, const Elem* logits, const float* q, const int32_t* draft,
                         const int32_t* cu, const float* temperature, int greedy_all, int32_t D, int32_t max_k,
                         int32_t V, uint64_t seed, const PhaseArgs& a, RowPartial* partials, Gathered* gath,
                         const ReqRecord* records, unsigned long long* cand, const int32_t* top_k,
                         const float* top_p, float* tmax, uint32_t* req_count) {
  phase_kernel<Elem, NV, TPT><<<(unsigned)(a.n_row + a.n_race), kRowThreads, 0, stream>>>(
      logits, q, draft, cu, temperature, greedy_all, D, max_k, V, seed, a.j_begin, a.j_count, a.nsplit, a.n_row,
      a.race_chunks, a.n_race, a.race_phase, partials, gath, records, cand, top_k, top_p, tmax, req_count);
}

template <typename Elem>
static bool dispatch_phase(int nv, int tpt, hipStream_t stream, const Elem* logits, const float* q,
                           const int32_t* draft, const int32_t* cu, const float* temperature, int greedy_all,
                           int32_t D, int32_t max_k, int32_t V, uint64_t seed, const PhaseArgs& a,
                           RowPartial* partials, Gathered* gath, const ReqRecord* records, unsigned long long* cand,
                           const int32_t* top_k, const float* top_p, float* tmax, uint32_t* req_count) {
#define RS_PHASE(NV, TPT)                                                                                           \
  if (nv == NV && tpt == TPT) {                                                                                     \
    launch_phase<Elem, NV, TPT>(stream, logits, q, draft, cu, temperature, greedy_all, D, max_k, V, seed, a,        \
                                partials, gath, records, cand, top_k, top_p, tmax, req_count);                      \
    return true;                                                                                                    \
  }
  RS_PHASE(16, 32)
  RS_PHASE(16, 8)
  RS_PHASE(4, 32)
  RS_PHASE(4, 8)
  RS_PHASE(1, 32)
  RS_PHASE(1, 8)
#undef RS_PHASE
  return false;
}

template <typename Elem, int NV, int TPT>
static bool launch_stream_kernels(StreamArgs<Elem>& a, hipStream_t stream, EventLog& evl) {
  stream_kernel<Elem, NV, TPT><<<(unsigned)a.n_tasks, kRowThreads, 0, stream>>>(a);
  if (!evl.after_kernel(stream)) return false;
  if (a.n_race > 0) {
    stream_race_tail_kernel<Elem, TPT><<<(unsigned)a.B, kRaceThreads, 0, stream>>>(a);
    if (!evl.after_kernel(stream)) return false;
  }
  return true;
}

// 1: launched, 0: a launch failed, -1: no such variant.
template <typename Elem>
static int dispatch_stream(int nv, int tpt, StreamArgs<Elem>& a, hipStream_t stream, EventLog& evl) {
#define RS_STREAM(NV, TPT) \
  if (nv == NV && tpt == TPT) return launch_stream_kernels<Elem, NV, TPT>(a, stream, evl) ? 1 : 0;
  RS_STREAM(16, 32)
  RS_STREAM(16, 8)
  RS_STREAM(4, 32)
  RS_STREAM(4, 8)
  RS_STREAM(1, 32)
  RS_STREAM(1, 8)
#undef RS_STREAM
  return -1;
}

template <typename Elem>
static rs_status launch(const void* logits_v, const float* q, const int32_t* draft, const int32_t* cu,
                        const float* temperature, const int32_t* top_k, const float* top_p, int greedy_all, int32_t B,
                        int32_t D, int32_t max_k, int32_t V, uint64_t seed, int32_t* out, int32_t* nacc, void* ws,
                        const Plan& p, const rs_debug* dbg, hipStream_t stream) {
  const Elem* logits = static_cast<const Elem*>(logits_v);
  char* w = static_cast<char*>(ws);
  RowPartial* partials = reinterpret_cast<RowPartial*>(w + p.off_partials);
  Gathered* gath = reinterpret_cast<Gathered*>(w + p.off_gath);
  ReqRecord* records = reinterpret_cast<ReqRecord*>(w + p.off_records);
  unsigned long long* cand = reinterpret_cast<unsigned long long*>(w + p.off_cand);
  FilterRec* frec = reinterpret_cast<FilterRec*>(w + p.off_frec);
  float* tmax = reinterpret_cast<float*>(w + p.off_tmax);
  const bool filtered = !greedy_all && (top_k || top_p);
  // the phased path's per-request filter arrivals reuse the stream path's row counters
  uint32_t* req_count = filtered ? reinterpret_cast<uint32_t*>(w + p.off_row_count) : nullptr;
  double* dbg_p = dbg ? dbg->draft_target_prob : nullptr;
  EventLog evl{dbg};
  evl.mark(stream);

  if (p.path == kPathStream) {
    StreamArgs<Elem> a;
    a.logits = logits;
    a.q = q;
    a.draft = draft;
    a.cu = cu;
    a.temperature = temperature;
    a.seed = seed;
    a.greedy_all = greedy_all;
    a.B = B;
    a.D = D;
    a.max_k = max_k;
    a.V = V;
    a.nsplit = p.nsplit;
    a.race_chunks = p.race_chunks;
    a.n_rows = (int64_t)(max_k + 1) * B * p.nsplit;
    a.n_lead = (int64_t)p.stream_lead * B * p.nsplit;
    a.n_race = greedy_all ? 0 : (int64_t)B * p.race_chunks;
    a.n_tasks = a.n_rows + a.n_race;
    a.partials = partials;
    a.gath = gath;
    a.records = records;
    a.cand = cand;
    a.row_count = reinterpret_cast<uint32_t*>(w + p.off_row_count);
    a.masks = reinterpret_cast<unsigned long long*>(w + p.off_masks);
    a.state = reinterpret_cast<int32_t*>(w + p.off_state);
    a.race_ctl = reinterpret_cast<uint32_t*>(w + p.off_race_ctl);
    a.queue = reinterpret_cast<int32_t*>(w + p.off_queue);
    a.tail = reinterpret_cast<uint32_t*>(w + p.off_tail);
    a.out = out;
    a.nacc = nacc;
    a.dbg_p = dbg_p;
    stream_init_kernel<<<(unsigned)B, 64, 0, stream>>>(draft, cu, B, D, max_k, V, a.row_count, a.masks, a.state,
                                                       a.race_ctl, a.queue, a.tail, out, nacc);
    if (!evl.after_kernel(stream)) return RS_ERR_HIP;
    const int launched = dispatch_stream<Elem>(p.row_nv, p.race_tpt, a, stream, evl);
    if (launched < 0) return RS_ERR_INVALID_ARG;
    if (launched == 0) return RS_ERR_HIP;
  } else if (p.path == kPathRequest) {
    if (p.request_nt == 1024)
      request_kernel<Elem, 1024><<<(unsigned)B, 1024, 0, stream>>>(logits, q, draft, cu, temperature, greedy_all, D,
                                                                  max_k, V, seed, out, nacc, dbg_p);
    else
      request_kernel<Elem, 256><<<(unsigned)B, 256, 0, stream>>>(logits, q, draft, cu, temperature, greedy_all, D,
                                                                max_k, V, seed, out, nacc, dbg_p);
    if (!evl.after_kernel(stream)) return RS_ERR_HIP;
  } else {
    for (int ph = 1; ph <= p.nphases; ++ph) {
      PhaseArgs a;
      a.j_begin = p.bounds[ph - 1];
      a.j_count = p.bounds[ph] - p.bounds[ph - 1];
      a.nsplit = p.nsplit;
      a.n_row = p.nsplit * a.j_count * B;
      a.race_chunks = p.race_chunks;
      a.n_race = (ph >= 2 && !greedy_all) ? p.race_chunks * B : 0;
      a.race_phase = ph - 1;
      if (!dispatch_phase<Elem>(p.row_nv, p.race_tpt, stream, logits, q, draft, cu, temperature, greedy_all, D,
                                max_k, V, seed, a, partials, gath, records, cand, top_k, top_p,
                                filtered ? tmax : nullptr, req_count))
        return RS_ERR_INVALID_ARG;
      if (!evl.after_kernel(stream)) return RS_ERR_HIP;
      if (filtered) {  // thresholds and kept mass of this phase's rows, then the scans
        filter_scan_kernel<Elem><<<(unsigned)(a.j_count * B), kFilterThreads, 0, stream>>>(
            logits, q, draft, cu, temperature, top_k, top_p, D, max_k, V, a.j_begin, a.j_count, ph, p.nsplit, seed,
            partials, gath, tmax, records, frec, req_count, out, nacc, dbg_p);
      } else {
        scan_kernel<Elem><<<(unsigned)B, kScanThreads, 0, stream>>>(q, draft, cu, temperature, greedy_all, D, max_k,
                                                                    V, p.nsplit, seed, partials, gath, a.j_begin,
                                                                    p.bounds[ph], ph, records, out, nacc, dbg_p,
                                                                    top_k, top_p, frec);
      }
      if (!evl.after_kernel(stream)) return RS_ERR_HIP;
      if (dbg && dbg->probs && !greedy_all) {
        probs_kernel<Elem><<<(unsigned)((max_k + 1) * B), 256, 0, stream>>>(
            logits, cu, temperature, D, max_k, V, p.nsplit, partials, dbg->probs, top_k, top_p, frec);
        if (!evl.after_kernel(stream)) return RS_ERR_HIP;
      }
    }
    if (!greedy_all) {  // race of the requests decided in the last phase, then the output rows
      PhaseArgs a;
      a.j_begin = 0;
      a.j_count = 1;
      a.nsplit = p.nsplit;
      a.n_row = 0;
      a.race_chunks = p.race_chunks;
      a.n_race = p.race_chunks * B;
      a.race_phase = p.nphases;
      if (!dispatch_phase<Elem>(p.row_nv, p.race_tpt, stream, logits, q, draft, cu, temperature, greedy_all, D,
                                max_k, V, seed, a, partials, gath, records, cand, top_k, top_p, nullptr, nullptr))
        return RS_ERR_INVALID_ARG;
      if (!evl.after_kernel(stream)) return RS_ERR_HIP;
      emit_kernel<Elem><<<(unsigned)B, 64, 0, stream>>>(logits, draft, max_k, V, p.race_chunks, seed, records, cand,
                                                        out, nacc);
      if (!evl.after_kernel(stream)) return RS_ERR_HIP;
    }
  }
  if (dbg && dbg->kernels_launched) *dbg->kernels_launched = evl.launched;
  if (dbg && dbg->path_taken) *dbg->path_taken = p.path;
  return RS_OK;
}

// ---------------------------------------------------- library-owned scratch
// rs_verify_noalloc's workspace: one array per GPU, in the library's code
// object, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory; its device address is looked up once
// per device (hipGetSymbolAddress, with that device current) and only that
// address is ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[RS_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_addr[kMaxDevices];

// Device address of the current device's scratch array.
static rs_status library_scratch(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return RS_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return RS_ERR_UNSUPPORTED;
  void* a = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!a) {
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return RS_ERR_HIP;
    g_scratch_addr[dev].store(a, std::memory_order_release);  // racing first calls store the same address
  }
  *addr = a;
  return RS_OK;
}

static rs_status verify_impl(const void* logits, rs_dtype dt, const float* q, const int32_t* draft, const int32_t* cu,
                             const float* temperature, const int32_t* top_k, const float* top_p, int greedy_all,
                             int32_t B, int32_t D, int32_t max_k, int32_t V, uint64_t seed, int32_t* out,
                             int32_t* nacc, void* ws, size_t ws_bytes, const rs_debug* dbg, hipStream_t stream,
                             bool lib_scratch = false) {
  // Every check below runs before the first HIP call.
  if (B < 0 || D < 0 || V < 1 || max_k < 0) return RS_ERR_INVALID_ARG;
  if (dt != RS_F32 && dt != RS_BF16) return RS_ERR_UNSUPPORTED;
  if (B == 0) return RS_OK;
  if (!sizes_ok(B, D, max_k, V)) return RS_ERR_INVALID_ARG;
  if (!logits || !cu || !out || !nacc || (D > 0 && !draft) || (!greedy_all && !temperature))
    return RS_ERR_INVALID_ARG;
  const size_t es = dt == RS_BF16 ? 2 : 4;
  if (!aligned(logits, es) || (q && !aligned(q, 4)) || !aligned(cu, 4) || !aligned(out, 4) || !aligned(nacc, 4) ||
      (draft && !aligned(draft, 4)) || (temperature && !aligned(temperature, 4)) || (top_k && !aligned(top_k, 4)) ||
      (top_p && !aligned(top_p, 4)))
    return RS_ERR_UNSUPPORTED;
  // fixed-point masses of the top-p selection stay below 2^64 for V < 2^20
  if ((top_k || top_p) && V >= (1 << 20)) return RS_ERR_UNSUPPORTED;
  if (dbg) {
    const int nv = dbg->row_vectors_per_thread, tpt = dbg->race_tokens_per_thread;
    if (!(nv == 0 || nv == 1 || nv == 4 || nv == 16)) return RS_ERR_INVALID_ARG;
    if (!(tpt == 0 || tpt == 8 || tpt == 32)) return RS_ERR_INVALID_ARG;
    if (dbg->sampling_path < 0 || dbg->sampling_path > 3) return RS_ERR_INVALID_ARG;
    if (dbg->num_events < 0 || (dbg->num_events > 0 && !dbg->events)) return RS_ERR_INVALID_ARG;
    if ((dbg->draft_target_prob && !aligned(dbg->draft_target_prob, 8)) || (dbg->probs && !aligned(dbg->probs, 4)))
      return RS_ERR_UNSUPPORTED;
  }
  Plan p;
  if (!make_plan(B, D, max_k, V, dt, dbg, !greedy_all && (top_k || top_p), p)) return RS_ERR_UNSUPPORTED;
  if (lib_scratch) {  // the library's own array instead of a caller's workspace
    if (p.total > RS_NOALLOC_SCRATCH_BYTES) return RS_ERR_WORKSPACE;
    const rs_status st = library_scratch(&ws);
    if (st != RS_OK) return st;
    ws_bytes = RS_NOALLOC_SCRATCH_BYTES;
  }
  if (!ws || !aligned(ws, 16) || ws_bytes < p.total) return RS_ERR_WORKSPACE;
  if (dt == RS_BF16)
    return launch<uint16_t>(logits, q, draft, cu, temperature, top_k, top_p, greedy_all, B, D, max_k, V, seed, out,
                            nacc, ws, p, dbg, stream);
  return launch<float>(logits, q, draft, cu, temperature, top_k, top_p, greedy_all, B, D, max_k, V, seed, out, nacc,
                       ws, p, dbg, stream);
}

// Tree workspace: walk words, per-step arrival counters and partial
// statistics (for up to RS_MAX_TREE_NODES + 1 steps), race winners, records.
struct TreeLayout {
  int32_t nsplit_max, race_chunks;
  size_t off_mail, off_count, off_race_count, off_partials, off_cand, total;
};

// Row chunks of a row: 16-byte vectors per row over vectors per chunk (nv per thread).
template <typename Elem>
static int32_t tree_nsplit(int32_t vocab, int nv) {
  const int64_t nvec = vocab / Vec<Elem>::W;
  return (int32_t)std::max<int64_t>(1, (nvec + nv * kRowThreads - 1) / (nv * kRowThreads));
}

static TreeLayout tree_layout(int32_t batch, int32_t vocab) {
  TreeLayout t;
  t.nsplit_max = tree_nsplit<float>(vocab, kTreeNV);  // fp32 rows at the smaller chunks have the most
  constexpr int32_t kChunk = kRaceThreads * kTreeRaceTPT;
  t.race_chunks = (vocab + kChunk - 1) / kChunk;
  const size_t B = (size_t)batch;
  t.off_mail = 0;
  t.off_count = align_up(B * kMailboxWords * sizeof(unsigned long long));
  t.off_race_count = t.off_count + align_up(B * kTreeRows * sizeof(uint32_t));
  t.off_partials = t.off_race_count + align_up(B * sizeof(uint32_t));
  t.off_cand = t.off_partials + align_up(B * kTreeRows * (size_t)t.nsplit_max * sizeof(RowPartial));
  t.total = t.off_cand + align_up(B * (size_t)t.race_chunks * sizeof(unsigned long long));
  return t;
}

// Workgroups the device holds at once for the walk kernel (queried once per
// device, element type and chunk size).
template <typename Elem, int NV>
static int64_t tree_resident() {
  static int64_t cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, tree_walk_kernel<Elem, NV>, kRowThreads, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu < 1 ||
        cus < 1)
      return 256;
    cached[dev] = (int64_t)per_cu * cus;
  }
  return cached[dev];
}

template <typename Elem>
static rs_status launch_tree(const void* logits, const float* q, const int32_t* node_tokens,
                             const int32_t* node_parents, const int32_t* cu, const float* temperature, int32_t B, int32_t N, int32_t max_nodes,
                             int32_t max_depth, int32_t V, uint64_t seed, int32_t* out, int32_t* path,
                             int32_t* nacc, void* ws, hipStream_t stream) {
  const TreeLayout t = tree_layout(B, V);
  char* w = static_cast<char*>(ws);
  TreeArgs<Elem> a;
  a.logits = static_cast<const Elem*>(logits);
  a.q = q;
  a.tokens = node_tokens;
  a.parents = node_parents;
  a.cu = cu;
  a.temperature = temperature;
  a.seed = seed;
  a.B = B;
  a.N = N;
  a.max_nodes = max_nodes;
  a.max_depth = max_depth;
  a.V = V;
  a.race_chunks = t.race_chunks;
  // K workgroups per request, enough to fill the device once (any of a
  // request's workgroups can take any of its chunks, so none waits on one
  // that is not resident).
  auto per_request = [&](int64_t resident) {
    return (int32_t)std::max<int64_t>(1, std::min<int64_t>(kTreeMaxK, resident / B));
  };
  a.K = per_request(tree_resident<Elem, kTreeNV>());
  bool wide = false;
  if constexpr (sizeof(Elem) == 2) {
    if (a.K <= kTreeWideK) {
      wide = true;
      a.K = per_request(tree_resident<Elem, kTreeNVWide>());
    }
  }
  a.nsplit = tree_nsplit<Elem>(V, wide ? kTreeNVWide : kTreeNV);
  a.out = out;
  a.path = path;
  a.nacc = nacc;
  a.mail = reinterpret_cast<unsigned long long*>(w + t.off_mail);
  a.count = reinterpret_cast<uint32_t*>(w + t.off_count);
  a.race_count = reinterpret_cast<uint32_t*>(w + t.off_race_count);
  a.partials = reinterpret_cast<RowPartial*>(w + t.off_partials);
  a.cand = reinterpret_cast<unsigned long long*>(w + t.off_cand);
  tree_init_kernel<Elem><<<(unsigned)B, kRowThreads, 0, stream>>>(a);
  if (hipGetLastError() != hipSuccess) return RS_ERR_HIP;
  if constexpr (sizeof(Elem) == 2) {
    if (wide) {
      tree_walk_kernel<Elem, kTreeNVWide><<<(unsigned)((int64_t)B * a.K), kRowThreads, 0, stream>>>(a);
      return hipGetLastError() == hipSuccess ? RS_OK : RS_ERR_HIP;
    }
  }
  tree_walk_kernel<Elem, kTreeNV><<<(unsigned)((int64_t)B * a.K), kRowThreads, 0, stream>>>(a);
  return hipGetLastError() == hipSuccess ? RS_OK : RS_ERR_HIP;
}

}  // namespace rsv

extern "C" {

static size_t workspace_size(int32_t batch, int32_t total_draft_tokens, int32_t max_k, int32_t vocab,
                             rs_dtype logits_dtype, bool filtered) {
  if (logits_dtype != RS_F32 && logits_dtype != RS_BF16) return 0;
  if (batch == 0 && total_draft_tokens == 0 && vocab >= 1 && max_k >= 0 && max_k <= RS_MAX_SPEC_LEN) return 0;
  if (!rsv::sizes_ok(batch, total_draft_tokens, max_k, vocab)) return 0;
  rsv::Plan p;
  if (!rsv::make_plan(batch, total_draft_tokens, max_k, vocab, logits_dtype, nullptr, filtered, p)) return 0;
  return p.total;
}

size_t rs_verify_workspace_size(int32_t batch, int32_t total_draft_tokens, int32_t max_k, int32_t vocab,
                                rs_dtype logits_dtype) {
  return workspace_size(batch, total_draft_tokens, max_k, vocab, logits_dtype, false);
}

size_t rs_verify_filtered_workspace_size(int32_t batch, int32_t total_draft_tokens, int32_t max_k, int32_t vocab,
                                         rs_dtype logits_dtype) {
  return workspace_size(batch, total_draft_tokens, max_k, vocab, logits_dtype, true);
}

rs_status rs_verify(const void* target_logits, rs_dtype logits_dtype, const float* draft_probs,
                    const int32_t* draft_token_ids, const int32_t* cu_num_draft_tokens, const float* temperature,
                    int32_t batch, int32_t total_draft_tokens, int32_t max_k, int32_t vocab, uint64_t seed,
                    int32_t* output_token_ids, int32_t* num_accepted, void* workspace, size_t workspace_bytes,
                    const rs_debug* debug, hipStream_t stream) {
  return rsv::verify_impl(target_logits, logits_dtype, draft_probs, draft_token_ids, cu_num_draft_tokens, temperature,
                          nullptr, nullptr, 0, batch, total_draft_tokens, max_k, vocab, seed, output_token_ids,
                          num_accepted, workspace, workspace_bytes, debug, stream);
}

rs_status rs_verify_noalloc(const void* target_logits, rs_dtype logits_dtype, const float* draft_probs,
                            const int32_t* draft_token_ids, const int32_t* cu_num_draft_tokens,
                            const float* temperature, int32_t batch, int32_t total_draft_tokens, int32_t max_k,
                            int32_t vocab, uint64_t seed, int32_t* output_token_ids, int32_t* num_accepted,
                            const rs_debug* debug, hipStream_t stream) {
  return rsv::verify_impl(target_logits, logits_dtype, draft_probs, draft_token_ids, cu_num_draft_tokens, temperature,
                          nullptr, nullptr, 0, batch, total_draft_tokens, max_k, vocab, seed, output_token_ids,
                          num_accepted, nullptr, 0, debug, stream, true);
}

rs_status rs_verify_filtered(const void* target_logits, rs_dtype logits_dtype, const float* draft_probs,
                             const int32_t* draft_token_ids, const int32_t* cu_num_draft_tokens,
                             const float* temperature, const int32_t* top_k, const float* top_p, int32_t batch,
                             int32_t total_draft_tokens, int32_t max_k, int32_t vocab, uint64_t seed,
                             int32_t* output_token_ids, int32_t* num_accepted, void* workspace,
                             size_t workspace_bytes, const rs_debug* debug, hipStream_t stream) {
  return rsv::verify_impl(target_logits, logits_dtype, draft_probs, draft_token_ids, cu_num_draft_tokens, temperature,
                          top_k, top_p, 0, batch, total_draft_tokens, max_k, vocab, seed, output_token_ids,
                          num_accepted, workspace, workspace_bytes, debug, stream);
}

rs_status rs_verify_greedy(const void* target_logits, rs_dtype logits_dtype, const int32_t* draft_token_ids,
                           const int32_t* cu_num_draft_tokens, int32_t batch, int32_t total_draft_tokens,
                           int32_t max_k, int32_t vocab, int32_t* output_token_ids, int32_t* num_accepted,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return rsv::verify_impl(target_logits, logits_dtype, nullptr, draft_token_ids, cu_num_draft_tokens, nullptr,
                          nullptr, nullptr, 1, batch, total_draft_tokens, max_k, vocab, 0, output_token_ids,
                          num_accepted, workspace, workspace_bytes, nullptr, stream);
}

size_t rs_verify_tree_workspace_size(int32_t batch, int32_t vocab) {
  if (batch < 0 || vocab < 1) return 0;
  if (batch == 0) return 0;
  return rsv::tree_layout(batch, vocab).total;
}

rs_status rs_verify_tree(const void* target_logits, rs_dtype logits_dtype, const float* draft_probs,
                         const int32_t* node_tokens, const int32_t* node_parents, const int32_t* cu_num_nodes,
                         const float* temperature,
                         int32_t batch, int32_t total_nodes, int32_t max_nodes, int32_t max_depth, int32_t vocab,
                         uint64_t seed, int32_t* output_token_ids, int32_t* accepted_nodes, int32_t* num_accepted,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  // Every check below runs before the first launch.
  if (batch < 0 || total_nodes < 0 || vocab < 1 || max_nodes < 0 || max_depth < 0) return RS_ERR_INVALID_ARG;
  if (logits_dtype != RS_F32 && logits_dtype != RS_BF16) return RS_ERR_UNSUPPORTED;
  if (batch == 0) return RS_OK;
  if (max_nodes > RS_MAX_TREE_NODES || max_depth > max_nodes || (int64_t)total_nodes > (int64_t)batch * max_nodes)
    return RS_ERR_INVALID_ARG;
  if (!target_logits || !cu_num_nodes || !temperature || !output_token_ids || !num_accepted ||
      (max_depth > 0 && !accepted_nodes) || (total_nodes > 0 && (!node_tokens || !node_parents)))
    return RS_ERR_INVALID_ARG;
  const size_t es = logits_dtype == RS_BF16 ? 2 : 4;
  if (((uintptr_t)target_logits % es) || ((uintptr_t)node_tokens % 4) || ((uintptr_t)node_parents % 4) ||
      ((uintptr_t)cu_num_nodes % 4) || ((uintptr_t)temperature % 4) || ((uintptr_t)output_token_ids % 4) ||
      ((uintptr_t)accepted_nodes % 4) || ((uintptr_t)num_accepted % 4) || ((uintptr_t)draft_probs % 16))
    return RS_ERR_UNSUPPORTED;
  // entry words hold a row's chunk count in 24 bits; the grid, B * K <= max(B, resident), stays below 2^31
  const rsv::TreeLayout t = rsv::tree_layout(batch, vocab);
  if (t.nsplit_max >= (1 << 24) || t.race_chunks >= (1 << 24)) return RS_ERR_UNSUPPORTED;
  if (!workspace || ((uintptr_t)workspace % 16) || workspace_bytes < t.total) return RS_ERR_WORKSPACE;
  if (logits_dtype == RS_BF16)
    return rsv::launch_tree<uint16_t>(target_logits, draft_probs, node_tokens, node_parents, cu_num_nodes,
                                      temperature, batch, total_nodes, max_nodes, max_depth, vocab, seed,
                                      output_token_ids, accepted_nodes, num_accepted, workspace, stream);
  return rsv::launch_tree<float>(target_logits, draft_probs, node_tokens, node_parents, cu_num_nodes, temperature,
                                 batch, total_nodes, max_nodes, max_depth, vocab, seed, output_token_ids,
                                 accepted_nodes, num_accepted, workspace, stream);
}

rs_status rs_ngram_propose(const int32_t* context_token_ids, const int32_t* cu_context, int32_t batch,
                           int32_t total_context_tokens, int32_t min_n, int32_t max_n, int32_t k,
                           int64_t max_model_len, int32_t* draft_token_ids, int32_t* num_draft_tokens,
                           int32_t* cu_num_draft_tokens, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  // Every check below runs before the first launch.
  if (batch < 0 || total_context_tokens < 0) return RS_ERR_INVALID_ARG;
  if (min_n < 1 || max_n < min_n || max_n > RS_NGRAM_MAX_N || k < 1 || k > RS_MAX_SPEC_LEN) return RS_ERR_INVALID_ARG;
  if (batch == 0) return RS_OK;
  if (!cu_context || !draft_token_ids || !num_draft_tokens || !cu_num_draft_tokens ||
      (total_context_tokens > 0 && !context_token_ids))
    return RS_ERR_INVALID_ARG;
  if (((uintptr_t)context_token_ids % 4) || ((uintptr_t)cu_context % 4) || ((uintptr_t)draft_token_ids % 4) ||
      ((uintptr_t)num_draft_tokens % 4) || ((uintptr_t)cu_num_draft_tokens % 4))
    return RS_ERR_UNSUPPORTED;
  if (!workspace || ((uintptr_t)workspace % 4) || workspace_bytes < (size_t)batch * k * sizeof(int32_t))
    return RS_ERR_WORKSPACE;
  int32_t* padded = static_cast<int32_t*>(workspace);
  rsv::ngram_kernel<<<(unsigned)batch, rsv::kNgramThreads, 0, stream>>>(
      context_token_ids, cu_context, total_context_tokens, min_n, max_n, k, max_model_len, padded, num_draft_tokens);
  if (hipGetLastError() != hipSuccess) return RS_ERR_HIP;
  rsv::ngram_pack_kernel<<<1, 1024, 0, stream>>>(padded, num_draft_tokens, batch, k, draft_token_ids,
                                                 cu_num_draft_tokens);
  return hipGetLastError() == hipSuccess ? RS_OK : RS_ERR_HIP;
}

rs_status rs_accept_stats_accumulate(const int32_t* num_accepted, const int32_t* cu_num_draft_tokens, int32_t batch,
                                     int64_t* counters, hipStream_t stream) {
  if (batch < 0) return RS_ERR_INVALID_ARG;
  if (batch == 0) return RS_OK;
  if (!num_accepted || !cu_num_draft_tokens || !counters) return RS_ERR_INVALID_ARG;
  if (((uintptr_t)num_accepted % 4) || ((uintptr_t)cu_num_draft_tokens % 4) || ((uintptr_t)counters % 8))
    return RS_ERR_UNSUPPORTED;
  const unsigned grid = (unsigned)((batch + rsv::kStatsThreads - 1) / rsv::kStatsThreads);
  rsv::stats_kernel<<<grid, rsv::kStatsThreads, 0, stream>>>(num_accepted, cu_num_draft_tokens, batch,
                                                              reinterpret_cast<unsigned long long*>(counters));
  return hipGetLastError() == hipSuccess ? RS_OK : RS_ERR_HIP;
}

double rs_accept_rate(const int64_t* c) {
  return (c && c[1] > 0) ? (double)c[2] / (double)c[1] : __builtin_nan("");
}

double rs_accept_length(const int64_t* c) {
  return (c && c[4] > 0) ? (double)c[3] / (double)c[4] : __builtin_nan("");
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
      return "RS_ERR_WORKSPACE: workspace missing, misaligned or too small (rs_verify_noalloc: the call needs more "
             "than the library's RS_NOALLOC_SCRATCH_BYTES of scratch)";
    case RS_ERR_HIP:
      return "RS_ERR_HIP: a HIP launch or event call failed";
    default:
      break;
  }
  return "unknown rs_status";
}

int32_t rs_abi_version(void) { return RS_VERIFY_ABI_VERSION; }

}  // extern "C"
