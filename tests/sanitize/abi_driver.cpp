// Host sanitizer driver for the library's host side (test infrastructure):
// every entry point's argument validation with pointers that are never
// dereferenced, the workspace size queries (the launch planning) over a grid
// of sizes, empty batches, the debug-knob checks, the counters' host helpers
// and the status strings.  No call here reaches a HIP call, so it runs on a
// machine without a GPU.  Built with host-side -fsanitize=address,undefined
// by tests/test_host_sanitizers.py; any sanitizer report fails the test.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "rs_verify.h"

static int fails = 0;
#define EXPECT(call, status)                                                                 \
  do {                                                                                       \
    const rs_status got_ = (call);                                                           \
    if (got_ != (status)) {                                                                  \
      std::fprintf(stderr, "line %d: %s gave %d, expected %d\n", __LINE__, #call, (int)got_, \
                   (int)(status));                                                           \
      ++fails;                                                                               \
    }                                                                                        \
  } while (0)

int main() {
  // never dereferenced: every call below fails validation or is empty
  void* const P = reinterpret_cast<void*>(uintptr_t(0x10000));
  const float* F = static_cast<const float*>(P);
  const int32_t* I = static_cast<const int32_t*>(P);
  int32_t* O = static_cast<int32_t*>(P);

  // workspace sizes: the launch plan over a grid of shapes
  size_t prev = 0;
  for (int32_t B : {1, 2, 8, 64, 256, 1000})
    for (int32_t K : {0, 1, 3, 8, 32})
      for (int32_t V : {1, 7, 1024, 32000, 151936, 1 << 20})
        for (rs_dtype dt : {RS_F32, RS_BF16}) {
          const size_t a = rs_verify_workspace_size(B, B * K, K, V, dt);
          const size_t f = rs_verify_filtered_workspace_size(B, B * K, K, V, dt);
          if (a == 0 || f < a || a % 256) {
            std::fprintf(stderr, "size B=%d K=%d V=%d: %zu %zu\n", B, K, V, a, f);
            ++fails;
          }
          prev += a;
        }
  if (rs_verify_workspace_size(-1, 0, 1, 10, RS_BF16) || rs_verify_workspace_size(2, 9, 4, 10, RS_BF16) ||
      rs_verify_workspace_size(2, 0, 33, 10, RS_BF16) || rs_verify_workspace_size(2, 0, 4, 0, RS_BF16) ||
      rs_verify_workspace_size(2, 0, 4, 10, static_cast<rs_dtype>(9)) ||
      rs_verify_filtered_workspace_size(1, 2, 1, 10, RS_BF16) || rs_verify_tree_workspace_size(-1, 10) ||
      rs_verify_tree_workspace_size(4, 0) || rs_verify_tree_workspace_size(64, 151936) == 0) {
    std::fprintf(stderr, "invalid sizes not refused\n");
    ++fails;
  }

  // rs_verify: validation before any HIP call
  auto verify = [&](const void* lg, int dt, const float* q, const int32_t* d, const int32_t* cu, const float* T,
                    int32_t B, int32_t D, int32_t mk, int32_t V, void* ws, size_t wsb, const rs_debug* dbg) {
    return rs_verify(lg, static_cast<rs_dtype>(dt), q, d, cu, T, B, D, mk, V, 1, O, O, ws, wsb, dbg, nullptr);
  };
  EXPECT(verify(P, 1, nullptr, I, I, F, -1, 4, 2, 100, P, 1 << 30, nullptr), RS_ERR_INVALID_ARG);
  EXPECT(verify(P, 1, nullptr, I, I, F, 2, 5, 2, 100, P, 1 << 30, nullptr), RS_ERR_INVALID_ARG);
  EXPECT(verify(P, 1, nullptr, I, I, F, 2, 4, 33, 100, P, 1 << 30, nullptr), RS_ERR_INVALID_ARG);
  EXPECT(verify(P, 1, nullptr, I, I, F, 2, 4, 2, 0, P, 1 << 30, nullptr), RS_ERR_INVALID_ARG);
  EXPECT(verify(P, 5, nullptr, I, I, F, 2, 4, 2, 100, P, 1 << 30, nullptr), RS_ERR_UNSUPPORTED);
  EXPECT(verify(nullptr, 1, nullptr, I, I, F, 2, 4, 2, 100, P, 1 << 30, nullptr), RS_ERR_INVALID_ARG);
  EXPECT(verify(P, 1, nullptr, nullptr, I, F, 2, 4, 2, 100, P, 1 << 30, nullptr), RS_ERR_INVALID_ARG);
  EXPECT(verify(P, 1, nullptr, I, I, nullptr, 2, 4, 2, 100, P, 1 << 30, nullptr), RS_ERR_INVALID_ARG);
  EXPECT(verify(static_cast<char*>(P) + 1, 1, nullptr, I, I, F, 2, 4, 2, 100, P, 1 << 30, nullptr),
         RS_ERR_UNSUPPORTED);
  EXPECT(verify(P, 1, reinterpret_cast<const float*>(static_cast<char*>(P) + 2), I, I, F, 2, 4, 2, 100, P, 1 << 30,
                nullptr),
         RS_ERR_UNSUPPORTED);
  EXPECT(verify(P, 1, nullptr, I, I, F, 2, 4, 2, 100, nullptr, 1 << 30, nullptr), RS_ERR_WORKSPACE);
  EXPECT(verify(P, 1, nullptr, I, I, F, 2, 4, 2, 100, static_cast<char*>(P) + 8, 1 << 30, nullptr),
         RS_ERR_WORKSPACE);
  EXPECT(verify(P, 1, nullptr, I, I, F, 2, 4, 2, 100, P, 16, nullptr), RS_ERR_WORKSPACE);
  EXPECT(verify(nullptr, 1, nullptr, nullptr, I, F, 0, 0, 2, 100, nullptr, 0, nullptr), RS_OK);
  rs_debug dbg;
  std::memset(&dbg, 0, sizeof dbg);
  dbg.row_vectors_per_thread = 3;
  EXPECT(verify(P, 1, nullptr, I, I, F, 2, 4, 2, 100, P, 1 << 30, &dbg), RS_ERR_INVALID_ARG);
  dbg.row_vectors_per_thread = 0;
  dbg.race_tokens_per_thread = 5;
  EXPECT(verify(P, 1, nullptr, I, I, F, 2, 4, 2, 100, P, 1 << 30, &dbg), RS_ERR_INVALID_ARG);
  dbg.race_tokens_per_thread = 0;
  dbg.sampling_path = 7;
  EXPECT(verify(P, 1, nullptr, I, I, F, 2, 4, 2, 100, P, 1 << 30, &dbg), RS_ERR_INVALID_ARG);
  dbg.sampling_path = 0;
  dbg.num_events = 2;
  EXPECT(verify(P, 1, nullptr, I, I, F, 2, 4, 2, 100, P, 1 << 30, &dbg), RS_ERR_INVALID_ARG);
  dbg.num_events = 0;
  dbg.draft_target_prob = reinterpret_cast<double*>(static_cast<char*>(P) + 4);
  EXPECT(verify(P, 1, nullptr, I, I, F, 2, 4, 2, 100, P, 1 << 30, &dbg), RS_ERR_UNSUPPORTED);

  // the other entry points
  EXPECT(rs_verify_filtered(P, RS_BF16, nullptr, I, I, F, I, F, 2, 4, 2, 1 << 20, 1, O, O, P, 1 << 30, nullptr,
                            nullptr),
         RS_ERR_UNSUPPORTED);  // V >= 2^20 with a filter
  EXPECT(rs_verify_filtered(P, RS_BF16, nullptr, I, I, F, I, nullptr, 2, 4, 2, 100, 1, O, O, P, 64, nullptr,
                            nullptr),
         RS_ERR_WORKSPACE);
  EXPECT(rs_verify_greedy(P, RS_BF16, I, I, 2, 4, 40, 100, O, O, P, 1 << 30, nullptr), RS_ERR_INVALID_ARG);
  EXPECT(rs_verify_greedy(P, RS_BF16, I, I, 2, 4, 2, 100, O, O, P, 0, nullptr), RS_ERR_WORKSPACE);
  EXPECT(rs_verify_greedy(nullptr, RS_BF16, nullptr, I, 0, 0, 2, 100, nullptr, nullptr, nullptr, 0, nullptr), RS_OK);
  EXPECT(rs_verify_noalloc(P, RS_BF16, nullptr, I, I, F, 1024, 8192, 8, 151936, 1, O, O, nullptr, nullptr),
         RS_ERR_WORKSPACE);  // beyond the fixed scratch
  EXPECT(rs_verify_noalloc(P, RS_BF16, nullptr, I, I, F, 2, 4, 40, 100, 1, O, O, nullptr, nullptr),
         RS_ERR_INVALID_ARG);
  EXPECT(rs_verify_noalloc(nullptr, RS_BF16, nullptr, nullptr, I, F, 0, 0, 2, 100, 1, nullptr, nullptr, nullptr,
                           nullptr),
         RS_OK);
  EXPECT(rs_verify_tree(P, RS_BF16, nullptr, I, I, I, F, 2, 10, 65, 4, 100, 1, O, O, O, P, 1 << 30, nullptr),
         RS_ERR_INVALID_ARG);  // max_nodes > 64
  EXPECT(rs_verify_tree(P, RS_BF16, nullptr, I, I, I, F, 2, 10, 8, 9, 100, 1, O, O, O, P, 1 << 30, nullptr),
         RS_ERR_INVALID_ARG);  // max_depth > max_nodes
  EXPECT(rs_verify_tree(P, RS_BF16, nullptr, I, I, I, F, 2, 10, 8, 4, 100, 1, O, O, O, P, 16, nullptr), RS_ERR_WORKSPACE);
  EXPECT(rs_verify_tree(P, RS_BF16, F + 2, I, I, I, F, 2, 10, 8, 4, 100, 1, O, O, O, P, 1 << 30, nullptr),
         RS_ERR_UNSUPPORTED);  // draft rows not 16-byte aligned
  EXPECT(rs_verify_tree(nullptr, RS_BF16, nullptr, nullptr, nullptr, I, F, 0, 0, 8, 4, 100, 1, nullptr, nullptr, nullptr,
                        nullptr, 0, nullptr),
         RS_OK);
  EXPECT(rs_ngram_propose(I, I, 2, 10, 0, 3, 5, 100, O, O, O, P, 1 << 20, nullptr), RS_ERR_INVALID_ARG);
  EXPECT(rs_ngram_propose(I, I, 2, 10, 1, 65, 5, 100, O, O, O, P, 1 << 20, nullptr), RS_ERR_INVALID_ARG);
  EXPECT(rs_ngram_propose(I, I, 2, 10, 1, 3, 33, 100, O, O, O, P, 1 << 20, nullptr), RS_ERR_INVALID_ARG);
  EXPECT(rs_ngram_propose(I, I, 2, 10, 1, 3, 5, 100, O, O, O, P, 8, nullptr), RS_ERR_WORKSPACE);
  EXPECT(rs_accept_stats_accumulate(I, I, -1, reinterpret_cast<int64_t*>(P), nullptr), RS_ERR_INVALID_ARG);
  EXPECT(rs_accept_stats_accumulate(I, I, 4, reinterpret_cast<int64_t*>(static_cast<char*>(P) + 4), nullptr),
         RS_ERR_UNSUPPORTED);
  EXPECT(rs_accept_stats_accumulate(nullptr, nullptr, 0, nullptr, nullptr), RS_OK);

  // host helpers of the counters and the status strings
  int64_t c[RS_STATS_COUNTERS] = {4, 40, 25, 35, 10};
  if (std::fabs(rs_accept_rate(c) - 0.625) > 1e-15 || std::fabs(rs_accept_length(c) - 3.5) > 1e-15 ||
      !std::isnan(rs_accept_rate(nullptr)) || !std::isnan(rs_accept_length(nullptr))) {
    std::fprintf(stderr, "counter helpers\n");
    ++fails;
  }
  int64_t z[RS_STATS_COUNTERS] = {0};
  if (!std::isnan(rs_accept_rate(z)) || !std::isnan(rs_accept_length(z))) ++fails;
  for (int s = 0; s <= 5; ++s)
    if (!rs_status_string(static_cast<rs_status>(s))[0]) ++fails;
  if (rs_abi_version() != RS_VERIFY_ABI_VERSION) ++fails;
  if (fails) return 1;
  std::printf("abi sanitizer driver: ok (%zu workspace bytes planned)\n", prev);
  return 0;
}
