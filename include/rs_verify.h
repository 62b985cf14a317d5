/*
 * rs_verify.h -- C ABI of the MI355X (gfx950) batched speculative-sampling
 * verify step.
 *
 * The verify step takes the target model's logits for every draft position
 * plus one bonus position per request, the draft tokens and (optionally) the
 * draft distributions q, and decides how many drafts each request keeps and
 * which one extra target token it emits.  Definitions, by page title and
 * section:
 *
 *   - p = softmax(l / T), temperature on the target only
 *       [第12章 投机解码：以小博大 §12.2.3; §12.9 (compute_probs)]
 *   - accept draft x* at position j iff u_j * q(x*) < p(x*), u_j ~ U[0,1),
 *     i.e. with probability min(1, p(x*)/q(x*)); with no q the draft is
 *     deterministic and q(x*) = 1
 *       [§12.2.1; 投机解码（Speculative Decoding）端到端深挖 §7.3]
 *   - drafts after the first rejection are discarded; at the first rejected
 *     position the extra token is drawn from max(0, p - q) / sum max(0, p - q)
 *     (no q: p with p(x*) zeroed); if all are accepted it is drawn from p at
 *     the bonus position
 *       [§12.2.1 step 3; §12.3.2; §12.9 (recovered tokens)]
 *   - temperature <= 0 marks a greedy request: accept iff x* == argmax l, the
 *     extra token is the target argmax
 *       [§12.2.4; §12.9 (GREEDY_TEMPERATURE sentinel)]
 *   - ragged batches: flat draft ids with prefix sums cu_num_draft_tokens
 *       [§12.3.5; vllm v1 源码精读（五） §5.1, §8 (SpecDecodeMetadata)]
 *   - at most 32 drafts per request per step
 *       [§12.5.4 (MAX_SPEC_LEN = 32)]
 *
 * Random numbers come from counter-based Philox4x32-10 keyed by the 64-bit
 * seed: accept uniform u_j = (w0 >> 8) 2^-24 with counter (0, j, b, 0); the
 * sampled token is argmax_x r(x) / E_x with E_x = -ln U_x,
 * U_x = ((w >> 9) + 1/2) 2^-23, w = word (x & 3) of counter (x >> 2, j, b, 1).
 * Output is therefore a pure function of (inputs, seed): re-running a call
 * reproduces it bit for bit.  Vary the seed per decode step.
 *
 * Layout (row-major, no padding):
 *   B = batch, D = total_draft_tokens, R = D + B, V = vocab.
 *   cu_num_draft_tokens [B+1] int32: cu[0] = 0, cu[b+1] - cu[b] = K_b,
 *       0 <= K_b <= max_k, cu[B] = D.
 *   target_logits [R, V] (fp32 or bf16): request b owns rows
 *       cu[b] + b ... cu[b+1] + b; row cu[b] + b + j scores draft j, the last
 *       row (j = K_b) is the bonus row.  Uniform K is a plain [B, K+1, V].
 *   draft_probs [D, V] fp32 (row cu[b] + j = q of draft j of request b), or NULL.
 *   draft_token_ids [D] int32, temperature [B] fp32.
 *   output_token_ids [B, max_k+1] int32: the n_b accepted drafts, then the
 *       extra token, then -1; num_accepted [B] int32 = n_b (n_b + 1 tokens
 *       are emitted).
 *
 * Ownership: every array pointer is a DEVICE pointer owned by the caller; the
 * library never allocates, frees or keeps a pointer after returning.  Scratch
 * memory is the caller's workspace (rs_verify_workspace_size bytes, 16-byte
 * aligned).  All work is enqueued asynchronously on `stream`; the call never
 * synchronises with the host, so it can be captured in a HIP graph.  Calls
 * sharing one workspace must not overlap.  The library holds no global state
 * and is safe to call from several threads on distinct workspaces.
 *
 * Errors: every host-side argument check runs before the first HIP call and
 * returns a status (never aborts, never throws).  Device-resident values are
 * not read on the host; instead the kernels bound every access by the sizes
 * given here and treat a request whose metadata is out of range (cu[b] < 0,
 * cu[b+1] > D, K_b < 0 or > max_k, or a draft id outside [0, V)) as invalid:
 * its output row is all -1 and num_accepted[b] = -1.  Logits must be finite
 * or -inf with at least one finite value per row; q must be non-negative;
 * for T > 0, |l| * log2(e) / T must stay finite in fp32.
 */
#ifndef RS_VERIFY_H
#define RS_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RS_VERIFY_ABI_VERSION 2
#define RS_MAX_SPEC_LEN 32 /* [第12章 §12.5.4: MAX_SPEC_LEN = 32] */

/* Both enums span every 32-bit value (the *_ENUM_MAX sentinels), so any int a
 * caller passes is a valid value of the type; unknown values are reported,
 * not undefined. */
typedef enum rs_status {
  RS_OK = 0,
  RS_ERR_INVALID_ARG = 1, /* NULL pointer, negative size, max_k > 32, D > B*max_k, ... */
  RS_ERR_UNSUPPORTED = 2, /* unknown dtype, misaligned pointer, size beyond the grid */
  RS_ERR_WORKSPACE = 3,   /* workspace NULL, misaligned or smaller than required */
  RS_ERR_HIP = 4,         /* a kernel launch or event record failed */
  RS_STATUS_ENUM_MAX = 0x7FFFFFFF
} rs_status;

typedef enum rs_dtype { RS_F32 = 0, RS_BF16 = 1, RS_DTYPE_ENUM_MAX = 0x7FFFFFFF } rs_dtype;

/* Optional outputs and knobs for parity checks and profiling.  Pass NULL in
 * production.  Every pointer may be NULL independently. */
typedef struct rs_debug {
  /* [D] device, p(x*) as used by the accept test at every evaluated draft
   * position of a random request (fp64); NaN at greedy requests' positions;
   * positions after a request's first rejection may or may not be written. */
  double* draft_target_prob;
  /* [R, V] device, p at every row of every random request, in the fp32 form
   * the sampling race uses; rows of greedy requests are left untouched.
   * Costs an extra pass over every row (one phase): small shapes only. */
  float* probs;
  /* num_events caller-created events: events[0] is recorded on `stream`
   * before the first kernel, events[k] after the k-th kernel launch. */
  hipEvent_t* events;
  int32_t num_events;
  /* HOST pointer or NULL: receives the number of kernels the call launched. */
  int32_t* kernels_launched;
  /* 0 = automatic.  Otherwise force the row statistics to 1, 4 or 16 16-byte
   * vectors per thread, or the race to 8 or 32 tokens per thread.  Output
   * does not depend on these (the parity tests check that). */
  int32_t row_vectors_per_thread;
  int32_t race_tokens_per_thread;
  /* 0 = automatic: the per-request path for batches of at most 8 requests
   * whose rows take at most 10 load passes per request in all; else the
   * stream path when the logits total at most 128 MB or rows split into
   * 16-vector chunks give B times the chunks per row of at least 512; else
   * the phased split path.
   * 1 = per-request path: one workgroup per request walks its rows in order
   * and stops at the first rejection.  2 = phased split path: each phase
   * spreads every active
   * request's rows across the whole GPU, then scans.  3 = stream path: one
   * kernel streams rows position by position, decides requests as their
   * rows complete (skipping the rows behind a decided request's first
   * rejection) and races them as they are decided.  Requesting `probs`
   * selects the split path. */
  int32_t sampling_path;
  /* Phases of the split path, as the draft positions where phases end.
   * phase_ends[0] == 0: automatic (one phase for a filtered call whose
   * logits total at most 256 MB, else about the first third of the
   * positions, then the rest); phase_ends[0] < 0: one phase (every row is
   * read); otherwise strictly increasing ends P1 < P2 < ..., stopping at
   * the first entry that is 0 or >= max_k + 1 (the last phase always ends at
   * max_k + 1).  At most four phases.  On the stream path phase_ends[0] > 0
   * is the number of positions streamed before race tasks start to
   * interleave with rows (default max_k + 1: all rows first). */
  int32_t phase_ends[3];
  /* HOST pointer or NULL: receives the path the call took (1, 2 or 3). */
  int32_t* path_taken;
} rs_debug;

/* Bytes of workspace rs_verify / rs_verify_greedy need for these sizes
 * (independent of the debug knobs).  Returns 0 for invalid sizes. */
size_t rs_verify_workspace_size(int32_t batch, int32_t total_draft_tokens, int32_t max_k,
                                int32_t vocab, rs_dtype logits_dtype);

/* Bytes of workspace rs_verify_filtered needs with top_k or top_p given: the
 * rs_verify workspace plus one fp32 maximum per 4096-byte segment of every
 * logits row (5 KB per row at V = 151936 bf16).  Returns 0 for invalid sizes. */
size_t rs_verify_filtered_workspace_size(int32_t batch, int32_t total_draft_tokens, int32_t max_k,
                                         int32_t vocab, rs_dtype logits_dtype);

/* Batched verify (random and greedy requests mixed; T <= 0 is greedy).
 *   target_logits       [R, V] fp32 or bf16, element-aligned
 *   draft_probs         [D, V] fp32 or NULL (one-hot q at the draft)
 *   draft_token_ids     [D] int32
 *   cu_num_draft_tokens [B+1] int32
 *   temperature         [B] fp32
 *   seed                Philox key
 *   output_token_ids    [B, max_k+1] int32 (written)
 *   num_accepted        [B] int32 (written)
 *   workspace           >= rs_verify_workspace_size(...) bytes, 16-byte aligned
 *   debug               NULL or optional outputs
 *   stream              HIP stream the kernels are enqueued on
 * batch = 0 returns RS_OK without touching the GPU. */
rs_status rs_verify(const void* target_logits, rs_dtype logits_dtype, const float* draft_probs,
                    const int32_t* draft_token_ids, const int32_t* cu_num_draft_tokens,
                    const float* temperature, int32_t batch, int32_t total_draft_tokens,
                    int32_t max_k, int32_t vocab, uint64_t seed, int32_t* output_token_ids,
                    int32_t* num_accepted, void* workspace, size_t workspace_bytes,
                    const rs_debug* debug, hipStream_t stream);

/* rs_verify for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * takes no workspace; its scratch is an array of RS_NOALLOC_SCRATCH_BYTES in
 * the library's own device code object, one per GPU the library runs on, held
 * until the process ends.  The call allocates nothing (no hipMalloc, hipFree
 * or allocating library routine).  Arguments, layout, outputs, ownership and
 * errors are those of rs_verify; in addition:
 *   - a call whose rs_verify_workspace_size(...) exceeds
 *     RS_NOALLOC_SCRATCH_BYTES returns RS_ERR_WORKSPACE before any HIP call
 *     (8 MiB holds every measured workload, e.g. B=512, K=8, V=151936 with
 *     bf16 logits or B=256 with fp32 logits; not B=1024 or B=512 fp32);
 *   - the first call on a device, with that device current, looks the
 *     array's device address up (hipGetSymbolAddress); `stream` must belong to
 *     the current device;
 *   - every call on one GPU shares that GPU's array: calls that overlap on one
 *     GPU (concurrent streams, or threads) race and give wrong results; calls
 *     ordered on one stream are safe, each call leaving the array in whatever
 *     state and the next one initialising what it needs. */
#define RS_NOALLOC_SCRATCH_BYTES (8u << 20)
rs_status rs_verify_noalloc(const void* target_logits, rs_dtype logits_dtype, const float* draft_probs,
                            const int32_t* draft_token_ids, const int32_t* cu_num_draft_tokens,
                            const float* temperature, int32_t batch, int32_t total_draft_tokens, int32_t max_k,
                            int32_t vocab, uint64_t seed, int32_t* output_token_ids, int32_t* num_accepted,
                            const rs_debug* debug, hipStream_t stream);

/* rs_verify with top-k / top-p filtering of each random request's target
 * distribution before the accept test, the residual and the bonus: the
 * rejection sampler constrains the target distribution with temperature,
 * top-k and top-p [第12章 §12.2.3; §12.9 (compute_probs applies the
 * per-request top_k / top_p to every draft position)].  The pages do not print
 * the tie rules; the library's reading:
 *   top-k keeps token x iff fewer than top_k[b] tokens have a strictly larger
 *     logit (every token tied with the k-th largest stays);
 *   top-p then keeps x iff the probability mass, under the top-k-filtered
 *     softmax at temperature T_b, of the tokens with a strictly larger logit
 *     is below top_p[b] (tokens of equal logit stay or go together; the
 *     largest logit always stays);
 *   p' = the softmax restricted to the kept tokens.
 *   top_k        [B] int32 device, or NULL; top_k[b] <= 0 or >= V: no top-k
 *   top_p        [B] fp32 device, or NULL; top_p[b] outside (0, 1): no top-p
 * Greedy requests (T <= 0) ignore both.  Every other argument, the layout,
 * ownership and error rules are those of rs_verify, except that the workspace
 * must hold rs_verify_filtered_workspace_size bytes when top_k or top_p is
 * given (RS_ERR_WORKSPACE otherwise), and that V must then be below 2^20
 * (RS_ERR_UNSUPPORTED otherwise).  Filtered calls run the phased path: the
 * row statistics pass also records per-segment maxima of filtered rows, and a
 * small kernel per phase finds each such row's threshold by radix selection
 * over the few segments that can hold kept tokens before the accept tests.
 * With top_k and top_p both NULL this is exactly rs_verify. */
rs_status rs_verify_filtered(const void* target_logits, rs_dtype logits_dtype, const float* draft_probs,
                             const int32_t* draft_token_ids, const int32_t* cu_num_draft_tokens,
                             const float* temperature, const int32_t* top_k, const float* top_p,
                             int32_t batch, int32_t total_draft_tokens, int32_t max_k, int32_t vocab,
                             uint64_t seed, int32_t* output_token_ids, int32_t* num_accepted,
                             void* workspace, size_t workspace_bytes, const rs_debug* debug,
                             hipStream_t stream);

/* Greedy argmax-match for every request (no temperature, q or random numbers)
 * [第12章 §12.2.4; 投机解码（Speculative Decoding）端到端深挖 §7.1 path A].
 * Same layout, ownership and error rules as rs_verify. */
rs_status rs_verify_greedy(const void* target_logits, rs_dtype logits_dtype,
                           const int32_t* draft_token_ids, const int32_t* cu_num_draft_tokens,
                           int32_t batch, int32_t total_draft_tokens, int32_t max_k, int32_t vocab,
                           int32_t* output_token_ids, int32_t* num_accepted, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* ---- Tree verify --------------------------------------------------------
 * The drafts of a request form a tree: node i holds one draft token and its
 * parent (a node earlier in the request's node order, or -1 for a child of
 * the last prefix position).  One target forward over the whole tree scored
 * the prefix position and every node [投机解码深度实战 §四 (tree drafts and
 * tree attention)].  Verification walks the tree one depth at a time from the
 * root: among the current node's children it looks for an accepted one,
 * descends into it, and stops at the first depth where none is accepted; one
 * extra token then comes from the stop node's row
 * [投机解码（Speculative Decoding）端到端深挖 §6.2].
 *   greedy (T <= 0): the first child whose token is the row's argmax (lowest
 *     index on argmax ties); else emit the argmax [§7.1].
 *   random: p = softmax(row / T); one coin u_d per depth d (the accept uniform
 *     of position d, see above); children in node order, a child repeating an
 *     earlier sibling's token skipped; child i is accepted iff u_d < the sum
 *     of p over the siblings up to and including i [§7.2, both thresholds at
 *     their default 1]; if none, the extra token is the race over p without
 *     the children's tokens (exponentials of depth d); a childless stop node
 *     races over p (the bonus).
 * Every sibling is accepted with probability p(its token) and the residual is
 * p without the siblings, so each emitted token follows p; a tree with one
 * child per node is exactly the chain of rs_verify with draft_probs = NULL
 * (same tokens for the same seed).
 * With draft_probs (one draft distribution per tree position), the extra token
 * after a stop at node c is the race over max(0, p - q_c) instead, q_c the
 * stop node's row [§7.2: after a rejection, from relu(target_probs -
 * draft_probs)]; acceptance is the same roulette.  This is the page's rule
 * as written: it leaves each emitted token distributed as p when q_c is p on
 * c's children and 0 elsewhere (then it equals the rule above), not for an
 * arbitrary q (§7.4).  An all-zero residual falls back to the race over p.
 * A stop at a childless node rejected nothing: its extra token is the race
 * over p whatever its draft row holds.  A draft_probs pointer that is not
 * 16-byte aligned gives RS_ERR_UNSUPPORTED.
 * Layout:
 *   cu_num_nodes  [B+1] int32: request b owns nodes cu[b] .. cu[b+1]-1
 *   target_logits [N + B, V] fp32 / bf16: request b's rows start at
 *                 cu[b] + b; row 0 is the prefix position (it predicts the
 *                 children of the root), row 1 + i is node i
 *   draft_probs   [N + B, V] fp32 or NULL: rows aligned with target_logits
 *                 (row 0 of a request the draft distribution at the prefix
 *                 position, row 1 + i at node i), non-negative; a row
 *                 need not sum to 1; 16-byte aligned
 *   node_tokens   [N] int32 in [0, V); node_parents [N] int32, request-local,
 *                 -1 <= parent < node
 *   temperature   [B] fp32
 *   output_token_ids [B, max_depth + 1] int32: the accepted path's tokens,
 *                 then the extra token, then -1
 *   accepted_nodes   [B, max_depth] int32: request-local indices of the
 *                 accepted nodes, then -1
 *   num_accepted     [B] int32: accepted nodes (path length)
 * max_nodes <= RS_MAX_TREE_NODES bounds the nodes per request and max_depth
 * <= max_nodes the depth (a node with no parent has depth 0); a request whose
 * tree breaks these rules (too many nodes, a parent after its child, a token
 * out of range, a node of depth >= max_depth) gets -1 rows and
 * num_accepted = -1.  The walks run spread over the GPU: the rows of a
 * walk's next candidates are streamed by many workgroups ahead of the step
 * that needs them, and the stop row's race is split over the GPU too.
 *   workspace  >= rs_verify_tree_workspace_size(B, V) bytes, 16-byte aligned
 *              (RS_ERR_WORKSPACE otherwise); calls sharing one workspace must
 *              not overlap.
 * Ownership, asynchrony and error reporting as for rs_verify. */
#define RS_MAX_TREE_NODES 64
size_t rs_verify_tree_workspace_size(int32_t batch, int32_t vocab);
rs_status rs_verify_tree(const void* target_logits, rs_dtype logits_dtype, const float* draft_probs,
                         const int32_t* node_tokens, const int32_t* node_parents, const int32_t* cu_num_nodes,
                         const float* temperature,
                         int32_t batch, int32_t total_nodes, int32_t max_nodes, int32_t max_depth,
                         int32_t vocab, uint64_t seed, int32_t* output_token_ids,
                         int32_t* accepted_nodes, int32_t* num_accepted, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* ---- n-gram draft proposer -------------------------------------------------
 * Prompt-lookup drafts for a batch of requests, ready for rs_verify with
 * draft_probs = NULL [第12章 §12.4.4]: for n = max_n down to min_n, the
 * pattern is the context's last n tokens; the proposal is the tokens after
 * the leftmost earlier occurrence of the pattern (one ending before the
 * pattern begins), at most k_b = min(k, max_model_len - len(context_b)) of
 * them (fewer when the context ends first); the first n that matches wins;
 * no match (or k_b <= 0) proposes nothing.
 *   context_token_ids [total_context_tokens] int32 device, request b's tokens
 *                     at cu_context[b] .. cu_context[b+1]-1 (cu_context [B+1])
 *   1 <= min_n <= max_n <= RS_NGRAM_MAX_N, 1 <= k <= RS_MAX_SPEC_LEN
 *   draft_token_ids     [B * k] int32 device: the proposals packed in request
 *                       order (the first cu_num_draft_tokens[B] entries)
 *   num_draft_tokens    [B] int32 device: proposals per request
 *   cu_num_draft_tokens [B+1] int32 device: their prefix sums, from 0
 *   workspace           >= B * k * 4 bytes of device scratch, 4-byte aligned
 * A request whose context range is out of [0, total] proposes nothing.
 * Errors and ownership as for rs_verify (RS_ERR_WORKSPACE for a missing or
 * short workspace). */
#define RS_NGRAM_MAX_N 64
rs_status rs_ngram_propose(const int32_t* context_token_ids, const int32_t* cu_context, int32_t batch,
                           int32_t total_context_tokens, int32_t min_n, int32_t max_n, int32_t k,
                           int64_t max_model_len, int32_t* draft_token_ids, int32_t* num_draft_tokens,
                           int32_t* cu_num_draft_tokens, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* ---- Acceptance statistics ------------------------------------------------
 * Running counters a serving engine exports per verify step: draft proposals
 * (requests that proposed at least one draft -- proposals, not tokens),
 * proposed draft tokens, accepted draft tokens and accepted tokens per draft
 * position [第12章 §12.7.5]; acceptance rate = accepted / proposed (bonus
 * excluded) and acceptance length = emitted tokens / verifies, every verify
 * emitting its accepted drafts plus one extra token
 * [投机解码（Speculative Decoding）端到端深挖 §13].  One verify is one request
 * in one step; requests with num_accepted = -1 (invalid) are not counted. */
#define RS_STATS_SCALARS 5
#define RS_STATS_COUNTERS (RS_STATS_SCALARS + RS_MAX_SPEC_LEN)
/* counters[] layout (int64):
 *   [0] draft proposals      [1] proposed draft tokens   [2] accepted draft tokens
 *   [3] emitted tokens       [4] verifies
 *   [RS_STATS_SCALARS + j]   requests whose drafts 0 .. j were all accepted, j < 32 */

/* Adds one verify step's outcome to the counters, asynchronously on `stream`
 * (call it after rs_verify* on the same stream).
 *   num_accepted        [B] int32 device: rs_verify*'s output
 *   cu_num_draft_tokens [B+1] int32 device: the same prefix sums as the call
 *   counters            [RS_STATS_COUNTERS] int64 device, 8-byte aligned, owned by
 *                       the caller, zeroed by the caller to start; accumulated
 *                       with device atomics (calls may overlap)
 * batch = 0 returns RS_OK without touching the GPU; NULL pointers or B < 0:
 * RS_ERR_INVALID_ARG; misalignment: RS_ERR_UNSUPPORTED; a failed launch:
 * RS_ERR_HIP.  All checks run before the launch. */
rs_status rs_accept_stats_accumulate(const int32_t* num_accepted, const int32_t* cu_num_draft_tokens,
                                     int32_t batch, int64_t* counters, hipStream_t stream);

/* alpha = accepted / proposed draft tokens and tau = emitted tokens /
 * verifies from a HOST copy of the counters; NaN when the denominator is 0
 * or the pointer is NULL. */
double rs_accept_rate(const int64_t* counters);
double rs_accept_length(const int64_t* counters);

/* Static string naming a status. */
const char* rs_status_string(rs_status status);

/* RS_VERIFY_ABI_VERSION of the built library. */
int32_t rs_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RS_VERIFY_H */
