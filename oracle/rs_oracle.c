/*
 * rs_oracle.c -- plain, slow, fp64 CPU oracle for the batched speculative-
 * sampling verify step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with the
 * HIP library; its Philox4x32-10 is written here from the published
 * definition.
 *
 * What it computes (citations name the page title and section):
 *
 *  - Target distribution: temperature softmax of the target logits,
 *    p = softmax(l / T), applied to the target only.
 *      [Ch.12 "投机解码：以小博大" §12.2.3; §12.9, compute_probs bullet]
 *  - Accept test at each draft position j, in order: draw u ~ U[0,1) and
 *    accept the draft token x* iff u * q(x*) < p(x*), which accepts with
 *    probability min(1, p(x*)/q(x*)).
 *      [Ch.12 §12.2.1 steps 1-3; "投机解码（Speculative Decoding）端到端深挖"
 *       §7.3 path C (coin * q < p)]
 *    With no draft probabilities the draft is deterministic and q is one-hot
 *    at x*, so q(x*) = 1.  [Ch.12 §12.2.3; §12.9, last bullet]
 *  - First-rejection prefix: drafts after the first rejected one are
 *    discarded.  [Ch.12 §12.9 (each request's drafts are checked in order by
 *    one program); "vllm v1 源码精读（五）" §7]
 *  - At the first rejected position j = n < K: resample from the residual
 *    max(0, p - q) / sum max(0, p - q)  [Ch.12 §12.2.1 step 3, §12.2.2];
 *    with one-hot q this is p with p(x*) set to zero, renormalised
 *    [Ch.12 §12.9, last bullet].
 *  - If all K drafts are accepted, sample a bonus token from p at position K.
 *    [Ch.12 §12.3.2; "投机解码深度实战" §一 item 4]
 *  - Sampling is an exponential race: argmax_x r(x) / E_x with E_x ~ Exp(1),
 *    which samples r / sum(r) without normalising it.
 *      [Ch.12 §12.9, last bullet: argmax(prob / exponential)]
 *  - Greedy requests (temperature <= 0, or the greedy entry point): accept
 *    iff draft == argmax of the target logits; at the first mismatch, or as
 *    the bonus, emit the target argmax.
 *      [Ch.12 §12.2.4; §12.9 first bullet (temperature sentinel -1);
 *       "投机解码端到端深挖" §7.1 path A]
 *  - Output: the accepted drafts, then one target token; num_accepted = n,
 *    so n + 1 tokens are emitted.  [Ch.12 §12.3.4; "投机解码端到端深挖"
 *    §8 (accept_lens = num_correct_drafts + 1)]
 *
 *  - Optional top-k / top-p filtering of the target distribution, applied
 *    after the temperature and before the accept test, the residual and the
 *    bonus: rejection sampling constrains the target distribution with
 *    temperature, top-k and top-p (not min_p or penalties).
 *      [Ch.12 §12.2.3 (last sentences); §12.9, top-k / top-p bullet:
 *       batch-level top_k / top_p expanded to tokens, then applied in
 *       compute_probs]
 *    The pages name the step but not its tie rules; the reading taken:
 *      top-k keeps token x iff fewer than k tokens have a strictly larger
 *      logit (ties at the k-th value are all kept); k <= 0 or k >= V is off.
 *      top-p (after top-k) keeps x iff the probability mass, under the
 *      top-k-filtered softmax, of the tokens with a strictly larger logit is
 *      below top_p (tokens of equal logit are kept or dropped together; the
 *      largest logit is always kept); top_p outside (0, 1) is off.
 *      p' = softmax restricted to the kept tokens.  Greedy requests ignore
 *      both.
 *
 * Readings where the pages leave a step open (each is also listed in the
 * design notes):
 *  - Random stream: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
 *    Random Numbers: As Easy as 1, 2, 3", SC'11), key = 64-bit seed
 *    (low word, high word), counter = (c0, j, b, tag).
 *      accept uniform  u_j = (w0 >> 8) * 2^-24, counter (0, j, b, 0), word 0;
 *      race exponential E_x = -ln U_x, U_x = ((w >> 9) + 1/2) * 2^-23,
 *        counter (x >> 2, j, b, 1), word (x & 3).
 *  - Greedy and race ties: lowest token index wins.
 *  - All-zero residual after a rejection: max(0, p - q) / sum is undefined
 *    when p <= q everywhere [Ch.12 §12.2.1 step 3 normalises by that sum].
 *    With normalised q this happens only through rounding; with q that is
 *    not normalised (q >= p everywhere, e.g. q = 2p) it happens at every
 *    rejection.  Reading: race over p at that position instead
 *    (FLAG_ZERO_RESIDUAL).  This is an ordinary, exactly reproducible
 *    decision, not a near tie, unless the eps perturbation below could make
 *    the residual positive.
 *  - Requests whose metadata is out of range (cu not within [0, D], K_b >
 *    max_k, a draft id outside [0, V)) emit -1 everywhere and
 *    num_accepted = -1.
 *
 * Near-tie flags (a request is flagged when a decision on its taken path
 * would change under a relative perturbation eps of p and of E):
 *   accept test:  |p(x*) - u q(x*)| <= eps * p(x*)
 *   race:         lower bound of the winner's key <= upper bound of any
 *                 other key, the bounds taken with p -> p(1 -/+ eps) and
 *                 E -> E(1 +/- eps); or the choice between the residual race
 *                 and the zero-residual fallback could flip (some upper
 *                 residual bound positive although every residual is zero,
 *                 or the winner's lower residual bound zero).
 *   The near-tied alternatives of the race are reported per request (the
 *   winner first), so a flagged request can still be checked for a valid
 *   token.
 *   top-p:        for some group of equal logits, the mass of the larger
 *                 kept tokens is within eps * top_p * S_k of top_p * S_k
 *                 (S_k = the top-k-filtered mass) on a sampled or tested row.
 *
 * Parity unpinned: the specific token ids drawn at a given seed (the race
 * winners and the accept coins) are fixed by nothing on the pages, which name
 * no generator.  The laws they follow are pinned (the output marginal equals
 * p, the acceptance rate, the expected accept length, greedy brute force), and
 * the stream itself only by its published definition: this Philox4x32-10
 * against the Random123 known-answer tests and rocRAND, and a second,
 * independent implementation on the HIP side.
 *
 * Arithmetic: inputs are widened exactly (bf16 -> fp32 -> fp64; temperature
 * from fp32) and everything is computed in fp64 with the C library's exp/log.
 * Requests are independent; OpenMP runs them in parallel without changing
 * any request's arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define RSO_F32 0
#define RSO_BF16 1

#define RSO_FLAG_ACCEPT_TIE 1
#define RSO_FLAG_RACE_TIE 2
#define RSO_FLAG_ZERO_RESIDUAL 4
#define RSO_FLAG_INVALID 8
#define RSO_FLAG_TOPP_TIE 16
#define RSO_FLAG_CAND_OVERFLOW 32

/* ------------------------------------------------------------------------ */
/* Philox4x32-10.  One round maps (c0, c1, c2, c3) with key (k0, k1) to
 *   (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))
 * and the key is advanced by the Weyl constants between rounds. */
static const uint32_t PHILOX_M0 = 0xD2511F53u;
static const uint32_t PHILOX_M1 = 0xCD9E8D57u;
static const uint32_t PHILOX_W0 = 0x9E3779B9u;
static const uint32_t PHILOX_W1 = 0xBB67AE85u;

void rso_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += PHILOX_W0;
      k1 += PHILOX_W1;
    }
    uint64_t prod0 = (uint64_t)PHILOX_M0 * (uint64_t)c0;
    uint64_t prod1 = (uint64_t)PHILOX_M1 * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
    uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static void seed_key(uint64_t seed, uint32_t key[2]) {
  key[0] = (uint32_t)(seed & 0xFFFFFFFFu);
  key[1] = (uint32_t)(seed >> 32);
}

/* u_j for request b, position j: 24-bit uniform on [0, 1). */
double rso_accept_uniform(uint64_t seed, int32_t b, int32_t j) {
  uint32_t key[2], ctr[4], w[4];
  seed_key(seed, key);
  ctr[0] = 0u; ctr[1] = (uint32_t)j; ctr[2] = (uint32_t)b; ctr[3] = 0u;
  rso_philox4x32_10(ctr, key, w);
  return (double)(w[0] >> 8) * 0x1p-24;
}

/* U_x for request b, position j, token x: 23-bit midpoint uniform in (0, 1). */
double rso_race_uniform(uint64_t seed, int32_t b, int32_t j, int32_t x) {
  uint32_t key[2], ctr[4], w[4];
  seed_key(seed, key);
  ctr[0] = (uint32_t)x >> 2; ctr[1] = (uint32_t)j; ctr[2] = (uint32_t)b; ctr[3] = 1u;
  rso_philox4x32_10(ctr, key, w);
  return ((double)(w[x & 3] >> 9) + 0.5) * 0x1p-23;
}

/* E_x = -ln U_x ~ Exp(1). */
double rso_race_exponential(uint64_t seed, int32_t b, int32_t j, int32_t x) {
  return -log(rso_race_uniform(seed, b, j, x));
}

/* ------------------------------------------------------------------------ */
static double widen(const void* logits, int dtype, int64_t idx) {
  if (dtype == RSO_BF16) {
    uint32_t bits = (uint32_t)((const uint16_t*)logits)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return (double)((const float*)logits)[idx];
}

/* p = softmax(l / T) of one row, in fp64:
 *   M = max_y l_y / T,  p_x = exp(l_x / T - M) / sum_y exp(l_y / T - M). */
void rso_softmax_row(const double* l, int32_t V, double T, double* p) {
  double M = -INFINITY;
  for (int32_t x = 0; x < V; ++x) {
    double s = l[x] / T;
    if (s > M) M = s;
  }
  double Z = 0.0;
  for (int32_t x = 0; x < V; ++x) {
    p[x] = exp(l[x] / T - M);
    Z += p[x];
  }
  for (int32_t x = 0; x < V; ++x) p[x] /= Z;
}

/* Lowest index of the maximum of l. */
static int32_t argmax_lowest(const double* l, int32_t V) {
  int32_t best = 0;
  for (int32_t x = 1; x < V; ++x)
    if (l[x] > l[best]) best = x;
  return best;
}

static int cmp_desc(const void* a, const void* b) {
  double x = *(const double*)a, y = *(const double*)b;
  return (x < y) - (x > y);
}

/* Target distribution p' of one row with top-k / top-p filtering:
 *   M = max_y l_y / T;  w_x = exp(l_x / T - M);
 *   top-k: kept iff l_x >= v_k, v_k = the k-th largest logit (k-th entry of
 *          the logits sorted in descending order), so exactly the tokens with
 *          fewer than k strictly larger logits;
 *   top-p: walk the kept logits in descending order in groups of equal value;
 *          a group stays iff the mass of the groups before it is below
 *          top_p * S_k, S_k = sum of w over the top-k-kept tokens;
 *   p'_x = w_x / sum of w over the kept tokens (0 for dropped tokens).
 * k <= 0 or k >= V disables top-k; top_p outside (0, 1) disables top-p.
 * *near_tie is set when some group's preceding mass is within
 * eps * top_p * S_k of top_p * S_k.  sorted is scratch of length V. */
void rso_filtered_probs_row(const double* l, int32_t V, double T, int32_t k, double top_p, double eps,
                            double* p, double* sorted, int* near_tie) {
  *near_tie = 0;
  double M = -INFINITY;
  for (int32_t x = 0; x < V; ++x) {
    double s = l[x] / T;
    if (s > M) M = s;
  }
  double vk = -INFINITY; /* keep l >= vk */
  if (k > 0 && k < V) {
    memcpy(sorted, l, sizeof(double) * (size_t)V);
    qsort(sorted, (size_t)V, sizeof(double), cmp_desc);
    vk = sorted[k - 1];
  }
  double Sk = 0.0;
  for (int32_t x = 0; x < V; ++x) {
    p[x] = (l[x] >= vk) ? exp(l[x] / T - M) : 0.0;
    Sk += p[x];
  }
  double vp = -INFINITY;
  if (top_p > 0.0 && top_p < 1.0) {
    int32_t n = 0;
    for (int32_t x = 0; x < V; ++x)
      if (l[x] >= vk) sorted[n++] = l[x];
    qsort(sorted, (size_t)n, sizeof(double), cmp_desc);
    double target = top_p * Sk, before = 0.0;
    int32_t i = 0;
    while (i < n) {
      double v = sorted[i];
      if (fabs(before - target) <= eps * target) *near_tie = 1;
      if (!(before < target)) break;
      vp = v;
      double group = 0.0;
      while (i < n && sorted[i] == v) {
        group += exp(v / T - M);
        ++i;
      }
      before += group;
    }
  }
  double S = 0.0;
  for (int32_t x = 0; x < V; ++x) {
    if (l[x] < vp) p[x] = 0.0;
    S += p[x];
  }
  for (int32_t x = 0; x < V; ++x) p[x] /= S;
}

static void load_row(const void* logits, int dtype, int64_t row, int32_t V, double* l) {
  for (int32_t x = 0; x < V; ++x) l[x] = widen(logits, dtype, row * (int64_t)V + x);
}

/* Exponential race over r (r[x] > 0 are the candidates).  Returns the winner
 * (lowest index among equal keys) or -1 when every r[x] is zero.  *near_tie is
 * set if the winner's key taken with (rlo, E(1+eps)) does not exceed some
 * other token's key taken with (rhi, E(1-eps)).  cand (RSO_NCAND entries, or NULL) receives
 * the winner, then the tokens whose upper key reaches the winner's lower key,
 * -1 padded; *overflow is set when they do not all fit.  E is scratch of
 * length V. */
#define RSO_NCAND 8
static int32_t race(const double* r, const double* rlo, const double* rhi, int32_t V, uint64_t seed,
                    int32_t b, int32_t j, double eps, double* E, int* near_tie, int32_t* cand, int* overflow) {
  int32_t win = -1;
  double best = 0.0;
  for (int32_t x = 0; x < V; ++x) {
    E[x] = (rhi[x] > 0.0 || r[x] > 0.0) ? rso_race_exponential(seed, b, j, x) : INFINITY;
    if (!(r[x] > 0.0)) continue;
    double key = r[x] / E[x];
    if (win < 0 || key > best) {
      best = key;
      win = x;
    }
  }
  *near_tie = 0;
  *overflow = 0;
  if (cand)
    for (int i = 0; i < RSO_NCAND; ++i) cand[i] = -1;
  if (win < 0) return -1;
  int nc = 0;
  if (cand) cand[nc++] = win;
  double lo = rlo[win] / (E[win] * (1.0 + eps));
  for (int32_t x = 0; x < V; ++x) {
    if (x == win || !(rhi[x] > 0.0)) continue;
    double hi = rhi[x] / (E[x] * (1.0 - eps));
    if (hi >= lo) {
      *near_tie = 1;
      if (cand && nc < RSO_NCAND)
        cand[nc++] = x;
      else
        *overflow = 1;
    }
  }
  return win;
}

/* Appends token x to a -1 padded candidate list unless present; sets
 * *overflow when the list is full. */
static void cand_add(int32_t* cand, int32_t x, int* overflow) {
  if (!cand || x < 0) return;
  for (int i = 0; i < RSO_NCAND; ++i) {
    if (cand[i] == x) return;
    if (cand[i] < 0) {
      cand[i] = x;
      return;
    }
  }
  *overflow = 1;
}

/* The sampling race of one request at position n over r, with the
 * all-zero-residual fallback: when every r(x) is zero, race over p at the same
 * position instead (flag FLAG_ZERO_RESIDUAL).  The choice between the two
 * races is itself a decision; it is a near tie (FLAG_RACE_TIE) when the eps
 * perturbation could flip it:
 *   - the fallback was taken but some rhi(x) > 0: a perturbed residual would
 *     race over those tokens, which join the candidates;
 *   - the residual race was taken but its winner's rlo is 0: a perturbed
 *     residual could be all zero, so the fallback's candidates join.
 * cand (RSO_NCAND entries or NULL) receives the winner first, then every
 * near-tied alternative; FLAG_CAND_OVERFLOW marks a list that did not fit.
 * r, rlo and rhi are overwritten. */
static int32_t sample_with_fallback(double* r, double* rlo, double* rhi, const double* p, int32_t V,
                                    uint64_t seed, int32_t b, int32_t n, double eps, double* E, int32_t* flags,
                                    int32_t* cand) {
  int tie = 0, over = 0;
  int32_t token = race(r, rlo, rhi, V, seed, b, n, eps, E, &tie, cand, &over);
  int fallback_fragile = 0;
  int32_t alt[RSO_NCAND];
  int n_alt = 0;
  if (token < 0) {
    *flags |= RSO_FLAG_ZERO_RESIDUAL;
    for (int32_t x = 0; x < V; ++x)
      if (rhi[x] > 0.0) {
        fallback_fragile = 1;
        if (n_alt < RSO_NCAND) alt[n_alt++] = x;
        else over = 1;
      }
  }
  const int winner_fragile = token >= 0 && !(rlo[token] > 0.0);
  if (token < 0 || winner_fragile) {
    for (int32_t x = 0; x < V; ++x) {
      r[x] = p[x];
      rlo[x] = p[x] * (1.0 - eps);
      rhi[x] = p[x] * (1.0 + eps);
    }
    int tie2 = 0, over2 = 0;
    int32_t fb_cand[RSO_NCAND];
    int32_t fb = race(r, rlo, rhi, V, seed, b, n, eps, E, &tie2, fb_cand, &over2);
    if (token < 0) {
      token = fb;
      tie |= tie2;
      if (cand) memcpy(cand, fb_cand, sizeof fb_cand);
    } else {
      for (int i = 0; i < RSO_NCAND; ++i) cand_add(cand, fb_cand[i], &over);
    }
    over |= over2;
  }
  for (int i = 0; i < n_alt; ++i) cand_add(cand, alt[i], &over);
  if (tie || fallback_fragile || winner_fragile) *flags |= RSO_FLAG_RACE_TIE;
  if (over) *flags |= RSO_FLAG_CAND_OVERFLOW;
  return token;
}

/* ------------------------------------------------------------------------ */
/* Verify a batch.
 *   logits   [R, V] (fp32 or raw bf16 bits), R = D + B; request b owns rows
 *            cu[b] + b ... cu[b+1] + b (K_b + 1 rows, the last is the bonus row).
 *   q        [D, V] fp32 draft probabilities, or NULL for one-hot q.
 *   draft    [D] draft token ids; cu [B+1] prefix sums of draft counts.
 *   T        [B] temperatures; T <= 0 marks a greedy request.
 *   greedy_only: treat every request as greedy (T and q ignored).
 *   out      [B, max_k+1] tokens (-1 padded); num_accepted [B]; flags [B].
 *   top_k    [B] or NULL, top_p [B] or NULL: per-request filtering of the
 *            target distribution (see rso_filtered_probs_row).
 *   p_draft  [D] or NULL: p(x*) at each evaluated random position, NaN elsewhere.
 * Returns 0, or -1 on an argument error. */
int rso_verify_filtered(const void* logits, int32_t dtype, const float* q, const int32_t* draft,
                        const int32_t* cu, const float* T, const int32_t* top_k, const float* top_p,
                        int32_t B, int32_t D, int32_t max_k, int32_t V, uint64_t seed, int32_t greedy_only,
                        double eps, int32_t* out, int32_t* num_accepted, int32_t* flags, double* p_draft,
                        int32_t* cand, int32_t nthreads) {
  if (!logits || !draft || !cu || !out || !num_accepted || !flags) return -1;
  if (!greedy_only && !T) return -1;
  if (B < 0 || D < 0 || V < 1 || max_k < 0 || (dtype != RSO_F32 && dtype != RSO_BF16)) return -1;
  if (p_draft)
    for (int32_t i = 0; i < D; ++i) p_draft[i] = NAN;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int failed = 0;
#pragma omp parallel
  {
    double* l = (double*)malloc(sizeof(double) * (size_t)V);
    double* p = (double*)malloc(sizeof(double) * (size_t)V);
    double* r = (double*)malloc(sizeof(double) * (size_t)V);
    double* rlo = (double*)malloc(sizeof(double) * (size_t)V);
    double* rhi = (double*)malloc(sizeof(double) * (size_t)V);
    double* E = (double*)malloc(sizeof(double) * (size_t)V);
    double* srt = (double*)malloc(sizeof(double) * (size_t)V);
    if (!l || !p || !r || !rlo || !rhi || !E || !srt) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int32_t b = 0; b < B; ++b) {
      if (failed) continue;
      int32_t* ob = out + (int64_t)b * (max_k + 1);
      for (int32_t i = 0; i <= max_k; ++i) ob[i] = -1;
      num_accepted[b] = -1;
      flags[b] = 0;
      int32_t* cb = cand ? cand + (int64_t)b * RSO_NCAND : NULL;
      if (cb)
        for (int i = 0; i < RSO_NCAND; ++i) cb[i] = -1;
      int32_t s = cu[b], e = cu[b + 1];
      int32_t K = e - s;
      int valid = (s >= 0 && e <= D && K >= 0 && K <= max_k);
      for (int32_t i = 0; valid && i < K; ++i)
        if (draft[s + i] < 0 || draft[s + i] >= V) valid = 0;
      if (!valid) {
        flags[b] = RSO_FLAG_INVALID;
        continue;
      }
      int64_t row0 = (int64_t)s + b; /* row of position 0 */
      int greedy = greedy_only || !(T[b] > 0.0f);
      int32_t n = K, token = -1;
      if (greedy) {
        /* accept while draft_j == argmax of row j; emit the argmax at n */
        for (int32_t j = 0; j < K; ++j) {
          load_row(logits, dtype, row0 + j, V, l);
          if (draft[s + j] != argmax_lowest(l, V)) {
            n = j;
            break;
          }
        }
        load_row(logits, dtype, row0 + n, V, l);
        token = argmax_lowest(l, V);
      } else {
        double Tb = (double)T[b];
        int32_t kb = top_k ? top_k[b] : 0;
        double pb = top_p ? (double)top_p[b] : 1.0;
        int ptie = 0;
        for (int32_t j = 0; j < K; ++j) {
          load_row(logits, dtype, row0 + j, V, l);
          rso_filtered_probs_row(l, V, Tb, kb, pb, eps, p, srt, &ptie);
          if (ptie) flags[b] |= RSO_FLAG_TOPP_TIE;
          int32_t xs = draft[s + j];
          double qs = q ? (double)q[(int64_t)(s + j) * V + xs] : 1.0;
          double u = rso_accept_uniform(seed, b, j);
          double ps = p[xs];
          if (p_draft) p_draft[s + j] = ps;
          if (fabs(ps - u * qs) <= eps * ps) flags[b] |= RSO_FLAG_ACCEPT_TIE;
          if (!(u * qs < ps)) {
            n = j;
            break;
          }
        }
        /* p at the sampled position n (bonus row when n == K) */
        load_row(logits, dtype, row0 + n, V, l);
        rso_filtered_probs_row(l, V, Tb, kb, pb, eps, p, srt, &ptie);
        if (ptie) flags[b] |= RSO_FLAG_TOPP_TIE;
        if (n < K) {
          int32_t xs = draft[s + n];
          for (int32_t x = 0; x < V; ++x) {
            if (q) {
              double qx = (double)q[(int64_t)(s + n) * V + x];
              r[x] = fmax(0.0, p[x] - qx);
              rlo[x] = fmax(0.0, p[x] * (1.0 - eps) - qx);
              rhi[x] = fmax(0.0, p[x] * (1.0 + eps) - qx);
            } else {
              r[x] = (x == xs) ? 0.0 : p[x];
              rlo[x] = r[x] * (1.0 - eps);
              rhi[x] = r[x] * (1.0 + eps);
            }
          }
        } else {
          for (int32_t x = 0; x < V; ++x) {
            r[x] = p[x];
            rlo[x] = p[x] * (1.0 - eps);
            rhi[x] = p[x] * (1.0 + eps);
          }
        }
        token = sample_with_fallback(r, rlo, rhi, p, V, seed, b, n, eps, E, &flags[b], cb);
      }
      for (int32_t i = 0; i < n; ++i) ob[i] = draft[s + i];
      ob[n] = token;
      num_accepted[b] = n;
    }
    free(l); free(p); free(r); free(rlo); free(rhi); free(E); free(srt);
  }
  return failed ? -1 : 0;
}

/* rso_verify_filtered with no top-k / top-p. */
int rso_verify(const void* logits, int32_t dtype, const float* q, const int32_t* draft,
               const int32_t* cu, const float* T, int32_t B, int32_t D, int32_t max_k, int32_t V,
               uint64_t seed, int32_t greedy_only, double eps, int32_t* out, int32_t* num_accepted,
               int32_t* flags, double* p_draft, int32_t* cand, int32_t nthreads) {
  return rso_verify_filtered(logits, dtype, q, draft, cu, T, NULL, NULL, B, D, max_k, V, seed, greedy_only,
                             eps, out, num_accepted, flags, p_draft, cand, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Tree verify.  A request's drafts form a tree (each node one draft token,
 * its parent earlier in the node order or -1 for a child of the last prefix
 * position); the target scored the last prefix position (row 0) and every
 * node (row 1 + i), row r predicting the children of its node.  Verification
 * walks the tree from the root one depth at a time and stops at the first
 * depth where no child is accepted; one extra token is then emitted from the
 * stop node's row.  [投机解码深度实战 §四 (tree drafts, one forward over the
 * whole tree); 投机解码（Speculative Decoding）端到端深挖 §6.2 (per depth, match
 * among the current layer's siblings, descend into the match, stop when the
 * whole layer fails; a bonus follows the last accepted node), §7.1 (greedy),
 * §7.2 (random: one coin per layer against the siblings' accumulated target
 * probabilities; the extra token from the residual)]
 *   greedy (T <= 0): the child whose token is the row's argmax (lowest index
 *     on ties, first such child), else stop and emit the argmax.
 *   random: p = softmax(row / T); coin u_d = the accept uniform of depth d;
 *     children in node order, a child whose token repeats an earlier
 *     sibling's is skipped; child i is accepted iff u_d < (sum of p over the
 *     siblings up to and including i); if none, emit the race over p with
 *     the children's tokens removed (exponentials of depth d); a node
 *     without children emits the race over p (the bonus).
 * Reading (§7.2 with both thresholds at their default 1.0 and the draft
 * distribution one-hot on the siblings): each sibling is accepted with
 * probability p(its token) and the residual is p without the siblings, so the
 * emitted token at every depth is distributed as p.  A one-child-per-node tree
 * is the chain with one-hot q, with the same random numbers.
 * With draft distributions q (one row per tree position, aligned with the
 * target rows: row 0 the prefix position, row 1 + i node i), the extra token
 * after a stop at node c is the race over max(0, p - q_c) instead, q_c the
 * row of c [§7.2: after a rejection the extra token is sampled from
 * relu(target_probs - draft_probs)]; the acceptance roulette is unchanged.
 * This is the page's rule as written: it keeps p only when q_c is p on the
 * siblings and 0 elsewhere (then it is the rule above, the same tokens), not
 * for an arbitrary q (§7.4 calls the target-only path inexact).  An all-zero
 * residual falls back to the race over p, flagged, as in the chain.  A stop
 * at a childless node rejected nothing, so its extra token is the race over p
 * whatever q_c holds (the bonus after a full acceptance).
 *   tree tokens [N], parents [N] (request-local node index or -1), cu [B+1];
 *   out [B, max_depth + 1] tokens (-1 padded), path [B, max_depth] node
 *   indices (-1 padded), num_accepted [B]; flags as rso_verify (invalid:
 *   parent >= node or < -1, token outside [0, V), depth beyond max_depth,
 *   more than max_nodes nodes).
 * Returns 0, or -1 on an argument error. */
int rso_verify_tree(const void* logits, int32_t dtype, const float* q, const int32_t* tokens,
                    const int32_t* parents, const int32_t* cu, const float* T, int32_t B, int32_t N, int32_t max_nodes,
                    int32_t max_depth, int32_t V, uint64_t seed, double eps, int32_t* out, int32_t* path,
                    int32_t* num_accepted, int32_t* flags, int32_t* cand, int32_t nthreads) {
  if (!logits || !cu || !T || !out || !path || !num_accepted || !flags) return -1;
  if (B < 0 || N < 0 || V < 1 || max_nodes < 0 || max_depth < 0 || (N > 0 && (!tokens || !parents))) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int failed = 0;
#pragma omp parallel
  {
    double* l = (double*)malloc(sizeof(double) * (size_t)V);
    double* p = (double*)malloc(sizeof(double) * (size_t)V);
    double* r = (double*)malloc(sizeof(double) * (size_t)V);
    double* rlo = (double*)malloc(sizeof(double) * (size_t)V);
    double* rhi = (double*)malloc(sizeof(double) * (size_t)V);
    double* E = (double*)malloc(sizeof(double) * (size_t)V);
    int32_t* depth = (int32_t*)malloc(sizeof(int32_t) * (size_t)(max_nodes > 0 ? max_nodes : 1));
    if (!l || !p || !r || !rlo || !rhi || !E || !depth) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int32_t b = 0; b < B; ++b) {
      if (failed) continue;
      int32_t* ob = out + (int64_t)b * (max_depth + 1);
      int32_t* pb = path + (int64_t)b * max_depth;
      for (int32_t i = 0; i <= max_depth; ++i) ob[i] = -1;
      for (int32_t i = 0; i < max_depth; ++i) pb[i] = -1;
      num_accepted[b] = -1;
      flags[b] = 0;
      int32_t* cb = cand ? cand + (int64_t)b * RSO_NCAND : NULL;
      if (cb)
        for (int i = 0; i < RSO_NCAND; ++i) cb[i] = -1;
      int32_t s = cu[b], e = cu[b + 1], n = e - s;
      int valid = (s >= 0 && e <= N && n >= 0 && n <= max_nodes);
      for (int32_t i = 0; valid && i < n; ++i) {
        int32_t par = parents[s + i];
        if (par < -1 || par >= i || tokens[s + i] < 0 || tokens[s + i] >= V) valid = 0;
        else {
          depth[i] = par < 0 ? 0 : depth[par] + 1;
          if (depth[i] >= max_depth) valid = 0;
        }
      }
      if (!valid) {
        flags[b] = RSO_FLAG_INVALID;
        continue;
      }
      int64_t row0 = (int64_t)s + b; /* root row; node i is row row0 + 1 + i */
      int greedy = !(T[b] > 0.0f);
      double Tb = (double)T[b];
      int32_t cur = -1, d = 0, token = -1;
      for (;;) {
        load_row(logits, dtype, row0 + 1 + cur, V, l);
        int32_t next = -1;
        if (greedy) {
          int32_t g = argmax_lowest(l, V);
          for (int32_t i = 0; i < n && next < 0; ++i)
            if (parents[s + i] == cur && tokens[s + i] == g) next = i;
          if (next < 0) token = g;
        } else {
          rso_softmax_row(l, V, Tb, p);
          double u = rso_accept_uniform(seed, b, d), cum = 0.0;
          int32_t kids = 0;
          for (int32_t i = 0; i < n && next < 0; ++i) {
            if (parents[s + i] != cur) continue;
            ++kids;
            int dup = 0;
            for (int32_t k = 0; k < i; ++k)
              if (parents[s + k] == cur && tokens[s + k] == tokens[s + i]) dup = 1;
            if (dup) continue;
            cum += p[tokens[s + i]];
            if (fabs(u - cum) <= eps * cum) flags[b] |= RSO_FLAG_ACCEPT_TIE;
            if (u < cum) next = i;
          }
          if (next < 0 && q && kids > 0) {
            /* residual after the siblings were turned down: max(0, p - q) with
             * the stop node's draft row.  A childless node proposed nothing,
             * so nothing was rejected there and its extra token follows p
             * (the branch below, with no tokens to take out). */
            const float* qc = q + (row0 + 1 + cur) * (int64_t)V;
            for (int32_t x = 0; x < V; ++x) {
              double qx = (double)qc[x];
              r[x] = fmax(0.0, p[x] - qx);
              rlo[x] = fmax(0.0, p[x] * (1.0 - eps) - qx);
              rhi[x] = fmax(0.0, p[x] * (1.0 + eps) - qx);
            }
            token = sample_with_fallback(r, rlo, rhi, p, V, seed, b, d, eps, E, &flags[b], cb);
          } else if (next < 0) {
            /* residual: p without the children's tokens (a childless node: p) */
            for (int32_t x = 0; x < V; ++x) r[x] = p[x];
            for (int32_t i = 0; i < n; ++i)
              if (parents[s + i] == cur) r[tokens[s + i]] = 0.0;
            for (int32_t x = 0; x < V; ++x) {
              rlo[x] = r[x] * (1.0 - eps);
              rhi[x] = r[x] * (1.0 + eps);
            }
            token = sample_with_fallback(r, rlo, rhi, p, V, seed, b, d, eps, E, &flags[b], cb);
          }
        }
        if (next < 0) break;
        ob[d] = tokens[s + next];
        pb[d] = next;
        cur = next;
        ++d;
      }
      ob[d] = token;
      num_accepted[b] = d;
    }
    free(l); free(p); free(r); free(rlo); free(rhi); free(E); free(depth);
  }
  return failed ? -1 : 0;
}

/* Full p = softmax(l / T_b) for every row of every request (rows of greedy
 * requests, T <= 0, are filled with NaN).  Used to check the library's
 * optional full-probability output on small shapes. */
int rso_probs(const void* logits, int32_t dtype, const int32_t* cu, const float* T, int32_t B,
              int32_t V, double* probs) {
  if (!logits || !cu || !T || !probs || V < 1) return -1;
  double* l = (double*)malloc(sizeof(double) * (size_t)V);
  if (!l) return -1;
  for (int32_t b = 0; b < B; ++b) {
    for (int64_t row = (int64_t)cu[b] + b; row <= (int64_t)cu[b + 1] + b; ++row) {
      double* pr = probs + row * V;
      if (!(T[b] > 0.0f)) {
        for (int32_t x = 0; x < V; ++x) pr[x] = NAN;
        continue;
      }
      load_row(logits, dtype, row, V, l);
      rso_softmax_row(l, V, (double)T[b], pr);
    }
  }
  free(l);
  return 0;
}

/* Vector helpers for the statistical pins of the random stream. */
void rso_accept_uniforms(uint64_t seed, const int32_t* b, const int32_t* j, int64_t n, double* u) {
  for (int64_t i = 0; i < n; ++i) u[i] = rso_accept_uniform(seed, b[i], j[i]);
}
void rso_race_exponentials(uint64_t seed, int32_t b, int32_t j, int32_t x0, int64_t n, double* e) {
  for (int64_t i = 0; i < n; ++i) e[i] = rso_race_exponential(seed, b, j, (int32_t)(x0 + i));
}

/* n independent Philox4x32-10 evaluations: ctr [n,4], key [n,2], out [n,4]. */
void rso_philox_many(int64_t n, const uint32_t* ctr, const uint32_t* key, uint32_t* out) {
  for (int64_t i = 0; i < n; ++i) rso_philox4x32_10(ctr + 4 * i, key + 2 * i, out + 4 * i);
}
