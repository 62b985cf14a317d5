/* Host sanitizer driver for the CPU oracle (test infrastructure): calls every
 * oracle entry on small seeded inputs -- random and greedy requests, q present
 * and absent, q = 2p (the all-zero residual), top-k / top-p, K_b = 0, V = 1,
 * -inf logits, invalid metadata, trees -- and checks that the outputs are in
 * range.  Built with -fsanitize=address,undefined by
 * tests/test_host_sanitizers.py; any sanitizer report fails the test. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int rso_verify(const void*, int32_t, const float*, const int32_t*, const int32_t*, const float*, int32_t, int32_t,
               int32_t, int32_t, uint64_t, int32_t, double, int32_t*, int32_t*, int32_t*, double*, int32_t*,
               int32_t);
int rso_verify_filtered(const void*, int32_t, const float*, const int32_t*, const int32_t*, const float*,
                        const int32_t*, const float*, int32_t, int32_t, int32_t, int32_t, uint64_t, int32_t, double,
                        int32_t*, int32_t*, int32_t*, double*, int32_t*, int32_t);
int rso_verify_tree(const void*, int32_t, const float*, const int32_t*, const int32_t*, const int32_t*,
                    const float*, int32_t, int32_t, int32_t, int32_t, int32_t, uint64_t, double, int32_t*, int32_t*,
                    int32_t*, int32_t*, int32_t*, int32_t);
int rso_probs(const void*, int32_t, const int32_t*, const float*, int32_t, int32_t, double*);
void rso_filtered_probs_row(const double*, int32_t, double, int32_t, double, double, double*, double*, int*);

static uint64_t lcg = 88172645463325252ull;
static double unif(void) {  /* xorshift64, [0, 1) */
  lcg ^= lcg << 13;
  lcg ^= lcg >> 7;
  lcg ^= lcg << 17;
  return (double)(lcg >> 11) * 0x1p-53;
}
static double gauss(void) { return sqrt(-2.0 * log(1.0 - unif())) * cos(6.283185307179586 * unif()); }

static int fails = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++fails;                                                     \
    }                                                              \
  } while (0)

static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

/* One chain batch: ks[B] drafts, vocab V; q_mode 0 none, 1 softmax-like, 2 twice a softmax. */
static void chain_case(const int32_t* ks, int32_t B, int32_t V, int dtype, int q_mode, int greedy_only,
                       int filtered, int neg_inf) {
  int32_t D = 0, max_k = 0;
  for (int32_t b = 0; b < B; ++b) {
    D += ks[b];
    if (ks[b] > max_k) max_k = ks[b];
  }
  int32_t R = D + B;
  float* lf = malloc(sizeof(float) * (size_t)R * V);
  uint16_t* lb = malloc(sizeof(uint16_t) * (size_t)R * V);
  for (int64_t i = 0; i < (int64_t)R * V; ++i) {
    lf[i] = (float)(3.0 * gauss());
    if (neg_inf && (i % V) >= V / 2 && V > 1) lf[i] = -INFINITY;
    lb[i] = to_bf16(lf[i]);
  }
  int32_t* cu = malloc(sizeof(int32_t) * (size_t)(B + 1));
  cu[0] = 0;
  for (int32_t b = 0; b < B; ++b) cu[b + 1] = cu[b] + ks[b];
  float* q = NULL;
  if (q_mode && D > 0) {
    q = malloc(sizeof(float) * (size_t)D * V);
    for (int32_t s = 0; s < D; ++s) {
      double z = 0.0;
      for (int32_t x = 0; x < V; ++x) z += (q[(int64_t)s * V + x] = (float)exp(gauss()));
      for (int32_t x = 0; x < V; ++x) q[(int64_t)s * V + x] = (float)(q[(int64_t)s * V + x] / z * q_mode);
    }
  }
  int32_t* draft = malloc(sizeof(int32_t) * (size_t)(D > 0 ? D : 1));
  for (int32_t s = 0; s < D; ++s) draft[s] = neg_inf ? (int32_t)(unif() * (V / 2 > 0 ? V / 2 : 1)) : (int32_t)(unif() * V);
  float* T = malloc(sizeof(float) * (size_t)B);
  int32_t* tk = malloc(sizeof(int32_t) * (size_t)B);
  float* tp = malloc(sizeof(float) * (size_t)B);
  for (int32_t b = 0; b < B; ++b) {
    T[b] = (b % 4 == 3) ? 0.0f : (float)(0.3 + unif());
    tk[b] = (int32_t)(unif() * (V + 2)) - 1;
    tp[b] = (b % 3 == 0) ? 1.0f : (float)unif();
  }
  int32_t* out = malloc(sizeof(int32_t) * (size_t)B * (max_k + 1));
  int32_t* nacc = malloc(sizeof(int32_t) * (size_t)B);
  int32_t* flags = malloc(sizeof(int32_t) * (size_t)B);
  int32_t* cand = malloc(sizeof(int32_t) * (size_t)B * 8);
  double* pd = malloc(sizeof(double) * (size_t)(D > 0 ? D : 1));
  const void* lg = dtype ? (const void*)lb : (const void*)lf;
  int rc = filtered ? rso_verify_filtered(lg, dtype, q, draft, cu, T, tk, tp, B, D, max_k, V, 7, greedy_only, 1e-6,
                                          out, nacc, flags, pd, cand, 2)
                    : rso_verify(lg, dtype, q, draft, cu, T, B, D, max_k, V, 7, greedy_only, 1e-6, out, nacc, flags,
                                 pd, cand, 2);
  CHECK(rc == 0);
  for (int32_t b = 0; b < B; ++b) {
    CHECK(nacc[b] >= 0 && nacc[b] <= ks[b]);
    CHECK(out[(int64_t)b * (max_k + 1) + nacc[b]] >= 0 && out[(int64_t)b * (max_k + 1) + nacc[b]] < V);
  }
  double* P = malloc(sizeof(double) * (size_t)R * V);
  if (!greedy_only) CHECK(rso_probs(lg, dtype, cu, T, B, V, P) == 0);
  free(P);
  free(lf); free(lb); free(cu); free(q); free(draft); free(T); free(tk); free(tp);
  free(out); free(nacc); free(flags); free(cand); free(pd);
}

static void invalid_case(void) {
  const int32_t V = 10, B = 3, max_k = 2;
  float lg[7 * 10] = {0};
  int32_t cu[4] = {0, 2, 5, 4};  /* request 1 has K = 3 > max_k; request 2 goes backwards */
  int32_t draft[4] = {1, 2, 3, 99};
  float T[3] = {1.0f, 1.0f, 1.0f};
  int32_t out[3 * 3], nacc[3], flags[3], cand[3 * 8];
  double pd[4];
  CHECK(rso_verify(lg, 0, NULL, draft, cu, T, B, 4, max_k, V, 1, 0, 1e-6, out, nacc, flags, pd, cand, 1) == 0);
  CHECK(nacc[1] == -1 && nacc[2] == -1);
  CHECK(rso_verify(NULL, 0, NULL, draft, cu, T, B, 4, max_k, V, 1, 0, 1e-6, out, nacc, flags, pd, cand, 1) == -1);
}

static void tree_case(int32_t V, int dtype) {
  const int32_t B = 5, n = 12, max_depth = 4;
  int32_t par[12] = {-1, -1, -1, 0, 0, 1, 3, 3, 6, -1, 9, 10};
  int32_t tok[5 * 12], parents[5 * 12], cu[6];
  for (int32_t b = 0; b < B; ++b) {
    cu[b] = b * n;
    for (int32_t i = 0; i < n; ++i) {
      parents[b * n + i] = par[i];
      tok[b * n + i] = (int32_t)(unif() * V);
    }
  }
  cu[B] = B * n;
  parents[3 * n + 4] = 7;  /* request 3: a parent after its child (invalid) */
  int32_t R = B * (n + 1);
  float* lf = malloc(sizeof(float) * (size_t)R * V);
  uint16_t* lb = malloc(sizeof(uint16_t) * (size_t)R * V);
  for (int64_t i = 0; i < (int64_t)R * V; ++i) lb[i] = to_bf16(lf[i] = (float)(2.0 * gauss()));
  float T[5] = {1.0f, 0.0f, 0.7f, 1.2f, -1.0f};
  int32_t out[5 * 5], path[5 * 4], nacc[5], flags[5], cand[5 * 8];
  CHECK(rso_verify_tree(dtype ? (const void*)lb : (const void*)lf, dtype, NULL, tok, parents, cu, T, B, B * n, n,
                        max_depth, V, 3, 1e-6, out, path, nacc, flags, cand, 2) == 0);
  CHECK(nacc[3] == -1);
  for (int32_t b = 0; b < B; ++b)
    if (b != 3) CHECK(nacc[b] >= 0 && nacc[b] <= max_depth);
  /* with draft distributions: one row per tree position */
  float* q = malloc(sizeof(float) * (size_t)R * V);
  for (int64_t i = 0; i < (int64_t)R * V; ++i) q[i] = (float)(unif() * 2.0 / V);
  CHECK(rso_verify_tree(dtype ? (const void*)lb : (const void*)lf, dtype, q, tok, parents, cu, T, B, B * n, n,
                        max_depth, V, 3, 1e-6, out, path, nacc, flags, cand, 2) == 0);
  CHECK(nacc[3] == -1);
  free(q);
  free(lf);
  free(lb);
}

int main(void) {
  const int32_t k1[6] = {3, 0, 5, 2, 8, 1};
  for (int dt = 0; dt < 2; ++dt)
    for (int qm = 0; qm < 3; ++qm) {
      chain_case(k1, 6, 37, dt, qm, 0, 0, 0);
      chain_case(k1, 6, 37, dt, qm, 0, 1, 0);
    }
  chain_case(k1, 6, 37, 1, 1, 1, 0, 0);  /* greedy entry */
  chain_case(k1, 6, 1, 0, 1, 0, 0, 0);   /* V = 1 */
  chain_case(k1, 6, 64, 1, 1, 0, 1, 1);  /* -inf logits, filtered */
  const int32_t k0[3] = {0, 0, 0};
  chain_case(k0, 3, 16, 1, 0, 0, 0, 0);  /* no drafts at all */
  invalid_case();
  tree_case(9, 0);
  tree_case(300, 1);
  double l[8], p[8], srt[8];
  int tie = 0;
  for (int i = 0; i < 8; ++i) l[i] = (double)(i % 3);
  rso_filtered_probs_row(l, 8, 0.8, 3, 0.5, 1e-6, p, srt, &tie);
  double z = 0.0;
  for (int i = 0; i < 8; ++i) z += p[i];
  CHECK(fabs(z - 1.0) < 1e-12);
  if (fails) return 1;
  puts("oracle sanitizer driver: ok");
  return 0;
}
