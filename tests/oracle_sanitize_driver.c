/*
 * Runs every function of the CPU oracle (oracle/oracle.c) on seeded synthetic
 * streams, built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_oracle_sanitize.py: a stream is indexed (norms, transform,
 * projection, sorted lists, pages), grows by inserts, and is queried with
 * literal and closed-form walks, bounded and unbounded visit budgets, both GQA
 * readings, page selection and attention, including the empty and tiny
 * cases.  It checks the two walks agree, so a run that only "does not crash"
 * still has to compute.  Exit status 0 when everything ran and agreed.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void ora_key_norm_sq(const float *K, int64_t n, int d, double *nsq);
float ora_norm_bound(const double *nsq, int64_t n);
void ora_transform(const float *K, int64_t n, int d, float c, double *kt);
void ora_project(const float *K, int64_t n, int d, const float *U, int mL, float c, int D,
                 int32_t *codes, uint32_t *cell);
void ora_sort_list(const int32_t *codes, int64_t n, int mL, int t, int32_t *out_code,
                   int32_t *out_id);
void ora_list_insert(int32_t *lcode, int32_t *lid, int64_t n, int32_t code, int32_t id);
int64_t ora_tree(const uint32_t *cell, int64_t n, int D, int p, int32_t *page_of,
                 int32_t *slot_of, int32_t *page_tokens, int32_t *page_len, int32_t *page_cell,
                 int64_t Pcap);
int64_t ora_tree_append(int64_t tok, uint32_t cl, int p, int64_t npages, int32_t *page_of,
                        int32_t *slot_of, int32_t *page_tokens, int32_t *page_len,
                        int32_t *page_cell, int64_t Pcap);
double ora_dot_blocked(const float *a, const float *b, int d);
void ora_query_prep(const float *q, int g, int d, const float *U, int mL, float *qkv,
                    int32_t *qcode);
int64_t ora_pdci_literal(const int32_t *lcode, const int32_t *lid, int64_t n, int m,
                         const int32_t *qcode, int64_t k0, int64_t k1, int32_t *S,
                         int64_t *visits);
int64_t ora_pdci_closed(const int32_t *codes, int64_t n, int mL, int m, int l,
                        const int32_t *qcode, int64_t k0, int64_t k1, int32_t *S,
                        int64_t *visits);
double ora_score(const float *K, int d, const float *qkv, int64_t tok);
void ora_rerank(const float *K, int d, const float *qkv, const int32_t *C, int64_t nC,
                int32_t *ranked, double *scores);
void ora_rerank_max(const float *K, int d, const float *Q, int g, const int32_t *C, int64_t nC,
                    int32_t *ranked, double *scores);
int64_t ora_select_pages(const int32_t *ranked, int64_t nC, const int32_t *page_of, int64_t P,
                         int32_t *page_ids);
void ora_attention(const float *q, int g, int d, const float *poolK, const float *poolV, int p,
                   const int32_t *page_ids, int64_t n_sel, const int32_t *page_len, double *out);

static uint64_t rng_state;
static double uniform(void) { /* SplitMix64, 53-bit uniform in [0, 1) */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}
static float gauss(void) {
  double u = uniform(), v = uniform();
  return (float)(sqrt(-2.0 * log(u + 1e-300)) * cos(6.283185307179586 * v));
}

static int fails;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      ++fails;                                                     \
    }                                                              \
  } while (0)

/* One stream: build from n0 tokens, insert ins more, query with g heads. */
static void run(int n0, int ins, int d, int m, int L, int p, int k, int g, int64_t k1,
                uint64_t seed) {
  rng_state = seed;
  const int mL = m * L, n = n0 + ins, P = k / p;
  float *K = malloc(sizeof(float) * (size_t)(n > 0 ? n : 1) * d);
  float *V = malloc(sizeof(float) * (size_t)(n > 0 ? n : 1) * d);
  float *U = malloc(sizeof(float) * (size_t)mL * (d + 1));
  float *q = malloc(sizeof(float) * (size_t)g * d);
  for (int64_t i = 0; i < (int64_t)n * d; ++i) {
    K[i] = gauss();
    V[i] = gauss();
  }
  for (int t = 0; t < mL; ++t) {
    double nrm = 0.0;
    for (int e = 0; e <= d; ++e) {
      U[t * (d + 1) + e] = gauss();
      nrm += (double)U[t * (d + 1) + e] * U[t * (d + 1) + e];
    }
    for (int e = 0; e <= d; ++e) U[t * (d + 1) + e] = (float)(U[t * (d + 1) + e] / sqrt(nrm));
  }
  for (int i = 0; i < g * d; ++i) q[i] = gauss();

  double *nsq = malloc(sizeof(double) * (size_t)(n0 > 0 ? n0 : 1));
  ora_key_norm_sq(K, n0, d, nsq);
  const float c = ora_norm_bound(nsq, n0);
  double *kt = malloc(sizeof(double) * (size_t)(n0 > 0 ? n0 : 1) * (d + 1));
  ora_transform(K, n0, d, c, kt);
  const int D = 3;
  int32_t *codes = malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1) * mL);
  uint32_t *cell = malloc(sizeof(uint32_t) * (size_t)(n > 0 ? n : 1));
  ora_project(K, n, d, U, mL, c, D, codes, cell); /* the inserts use the stored c */
  int32_t *lc = malloc(sizeof(int32_t) * (size_t)mL * (n > 0 ? n : 1));
  int32_t *li = malloc(sizeof(int32_t) * (size_t)mL * (n > 0 ? n : 1));
  for (int t = 0; t < mL; ++t) ora_sort_list(codes, n0, mL, t, lc + (int64_t)t * n, li + (int64_t)t * n);
  const int64_t Pcap = (n + p - 1) / p + (1 << D);
  int32_t *page_of = malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  int32_t *slot_of = malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  int32_t *page_tokens = malloc(sizeof(int32_t) * (size_t)Pcap * p);
  int32_t *page_len = malloc(sizeof(int32_t) * (size_t)Pcap);
  int32_t *page_cell = malloc(sizeof(int32_t) * (size_t)Pcap);
  int64_t npages = ora_tree(cell, n0, D, p, page_of, slot_of, page_tokens, page_len, page_cell, Pcap);
  CHECK(npages >= 0);
  for (int i = n0; i < n; ++i) {
    for (int t = 0; t < mL; ++t)
      ora_list_insert(lc + (int64_t)t * n, li + (int64_t)t * n, i, codes[(int64_t)i * mL + t], i);
    npages = ora_tree_append(i, cell[i], p, npages, page_of, slot_of, page_tokens, page_len,
                             page_cell, Pcap);
    CHECK(npages >= 0);
  }
  /* queries: the mean reading (one head set), then each head alone */
  float *qkv = malloc(sizeof(float) * (size_t)d);
  int32_t *qcode = malloc(sizeof(int32_t) * (size_t)mL);
  const int64_t k0 = k;
  int32_t *S1 = malloc(sizeof(int32_t) * (size_t)(k0 > 0 ? k0 : 1));
  int32_t *S2 = malloc(sizeof(int32_t) * (size_t)(k0 > 0 ? k0 : 1));
  int32_t *C = malloc(sizeof(int32_t) * (size_t)((int64_t)g * L * k0 + 1));
  int64_t nC = 0;
  int32_t *lcl = malloc(sizeof(int32_t) * (size_t)m * (n > 0 ? n : 1));
  int32_t *lil = malloc(sizeof(int32_t) * (size_t)m * (n > 0 ? n : 1));
  for (int h = -1; h < g; ++h) {
    if (h < 0)
      ora_query_prep(q, g, d, U, mL, qkv, qcode);
    else
      ora_query_prep(q + (int64_t)h * d, 1, d, U, mL, qkv, qcode);
    for (int l = 0; l < L; ++l) {
      for (int j = 0; j < m; ++j) {
        memcpy(lcl + (int64_t)j * n, lc + (int64_t)(l * m + j) * n, sizeof(int32_t) * (size_t)n);
        memcpy(lil + (int64_t)j * n, li + (int64_t)(l * m + j) * n, sizeof(int32_t) * (size_t)n);
      }
      int64_t v1 = 0, v2 = 0;
      const int64_t a = ora_pdci_literal(lcl, lil, n, m, qcode + l * m, k0, k1, S1, &v1);
      const int64_t b = ora_pdci_closed(codes, n, mL, m, l, qcode, k0, k1, S2, &v2);
      CHECK(a == b && v1 == v2 && memcmp(S1, S2, sizeof(int32_t) * (size_t)a) == 0);
      if (h >= 0)
        for (int64_t x = 0; x < a; ++x) C[nC++] = S1[x];
    }
  }
  (void)ora_dot_blocked(q, q, d);
  (void)ora_score(K, d, q, 0);
  int32_t *ranked = malloc(sizeof(int32_t) * (size_t)(nC + 1));
  double *scores = malloc(sizeof(double) * (size_t)(nC + 1));
  /* de-duplicate the pooled candidates (the rerank expects a set) */
  int64_t u = 0;
  for (int64_t x = 0; x < nC; ++x) {
    int dup = 0;
    for (int64_t y = 0; y < u; ++y) dup |= C[y] == C[x];
    if (!dup) C[u++] = C[x];
  }
  ora_rerank(K, d, qkv, C, u, ranked, scores);
  ora_rerank_max(K, d, q, g, C, u, ranked, scores);
  for (int64_t x = 1; x < u; ++x) CHECK(scores[x - 1] >= scores[x]);
  int32_t *page_ids = malloc(sizeof(int32_t) * (size_t)(P > 0 ? P : 1));
  const int64_t ns = ora_select_pages(ranked, u, page_of, P, page_ids);
  CHECK(ns <= P && ns >= 0);
  float *pk = calloc((size_t)Pcap * p * d, sizeof(float));
  float *pv = calloc((size_t)Pcap * p * d, sizeof(float));
  for (int64_t pg = 0; pg < npages; ++pg)
    for (int sl = 0; sl < page_len[pg]; ++sl) {
      const int32_t tok = page_tokens[pg * p + sl];
      memcpy(pk + (pg * p + sl) * d, K + (int64_t)tok * d, sizeof(float) * (size_t)d);
      memcpy(pv + (pg * p + sl) * d, V + (int64_t)tok * d, sizeof(float) * (size_t)d);
    }
  double *out = malloc(sizeof(double) * (size_t)g * d);
  ora_attention(q, g, d, pk, pv, p, page_ids, ns, page_len, out);
  for (int i = 0; i < g * d; ++i) CHECK(isfinite(out[i]));
  free(K); free(V); free(U); free(q); free(nsq); free(kt); free(codes); free(cell); free(lc);
  free(li); free(page_of); free(slot_of); free(page_tokens); free(page_len); free(page_cell);
  free(qkv); free(qcode); free(S1); free(S2); free(C); free(lcl); free(lil); free(ranked);
  free(scores); free(page_ids); free(pk); free(pv); free(out);
}

int main(void) {
  run(700, 40, 64, 3, 2, 16, 64, 2, 0, 1);        /* unbounded walks */
  run(900, 25, 128, 4, 3, 8, 128, 4, 1500, 2);    /* bounded walks, page size 8 */
  run(100, 5, 16, 2, 2, 16, 256, 1, 0, 3);        /* fewer tokens than k0 */
  run(0, 30, 16, 2, 2, 16, 32, 2, 0, 4);          /* empty build, inserts only */
  run(300, 0, 32, 1, 1, 32, 64, 3, 7, 5);         /* one list, tiny budget */
  if (fails) fprintf(stderr, "%d checks failed\n", fails);
  return fails ? 1 : 0;
}
