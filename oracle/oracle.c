/*
 * IceCache decode hot path -- plain CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * generator with the HIP path.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -shared -fPIC
 * (no FMA contraction, IEEE double everywhere; products that must be exact
 * are exact by the operand widths noted at each step).
 *
 * Sources.  "IceCache paper page" = the IceCache paper summary page
 * (arXiv 2604.10539, abstract and figure captions).  "IceCache blog page" =
 * the technical-details section of the blog post on IceCache.  DCI and
 * Prioritized DCI are cited by title only in the paper's citation map
 * ("Builds on" list); the index and query rules below restate the published
 * DCI / P-DCI method in this project's own terms.  Every choice the pages
 * leave open is marked READING and is listed with its rationale in the
 * design notes at the repository root.
 *
 * Everything works on ONE stream (one KV head of one layer of one sequence):
 * the blog page states there is one tree per attention head.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* READING: projections are stored as signed fixed-point codes with 29
 * fractional bits (value * 2^29 rounded half-to-even, saturated at
 * +-(2^30 - 1)).  With exact integer codes the projected distance
 * |code - qcode| is exact, so the visit order of P-DCI is a strict total
 * order and the list walk and its closed form agree exactly. */
#define ORA_CODE_SCALE 536870912.0 /* 2^29 */
#define ORA_CODE_MAX 1073741823LL  /* 2^30 - 1 */

static int32_t ora_to_code(double x) {
  double v = rint(x * ORA_CODE_SCALE); /* scaling by 2^29 is exact */
  if (v > (double)ORA_CODE_MAX) v = (double)ORA_CODE_MAX;
  if (v < -(double)ORA_CODE_MAX) v = -(double)ORA_CODE_MAX;
  return (int32_t)v;
}

/* ------------------------------------------------------------------ */
/* Key transform (IceCache paper page, Figure 2 caption, step (1):     */
/* tokens are indexed in a "transformed key-embedding space").          */
/* READING: the standard MIPS-to-nearest-neighbour reduction,           */
/*   T_K(k) = [k / c, sqrt(1 - |k|^2 / c^2)],  T_Q(q) = [q / |q|, 0],   */
/* with c the largest key norm of the stream at build time.  It makes   */
/* |T_K(k)| = 1 and orders keys by Euclidean distance to T_Q(q) exactly */
/* as by inner product with q.  1/c is formed once and multiplied in.   */
/* ------------------------------------------------------------------ */

/* Squared L2 norm of every key, fp64, ascending element order. */
void ora_key_norm_sq(const float *K, int64_t n, int d, double *nsq) {
  for (int64_t i = 0; i < n; ++i) {
    double acc = 0.0;
    for (int e = 0; e < d; ++e) {
      double v = (double)K[i * d + e];
      acc = acc + v * v; /* exact square of a float */
    }
    nsq[i] = acc;
  }
}

/* c = largest key norm, rounded to fp32; 1 when every key is zero or n = 0. */
float ora_norm_bound(const double *nsq, int64_t n) {
  double mx = 0.0;
  for (int64_t i = 0; i < n; ++i)
    if (nsq[i] > mx) mx = nsq[i];
  float c = (float)sqrt(mx);
  return c > 0.0f ? c : 1.0f;
}

/* Transformed keys [n][d+1] in fp64 (used by the pins, not by the index). */
void ora_transform(const float *K, int64_t n, int d, float c, double *kt) {
  double inv_c = 1.0 / (double)c;
  double inv_c2 = inv_c * inv_c;
  for (int64_t i = 0; i < n; ++i) {
    double nsq = 0.0;
    for (int e = 0; e < d; ++e) {
      double v = (double)K[i * d + e];
      nsq = nsq + v * v;
    }
    double b = 1.0 - nsq * inv_c2;
    if (b < 0.0) b = 0.0; /* keys longer than c (late inserts) */
    for (int e = 0; e < d; ++e) kt[i * (d + 1) + e] = (double)K[i * d + e] * inv_c;
    kt[i * (d + 1) + d] = sqrt(b);
  }
}

/* ------------------------------------------------------------------ */
/* Projection onto the m*L random directions (published DCI index:     */
/* one sorted list per direction; direction t = l*m + j belongs to      */
/* composite l).  codes[i][t] = code( <T_K(k_i), u_t> ), evaluated as   */
/*   r = sum_e k_e u_te   (fp64, ascending e; each product is exact)    */
/*   x = r * (1/c) + s_i * u_td                                          */
/* and the DCI-tree cell of token i is the sign pattern of r on the     */
/* first D directions (READING: a sign-code tree of depth D; a leaf is  */
/* one cell, and it is stored as a chain of pages -- IceCache paper     */
/* page, Figure 2 caption: each leaf corresponds to a physical page).   */
/* U is [mL][d+1].                                                       */
/* ------------------------------------------------------------------ */
void ora_project(const float *K, int64_t n, int d, const float *U, int mL, float c, int D,
                 int32_t *codes, uint32_t *cell) {
  double inv_c = 1.0 / (double)c;
  double inv_c2 = inv_c * inv_c;
  for (int64_t i = 0; i < n; ++i) {
    const float *k = K + i * d;
    double nsq = 0.0;
    for (int e = 0; e < d; ++e) {
      double v = (double)k[e];
      nsq = nsq + v * v;
    }
    double b = 1.0 - nsq * inv_c2;
    if (b < 0.0) b = 0.0;
    double s = sqrt(b);
    uint32_t cl = 0;
    for (int t = 0; t < mL; ++t) {
      const float *u = U + (int64_t)t * (d + 1);
      double r = 0.0;
      for (int e = 0; e < d; ++e) r = r + (double)k[e] * (double)u[e];
      double x = r * inv_c + s * (double)u[d];
      codes[i * mL + t] = ora_to_code(x);
      if (t < D && r >= 0.0) cl |= (1u << t);
    }
    if (cell) cell[i] = cl;
  }
}

/* ------------------------------------------------------------------ */
/* Sorted list of direction t: all tokens ascending by (code, token).   */
/* ------------------------------------------------------------------ */
typedef struct {
  int32_t code, id;
} ora_entry;

static int ora_entry_cmp(const void *a, const void *b) {
  const ora_entry *x = (const ora_entry *)a, *y = (const ora_entry *)b;
  if (x->code != y->code) return x->code < y->code ? -1 : 1;
  return (x->id > y->id) - (x->id < y->id);
}

void ora_sort_list(const int32_t *codes, int64_t n, int mL, int t, int32_t *out_code,
                   int32_t *out_id) {
  ora_entry *a = (ora_entry *)malloc(sizeof(ora_entry) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) {
    a[i].code = codes[i * mL + t];
    a[i].id = (int32_t)i;
  }
  qsort(a, (size_t)n, sizeof(ora_entry), ora_entry_cmp);
  for (int64_t i = 0; i < n; ++i) {
    out_code[i] = a[i].code;
    out_id[i] = a[i].id;
  }
  free(a);
}

/* Dynamic update of one list (blog page: the tree is updated with no    */
/* rebuild when a token arrives).  Inserts (code, id) keeping the order; */
/* `n` is the current length, the arrays hold n + 1 slots.               */
void ora_list_insert(int32_t *lcode, int32_t *lid, int64_t n, int32_t code, int32_t id) {
  int64_t lo = 0, hi = n; /* first position whose (code, id) > (code, id_new) */
  while (lo < hi) {
    int64_t mid = lo + (hi - lo) / 2;
    if (lcode[mid] < code || (lcode[mid] == code && lid[mid] < id))
      lo = mid + 1;
    else
      hi = mid;
  }
  memmove(lcode + lo + 1, lcode + lo, sizeof(int32_t) * (size_t)(n - lo));
  memmove(lid + lo + 1, lid + lo, sizeof(int32_t) * (size_t)(n - lo));
  lcode[lo] = code;
  lid[lo] = id;
}

/* ------------------------------------------------------------------ */
/* DCI-tree leaves -> physical pages (IceCache paper page, Figure 2:    */
/* each leaf node is a physical memory page; Figure 3: a mapping table  */
/* locates the memory region of each selected node).                    */
/* READING: the tokens of one cell, in token order, are cut into pages  */
/* of p; pages are numbered by the index of their first token.          */
/* Outputs: page_of[n], slot_of[n], page_tokens[Pcap*p] (-1 = empty),   */
/* page_len[Pcap], page_cell[Pcap].  Returns the page count, -1 when    */
/* Pcap is too small.                                                    */
/* ------------------------------------------------------------------ */
typedef struct {
  int64_t first;  /* token index of the page's first token */
  int64_t start;  /* offset of the page's first token in the cell order */
  int32_t len, cl;
} ora_page;

static int ora_page_cmp(const void *a, const void *b) {
  const ora_page *x = (const ora_page *)a, *y = (const ora_page *)b;
  return (x->first > y->first) - (x->first < y->first);
}

int64_t ora_tree(const uint32_t *cell, int64_t n, int D, int p, int32_t *page_of,
                 int32_t *slot_of, int32_t *page_tokens, int32_t *page_len, int32_t *page_cell,
                 int64_t Pcap) {
  int64_t ncell = (int64_t)1 << D;
  int64_t *cnt = (int64_t *)calloc((size_t)ncell + 1, sizeof(int64_t));
  int64_t *order = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) cnt[cell[i] + 1]++;
  for (int64_t c = 0; c < ncell; ++c) cnt[c + 1] += cnt[c]; /* cell starts */
  int64_t *fill = (int64_t *)malloc(sizeof(int64_t) * (size_t)ncell);
  memcpy(fill, cnt, sizeof(int64_t) * (size_t)ncell);
  for (int64_t i = 0; i < n; ++i) order[fill[cell[i]]++] = i; /* token order kept */

  int64_t npages = 0;
  for (int64_t c = 0; c < ncell; ++c) npages += (cnt[c + 1] - cnt[c] + p - 1) / p;
  if (npages > Pcap) {
    free(cnt); free(order); free(fill);
    return -1;
  }
  ora_page *pages = (ora_page *)malloc(sizeof(ora_page) * (size_t)(npages > 0 ? npages : 1));
  int64_t np = 0;
  for (int64_t c = 0; c < ncell; ++c)
    for (int64_t s = cnt[c]; s < cnt[c + 1]; s += p) {
      pages[np].first = order[s];
      pages[np].start = s;
      pages[np].len = (int32_t)((cnt[c + 1] - s) < p ? (cnt[c + 1] - s) : p);
      pages[np].cl = (int32_t)c;
      ++np;
    }
  qsort(pages, (size_t)np, sizeof(ora_page), ora_page_cmp);
  for (int64_t g = 0; g < Pcap * p; ++g) page_tokens[g] = -1;
  for (int64_t g = 0; g < Pcap; ++g) {
    page_len[g] = 0;
    page_cell[g] = -1;
  }
  for (int64_t g = 0; g < np; ++g) {
    page_len[g] = pages[g].len;
    page_cell[g] = pages[g].cl;
    for (int32_t s = 0; s < pages[g].len; ++s) {
      int64_t tok = order[pages[g].start + s];
      page_of[tok] = (int32_t)g;
      slot_of[tok] = s;
      page_tokens[g * p + s] = (int32_t)tok;
    }
  }
  free(cnt); free(order); free(fill); free(pages);
  return np;
}

/* Dynamic update of the pages: token `tok` of cell `cl` joins the last  */
/* page of its cell when that page has room, else opens page `npages`.   */
/* Returns the new page count, -1 when Pcap is exhausted.                */
int64_t ora_tree_append(int64_t tok, uint32_t cl, int p, int64_t npages, int32_t *page_of,
                        int32_t *slot_of, int32_t *page_tokens, int32_t *page_len,
                        int32_t *page_cell, int64_t Pcap) {
  int64_t last = -1;
  for (int64_t g = 0; g < npages; ++g)
    if (page_cell[g] == (int32_t)cl) last = g; /* pages of a cell rise with their first token */
  if (last < 0 || page_len[last] == p) {
    if (npages >= Pcap) return -1;
    last = npages++;
    page_cell[last] = (int32_t)cl;
    page_len[last] = 0;
  }
  int32_t s = page_len[last]++;
  page_of[tok] = (int32_t)last;
  slot_of[tok] = s;
  page_tokens[last * p + s] = (int32_t)tok;
  return npages;
}

/* ------------------------------------------------------------------ */
/* Dot products of the query side (the query's projections and norm and */
/* the rerank scores).  READING (the pages fix no evaluation order): a   */
/* fixed blocked order in fp64.  The elements are cut into blocks of 16; */
/* each block's products are added in ascending element order (every     */
/* product of two floats is exact in fp64, so each addition rounds once);*/
/* then the block sums are added pairwise, neighbours first:             */
/* ((b0 + b1) + (b2 + b3)) + ((b4 + b5) + (b6 + b7)) for d = 128.        */
/* d must be 16 times a power of two.                                    */
/* ------------------------------------------------------------------ */
double ora_dot_blocked(const float *a, const float *b, int d) {
  double part[64];
  int nb = d / 16;
  for (int j = 0; j < nb; ++j) {
    double acc = 0.0;
    for (int e = 16 * j; e < 16 * j + 16; ++e) acc = acc + (double)a[e] * (double)b[e];
    part[j] = acc;
  }
  for (int w = 1; w < nb; w *= 2) /* tree level: neighbours w apart */
    for (int j = 0; j + w < nb; j += 2 * w) part[j] = part[j] + part[j + w];
  return part[0];
}

/* ------------------------------------------------------------------ */
/* Query preparation.  READING (GQA is only cited by title): the g      */
/* query heads that share a KV head are averaged in fp32 (left fold,    */
/* then times fp32(1/g)); T_Q normalises; q̄_t = <q, u_t[:d]> / |q|,    */
/* the dot products and |q|^2 in the blocked order above.               */
/* q is [g][d]; outputs qkv[d] (fp32) and qcode[mL].                    */
/* ------------------------------------------------------------------ */
void ora_query_prep(const float *q, int g, int d, const float *U, int mL, float *qkv,
                    int32_t *qcode) {
  float inv_g = (float)(1.0 / (double)g);
  for (int e = 0; e < d; ++e) {
    float acc = q[e];
    for (int h = 1; h < g; ++h) acc = acc + q[h * d + e];
    qkv[e] = acc * inv_g;
  }
  double qsq = ora_dot_blocked(qkv, qkv, d);
  double qn = sqrt(qsq);
  for (int t = 0; t < mL; ++t) {
    const float *u = U + (int64_t)t * (d + 1);
    double z = ora_dot_blocked(qkv, u, d);
    double qb = qn > 0.0 ? z / qn : 0.0;
    qcode[t] = ora_to_code(qb);
  }
}

/* ------------------------------------------------------------------ */
/* Prioritized DCI on one composite (blog page: P-DCI is the per-head   */
/* ANN search; IceCache paper page, Figure 2 step (2): a tree search    */
/* finds the top-k tokens for q).                                        */
/* The composite owns m sorted lists.  Entries are visited in ascending */
/* (|code - qcode|, token, list) order; each visit counts one hit for   */
/* its token; a token becomes a candidate when all m of its entries     */
/* have been visited.  The walk stops at k0 candidates or after k1      */
/* visits (k1 <= 0: no visit limit) or when every entry is visited.     */
/* ------------------------------------------------------------------ */

/* One of the two frontiers of a list: upward from the query position,  */
/* or downward.  The downward frontier hands out a run of equal codes   */
/* in ascending token order, so every frontier yields entries in        */
/* ascending (distance, token) order.                                    */
typedef struct {
  const int32_t *code, *id;
  int64_t n, cur, run_lo, run_hi; /* down: current run [run_lo, run_hi], cursor cur */
  int up, j, live;
  uint32_t dist;
  int32_t tok;
} ora_front;

static void ora_front_load(ora_front *f, int32_t q) {
  if (f->up) {
    if (f->cur >= f->n) { f->live = 0; return; }
    f->dist = (uint32_t)((int64_t)f->code[f->cur] - q);
    f->tok = f->id[f->cur];
  } else {
    if (f->cur < 0) { f->live = 0; return; }
    f->dist = (uint32_t)((int64_t)q - f->code[f->cur]);
    f->tok = f->id[f->cur];
  }
  f->live = 1;
}

static void ora_front_start_down_run(ora_front *f, int64_t hi) {
  if (hi < 0) { f->cur = -1; return; }
  int64_t lo = hi;
  while (lo > 0 && f->code[lo - 1] == f->code[hi]) --lo;
  f->run_lo = lo;
  f->run_hi = hi;
  f->cur = lo;
}

static void ora_front_advance(ora_front *f, int32_t q) {
  if (f->up) {
    f->cur++;
  } else if (f->cur < f->run_hi) {
    f->cur++;
  } else {
    ora_front_start_down_run(f, f->run_lo - 1);
  }
  ora_front_load(f, q);
}

static int ora_front_less(const ora_front *a, const ora_front *b) {
  if (a->dist != b->dist) return a->dist < b->dist;
  if (a->tok != b->tok) return a->tok < b->tok;
  return a->j < b->j;
}

/* Literal walk.  lcode/lid: the composite's m lists, [m][n] each.      */
/* Writes the candidates in completion order to S (room for k0) and the */
/* number of visits to *visits; returns the candidate count.            */
int64_t ora_pdci_literal(const int32_t *lcode, const int32_t *lid, int64_t n, int m,
                         const int32_t *qcode, int64_t k0, int64_t k1, int32_t *S,
                         int64_t *visits) {
  *visits = 0;
  if (k0 <= 0 || n == 0) {
    if (n == 0) *visits = 0;
    return 0;
  }
  ora_front *f = (ora_front *)calloc((size_t)(2 * m), sizeof(ora_front));
  int *cnt = (int *)calloc((size_t)n, sizeof(int));
  for (int j = 0; j < m; ++j) {
    const int32_t *c = lcode + (int64_t)j * n;
    int64_t lo = 0, hi = n; /* first position with code >= q */
    while (lo < hi) {
      int64_t mid = lo + (hi - lo) / 2;
      if (c[mid] < qcode[j]) lo = mid + 1; else hi = mid;
    }
    ora_front *u = &f[2 * j], *dn = &f[2 * j + 1];
    u->code = dn->code = c;
    u->id = dn->id = lid + (int64_t)j * n;
    u->n = dn->n = n;
    u->j = dn->j = j;
    u->up = 1;
    dn->up = 0;
    u->cur = lo;
    ora_front_load(u, qcode[j]);
    ora_front_start_down_run(dn, lo - 1);
    ora_front_load(dn, qcode[j]);
  }
  int64_t ns = 0, v = 0;
  for (;;) {
    int best = -1; /* linear scan over the 2m frontiers: a priority queue in its plainest form */
    for (int x = 0; x < 2 * m; ++x)
      if (f[x].live && (best < 0 || ora_front_less(&f[x], &f[best]))) best = x;
    if (best < 0) break; /* every entry visited */
    int32_t tok = f[best].tok;
    ++v;
    if (++cnt[tok] == m) S[ns++] = tok;
    ora_front_advance(&f[best], qcode[f[best].j]);
    if (ns == k0) break;
    if (k1 > 0 && v == k1) break;
  }
  *visits = v;
  free(f);
  free(cnt);
  return ns;
}

/* Closed form of the same walk.  A token completes when its largest     */
/* entry key (M_i, i, j_i) is visited, where M_i = max_j |code - qcode|  */
/* and j_i the last list attaining it, so candidates are the tokens in   */
/* ascending (M_i, i) order, cut at k0 and at the visit budget k1.       */
/* codes: token-major [n][mL]; the composite is directions l*m .. l*m+m-1 */
typedef struct {
  uint32_t dist;
  int32_t tok, j;
} ora_key;

static int ora_key_cmp(const void *a, const void *b) {
  const ora_key *x = (const ora_key *)a, *y = (const ora_key *)b;
  if (x->dist != y->dist) return x->dist < y->dist ? -1 : 1;
  if (x->tok != y->tok) return x->tok < y->tok ? -1 : 1;
  return (x->j > y->j) - (x->j < y->j);
}

int64_t ora_pdci_closed(const int32_t *codes, int64_t n, int mL, int m, int l,
                        const int32_t *qcode, int64_t k0, int64_t k1, int32_t *S,
                        int64_t *visits) {
  *visits = 0;
  if (k0 <= 0 || n == 0) return 0;
  ora_key *mx = (ora_key *)malloc(sizeof(ora_key) * (size_t)n);
  for (int64_t i = 0; i < n; ++i) {
    mx[i].dist = 0;
    mx[i].tok = (int32_t)i;
    mx[i].j = 0;
    for (int j = 0; j < m; ++j) {
      int t = l * m + j;
      int64_t df = (int64_t)codes[i * mL + t] - qcode[t];
      uint32_t dd = (uint32_t)(df < 0 ? -df : df);
      if (j == 0 || dd >= mx[i].dist) { mx[i].dist = dd; mx[i].j = j; }
    }
  }
  qsort(mx, (size_t)n, sizeof(ora_key), ora_key_cmp); /* (M_i, i) order */

  /* every entry key, sorted, gives the visit rank of each token's largest entry */
  int64_t ne = n * m;
  ora_key *all = (ora_key *)malloc(sizeof(ora_key) * (size_t)ne);
  for (int64_t i = 0; i < n; ++i)
    for (int j = 0; j < m; ++j) {
      int t = l * m + j;
      int64_t df = (int64_t)codes[i * mL + t] - qcode[t];
      all[i * m + j].dist = (uint32_t)(df < 0 ? -df : df);
      all[i * m + j].tok = (int32_t)i;
      all[i * m + j].j = j;
    }
  qsort(all, (size_t)ne, sizeof(ora_key), ora_key_cmp);

  int64_t limit = (k1 > 0 && k1 < ne) ? k1 : ne;
  int64_t ns = 0, last_rank = 0;
  for (int64_t r = 0; r < n && ns < k0; ++r) {
    /* rank (1-based) of this token's largest entry */
    int64_t lo = 0, hi = ne;
    while (lo < hi) {
      int64_t mid = lo + (hi - lo) / 2;
      if (ora_key_cmp(&all[mid], &mx[r]) < 0) lo = mid + 1; else hi = mid;
    }
    int64_t rank = lo + 1;
    if (rank > limit) break;
    S[ns++] = mx[r].tok;
    last_rank = rank;
  }
  *visits = (ns == k0) ? last_rank : limit;
  free(mx);
  free(all);
  return ns;
}

/* ------------------------------------------------------------------ */
/* Exact rerank (IceCache paper page, Figure 2 step (2): the top-k      */
/* tokens most relevant to q).  READING: score_i = <qkv, k_i> in fp64,  */
/* in the blocked order above (each product of an fp32 and a key element */
/* is exact in fp64); rank by score descending, then token ascending.   */
/* ------------------------------------------------------------------ */
typedef struct {
  double score;
  int32_t tok;
} ora_scored;

static int ora_scored_cmp(const void *a, const void *b) {
  const ora_scored *x = (const ora_scored *)a, *y = (const ora_scored *)b;
  if (x->score != y->score) return x->score > y->score ? -1 : 1;
  return (x->tok > y->tok) - (x->tok < y->tok);
}

double ora_score(const float *K, int d, const float *qkv, int64_t tok) {
  return ora_dot_blocked(qkv, K + tok * d, d);
}

void ora_rerank(const float *K, int d, const float *qkv, const int32_t *C, int64_t nC,
                int32_t *ranked, double *scores) {
  ora_scored *a = (ora_scored *)malloc(sizeof(ora_scored) * (size_t)(nC > 0 ? nC : 1));
  for (int64_t x = 0; x < nC; ++x) {
    a[x].tok = C[x];
    a[x].score = ora_score(K, d, qkv, C[x]);
  }
  qsort(a, (size_t)nC, sizeof(ora_scored), ora_scored_cmp);
  for (int64_t x = 0; x < nC; ++x) {
    ranked[x] = a[x].tok;
    if (scores) scores[x] = a[x].score;
  }
  free(a);
}

/* GQA "max" reading (BASELINE's 36k configuration lets the query heads */
/* of a KV head be averaged or maxed; GQA itself is cited by title on    */
/* the citation-map page).  READING: each of the g heads walks every     */
/* composite with its own query; the pooled candidates are scored by the */
/* largest of the heads' exact scores, score_i = max_h <q_h, k_i> (each  */
/* in the blocked order above), and ranked by score descending, then     */
/* token ascending.  Q is [g][d].                                         */
void ora_rerank_max(const float *K, int d, const float *Q, int g, const int32_t *C, int64_t nC,
                    int32_t *ranked, double *scores) {
  ora_scored *a = (ora_scored *)malloc(sizeof(ora_scored) * (size_t)(nC > 0 ? nC : 1));
  for (int64_t x = 0; x < nC; ++x) {
    double best = ora_score(K, d, Q, C[x]);
    for (int h = 1; h < g; ++h) {
      double sc = ora_score(K, d, Q + (int64_t)h * d, C[x]);
      if (sc > best) best = sc;
    }
    a[x].tok = C[x];
    a[x].score = best;
  }
  qsort(a, (size_t)nC, sizeof(ora_scored), ora_scored_cmp);
  for (int64_t x = 0; x < nC; ++x) {
    ranked[x] = a[x].tok;
    if (scores) scores[x] = a[x].score;
  }
  free(a);
}

/* ------------------------------------------------------------------ */
/* Page selection (IceCache paper page, Figure 2 step (3): the pages    */
/* that contain the relevant tokens are selected).  READING: walk the   */
/* ranked candidates and keep each token's page the first time it is    */
/* seen, until P = k / p pages.  Returns the number selected.            */
/* ------------------------------------------------------------------ */
int64_t ora_select_pages(const int32_t *ranked, int64_t nC, const int32_t *page_of, int64_t P,
                         int32_t *page_ids) {
  int64_t np = 0;
  for (int64_t x = 0; x < nC && np < P; ++x) {
    int32_t pg = page_of[ranked[x]];
    int seen = 0;
    for (int64_t y = 0; y < np; ++y)
      if (page_ids[y] == pg) { seen = 1; break; }
    if (!seen) page_ids[np++] = pg;
  }
  return np;
}

/* ------------------------------------------------------------------ */
/* Sparse attention over every token of the selected pages (IceCache    */
/* paper page, Figure 2 step (3)).  For each of the g query heads:      */
/* softmax(q k^T / sqrt(d)) V over the pages in selection order, slots  */
/* in order, in fp64.  pool{K,V}: [Pcap][p][d].  out: [g][d].            */
/* ------------------------------------------------------------------ */
void ora_attention(const float *q, int g, int d, const float *poolK, const float *poolV, int p,
                   const int32_t *page_ids, int64_t n_sel, const int32_t *page_len,
                   double *out) {
  int64_t ntok = 0;
  for (int64_t x = 0; x < n_sel; ++x) ntok += page_len[page_ids[x]];
  double *z = (double *)malloc(sizeof(double) * (size_t)(ntok > 0 ? ntok : 1));
  double scale = sqrt((double)d);
  for (int h = 0; h < g; ++h) {
    const float *qh = q + (int64_t)h * d;
    for (int e = 0; e < d; ++e) out[h * d + e] = 0.0;
    if (ntok == 0) continue;
    int64_t t = 0;
    double zmax = -INFINITY;
    for (int64_t x = 0; x < n_sel; ++x) {
      int64_t pg = page_ids[x];
      for (int s = 0; s < page_len[pg]; ++s) {
        const float *k = poolK + (pg * p + s) * (int64_t)d;
        double acc = 0.0;
        for (int e = 0; e < d; ++e) acc = acc + (double)qh[e] * (double)k[e];
        z[t] = acc / scale;
        if (z[t] > zmax) zmax = z[t];
        ++t;
      }
    }
    double den = 0.0;
    t = 0;
    for (int64_t x = 0; x < n_sel; ++x) {
      int64_t pg = page_ids[x];
      for (int s = 0; s < page_len[pg]; ++s) {
        double w = exp(z[t] - zmax);
        den = den + w;
        const float *v = poolV + (pg * p + s) * (int64_t)d;
        for (int e = 0; e < d; ++e) out[h * d + e] = out[h * d + e] + w * (double)v[e];
        ++t;
      }
    }
    for (int e = 0; e < d; ++e) out[h * d + e] = out[h * d + e] / den;
  }
  free(z);
}
