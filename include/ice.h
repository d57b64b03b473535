/*
 * ice.h -- C ABI of the IceCache decode hot path on AMD Instinct MI355X.
 *
 * IceCache (IceCache paper page, abstract and Figures 2-3) keeps each
 * attention head's keys in a DCI-tree whose leaves are physical KV pages:
 *   (1) prefill indexes the keys by similarity in a transformed key space;
 *   (2) each decode step runs a tree search (prioritized DCI, one search per
 *       head -- IceCache blog page, technical details) for the query's top-k
 *       tokens;
 *   (3) the pages holding those tokens are selected and every token in them
 *       takes part in sparse attention with the query.
 * The tree is updated in place as tokens arrive (blog page: no rebuild).
 *
 * Terms.  A "stream" is one KV head of one layer of one sequence; an index
 * holds S streams of the same shape and each stream has its own tree, lists
 * and pages.  All tensors are row-major.  "dtype" is the element type of K, V,
 * the query and the directions: fp32 or bf16.
 *
 * Memory.  Every pointer named "device" is HIP device memory owned by the
 * caller.  The library never allocates device memory: the index lives in the
 * caller's workspace (size from ice_workspace_bytes, 256-byte aligned), and
 * the build uses a caller scratch buffer (ice_build_scratch_bytes) that may be
 * reused or freed once the build's stream work has finished.  The only host
 * allocation is the small ice_index handle.
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 * stream).  Every call enqueues kernels and returns without synchronising.
 * One index must be used from one stream at a time; calls on one index in
 * stream order see each other's results.
 *
 * Errors.  Arguments and capacities are checked on the host before anything
 * is enqueued; a call that fails a check returns a negative status and has no
 * effect.  ICE_ERR_HIP reports a launch error (asynchronous faults surface on
 * the caller's next synchronisation).  NaN/Inf inputs are outside the
 * contract.  Keys longer than the stored norm bound c are allowed (see
 * ice_insert).
 */
#ifndef ICE_H
#define ICE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ICE_OK = 0,
  ICE_ERR_INVALID_ARG = -1, /* a bad size, pointer or parameter */
  ICE_ERR_CAPACITY = -2,    /* an insert past capacity_tokens */
  ICE_ERR_UNSUPPORTED = -3, /* a valid setting this build does not implement */
  ICE_ERR_WORKSPACE = -4,   /* workspace or scratch too small or misaligned */
  ICE_ERR_HIP = -5,         /* a HIP launch error */
  ICE_ERR_SCRATCH_LIMIT = -6 /* ice_build_index_noalloc: the build needs more
                                scratch than the library's fixed array */
} ice_status;

typedef enum { ICE_F32 = 0, ICE_BF16 = 1 } ice_dtype;

/* Index parameters.  The pages state the problem in these terms: a token
 * budget k, a page size p, and the DCI parameters m and L (IceCache paper
 * page, abstract: budgets in tokens; the DCI and prioritized-DCI papers are
 * cited in the paper's citation map). */
typedef struct {
  int32_t head_dim;   /* d: 64 or 128                                          */
  int32_t page_size;  /* p: 8, 16, 32 or 64 tokens per page                    */
  int32_t budget_k;   /* k: tokens; a multiple of p; P = k / p pages per query;
                         above 65536: UNSUPPORTED                              */
  int32_t m;          /* simple indices (lists) per composite index, >= 1      */
  int32_t L;          /* composite indices, >= 1; m * L <= 128                 */
  int32_t gqa_group;  /* g: query heads per KV head, 1..16                      */
  int32_t k0;         /* candidates retrieved per composite; 0 -> budget_k;
                         L * k0 <= 12288 (larger: UNSUPPORTED)                 */
  int64_t k1;         /* visit budget per composite: the walk stops after k1
                         list entries (see ice_query_pages); 0 -> unbounded    */
  int32_t tree_depth; /* D, 1..13 and <= m*L; 0 -> derived from the build size:
                         D = round(log2(n_tokens / (4p))) clamped to [1, min(mL,13)] */
  float c;            /* key-norm bound of the transform; 0 -> the largest key
                         norm of each stream at build, rounded to fp32          */
  int32_t dtype;      /* ice_dtype of K, V, q and the directions                */
  int32_t gqa_mode;   /* ice_gqa_mode: how the g query heads of a KV head query
                         the index (0 = their mean; 1 = per-head walks, max score) */
  int32_t offload;    /* 0: the page pool lives in the workspace (HBM); 1: in
                         caller-owned pinned host memory (ice_build_index_offload);
                         2: its values there, its keys in the workspace      */
} ice_params;

/* GQA query modes (the query heads sharing a KV head "averaged or maxed"):
 *   ICE_GQA_MEAN  one walk per composite with the fp32 mean of the g heads;
 *                 candidates reranked by <q_kv, k>.
 *   ICE_GQA_MAX   every head walks every composite with its own query (g * L
 *                 walks, g * L <= 32 and g * L * k0 <= 4096, else
 *                 ICE_ERR_UNSUPPORTED); the pooled candidates are reranked by
 *                 max over the heads of <q_h, k>.
 * Both select P = k / p pages and attend every head over them. */
typedef enum { ICE_GQA_MEAN = 0, ICE_GQA_MAX = 1 } ice_gqa_mode;

typedef struct ice_index ice_index; /* opaque host handle */

/* Bytes of workspace for an index of n_streams streams built from n_tokens
 * tokens each with room for capacity_tokens >= n_tokens.  0 on bad input. */
size_t ice_workspace_bytes(const ice_params *prm, int32_t n_streams, int64_t n_tokens,
                           int64_t capacity_tokens);

/* Bytes of build scratch for ice_build_index.  0 on bad input. */
size_t ice_build_scratch_bytes(const ice_params *prm, int32_t n_streams, int64_t n_tokens);

/* Prefill indexing (IceCache paper page, Figure 2 step (1)).
 *   K, V   device [S][n_tokens][d] dtype: the keys and values of each stream.
 *   dirs   device [m*L][d+1] dtype: the DCI directions (unit vectors drawn by
 *          the caller; composite l owns directions l*m .. l*m+m-1).
 * For each stream: c (the key-norm bound), the transformed keys
 * [k/c, sqrt(max(0, 1 - |k|^2/c^2))] projected on every direction and stored as
 * fixed-point codes round(x * 2^29) saturated at +-(2^30-1); one list per
 * direction sorted by (code, token); the DCI-tree cell of each token (the sign
 * pattern of <k, u_t[:d]> on the first D directions); the cells' tokens, in
 * token order, cut into pages of p numbered by their first token; and a page
 * pool holding a copy of every key and value at its page slot.
 * K, V and dirs are read only by work enqueued here; once it has finished the
 * caller may free them.  The workspace must outlive the index.
 * n_tokens above 2^24 per stream: ICE_ERR_UNSUPPORTED (later inserts may grow
 * the index to capacity_tokens).
 * On success *out receives a new handle. */
ice_status ice_build_index(const ice_params *prm, int32_t n_streams, int64_t n_tokens,
                           int64_t capacity_tokens, const void *K, const void *V,
                           const void *dirs, void *workspace, size_t workspace_bytes,
                           void *scratch, size_t scratch_bytes, void *stream,
                           ice_index **out);

/* ice_build_index for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same build with the same results, except that the build scratch is a
 * fixed array inside the library (ICE_NOALLOC_SCRATCH_BYTES of device memory
 * on each GPU the library runs on, held until the process ends) instead of a
 * caller buffer; the caller still passes the inputs and the workspace.  It
 * calls no allocator.  ICE_ERR_SCRATCH_LIMIT (nothing enqueued) when
 * ice_build_scratch_bytes for these arguments exceeds
 * ICE_NOALLOC_SCRATCH_BYTES (an 8-head layer of 36,864 tokens with 32
 * directions needs about 122 MiB).  Every call on one GPU uses the same
 * array, which keeps the last build's contents (the build clears what it
 * needs itself): builds that may overlap in time on one GPU (several streams
 * or host threads) race, and the caller must serialise them. */
#define ICE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
ice_status ice_build_index_noalloc(const ice_params *prm, int32_t n_streams, int64_t n_tokens,
                                   int64_t capacity_tokens, const void *K, const void *V,
                                   const void *dirs, void *workspace, size_t workspace_bytes,
                                   void *stream, ice_index **out);

/* Host-offloaded page pool (IceCache paper page, abstract: most of the KV
 * cache is offloaded to the CPU; blog page: only the pages selected at a
 * decode step are brought to the GPU).  With prm->offload = 1 the K and V
 * pages live in host memory the caller allocated pinned and device-mapped
 * (hipHostMalloc; the library resolves it with hipHostGetDevicePointer and
 * never registers memory); the workspace holds the index and a staging area
 * of P pages per stream instead of the pool.  Per decode step the query's
 * exact rerank reads its candidates' key rows from host memory, k_fetch_pages
 * copies the P selected pages (K and V) into the staging area, and the
 * attention runs on the staging area: results equal the resident pool's bit
 * for bit.  The build and the inserts write the pool rows to host memory.
 * With prm->offload = 2 only the value pages live in host memory and the key
 * pages stay in the workspace: the rerank reads its key rows from HBM, the
 * host link carries the selected pages' values alone (the staging copy of
 * their keys is an HBM copy), and the host pool is half the size.
 *   host_pool  pinned host memory, ice_host_pool_bytes of it, 256-byte
 *              aligned; it must outlive the index.
 * ice_build_index refuses prm->offload = 1 or 2, and this call
 * prm->offload = 0 (ICE_ERR_INVALID_ARG); ICE_ERR_INVALID_ARG also when
 * host_pool is not device-mapped pinned memory, ICE_ERR_WORKSPACE when it is
 * too small.  The page pool's layout is the resident one (ice_index_layout's
 * pool_k and pool_v become byte offsets into host_pool; with offload 2
 * pool_k stays a workspace offset). */
size_t ice_host_pool_bytes(const ice_params *prm, int32_t n_streams, int64_t n_tokens,
                           int64_t capacity_tokens);
ice_status ice_build_index_offload(const ice_params *prm, int32_t n_streams, int64_t n_tokens,
                                   int64_t capacity_tokens, const void *K, const void *V,
                                   const void *dirs, void *workspace, size_t workspace_bytes,
                                   void *scratch, size_t scratch_bytes, void *host_pool,
                                   size_t host_pool_bytes, void *stream, ice_index **out);

/* Dynamic update (IceCache blog page: the tree takes new tokens with no
 * rebuild).  Appends one token to every stream.
 *   k_new, v_new  device [S][d] dtype.
 * The token gets index n (the stream's current length), is projected with the
 * stored c (the extra coordinate clamps at 0 for keys longer than c), enters
 * every list after all equal codes, and joins the last page of its cell when
 * that page has room, else opens page number n_pages.  The result equals a
 * rebuild over n+1 tokens with the same c, D and directions.
 * ICE_ERR_CAPACITY when the index already holds capacity_tokens tokens. */
ice_status ice_insert(ice_index *idx, const void *k_new, const void *v_new, void *stream);

/* Per-stream statistics of one query (the work the prioritized-DCI walk and
 * the attention do), written when a query or decode step is given a non-NULL
 * `stats` (device memory, one entry per stream; 8-byte aligned).
 *   visits[l]  V_l, the list entries composite l's walk visits (l < L): the
 *              visit rank of the entry that completes its k0-th candidate,
 *              or every entry it may visit (m * n, or k1 when the visit budget
 *              is smaller) when it completes fewer than k0 tokens
 *   n_cand     |C|, the tokens in the union of the composites' candidates
 *   n_pages    pages selected
 *   n_tokens   tokens attended: the valid slots of the selected pages
 * Entries l >= L are left untouched.  Collecting visits takes one extra pass
 * over the projection codes; with stats == NULL nothing extra runs. */
#define ICE_STATS_MAX_L 32
typedef struct {
  int64_t visits[ICE_STATS_MAX_L];
  int32_t n_cand, n_pages, n_tokens, reserved;
} ice_query_stats;

/* Delta-merge of the per-direction lists (the DCI index; IceCache blog page:
 * the tree takes new tokens with no rebuild).  Inserts append each list's new
 * entries after its sorted part in insertion order (see ice_index_layout);
 * this call folds them in, so that every list [0, n) is sorted by (code,
 * token) again and n_build becomes n.  Queries do not need it (they read the
 * projection codes); it keeps the lists a sorted DCI index.
 *   scratch  device, ice_merge_scratch_bytes(idx) bytes, 256-byte aligned;
 *            free to reuse once the call's stream work has finished.
 * Nothing to merge: ICE_OK with nothing enqueued.  More than 8192 entries
 * inserted since the build or the last merge: ICE_ERR_UNSUPPORTED. */
size_t ice_merge_scratch_bytes(const ice_index *idx);
ice_status ice_merge_lists(ice_index *idx, void *scratch, size_t scratch_bytes, void *stream);

/* Query: P-DCI candidates, exact rerank, page selection (IceCache paper page,
 * Figure 2 steps (2)-(3)).
 *   q         device [S*g][d] dtype: query heads, head j uses stream j / g;
 *             16-byte aligned.
 *   page_ids  device [S][P] int32 out: selected pages in selection order,
 *             -1 after the last.
 *   n_pages   device [S] int32 out.
 *   topk_ids  device [S][k] int32 out or NULL: the reranked top-k tokens,
 *             -1 after the last.
 *   stats     device [S] out or NULL: see ice_query_stats.
 * Per stream: the g query heads are averaged in fp32 (q_kv) and normalised;
 * composite l's candidates are the k0 tokens with the smallest
 * max_j |code_j - qcode_j| over its m directions (ties by token), which is
 * the set a prioritized-DCI walk over the sorted lists retrieves.  With a
 * visit budget k1 < m * n the walk visits only the first k1 of the
 * composite's m * n list entries in ascending (|code - qcode|, token, list)
 * order, and the candidates are the first min(k0, n_l) tokens of that order,
 * n_l being the tokens whose every entry is among those k1.  The union
 * of all composites is scored exactly, <q_kv, k> in fp64, and ranked by
 * (score desc, token asc); pages are taken in rank order, each the first time
 * one of its tokens appears, up to P = k/p pages.  Outputs are bit-exact and
 * deterministic. */
ice_status ice_query_pages(ice_index *idx, const void *q, int32_t *page_ids, int32_t *n_pages,
                           int32_t *topk_ids, ice_query_stats *stats, void *stream);

/* Sparse attention over every token of the selected pages (IceCache paper
 * page, Figure 2 step (3)).
 *   q         device [S*g][d] dtype, 16-byte aligned.
 *   page_ids  device [S][P] int32, n_pages device [S] int32 (as written by
 *             ice_query_pages; any valid page numbers may be passed).
 *   out       device [S*g][d] fp32: softmax(q k^T / sqrt(d)) V per head,
 *             accumulated in fp32; zero when a stream selects no page. */
ice_status ice_sparse_attn(const ice_index *idx, const void *q, const int32_t *page_ids,
                           const int32_t *n_pages, float *out, void *stream);

/* One decode step: ice_insert(k_new, v_new), then ice_query_pages(q, ...)
 * over the n+1 tokens, then ice_sparse_attn(q, page_ids, n_pages, out), with
 * results identical to those three calls (IceCache paper page, Figure 2 steps
 * (2)-(3); blog page: new tokens join the tree with no rebuild).  The insert
 * and the query's projection share one kernel, so the step takes fewer
 * launches.  Arguments as for those calls; q must be 16-byte aligned.
 * ICE_ERR_CAPACITY (nothing enqueued) when the index is full. */
ice_status ice_decode_step(ice_index *idx, const void *k_new, const void *v_new, const void *q,
                           int32_t *page_ids, int32_t *n_pages, int32_t *topk_ids, float *out,
                           ice_query_stats *stats, void *stream);

/* A decode step that reuses an earlier page selection (the pages name an
 * "IceCache (reuse)" variant, paper page Table 5 and the blog's comparison,
 * without its mechanism; reading: the selection of a query step is reused by
 * the following decode steps, and the caller re-runs the query every r steps,
 * which saves the P-DCI query the blog puts at about half of a decode step).
 * The new token is inserted as by ice_insert, then every head attends over
 * the pages in page_ids / n_pages (as written by an earlier query, or any
 * valid page numbers), as by ice_sparse_attn: the new token takes part only
 * when its page is among them.  Same arguments, alignment and errors as
 * ice_decode_step; page_ids and n_pages are read, not written.  With a budget
 * of one attention block (k <= 256) and the pool in HBM this is one kernel:
 * the index ends as ice_insert leaves it, and the attention equals ice_insert
 * + ice_sparse_attn up to the fp32 rounding of the new token's logit (summed
 * in element order, then joined to the pages' softmax). */
ice_status ice_decode_step_reuse(ice_index *idx, const void *k_new, const void *v_new,
                                 const void *q, const int32_t *page_ids, const int32_t *n_pages,
                                 float *out, void *stream);

/* Frees the handle (not the workspace). NULL is allowed. */
void ice_destroy_index(ice_index *idx);

const char *ice_status_string(ice_status s);

/* Byte offsets of the index arrays inside the workspace, for inspection and
 * tests.  Element types and shapes (S streams, Ncap = capacity_tokens,
 * Pcap = page_capacity, mL = m*L):
 *   norm_c        float   [S]            the key-norm bound c
 *   codes         int32   [S][ceil(Ncap/64)][mL][64]  projection codes in tiles
 *                 of 64 tokens: code t of token i at [i/64][t][i%64]
 *   list_code/id  int32   [S][mL][Ncap]  per-direction lists: entries
 *                 [0, n_build) sorted by (code, token); entries inserted later
 *                 follow in insertion order (the logical list merges both)
 *   loc           int32   [S][Ncap]      page * p + slot of every token
 *   page_tokens   int32   [S][Pcap][p]   token of each page slot, -1 = empty
 *   page_len      int32   [S][Pcap]
 *   page_cell     int32   [S][Pcap]      -1 for unused pages
 *   npages        int32   [S]
 *   cell_count    int32   [S][n_cells]   tokens per cell
 *   pool_k        dtype   [S][Pcap][p][d]  key of each page slot
 *   pool_v        dtype   [S][Pcap][d][p]  values, element-major inside a
 *                 page (value element e of slot j at [e][j]); with offload
 *                 1 both are offsets into the host pool, not the workspace
 *                 (offload 2: pool_v only)
 *   qcode         int32   [S][G][mL]     last query's projection codes (G = g
 *                 in the GQA max mode, one set per head; else 1)
 *   cand          int32   [S][Lq][k0]    last query's candidates per walk (Lq =
 *                 L, or g * L in the GQA max mode: walk h * L + l is head h on
 *                 composite l), cand_count int32 [S][Lq] of them valid, in no
 *                 fixed order */
typedef struct {
  int64_t n_streams, n_tokens, n_build, capacity_tokens, page_capacity, n_cells;
  int32_t tree_depth, mL, k0, elem_bytes, Lq, Gq, offload;
  int64_t norm_c, codes, list_code, list_id, loc, page_tokens, page_len, page_cell, npages,
      cell_count, pool_k, pool_v, qcode, cand, cand_count;
  int64_t workspace_bytes;
} ice_layout;

ice_status ice_index_layout(const ice_index *idx, ice_layout *out);

/* Per-kernel timing for benchmarks.  When enabled, every decode-time call
 * (ice_insert, ice_query_pages, ice_sparse_attn, ice_decode_step) records HIP events on its
 * stream around each kernel it launches; ice_timing_read waits for the
 * recorded events, writes the summed milliseconds and launch counts per
 * kernel (arrays of ICE_TIMED_KERNELS, in the order of ice_timing_name) and
 * clears the record.  The event records add a little time between kernels;
 * leave timing off for end-to-end latency. */
#define ICE_TIMED_KERNELS 9 /* insert, qscan, qcollect, qfinal, attn, amerge, visit,
                              fetch (the offloaded pool's page copy), reuse (the
                              one-kernel ice_decode_step_reuse) */
ice_status ice_timing_enable(ice_index *idx, int enable);
ice_status ice_timing_read(ice_index *idx, double *total_ms, int64_t *launches);
const char *ice_timing_name(int kernel);

#ifdef __cplusplus
}
#endif
#endif /* ICE_H */
