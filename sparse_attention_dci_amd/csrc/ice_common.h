// Internal declarations shared by the HIP kernels and the host side of the
// C ABI.  Not installed; include/ice.h is the public surface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ice.h"

namespace ice {

// Projection codes are fixed point with 29 fractional bits, saturated at
// +-(2^30 - 1), so every |code - qcode| fits in 31 bits.
constexpr double kCodeScale = 536870912.0;  // 2^29
constexpr int32_t kCodeMax = 1073741823;     // 2^30 - 1
constexpr int kMaxTreeDepth = 13;
constexpr int kMaxMl = 128;
constexpr int kMaxGroup = 16;
// First-level histogram of the candidate selection: bins of the top 11 bits of
// a 31-bit distance.
constexpr int kHistBits = 11;
constexpr int kHistBins = 1 << kHistBits;
constexpr int kHistShift = 31 - kHistBits;
// Largest candidate union per stream (L*k0) that the finaliser keeps in LDS;
// up to kMaxCandBig the union stays in global memory and is ranked in windows.
constexpr int kMaxCand = 4096;
constexpr int kMaxCandBig = 12288;
// Directions are stored in fp64, 16 per chunk, [chunk][d+1][16].
constexpr int kDirChunk = 16;
// Projection codes are stored in tiles of 64 tokens, [S][tile][mL][64]: a
// wave reads code t of its 64 tokens as one contiguous 256-byte load.
constexpr int kCodeTile = 64;
// Sparse attention: tokens of the selected pages per block (16 waves of 16).
constexpr int kAttnTpb = 256;
// Tokens per wave chunk of the sparse attention (16 or 32, a multiple of the
// logits product's 16-token tile).  16: twice the waves with loads in flight
// per block; 32-token chunks halve the values products but measured slower
// (36k decode step 45.9 -> 48.7 us).
constexpr int kAttnChunk = 16;
// Largest budget the standalone attention merges (blocks of kAttnTpb tokens).
constexpr int kMaxBudget = 65536;
// Token ranges of the visit-budget passes (one block per range and stream).
constexpr int kVisitRange = 1024;
// Largest list tail (entries inserted since the build or the last merge) that
// ice_merge_lists sorts in one block's LDS.
constexpr int kMaxMergeTail = 8192;

// Every device array of one index, resolved from the caller's workspace.
struct Dev {
  int S;
  int d, p, m, L, mL, g, D, k, P, k0, dtype, elem;  // elem = bytes per element
  // GQA max mode (gmax = 1): every head walks every composite, Lq = g * L
  // walks, Gq = g query-code sets; the mean mode has Lq = L, Gq = 1.  Every
  // query-side array indexed by composite uses Lq (walk h * L + l).
  int gmax, Lq, Gq;
  int64_t ncap, pcap, ncell, nbuild;
  int nchunk;          // direction chunks of kDirChunk
  int attn_nsplit;     // attention blocks per stream, ceil(k / kAttnTpb)
  int ncu;             // compute units of the device the index was built on
  int lp;              // log2 of the page size (a power of two)

  double *dirs;        // [nchunk][d+1][16]
  float *dirs32;       // [d+1][mLp] element-major, mLp = mL rounded up to 32, zero past mL
  int mLp;
  float *norm_c;       // [S]
  double *inv_c;       // [S]
  double *inv_c2;      // [S]
  unsigned long long *maxnsq;  // [S] bit pattern of the largest |k|^2
  int32_t *codes;      // [S][ntile][mL][64], ntile = ceil(ncap / 64)
  int64_t ntile;
  int32_t *list_code;  // [S][mL][ncap]
  int32_t *list_id;    // [S][mL][ncap]
  int32_t *loc;        // [S][ncap]
  int32_t *page_tokens;  // [S][pcap][p]
  int32_t *page_len;     // [S][pcap]
  int32_t *page_cell;    // [S][pcap]
  int32_t *npages;       // [S]
  int32_t *cell_count;   // [S][ncell]
  int32_t *cell_last;    // [S][ncell]
  void *pool_k;          // [S][pcap][p][d]  key rows, slot-major
  void *pool_v;          // [S][pcap][d][p]  value columns, element-major within a page
  // host-offloaded pool (offload = 1: pool_k / pool_v point into pinned host
  // memory): the selected pages are copied here before the attention
  int offload;
  void *stage_k;         // [S][P][p][d]
  void *stage_v;         // [S][P][d][p]
  int32_t *stage_len;    // [S][P] valid slots of each staged page (0: none)

  // per-query state (walks: Lq per stream)
  float *qkv;            // [S][Gq][d]
  int32_t *qcode;        // [S][Gq][mL]
  uint32_t *mbuf;        // [S][Lq][ncap] every walk of a query (all passes)
  uint32_t *hist;        // [S][Lq][kHistBins]
  uint32_t *hist2;       // [S][Lq][kHistBins] second level: the boundary bin's next 11 bits
  int32_t *cand;         // [S][Lq][k0]
  uint32_t *cand_count;  // [S][Lq]
  unsigned long long *bnd;  // [S][Lq][ncap] boundary-bin entries (M << 32 | token)
  unsigned long long *bnd_rk;  // [S][Lq][ncap] their rank keys
  int32_t *bnd_pg;          // [S][Lq][ncap] their pages
  uint32_t *bnd_count;      // [S][Lq]
  unsigned long long *rr_key;  // [S][Lq*k0] rank key of each scored candidate
  int32_t *rr_id;              // [S][Lq*k0]
  int32_t *rr_pg;              // [S][Lq*k0] its page
  uint32_t *rr_count;          // [S]
  float *attn_part;         // [S][nsplit][g][d+2] (values, max logit, softmax sum)

  // visit budget k1 (bounded walks only)
  int64_t nvrange;          // ceil(ncap / kVisitRange)
  uint32_t *vhist;          // [S][Lq][kHistBins] selection histogram, left cleared
  uint32_t *vstate;         // [S][Lq][4] prefix / d*, remaining rank, t*, t* completes
  uint32_t *vtie;           // [S][Lq][nvrange] entries at distance d* per token range
  uint32_t *vcount;         // [S][Lq] n_l, the tokens the bounded walk completes
  uint32_t *bsel;           // [S][Lq][2] the collect pass's threshold bin b* of each walk and
                            // the count of tokens below it (for the finaliser)
  unsigned long long *vlast;  // [S][Lq] query statistics: the (M, token) key of each walk's
                              // k0-th candidate, ~0 when it completed fewer
};

// Build scratch (caller-owned, only used while the build runs).
// Address of code t of token i of stream s.
__host__ __device__ inline int64_t code_index(int64_t ntile, int mL, int s, int64_t i, int t) {
  return (((int64_t)s * ntile + (i >> 6)) * mL + t) * kCodeTile + (i & 63);
}

struct BuildScratch {
  int32_t *codes_dm;  // [S][mL][n]
  int32_t *tmp_code;  // [S][mL][n]
  int32_t *tmp_id;    // [S][mL][n]
  uint32_t *cell;     // [S][n]
  // page assignment (chunks of kPageChunk tokens, cmax = 2^min(mL, 13) cells)
  int32_t *chunk_cnt;   // [S][nchunk][cmax] tokens of each cell per chunk, then their prefix
  int32_t *rank;        // [S][n] a token's rank among its cell's tokens
  int32_t *chunk_pg;    // [S][nchunk + 1] pages opened per chunk, then their prefix
  int32_t *cell_pg;     // [S][cmax + 1] prefix of the cells' page counts
  int32_t *page_of;     // [S][n / 8 + cmax + 1] page id by (cell_pg[c] + ordinal in the cell)
  double *nsq;          // [S][n] |k|^2 of every key row (fp64, ascending element order)
};

// Tokens per chunk of the build's page assignment.
constexpr int kPageChunk = 1024;

// Decode-time kernels that the optional event timer reports separately.
// KID_INSERT is the standalone insert; a decode step's insert and query prep
// run inside the scan and are timed with it.
enum KernelId { KID_INSERT = 0, KID_QSCAN, KID_QCOLLECT, KID_QFINAL, KID_ATTN, KID_AMERGE,
                KID_VISIT, KID_FETCH, KID_REUSE, KID_COUNT };

// Optional host-side event timer (owned by an index); null when timing is off.
struct Timer;
void timer_begin(Timer *tm, hipStream_t st);           // before a call's first launch
void timer_mark(Timer *tm, int kid, hipStream_t st);    // after each launch

// Host launchers (each returns the hipGetLastError of its launches).
hipError_t launch_build(const Dev &dv, const BuildScratch &bs, int64_t n, const void *K,
                        const void *V, const void *dirs, float c_fixed, hipStream_t st);
hipError_t launch_insert(const Dev &dv, int64_t n, const void *k_new, const void *v_new,
                         hipStream_t st, Timer *tm);
// k1: the visit budget per composite, 0 = unbounded
hipError_t launch_query(const Dev &dv, int64_t n, int64_t k1, const void *q, int32_t *page_ids,
                        int32_t *n_pages, int32_t *topk_ids, ice_query_stats *stats,
                        hipStream_t st, Timer *tm);
// the visit counts and attended tokens of the query just enqueued (stats non-null)
hipError_t launch_stats(const Dev &dv, int64_t n, ice_query_stats *stats, const int32_t *page_ids,
                        const int32_t *n_pages, hipStream_t st);
hipError_t launch_reuse(const Dev &dv, int64_t n, const void *k_new, const void *v_new,
                        const void *q, const int32_t *page_ids, const int32_t *n_pages,
                        float *out, hipStream_t st, Timer *tm);
hipError_t launch_attn(const Dev &dv, const void *q, const int32_t *page_ids,
                       const int32_t *n_pages, float *out, hipStream_t st, Timer *tm);
// the list merge: scratch bytes for n tokens, and the merge of entries nb .. n-1
int64_t merge_scratch_bytes(const Dev &dv, int64_t n);
hipError_t launch_merge(const Dev &dv, int64_t nb, int64_t n, void *scratch, hipStream_t st);
// n_l of every composite for a walk bounded at k1 visits (1 <= k1 < m * n)
hipError_t launch_visit_budget(const Dev &dv, int64_t n, uint32_t k1, int head, hipStream_t st);
// insert of token n, then the query over n + 1 tokens and the attention
hipError_t launch_decode(const Dev &dv, int64_t n, int64_t k1, const void *k_new,
                         const void *v_new, const void *q, int32_t *page_ids, int32_t *n_pages,
                         int32_t *topk_ids, float *out, ice_query_stats *stats, hipStream_t st,
                         Timer *tm);

}  // namespace ice
