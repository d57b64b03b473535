// Internal declarations shared by the HIP kernels and the host side of the
// C ABI.  Not installed; include/ice.h is the public surface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
// Largest reranked candidate set per stream that the finaliser sorts in LDS.
constexpr int kMaxCand = 4096;
// Directions are stored in fp64, 16 per chunk, [chunk][d+1][16].
constexpr int kDirChunk = 16;

// Every device array of one index, resolved from the caller's workspace.
struct Dev {
  int S;
  int d, p, m, L, mL, g, D, k, P, k0, dtype, elem;  // elem = bytes per element
  int64_t ncap, pcap, ncell, nbuild;
  int nchunk;          // direction chunks of kDirChunk
  int attn_tps;        // attention tokens per split
  int attn_nsplit;     // attention splits per stream

  double *dirs;        // [nchunk][d+1][16]
  float *norm_c;       // [S]
  double *inv_c;       // [S]
  double *inv_c2;      // [S]
  unsigned long long *maxnsq;  // [S] bit pattern of the largest |k|^2
  int32_t *codes;      // [S][ncap][mL]
  int32_t *list_code;  // [S][mL][ncap]
  int32_t *list_id;    // [S][mL][ncap]
  int32_t *loc;        // [S][ncap]
  int32_t *page_tokens;  // [S][pcap][p]
  int32_t *page_len;     // [S][pcap]
  int32_t *page_cell;    // [S][pcap]
  int32_t *npages;       // [S]
  int32_t *cell_count;   // [S][ncell]
  int32_t *cell_last;    // [S][ncell]
  void *pool_k;          // [S][pcap][p][d]
  void *pool_v;
  uint32_t *mark;        // [S][ncap] query epoch that claimed the token

  // per-query state
  float *qkv;            // [S][d]
  int32_t *qcode;        // [S][mL]
  uint32_t *mbuf;        // [S][L][ncap]
  uint32_t *hist;        // [S][L][kHistBins]
  int32_t *cand;         // [S][L][k0]
  uint32_t *cand_count;  // [S][L]
  unsigned long long *bnd;  // [S][L][ncap]
  uint32_t *bnd_count;      // [S][L]
  unsigned long long *cs_key;  // [S][L*k0]
  int32_t *cs_id;              // [S][L*k0]
  uint32_t *c_count;           // [S]
  float *attn_part;            // [S][nsplit][g][d+2]
};

// Build scratch (caller-owned, only used while the build runs).
struct BuildScratch {
  int32_t *codes_dm;  // [S][mL][n]
  int32_t *tmp_code;  // [S][mL][n]
  int32_t *tmp_id;    // [S][mL][n]
  uint32_t *cell;     // [S][n]
};

// Decode-time kernels that the optional event timer reports separately.
enum KernelId { KID_INSERT = 0, KID_QSCAN, KID_QCOLLECT, KID_QFINAL, KID_ATTN_PART,
                KID_ATTN_COMBINE, KID_COUNT };

// Optional host-side event timer (owned by an index); null when timing is off.
struct Timer;
void timer_begin(Timer *tm, hipStream_t st);           // before a call's first launch
void timer_mark(Timer *tm, int kid, hipStream_t st);    // after each launch

// Host launchers (each returns the hipGetLastError of its launches).
hipError_t launch_build(const Dev &dv, const BuildScratch &bs, int64_t n, const void *K,
                        const void *V, const void *dirs, float c_fixed, hipStream_t st);
hipError_t launch_build_reset_marks(const Dev &dv, hipStream_t st);
hipError_t launch_insert(const Dev &dv, int64_t n, const void *k_new, const void *v_new,
                         hipStream_t st, Timer *tm);
hipError_t launch_query(const Dev &dv, int64_t n, const void *q, uint32_t epoch,
                        int32_t *page_ids, int32_t *n_pages, int32_t *topk_ids,
                        hipStream_t st, Timer *tm);
hipError_t launch_attn(const Dev &dv, const void *q, const int32_t *page_ids,
                       const int32_t *n_pages, float *out, hipStream_t st, Timer *tm);

}  // namespace ice
