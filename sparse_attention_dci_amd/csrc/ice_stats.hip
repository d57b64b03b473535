// Query statistics (optional output of ice_query_pages / ice_decode_step):
// how many list entries each composite's prioritized-DCI walk visits, and how
// many tokens the attention covers (IceCache paper page, Figure 2 steps
// (2)-(3); the blog page's TPOT table puts almost half of a decode step in the
// DCI query).
//
// A walk visits its composite's entries in ascending (|code - qcode|, token,
// list) order and stops when its k0-th candidate completes, i.e. when that
// token's largest entry E* = (M*, i*, j*) is visited (j* the last list
// attaining M*).  It has then visited exactly the entries whose key is at most
// E*: every entry closer than M*, the entries at M* of tokens below i*, and
// those of i* up to list j*.  The finaliser starts each visit count (0 for such
// a walk, else every entry the walk may visit) and leaves E*'s (M*, i*) key in
// vlast; this pass counts the entries up to E* over the tiled codes and adds
// them, and totals the valid slots of the selected pages.
#include "ice_device.h"

namespace ice {

constexpr int kStatsThreads = 1024;
constexpr int kStatsTpb = 1024;  // tokens per block (one per thread: 16 waves keep the loads in flight)

// Grid (ceil(n / kStatsTpb), S).
__global__ __launch_bounds__(kStatsThreads) void k_qstats(Dev dv, int64_t n,
                                                          ice_query_stats *stats,
                                                          const int32_t *page_ids,
                                                          const int32_t *n_pages) {
  const int s = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  // walk l = h * L + c: composite c's codes against head h's query codes (one
  // head, h = 0, in the mean mode)
  const int m = dv.m, Lc = dv.L, L = dv.Lq, mL = dv.mL;
  const int64_t i0 = (int64_t)blockIdx.x * kStatsTpb;
  __shared__ int32_t qc[kMaxGroup * kMaxMl];
  __shared__ uint32_t Ms[32];
  __shared__ int32_t is[32], js[32];
  __shared__ uint32_t cnt[32];
  for (int x = tid; x < dv.Gq * mL; x += kStatsThreads) qc[x] = dv.qcode[(int64_t)s * dv.Gq * mL + x];
  if (tid < L) {
    const unsigned long long key = dv.vlast[(int64_t)s * L + tid];
    Ms[tid] = (uint32_t)(key >> 32);
    is[tid] = key == ~0ull ? -1 : (int32_t)(key & 0xffffffffull);
    cnt[tid] = 0;
  }
  __syncthreads();
  if (tid < L && is[tid] >= 0) {  // j*: the last list at distance M* for token i*
    const int h = tid / Lc, c = tid % Lc;
    int jl = 0;
    for (int j = 0; j < m; ++j) {
      const int t = c * m + j;
      if (absdiff(dv.codes[code_index(dv.ntile, mL, s, is[tid], t)], qc[h * mL + t]) == Ms[tid])
        jl = j;
    }
    js[tid] = jl;
  }
  __syncthreads();
  for (int l = 0; l < L; ++l) {
    if (is[l] < 0) continue;  // uniform: this walk completed fewer than k0 tokens
    const uint32_t M = Ms[l];
    const int64_t ist = is[l];
    const int jst = js[l];
    const int h = l / Lc, cmp = l % Lc;
    constexpr int U = kStatsTpb / kStatsThreads;  // tokens per thread
    const int64_t ilast = n > 0 ? n - 1 : 0;  // a valid address for every lane
    uint32_t c = 0;
    // list by list, the thread's U codes requested together (clamped
    // addresses; tokens past n count nothing)
#pragma unroll 2
    for (int j = 0; j < m; ++j) {
      const int t = cmp * m + j;
      const int32_t qv = qc[h * mL + t];
      int32_t cd[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = min(i0 + tid + (int64_t)kStatsThreads * u, ilast);
        cd[u] = dv.codes[code_index(dv.ntile, mL, s, i, t)];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = i0 + tid + (int64_t)kStatsThreads * u;
        const uint32_t dd = absdiff(cd[u], qv);
        c += i < n && (dd < M || (dd == M && (i < ist || (i == ist && j <= jst))));
      }
    }
    const uint32_t tot = wave_incl_scan(c);
    if (lane == 63 && tot) atomicAdd(&cnt[l], tot);
  }
  __syncthreads();
  if (tid < L && is[tid] >= 0 && cnt[tid])
    atomicAdd(reinterpret_cast<unsigned long long *>(&stats[s].visits[tid]),
              (unsigned long long)cnt[tid]);
  if (blockIdx.x == 0 && tid == 0) {  // the valid slots of the selected pages
    const int np = min(n_pages[s], dv.P);
    int32_t tot = 0;
    for (int x = 0; x < np; ++x) {
      const int32_t pg = page_ids[(int64_t)s * dv.P + x];
      if (pg >= 0 && pg < dv.pcap) tot += dv.page_len[(int64_t)s * dv.pcap + pg];
    }
    stats[s].n_tokens = tot;
  }
}

hipError_t launch_stats(const Dev &dv, int64_t n, ice_query_stats *stats, const int32_t *page_ids,
                        const int32_t *n_pages, hipStream_t st) {
  const int64_t nb = n > 0 ? (n + kStatsTpb - 1) / kStatsTpb : 1;
  hipLaunchKernelGGL(k_qstats, dim3((unsigned)nb, dv.S), dim3(kStatsThreads), 0, st, dv, n, stats,
                     page_ids, n_pages);
  return hipGetLastError();
}

}  // namespace ice
