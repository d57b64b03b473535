// Bounded visit budget k1 of the prioritized DCI walk (the DCI papers cited
// on the IceCache paper page; IceCache paper page, Figure 2 step (2)).
//
// A composite's walk visits its m*n list entries in ascending
// (|code - qcode|, token, list) order and stops after k1 visits.  Token i
// completes when its largest entry (M_i, i, j_i) is visited (j_i the last list
// attaining M_i), and those entries come in ascending (M_i, i) order, so the
// walk returns the first min(k0, n_l) tokens of that order, where n_l counts
// the tokens whose largest entry is among the first k1 entries.  With E* =
// (d*, t*, j*) the k1-th entry, those are the tokens with M_i < d*, the tokens
// with M_i = d* and i < t*, and t* itself when E* is its largest entry.
//
// The GPU finds E* by an exact radix selection over the entry distances
// (three passes over the codes: the top 11 bits, the next 11, the low 9), then
// the token t* among the entries at distance d* (per-range counts, then one
// wave walks the range that holds it), then counts n_l over the stored M
// values.  The query's selection then uses k0_l = min(k0, n_l) per composite.
#include "ice_device.h"

namespace ice {

constexpr int kVisitThreads = 1024;  // one token of a 1,024-token range per thread: 16 waves keep the code loads in flight
constexpr uint32_t kLowMask = (1u << (kHistShift - kHistBits)) - 1u;  // the last 9 bits

// GQA max mode: each kernel serves the walks of one head's pass, walk
// head * L + l of the stream (composite l, the head's query codes); the mean
// mode has the one pass, head 0.
__device__ __forceinline__ int64_t walk_of(const Dev &dv, int s, int head, int l) {
  return (int64_t)s * dv.Lq + head * dv.L + l;
}
__device__ __forceinline__ const int32_t *qcode_of(const Dev &dv, int s, int head) {
  return dv.qcode + ((int64_t)s * dv.Gq + (dv.gmax ? head : 0)) * dv.mL;
}

// The three selection passes; the state of walk w = walk_of(s, head, l) is
// vstate[4 * w + {0: selected prefix, 1: remaining rank (1-based),
// 2: t*, 3: whether t* completes}].
template <int LEVEL>
__device__ __forceinline__ void visit_bin(uint32_t dd, uint32_t pre, uint32_t *h) {
  if (LEVEL == 0) {
    atomicAdd(&h[dd >> kHistShift], 1u);
  } else if (LEVEL == 1) {
    if ((dd >> kHistShift) == pre) atomicAdd(&h[(dd >> (kHistShift - kHistBits)) & (kHistBins - 1)], 1u);
  } else {
    if ((dd >> (kHistShift - kHistBits)) == pre) atomicAdd(&h[dd & kLowMask], 1u);
  }
}

// Grid S * ceil(n / kScanRange) blocks (block b: stream b % S, token range
// b / S); per composite, an LDS histogram of the range's entries, added to the
// stream's global one.
template <int LEVEL>
__global__ __launch_bounds__(kVisitThreads) void k_visit_hist(Dev dv, int64_t n, int head) {
  const int S = dv.S, s = blockIdx.x % S, tid = threadIdx.x;
  const int m = dv.m, L = dv.L, mL = dv.mL;
  const int64_t r = blockIdx.x / S;
  const int64_t i0 = r * kVisitRange, i1 = min(i0 + kVisitRange, n);
  __shared__ uint32_t h[kHistBins];
  __shared__ int32_t qc[kMaxMl];
  if (tid < mL) qc[tid] = qcode_of(dv, s, head)[tid];
  for (int l = 0; l < L; ++l) {
    const uint32_t pre = LEVEL > 0 ? dv.vstate[4 * walk_of(dv, s, head, l)] : 0u;
    for (int x = tid; x < kHistBins; x += kVisitThreads) h[x] = 0;
    __syncthreads();
    for (int64_t i = i0 + tid; i < i1; i += kVisitThreads)
      for (int j = 0; j < m; ++j) {
        const int t = l * m + j;
        visit_bin<LEVEL>(absdiff(dv.codes[code_index(dv.ntile, mL, s, i, t)], qc[t]), pre, h);
      }
    __syncthreads();
    uint32_t *g = dv.vhist + walk_of(dv, s, head, l) * kHistBins;
    for (int x = tid; x < kHistBins; x += kVisitThreads) {
      const uint32_t c = h[x];
      if (c) atomicAdd(&g[x], c);
    }
    __syncthreads();
  }
}

// One wave per composite (block s * L + l): the bin holding the remaining
// rank, the new prefix and rank; the histogram is left cleared.
template <int LEVEL>
__global__ __launch_bounds__(64) void k_visit_pick(Dev dv, uint32_t k1, int head) {
  const int lane = threadIdx.x;
  const int64_t wk = walk_of(dv, blockIdx.x / dv.L, head, blockIdx.x % dv.L);
  uint32_t *g = dv.vhist + wk * kHistBins;
  uint32_t *st = dv.vstate + 4 * wk;
  const uint32_t target = LEVEL == 0 ? k1 : st[1];
  const uint32_t pre = LEVEL == 0 ? 0u : st[0];
  uint32_t v[kBinsPerLane];
  wave_hist_load(g, v);
  uint32_t bin, below;
  wave_find_bin_regs(v, target, bin, below);
  uint4 *g4 = reinterpret_cast<uint4 *>(g) + lane;  // the bins this lane read
#pragma unroll
  for (int c = 0; c < kHistChunks; ++c) g4[64 * c] = make_uint4(0u, 0u, 0u, 0u);
  if (lane == 0) {
    st[0] = LEVEL == 0 ? bin
                       : (LEVEL == 1 ? ((pre << kHistBits) | bin)
                                     : ((pre << (kHistShift - kHistBits)) | bin));
    st[1] = target - below;
  }
}

__device__ __forceinline__ uint32_t block_sum(uint32_t c, uint32_t *red) {
  const int tid = threadIdx.x;
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
  if ((tid & 63) == 0) red[tid >> 6] = c;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int k = 0; k < kVisitThreads / 64; ++k) t += red[k];
  __syncthreads();
  return t;
}

// Per range and composite: the entries at distance exactly d*.
__global__ __launch_bounds__(kVisitThreads) void k_visit_ties(Dev dv, int64_t n, int head) {
  const int S = dv.S, s = blockIdx.x % S, tid = threadIdx.x;
  const int m = dv.m, L = dv.L, mL = dv.mL;
  const int64_t r = blockIdx.x / S;
  const int64_t i0 = r * kVisitRange, i1 = min(i0 + kVisitRange, n);
  __shared__ int32_t qc[kMaxMl];
  __shared__ uint32_t red[kVisitThreads / 64];
  if (tid < mL) qc[tid] = qcode_of(dv, s, head)[tid];
  __syncthreads();
  for (int l = 0; l < L; ++l) {
    const uint32_t ds = dv.vstate[4 * walk_of(dv, s, head, l)];
    uint32_t c = 0;
    for (int64_t i = i0 + tid; i < i1; i += kVisitThreads)
      for (int j = 0; j < m; ++j) {
        const int t = l * m + j;
        c += absdiff(dv.codes[code_index(dv.ntile, mL, s, i, t)], qc[t]) == ds;
      }
    c = block_sum(c, red);
    if (tid == 0) dv.vtie[walk_of(dv, s, head, l) * dv.nvrange + r] = c;
  }
}

// One wave per composite: the range, then the token t* holding the
// remaining-rank-th entry at distance d* (entries in (token, list) order),
// the list j* of that entry, and whether it is t*'s largest entry (M_t* = d*
// and no later list of t* at d*).  Also seeds the completed-token count.
__global__ __launch_bounds__(64) void k_visit_resolve(Dev dv, int64_t n, int head) {
  const int sl = blockIdx.x, lane = threadIdx.x;
  const int L = dv.L, s = sl / L, l = sl % L, m = dv.m, mL = dv.mL;
  const int64_t wk = walk_of(dv, s, head, l);
  uint32_t *st = dv.vstate + 4 * wk;
  const uint32_t ds = st[0];
  uint32_t rr = st[1];
  const int64_t nr = (n + kVisitRange - 1) / kVisitRange;
  const uint32_t *tc = dv.vtie + wk * dv.nvrange;
  int64_t rg = -1;
  for (int64_t b0 = 0; b0 < nr; b0 += 64) {  // uniform loop: rr and the ballot are wave-wide
    const uint32_t c = b0 + lane < nr ? tc[b0 + lane] : 0u;
    const uint32_t incl = wave_incl_scan(c);
    const unsigned long long bal = __ballot(incl >= rr);
    if (bal) {
      const int src = __ffsll((long long)bal) - 1;
      rr -= __shfl(incl - c, src);
      rg = b0 + src;
      break;
    }
    rr -= __shfl(incl, 63);
  }
  const int32_t *qs = qcode_of(dv, s, head) + l * m;
  auto dist = [&](int64_t i, int j) {
    return absdiff(dv.codes[code_index(dv.ntile, mL, s, i, l * m + j)], qs[j]);
  };
  int64_t ts = -1;
  if (rg >= 0) {
    const int64_t i0 = rg * kVisitRange, i1 = min(i0 + kVisitRange, n);
    for (int64_t b0 = i0; b0 < i1; b0 += 64) {
      const int64_t i = b0 + lane;
      uint32_t c = 0;
      if (i < i1)
        for (int j = 0; j < m; ++j) c += dist(i, j) == ds;
      const uint32_t incl = wave_incl_scan(c);
      const unsigned long long bal = __ballot(incl >= rr);
      if (bal) {
        const int src = __ffsll((long long)bal) - 1;
        rr -= __shfl(incl - c, src);
        ts = b0 + src;
        break;
      }
      rr -= __shfl(incl, 63);
    }
  }
  if (lane == 0) {
    uint32_t done = 0;
    if (ts >= 0) {
      uint32_t seen = 0, mx = 0;
      int js = -1;
      bool later = false;
      for (int j = 0; j < m; ++j) {
        const uint32_t dj = dist(ts, j);
        mx = max(mx, dj);
        if (dj == ds) {
          ++seen;
          if (seen == rr) js = j;
          if (js >= 0 && j > js) later = true;
        }
      }
      done = (js >= 0 && mx == ds && !later) ? 1u : 0u;
    }
    st[2] = ts >= 0 ? (uint32_t)ts : (uint32_t)n;
    st[3] = done;
    dv.vcount[wk] = done;
  }
}

// Per range and composite: tokens with M < d*, or M = d* and token < t*.
__global__ __launch_bounds__(kVisitThreads) void k_visit_count(Dev dv, int64_t n, int head) {
  const int S = dv.S, s = blockIdx.x % S, tid = threadIdx.x, L = dv.L;
  const int64_t r = blockIdx.x / S;
  const int64_t i0 = r * kVisitRange, i1 = min(i0 + kVisitRange, n);
  __shared__ uint32_t red[kVisitThreads / 64];
  for (int l = 0; l < L; ++l) {
    const uint32_t *st = dv.vstate + 4 * walk_of(dv, s, head, l);
    const uint32_t ds = st[0], ts = st[2];
    const uint32_t *mrow = dv.mbuf + walk_of(dv, s, head, l) * dv.ncap;
    uint32_t c = 0;
    for (int64_t i = i0 + tid; i < i1; i += kVisitThreads) {
      const uint32_t M = mrow[i];
      c += (M < ds) || (M == ds && (uint32_t)i < ts);
    }
    c = block_sum(c, red);
    if (tid == 0 && c) atomicAdd(&dv.vcount[walk_of(dv, s, head, l)], c);
  }
}

hipError_t launch_visit_budget(const Dev &dv, int64_t n, uint32_t k1, int head, hipStream_t st) {
  const int64_t nr = (n + kVisitRange - 1) / kVisitRange;
  const dim3 grid((unsigned)(nr * dv.S)), sl((unsigned)(dv.S * dv.L));
  hipLaunchKernelGGL(k_visit_hist<0>, grid, dim3(kVisitThreads), 0, st, dv, n, head);
  hipLaunchKernelGGL(k_visit_pick<0>, sl, dim3(64), 0, st, dv, k1, head);
  hipLaunchKernelGGL(k_visit_hist<1>, grid, dim3(kVisitThreads), 0, st, dv, n, head);
  hipLaunchKernelGGL(k_visit_pick<1>, sl, dim3(64), 0, st, dv, k1, head);
  hipLaunchKernelGGL(k_visit_hist<2>, grid, dim3(kVisitThreads), 0, st, dv, n, head);
  hipLaunchKernelGGL(k_visit_pick<2>, sl, dim3(64), 0, st, dv, k1, head);
  hipLaunchKernelGGL(k_visit_ties, grid, dim3(kVisitThreads), 0, st, dv, n, head);
  hipLaunchKernelGGL(k_visit_resolve, sl, dim3(64), 0, st, dv, n, head);
  hipLaunchKernelGGL(k_visit_count, grid, dim3(kVisitThreads), 0, st, dv, n, head);
  return hipGetLastError();
}

}  // namespace ice
