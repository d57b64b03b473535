// Delta-merge of the per-direction lists (the DCI index the prioritized walk
// visits; IceCache blog page: the tree takes new tokens with no rebuild).
//
// The build leaves each list sorted by (code, token); inserts append their
// entries after it in insertion order (tokens n_build, n_build + 1, ...).
// ice_merge_lists folds those tails in, so that every list [0, n) is sorted
// again and n_build becomes n:
//   k_merge_tail  one block per list sorts its tail in LDS (bitonic over the
//                 64-bit key (order-preserving code image, token)) into scratch;
//   k_merge_place every entry's place in the merged list is its rank in its
//                 own sorted run plus the number of entries of the other run
//                 below it (a binary search; keys are distinct because tokens
//                 are), written to scratch;
//   k_merge_copy  the merged lists back into the index.
#include "ice_device.h"

namespace ice {

constexpr int kMergeThreads = 1024;

__device__ __forceinline__ unsigned long long list_key(int32_t code, int32_t tok) {
  return ((unsigned long long)((uint32_t)code ^ 0x80000000u) << 32) | (uint32_t)tok;
}

// Grid S * mL blocks: list b's tail entries nb .. n-1 (at most kMaxMergeTail),
// sorted ascending, to tail[b][0 .. n-nb).
__global__ __launch_bounds__(kMergeThreads) void k_merge_tail(Dev dv, int64_t nb, int64_t n,
                                                              unsigned long long *tail) {
  const int64_t b = blockIdx.x;
  const int t = (int)(n - nb);
  __shared__ unsigned long long key[kMaxMergeTail];
  int np2 = 1;
  while (np2 < t) np2 <<= 1;
  const int32_t *lc = dv.list_code + b * dv.ncap + nb, *li = dv.list_id + b * dv.ncap + nb;
  for (int x = threadIdx.x; x < np2; x += kMergeThreads) key[x] = x < t ? list_key(lc[x], li[x]) : ~0ull;
  __syncthreads();
  for (int k = 2; k <= np2; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int x = threadIdx.x; x < np2; x += kMergeThreads) {
        const int y = x ^ j;
        if (y > x) {
          const unsigned long long a = key[x], c = key[y];
          const bool up = (x & k) == 0;
          if ((a > c) == up) {
            key[x] = c;
            key[y] = a;
          }
        }
      }
      __syncthreads();
    }
  for (int x = threadIdx.x; x < t; x += kMergeThreads) tail[b * kMaxMergeTail + x] = key[x];
}

// Grid (S * mL, ceil(n / kMergeThreads)): entry x of list b (base run for
// x < nb, else tail entry x - nb) to its merged place in out[b][0 .. n).
__global__ __launch_bounds__(kMergeThreads) void k_merge_place(Dev dv, int64_t nb, int64_t n,
                                                               const unsigned long long *tail,
                                                               int2 *out) {
  const int64_t b = blockIdx.x;
  const int64_t x = (int64_t)blockIdx.y * kMergeThreads + threadIdx.x;
  if (x >= n) return;
  const int64_t t = n - nb;
  const int32_t *lc = dv.list_code + b * dv.ncap, *li = dv.list_id + b * dv.ncap;
  const unsigned long long *tk = tail + b * kMaxMergeTail;
  int32_t code, tok;
  int64_t dest;
  if (x < nb) {  // base entry: tail keys below it
    code = lc[x];
    tok = li[x];
    const unsigned long long k = list_key(code, tok);
    int64_t lo = 0, hi = t;
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if (tk[mid] < k) lo = mid + 1; else hi = mid;
    }
    dest = x + lo;
  } else {  // tail entry: base keys below it
    const int64_t j = x - nb;
    const unsigned long long k = tk[j];
    code = (int32_t)((uint32_t)(k >> 32) ^ 0x80000000u);
    tok = (int32_t)(k & 0xffffffffull);
    int64_t lo = 0, hi = nb;
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if (list_key(lc[mid], li[mid]) < k) lo = mid + 1; else hi = mid;
    }
    dest = j + lo;
  }
  out[b * n + dest] = make_int2(code, tok);
}

__global__ __launch_bounds__(kMergeThreads) void k_merge_copy(Dev dv, int64_t n, const int2 *out) {
  const int64_t b = blockIdx.x;
  const int64_t x = (int64_t)blockIdx.y * kMergeThreads + threadIdx.x;
  if (x >= n) return;
  const int2 e = out[b * n + x];
  dv.list_code[b * dv.ncap + x] = e.x;
  dv.list_id[b * dv.ncap + x] = e.y;
}

int64_t merge_scratch_bytes(const Dev &dv, int64_t n) {
  const int64_t lists = (int64_t)dv.S * dv.mL;
  return lists * kMaxMergeTail * 8 + lists * n * 8;
}

hipError_t launch_merge(const Dev &dv, int64_t nb, int64_t n, void *scratch, hipStream_t st) {
  if (n <= nb) return hipSuccess;
  const int64_t lists = (int64_t)dv.S * dv.mL;
  unsigned long long *tail = reinterpret_cast<unsigned long long *>(scratch);
  int2 *out = reinterpret_cast<int2 *>(tail + lists * kMaxMergeTail);
  const dim3 grid((unsigned)lists, (unsigned)((n + kMergeThreads - 1) / kMergeThreads));
  hipLaunchKernelGGL(k_merge_tail, dim3((unsigned)lists), dim3(kMergeThreads), 0, st, dv, nb, n,
                     tail);
  hipLaunchKernelGGL(k_merge_place, grid, dim3(kMergeThreads), 0, st, dv, nb, n, tail, out);
  hipLaunchKernelGGL(k_merge_copy, grid, dim3(kMergeThreads), 0, st, dv, n, out);
  return hipGetLastError();
}

}  // namespace ice
