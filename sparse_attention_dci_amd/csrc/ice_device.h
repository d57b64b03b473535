// Device helpers for the gfx950 kernels (64-wide wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ice_common.h"

namespace ice {

constexpr int kWave = 64;

// Element loads: K, V, q and directions are fp32 or bf16 (dtype 0 / 1).
__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
  return __uint_as_float(b << 16);
}

template <int DT>
__device__ __forceinline__ float load_elem(const void *base, int64_t i) {
  if constexpr (DT == 0) {
    return reinterpret_cast<const float *>(base)[i];
  } else {
    return bf16_bits_to_float(reinterpret_cast<const uint16_t *>(base)[i]);
  }
}

// Eight consecutive elements starting at an index that is a multiple of 8.
template <int DT>
__device__ __forceinline__ void load8(const void *base, int64_t i, float (&v)[8]) {
  if constexpr (DT == 0) {
    const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + i);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    uint4 a = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(base) + i);
    uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
}

// Workgroup barrier that orders LDS only: global loads and stores stay in
// flight across it (__syncthreads would wait for every outstanding one).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ int32_t to_code(double x) {
  double v = rint(x * kCodeScale);  // scaling by 2^29 is exact
  v = fmin(fmax(v, -(double)kCodeMax), (double)kCodeMax);
  return (int32_t)v;
}

__device__ __forceinline__ uint32_t absdiff(int32_t a, int32_t b) {
  int64_t d = (int64_t)a - (int64_t)b;
  return (uint32_t)(d < 0 ? -d : d);
}

// Rank key of a reranked candidate: ascending key == descending score.
__device__ __forceinline__ unsigned long long score_rank_key(double s) {
  if (s == 0.0) s = 0.0;  // one zero
  unsigned long long b = (unsigned long long)__double_as_longlong(s);
  unsigned long long ord = (b >> 63) ? ~b : (b | 0x8000000000000000ull);  // ascending
  return ~ord;
}

__device__ __forceinline__ unsigned long long lanemask_lt() {
  const int lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__device__ __forceinline__ int popc64(unsigned long long x) { return __popcll(x); }

// Index of the n-th (0-based) set bit of m; m must have more than n bits set.
__device__ __forceinline__ int nth_set_bit(unsigned long long m, int n) {
  int pos = 0;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    unsigned long long low = m & ((1ull << w) - 1ull);
    int c = popc64(low);
    if (n >= c) {
      n -= c;
      m >>= w;
      pos += w;
    } else {
      m = low;
    }
  }
  return pos;
}

// Lanes of the wave whose `key` (restricted to `bits` low bits) equals this
// lane's, among the lanes in `active`.
__device__ __forceinline__ unsigned long long match_bits(uint32_t key, int bits,
                                                         unsigned long long active) {
  unsigned long long m = active;
  for (int b = 0; b < bits; ++b) {
    unsigned long long bal = __ballot((key >> b) & 1u);
    m &= ((key >> b) & 1u) ? bal : ~bal;
  }
  return m;
}

// Inclusive prefix sum over the 64 lanes of a wave.
// Inclusive prefix sum over the 64 lanes with DPP moves (no LDS round trips):
// row_shr 1, 2, 4, 8 scan each row of 16 lanes, row_bcast 15 and 31 carry
// the row totals into the rows above.  Lanes whose DPP source is outside the
// row, or rows the row mask excludes, add 0.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return (uint32_t)x;
}

// Smallest / largest 64-bit value over the 64 lanes (whole wave), by the
// same DPP sequence as wave_incl_scan on both halves (lane 63 ends with the
// result), broadcast.  Lanes without a DPP source take the identity.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long id,
                                                      unsigned long long v) {
  const int lo = __builtin_amdgcn_update_dpp((int)(uint32_t)id, (int)(uint32_t)v, CTRL, ROWMASK,
                                             0xf, false);
  const int hi = __builtin_amdgcn_update_dpp((int)(uint32_t)(id >> 32), (int)(uint32_t)(v >> 32),
                                             CTRL, ROWMASK, 0xf, false);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

template <bool MAX>
__device__ __forceinline__ unsigned long long wave_minmax_u64(unsigned long long x) {
  constexpr unsigned long long id = MAX ? 0ull : ~0ull;
  auto op = [](unsigned long long a, unsigned long long b) { return MAX ? max(a, b) : min(a, b); };
  x = op(x, dpp_u64<0x111, 0xf>(id, x));  // row_shr:1
  x = op(x, dpp_u64<0x112, 0xf>(id, x));  // row_shr:2
  x = op(x, dpp_u64<0x114, 0xf>(id, x));  // row_shr:4
  x = op(x, dpp_u64<0x118, 0xf>(id, x));  // row_shr:8
  x = op(x, dpp_u64<0x142, 0xa>(id, x));  // row_bcast:15
  x = op(x, dpp_u64<0x143, 0xc>(id, x));  // row_bcast:31
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), 63);
  return ((unsigned long long)hi << 32) | lo;
}

// One whole wave: smallest bin b of a kHistBins histogram whose inclusive
// prefix reaches `target` (1 <= target <= total) and the count below b.  The
// histogram is read by wave_hist_load in chunks of 256 bins, one contiguous
// 16-byte read per lane and chunk (lane j holds bins 256c + 4j .. 256c + 4j
// + 3 of chunk c in v[4c .. 4c + 3]), so that several can be in flight
// before any is searched, and a wave's read of a chunk is one contiguous
// kilobyte (no LDS bank conflicts, whole lines from memory).
constexpr int kBinsPerLane = kHistBins / 64;
constexpr int kHistChunks = kHistBins / 256;

__device__ __forceinline__ void wave_hist_load(const uint32_t *h, uint32_t (&v)[kBinsPerLane]) {
  const uint4 *h4 = reinterpret_cast<const uint4 *>(h) + __lane_id();
#pragma unroll
  for (int c = 0; c < kHistChunks; ++c) {
    const uint4 x = h4[64 * c];
    v[4 * c] = x.x;
    v[4 * c + 1] = x.y;
    v[4 * c + 2] = x.z;
    v[4 * c + 3] = x.w;
  }
}

// The bin within a 256-bin chunk (lane j holds c[0..3] = bins 4j .. 4j+3)
// whose inclusive prefix reaches target, given the lane's inclusive prefix
// incl of the chunk and its sum (the chunk's total reaches target).
__device__ __forceinline__ void chunk_find(const uint32_t (&c)[4], uint32_t incl, uint32_t sum,
                                           uint32_t target, uint32_t &bin, uint32_t &below) {
  const int lane = __lane_id();
  const uint32_t excl = incl - sum;
  const bool mine = excl < target && incl >= target;
  const unsigned long long bal = __ballot(mine);
  const int src = bal ? __ffsll((long long)bal) - 1 : 0;
  uint32_t b = 0, bl = 0;
  if (mine) {
    uint32_t run = excl;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (run < target && run + c[k] >= target) {
        b = 4 * lane + k;
        bl = run;
      }
      run += c[k];
    }
  }
  bin = (uint32_t)__builtin_amdgcn_readlane((int)b, src);  // src is wave-uniform
  below = (uint32_t)__builtin_amdgcn_readlane((int)bl, src);
}

__device__ void wave_find_bin_regs(const uint32_t (&v)[kBinsPerLane], uint32_t target,
                                   uint32_t &bin, uint32_t &below) {
  uint32_t sum[kHistChunks], incl[kHistChunks], tot[kHistChunks];
#pragma unroll
  for (int c = 0; c < kHistChunks; ++c) {  // independent scans, all in flight
    sum[c] = v[4 * c] + v[4 * c + 1] + v[4 * c + 2] + v[4 * c + 3];
    incl[c] = wave_incl_scan(sum[c]);
    tot[c] = (uint32_t)__builtin_amdgcn_readlane((int)incl[c], 63);
  }
  uint32_t base = 0;  // the count below the chunk that holds the target (uniform)
  int cs = kHistChunks - 1;
#pragma unroll
  for (int c = 0; c < kHistChunks - 1; ++c) {
    if (cs == kHistChunks - 1 && base + tot[c] >= target) cs = c;
    if (cs == kHistChunks - 1) base += tot[c];
  }
  uint32_t cv[4] = {0u, 0u, 0u, 0u}, ci = 0, csum = 0;
#pragma unroll
  for (int c = 0; c < kHistChunks; ++c)
    if (c == cs) {
      cv[0] = v[4 * c];
      cv[1] = v[4 * c + 1];
      cv[2] = v[4 * c + 2];
      cv[3] = v[4 * c + 3];
      ci = incl[c];
      csum = sum[c];
    }
  uint32_t b, bl;
  chunk_find(cv, ci, csum, target - base, b, bl);
  bin = 256u * (uint32_t)cs + b;
  below = base + bl;
}

// The low kLowBins bins of a histogram (its first chunk), four per lane.
constexpr int kLowBins = 256;
static_assert(kLowBins == 4 * 64 && kLowBins <= kHistBins, "four low bins per lane");

__device__ __forceinline__ uint4 wave_hist_load_low(const uint32_t *h) {
  return reinterpret_cast<const uint4 *>(h)[__lane_id()];
}

// wave_find_bin_regs over the low bins only: found (wave-uniform) when their
// total reaches `target`, and then bin and below are those of the whole
// histogram (the smallest bin whose inclusive prefix reaches the target is
// among them).
__device__ __forceinline__ bool wave_find_bin_low(uint4 v, uint32_t target, uint32_t &bin,
                                                  uint32_t &below) {
  const uint32_t sum = v.x + v.y + v.z + v.w;
  const uint32_t incl = wave_incl_scan(sum);
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  if (total < target) return false;
  const uint32_t c[4] = {v.x, v.y, v.z, v.w};
  chunk_find(c, incl, sum, target, bin, below);
  return true;
}

// wave_find_bin one chunk at a time (four registers per lane instead of 32;
// a chunk is read only when the ones below it do not reach the target).
__device__ __forceinline__ void wave_find_bin_seq(const uint32_t *h, uint32_t target,
                                                  uint32_t &bin, uint32_t &below) {
  uint32_t base = 0;
  for (int c = 0; c < kHistChunks; ++c) {
    const uint4 v = reinterpret_cast<const uint4 *>(h)[64 * c + __lane_id()];
    const uint32_t sum = v.x + v.y + v.z + v.w;
    const uint32_t incl = wave_incl_scan(sum);
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    if (base + tot >= target || c == kHistChunks - 1) {
      const uint32_t cv[4] = {v.x, v.y, v.z, v.w};
      uint32_t b, bl;
      chunk_find(cv, incl, sum, target - base, b, bl);
      bin = 256u * (uint32_t)c + b;
      below = base + bl;
      return;
    }
    base += tot;
  }
}

__device__ __forceinline__ void wave_find_bin(const uint32_t *h, uint32_t target, uint32_t &bin,
                                              uint32_t &below) {
  uint32_t v[kBinsPerLane];
  wave_hist_load(h, v);
  wave_find_bin_regs(v, target, bin, below);
}

}  // namespace ice
