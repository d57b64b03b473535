// Decode-time query (IceCache paper page, Figure 2 steps (2)-(3); blog page,
// technical details: one prioritized-DCI search per head).
//
// Prioritized DCI visits the entries of a composite's m sorted lists in
// ascending |code - qcode| order and returns tokens in the order their m-th
// entry is visited; with exact integer distances that order is ascending
// (M_i, i) with M_i = max_j |code_ij - qcode_j|, so the k0 candidates of a
// composite are the k0 smallest (M_i, i).  On the GPU the walk becomes one
// coalesced pass over the token-major codes (on the synthetic caches a walk
// visits 60-85% of all list entries before k0 tokens complete, so it would
// touch most of them anyway) followed by an exact selection:
//
//   k_qprep     one block per stream: fp32 GQA mean, fp64 projection of the
//               normalised query to codes (directions staged in LDS), and the
//               per-query counters and histogram cleared;
//   k_qscan     M_i for every token and composite, a histogram of its top 11
//               bits;
//   k_qcollect  tokens in bins below the k0-th smallest bin are candidates;
//               boundary-bin tokens are parked with their (M_i, i) key;
//   k_qfinal    one 1024-thread block per stream: exact selection inside the
//               boundary bins, union of the composites (a per-query token bitmap), exact fp64
//               rerank, bitonic sort by (score desc, token asc), top-k and the
//               page walk.
#include "ice_device.h"

namespace ice {

constexpr int kFinalThreads = 1024;
constexpr int kHashSlots = 8192;  // 2 * kMaxCand
constexpr int kBndLds = 4096;      // boundary keys ranked in LDS

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = __lane_id();
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  return v;
}

// One whole wave: smallest bin b of h[0..kHistBins) whose inclusive prefix
// reaches `target` (1 <= target <= total) and the count below b.
__device__ void wave_find_bin(const uint32_t *h, uint32_t target, uint32_t &bin,
                              uint32_t &below) {
  constexpr int per = kHistBins / 64;
  const int lane = __lane_id();
  uint32_t v[per];
  uint32_t sum = 0;
  const uint4 *h4 = reinterpret_cast<const uint4 *>(h + lane * per);
#pragma unroll
  for (int k = 0; k < per / 4; ++k) {
    const uint4 x = h4[k];
    v[4 * k] = x.x;
    v[4 * k + 1] = x.y;
    v[4 * k + 2] = x.z;
    v[4 * k + 3] = x.w;
    sum += x.x + x.y + x.z + x.w;
  }
  const uint32_t incl = wave_incl_scan(sum);
  const uint32_t excl = incl - sum;
  const bool mine = excl < target && incl >= target;
  const unsigned long long bal = __ballot(mine);
  const int src = bal ? __ffsll((long long)bal) - 1 : 0;
  uint32_t b = 0, bl = 0;
  if (mine) {
    uint32_t run = excl;
#pragma unroll
    for (int k = 0; k < per; ++k) {
      if (run < target && run + v[k] >= target) {
        b = lane * per + k;
        bl = run;
      }
      run += v[k];
    }
  }
  bin = __shfl(b, src);
  below = __shfl(bl, src);
}

// Directions t0 .. t0+31 into LDS as dl[e * 32 + j] (fp64, zero past mL).
// For 256-thread blocks: each thread issues all of its loads before storing.
__device__ void stage_dirs32(const Dev &dv, int t0, double *dl) {
  constexpr int kIter = (129 * 32 + 255) / 256;
  const int d1 = dv.d + 1, tot = d1 * 32;
  double v[kIter];
#pragma unroll
  for (int k = 0; k < kIter; ++k) {
    // clamped addresses keep every load unconditional (a predicated load
    // would wait for its result at the branch join)
    const int x = min(threadIdx.x + 256 * k, tot - 1);
    const int e = x >> 5, j = x & 31, t = t0 + j;
    const int ch = min(t / kDirChunk, dv.nchunk - 1);
    v[k] = dv.dirs[((size_t)ch * d1 + e) * kDirChunk + (t % kDirChunk)];
  }
#pragma unroll
  for (int k = 0; k < kIter; ++k) {
    const int x = threadIdx.x + 256 * k;
    if (x < tot) dl[x] = (t0 + (x & 31)) < dv.nchunk * kDirChunk ? v[k] : 0.0;
  }
}

// Exact fp64 score <q_kv, k> in ascending element order (every product of an
// fp32 and a key element is exact in fp64).  Up to sixteen 16-byte loads of
// the row are in flight ahead of their part of the chain.
template <int DT, int D, int G>
__device__ __forceinline__ double exact_score_row(const float *qkv, const void *pool, int64_t row) {
  constexpr int kEpl = DT == 0 ? 4 : 8;   // elements per 16-byte load
  constexpr int kLoads = D / kEpl;        // loads per row
  constexpr int kGroup = kLoads < G ? kLoads : G;  // loads in flight: 4*G VGPRs
  const uint4 *src = reinterpret_cast<const uint4 *>(
      reinterpret_cast<const char *>(pool) + row * (DT == 0 ? 4 : 2));
  double acc = 0.0;
#pragma unroll 1
  for (int g0 = 0; g0 < kLoads; g0 += kGroup) {
    uint4 raw[kGroup];
#pragma unroll
    for (int k = 0; k < kGroup; ++k) raw[k] = src[g0 + k];
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      const uint32_t wv[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
      const int e0 = (g0 + k) * kEpl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (DT == 0) {
          acc = fma((double)qkv[e0 + j], (double)__uint_as_float(wv[j]), acc);
        } else {
          acc = fma((double)qkv[e0 + 2 * j], (double)__uint_as_float(wv[j] << 16), acc);
          acc = fma((double)qkv[e0 + 2 * j + 1], (double)__uint_as_float(wv[j] & 0xffff0000u), acc);
        }
      }
    }
  }
  return acc;
}

template <int DT, int G>
__device__ __forceinline__ double exact_score(const Dev &dv, const float *qkv, int s, int32_t lc) {
  const int64_t row = ((int64_t)s * dv.pcap * dv.p + lc) * dv.d;
  return dv.d == 128 ? exact_score_row<DT, 128, G>(qkv, dv.pool_k, row)
                     : exact_score_row<DT, 64, G>(qkv, dv.pool_k, row);
}

// Exact fp64 scores of ids[0..cnt) by a block of NT threads: per round of
// as many tokens as ROWBYTES of LDS holds, one round trip gathers their page
// slots, one stages their key rows in LDS, then one thread per row runs the
// ordered chain.  emit(x, id, slot, score) receives each result.  lcs needs
// ROWBYTES / 128 entries.
template <int DT, int NT, int ROWBYTES, typename Emit>
__device__ void block_score(const Dev &dv, int s, const int32_t *ids, uint32_t cnt,
                            const float *qkv, int32_t *lcs, uint32_t *rows, Emit emit) {
  const int tid = threadIdx.x;
  const int d = dv.d;
  const int row_bytes = d * dv.elem;
  const int row_words = row_bytes / 4;
  const uint32_t cap = ROWBYTES / row_bytes;  // rows per round (<= NT)
  const int cpr = row_bytes / 16;             // 16-byte chunks per row
  constexpr int kIter = (ROWBYTES / 16 + NT - 1) / NT;
  for (uint32_t b0 = 0; b0 < cnt; b0 += cap) {
    const uint32_t nr = min(cap, cnt - b0);
    if ((uint32_t)tid < nr) lcs[tid] = dv.loc[(int64_t)s * dv.ncap + ids[b0 + tid]];
    __syncthreads();
    uint4 v[kIter];
#pragma unroll
    for (int k = 0; k < kIter; ++k) {  // unconditional loads (row 0 stands in past nr)
      const int x = tid + NT * k;
      const int r = x / cpr, c = x % cpr;
      const int rr = (uint32_t)r < nr ? r : 0;
      const int64_t row = ((int64_t)s * dv.pcap * dv.p + lcs[rr]) * row_bytes;
      v[k] = reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(dv.pool_k) + row)[c];
    }
#pragma unroll
    for (int k = 0; k < kIter; ++k) {
      const int x = tid + NT * k;
      const int r = x / cpr, c = x % cpr;
      if ((uint32_t)r < nr) reinterpret_cast<uint4 *>(rows + r * row_words)[c] = v[k];
    }
    __syncthreads();
    if ((uint32_t)tid < nr) {
      const uint32_t *rw = rows + tid * row_words;
      double acc = 0.0;
      if constexpr (DT == 0) {
#pragma unroll 16
        for (int e = 0; e < d; ++e) acc = fma((double)qkv[e], (double)__uint_as_float(rw[e]), acc);
      } else {
#pragma unroll 8
        for (int e2 = 0; e2 < d / 2; ++e2) {
          const uint32_t wv = rw[e2];
          acc = fma((double)qkv[2 * e2], (double)__uint_as_float(wv << 16), acc);
          acc = fma((double)qkv[2 * e2 + 1], (double)__uint_as_float(wv & 0xffff0000u), acc);
        }
      }
      emit(b0 + tid, ids[b0 + tid], lcs[tid], acc);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- prep

// q_kv = fp32 mean of the g heads (left fold, then times fp32(1/g));
// qcode_t = code(<q_kv, u_t[:d]> / |q_kv|) with the dot products and the norm
// in fp64, ascending element order.  Also clears the query's counters and
// histogram.
template <int DT>
__global__ __launch_bounds__(256) void k_qprep(Dev dv, const void *q) {
  const int s = blockIdx.x;
  const int tid = threadIdx.x, d = dv.d, mL = dv.mL, g = dv.g, L = dv.L;
  __shared__ float qkv[128];
  __shared__ double dl[129 * 32];
  __shared__ double zs[kMaxMl];
  __shared__ double qsq;
  if (tid < d) {
    const float inv_g = (float)__ddiv_rn(1.0, (double)g);
    float acc = load_elem<DT>(q, (int64_t)s * g * d + tid);
    for (int h = 1; h < g; ++h)
      acc = __fadd_rn(acc, load_elem<DT>(q, ((int64_t)s * g + h) * d + tid));
    qkv[tid] = __fmul_rn(acc, inv_g);
  }
  if (tid < L) {
    dv.cand_count[s * L + tid] = 0;
    dv.bnd_count[s * L + tid] = 0;
  }
  if (tid == 0) dv.rr_count[s] = 0;
  for (int64_t x = tid; x < dv.mwords; x += 256) dv.cmark[(int64_t)s * dv.mwords + x] = 0;
  uint32_t *hist = dv.hist + (int64_t)s * L * kHistBins;
  for (int x = tid; x < L * kHistBins; x += 256) hist[x] = 0;
  __syncthreads();
  if (tid == 255) {
    double a = 0.0;
#pragma unroll 16
    for (int e = 0; e < d; ++e) a = fma((double)qkv[e], (double)qkv[e], a);
    qsq = a;
  }
  for (int t0 = 0; t0 < mL; t0 += 32) {
    stage_dirs32(dv, t0, dl);
    __syncthreads();
    if (tid < 32 && t0 + tid < mL) {
      double z = 0.0;
#pragma unroll 16
      for (int e = 0; e < d; ++e) z = fma((double)qkv[e], dl[e * 32 + tid], z);
      zs[t0 + tid] = z;
    }
    __syncthreads();
  }
  if (tid < mL) {
    const double qn = __dsqrt_rn(qsq);
    const double qb = qn > 0.0 ? __ddiv_rn(zs[tid], qn) : 0.0;
    dv.qcode[(int64_t)s * mL + tid] = to_code(qb);
  }
  if (tid < d) dv.qkv[(int64_t)s * d + tid] = qkv[tid];
}

// ---------------------------------------------------------------- scan

// Grid (blocks, S); each 512-thread block covers kScanTpb = 1024 tokens:
// wave w takes tiles 2w and 2w+1 of the block, lane j token j of a tile, and
// reads code t of its 64 tokens as one contiguous 256-byte load (32 codes of
// both tiles in flight at a time).  Histogram in LDS when L <= 6, else
// straight to global.
constexpr int kScanTpb = 1024;

template <bool LDS_HIST>
__global__ __launch_bounds__(512) void k_qscan(Dev dv, int64_t n) {
  const int s = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int mL = dv.mL, m = dv.m, L = dv.L;
  __shared__ int32_t qc[kMaxMl];
  __shared__ uint32_t hist[LDS_HIST ? 6 * kHistBins : 1];
  if (LDS_HIST)
    for (int x = tid; x < L * kHistBins; x += 512) hist[x] = 0;
  if (tid < mL) qc[tid] = dv.qcode[(int64_t)s * mL + tid];
  __syncthreads();
  uint32_t *ghist = dv.hist + (int64_t)s * L * kHistBins;
  const int64_t i0 = (int64_t)blockIdx.x * kScanTpb;
  const int64_t i1 = min(i0 + kScanTpb, n);
  const int64_t tile0 = (i0 >> 6) + 2 * w;  // this wave's first tile
  const int64_t ia = tile0 * 64 + lane, ib = ia + 64;
  const bool va = ia < i1, vb = ib < i1;
  // tiles past the array read tile 0 instead: every load is unconditional
  const int64_t tla = tile0 < dv.ntile ? tile0 : 0, tlb = tile0 + 1 < dv.ntile ? tile0 + 1 : 0;
  const int32_t *pa = dv.codes + ((int64_t)s * dv.ntile + tla) * mL * kCodeTile + lane;
  const int32_t *pb = dv.codes + ((int64_t)s * dv.ntile + tlb) * mL * kCodeTile + lane;
  struct Run {
    int l, j;
    uint32_t M;
  } ra{0, 0, 0u}, rb{0, 0, 0u};
  auto take = [&](Run &r, int64_t i, int32_t code, int t) {
    const uint32_t dd = absdiff(code, qc[t]);
    r.M = dd > r.M ? dd : r.M;
    if (++r.j == m) {
      dv.mbuf[((int64_t)s * L + r.l) * dv.ncap + i] = r.M;
      if (LDS_HIST)
        atomicAdd(&hist[r.l * kHistBins + (r.M >> kHistShift)], 1u);
      else
        atomicAdd(&ghist[r.l * kHistBins + (r.M >> kHistShift)], 1u);
      ++r.l;
      r.j = 0;
      r.M = 0;
    }
  };
  for (int t0 = 0; t0 < mL; t0 += 32) {
    int32_t a[32], b[32];
#pragma unroll
    for (int x = 0; x < 32; ++x) {
      const int t = min(t0 + x, mL - 1);
      a[x] = pa[(int64_t)t * kCodeTile];
      b[x] = pb[(int64_t)t * kCodeTile];
    }
#pragma unroll
    for (int x = 0; x < 32; ++x) {
      if (t0 + x < mL) {
        if (va) take(ra, ia, a[x], t0 + x);
        if (vb) take(rb, ib, b[x], t0 + x);
      }
    }
  }
  if (LDS_HIST) {
    __syncthreads();
    // Flush only the bins at or below this block's own k0-th smallest bin.
    // The k0-th smallest M of the whole stream is never in a higher bin of a
    // block that holds at least k0 tokens, so every bin up to the global
    // threshold bin still receives every block's count.
    __shared__ uint32_t blim[6];
    const int lane = tid & 63, w = tid >> 6;
    const uint32_t ntok = (uint32_t)(i1 > i0 ? i1 - i0 : 0);
    for (int l = w; l < L; l += 8) {
      uint32_t b = kHistBins - 1, bl;
      if (ntok >= (uint32_t)dv.k0 && dv.k0 > 0) wave_find_bin(hist + l * kHistBins, dv.k0, b, bl);
      if (lane == 0) blim[l] = b;
    }
    __syncthreads();
    for (int x = tid; x < L * kHistBins; x += 512) {
      const uint32_t h = hist[x];
      if (h && (uint32_t)(x % kHistBins) <= blim[x / kHistBins]) atomicAdd(&ghist[x], h);
    }
  }
}

// ---------------------------------------------------------------- collect

// Token i is a candidate of composite l when its bin is below the k0-th
// smallest bin b*, and its key (M << 32 | i) goes to the boundary list when
// the bin is b*.  Candidates are gathered per block (one device atomic per
// block and composite), each distinct candidate token is scored exactly here,
// in parallel, and its (rank key, token, page) appended to the rerank list.
template <int DT>
__global__ __launch_bounds__(512) void k_qcollect(Dev dv, int64_t n) {
  const int s = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int L = dv.L;
  __shared__ uint32_t bstar[32];
  __shared__ uint32_t ccount[32], cbase[32];
  __shared__ float qkv[128];
  __shared__ int32_t cid[kScanTpb];
  constexpr int kCollectRowBytes = 32 * 1024;
  __shared__ int32_t lcs[kCollectRowBytes / 128];
  __shared__ uint32_t rows[kCollectRowBytes / 4];
  __shared__ uint32_t nc, rbase;
  const uint32_t k0e = (uint32_t)min((int64_t)dv.k0, n);
  if (k0e == 0) return;
  const int64_t i0 = (int64_t)blockIdx.x * kScanTpb;
  const int64_t i1 = min(i0 + kScanTpb, n);
  const int64_t ii[2] = {i0 + tid, i0 + 512 + tid};
  const bool vv[2] = {ii[0] < i1, ii[1] < i1};
  // every composite distance of both tokens for the first 8 composites
  uint32_t Mv[2][8];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int l = 0; l < 8; ++l) {  // unconditional loads at clamped addresses
      const int lc = l < L ? l : 0;
      const int64_t ic = vv[u] ? ii[u] : 0;
      Mv[u][l] = dv.mbuf[((int64_t)s * L + lc) * dv.ncap + ic];
    }
  if (tid < dv.d) qkv[tid] = dv.qkv[(int64_t)s * dv.d + tid];
  if (tid < L) ccount[tid] = 0;
  if (tid == 0) nc = 0;
  for (int l = w; l < L; l += 8) {
    uint32_t b, bl;
    wave_find_bin(dv.hist + ((int64_t)s * L + l) * kHistBins, k0e, b, bl);
    if (lane == 0) bstar[l] = b;
  }
  __syncthreads();
  const unsigned long long lt = lanemask_lt();
  uint32_t masks[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t i = ii[u];
    const bool valid = vv[u];
    uint32_t mask = 0;
    for (int l = 0; l < L; ++l) {
      uint32_t M = 0xffffffffu;
      if (l < 8) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (q == l) M = Mv[u][q];
      } else {
        M = dv.mbuf[((int64_t)s * L + l) * dv.ncap + (valid ? i : 0)];
      }
      const uint32_t b = M >> kHistShift;
      if (valid && b < bstar[l]) mask |= 1u << l;
      const bool is_b = valid && b == bstar[l];
      const unsigned long long mb = __ballot(is_b);
      if (mb) {  // rare: wave-aggregated append of boundary keys
        const int first = __ffsll((long long)mb) - 1;
        uint32_t base = 0;
        if (lane == first) base = atomicAdd(&dv.bnd_count[s * L + l], (uint32_t)popc64(mb));
        base = __shfl(base, first);
        if (is_b)
          dv.bnd[((int64_t)s * L + l) * dv.ncap + base + popc64(mb & lt)] =
              ((unsigned long long)M << 32) | (uint32_t)i;
      }
    }
    masks[u] = mask;
    if (mask) {
      cid[atomicAdd(&nc, 1u)] = (int32_t)i;
      for (int l = 0; l < L; ++l)
        if ((mask >> l) & 1u) atomicAdd(&ccount[l], 1u);
    }
  }
  __syncthreads();
  if (tid < L) {
    cbase[tid] = ccount[tid] ? atomicAdd(&dv.cand_count[s * L + tid], ccount[tid]) : 0u;
    ccount[tid] = 0;
  }
  if (tid == 64 && nc) rbase = atomicAdd(&dv.rr_count[s], nc);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t mask = masks[u];
    for (int l = 0; l < L; ++l)
      if ((mask >> l) & 1u)
        dv.cand[((int64_t)s * L + l) * dv.k0 + cbase[l] + atomicAdd(&ccount[l], 1u)] =
            (int32_t)ii[u];
  }
  const int64_t obase = (int64_t)s * L * dv.k0 + rbase;
  unsigned long long *rk = dv.rr_key + obase;
  int32_t *ri = dv.rr_id + obase;
  int32_t *rp = dv.rr_pg + obase;
  uint32_t *mk = dv.cmark + (int64_t)s * dv.mwords;
  const int p = dv.p;
  block_score<DT, 512, kCollectRowBytes>(dv, s, cid, nc, qkv, lcs, rows,
                       [rk, ri, rp, mk, p](uint32_t x, int32_t id, int32_t lc, double sc) {
                         rk[x] = score_rank_key(sc);
                         ri[x] = id;
                         rp[x] = lc / p;
                         atomicOr(&mk[id >> 5], 1u << (id & 31));
                       });
}

// ---------------------------------------------------------------- final

// r-th smallest (1-based) of n distinct keys in global memory, by eight 8-bit
// MSB-first digit passes.  All threads of the block call it.
__device__ unsigned long long block_select(const unsigned long long *keys, uint32_t n,
                                           uint32_t r, uint32_t *cnt,
                                           unsigned long long *res, uint32_t *rr) {
  const int tid = threadIdx.x;
  unsigned long long prefix = 0, himask = 0;
  if (tid == 0) *rr = r;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    if (tid < 256) cnt[tid] = 0;
    __syncthreads();
    for (uint32_t x = tid; x < n; x += blockDim.x) {
      const unsigned long long k = keys[x];
      if ((k & himask) == prefix) atomicAdd(&cnt[(k >> shift) & 255ull], 1u);
    }
    __syncthreads();
    if (tid < 64) {  // one wave scans the 256 digit counts
      uint32_t c4[4], sum = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        c4[k] = cnt[tid * 4 + k];
        sum += c4[k];
      }
      const uint32_t incl = wave_incl_scan(sum);
      uint32_t run = incl - sum;
      const uint32_t want = *rr;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (run < want && run + c4[k] >= want) {
          *res = prefix | ((unsigned long long)(tid * 4 + k) << shift);
          *rr = want - run;
        }
        run += c4[k];
      }
    }
    __syncthreads();
    prefix = *res;
    himask |= 0xffull << shift;
    __syncthreads();
  }
  return prefix;
}

// Element of the rerank order: rank key, token, page.
struct RankEl {
  unsigned long long k;
  int32_t id, pg;
};

__device__ __forceinline__ bool rank_less(const RankEl &a, const RankEl &b) {
  return a.k < b.k || (a.k == b.k && a.id < b.id);
}

__device__ __forceinline__ RankEl shfl_xor_el(const RankEl &e, int m) {
  RankEl o;
  o.k = ((unsigned long long)(uint32_t)__shfl_xor((int)(uint32_t)(e.k >> 32), m) << 32) |
        (uint32_t)__shfl_xor((int)(uint32_t)e.k, m);
  o.id = __shfl_xor(e.id, m);
  o.pg = __shfl_xor(e.pg, m);
  return o;
}

// Bitonic step for element x against its partner's value o (partner index
// x ^ jj): in an ascending run the lower index keeps the smaller element.
__device__ __forceinline__ void bitonic_keep(RankEl &e, const RankEl &o, uint32_t x, uint32_t jj,
                                             uint32_t kk) {
  const bool asc = (x & kk) == 0;
  const bool lower = (x & jj) == 0;
  if ((lower == asc) == rank_less(o, e)) e = o;
}

// a holds element xa, b its partner (a higher index) in the same thread.
__device__ __forceinline__ void reg_pair(RankEl &a, RankEl &b, uint32_t xa, uint32_t kk) {
  const bool asc = (xa & kk) == 0;
  if (rank_less(b, a) == asc) {
    const RankEl t = a;
    a = b;
    b = t;
  }
}

// Sorts npad (a power of two <= NT*R) elements ascending by (key, token)
// across a block of NT threads.  Element x = r*NT + tid lives in registers;
// partner distances below 64 are wave shuffles, distances of NT and more are
// register swaps inside a thread, the rest go through the LDS arrays xk/xi/xg.
template <int NT, int R>
__device__ void block_bitonic(RankEl (&el)[R], uint32_t npad, unsigned long long *xk, int32_t *xi,
                              int32_t *xg) {
  const int tid = threadIdx.x;
  for (uint32_t kk = 2; kk <= npad; kk <<= 1) {
    for (uint32_t jj = kk >> 1; jj > 0; jj >>= 1) {
      if (jj >= (uint32_t)NT) {
        if constexpr (R >= 2) {
          if (jj == (uint32_t)NT) {
#pragma unroll
            for (int r = 0; r < R; r += 2) reg_pair(el[r], el[r + 1], r * NT + tid, kk);
          }
        }
        if constexpr (R >= 4) {
          if (jj == 2u * NT) {
            reg_pair(el[0], el[2], tid, kk);
            reg_pair(el[1], el[3], NT + tid, kk);
          }
        }
      } else if (jj >= 64) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t x = r * NT + tid;
          xk[x] = el[r].k;
          xi[x] = el[r].id;
          xg[x] = el[r].pg;
        }
        __syncthreads();
        RankEl o[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t y = (r * NT + tid) ^ jj;
          o[r].k = xk[y];
          o[r].id = xi[y];
          o[r].pg = xg[y];
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) bitonic_keep(el[r], o[r], r * NT + tid, jj, kk);
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const RankEl o = shfl_xor_el(el[r], (int)jj);
          bitonic_keep(el[r], o, r * NT + tid, jj, kk);
        }
      }
    }
  }
}

// Sorts the LDS arrays (sk, si, sp)[0..npad) in place through registers.
template <int NT, int R>
__device__ void sort_rank_arrays(unsigned long long *sk, int32_t *si, int32_t *sp, uint32_t npad) {
  RankEl el[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t x = r * NT + threadIdx.x;
    if (x < npad) {
      el[r].k = sk[x];
      el[r].id = si[x];
      el[r].pg = sp[x];
    } else {
      el[r].k = ~0ull;
      el[r].id = 0x7fffffff;
      el[r].pg = 0;
    }
  }
  __syncthreads();
  block_bitonic<NT, R>(el, npad, sk, si, sp);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t x = r * NT + threadIdx.x;
    if (x < npad) {
      sk[x] = el[r].k;
      si[x] = el[r].id;
      sp[x] = el[r].pg;
    }
  }
  __syncthreads();
}

// Inserts id into the LDS hash set; true when it was not there yet.
__device__ __forceinline__ bool hash_insert(uint32_t *tab, int32_t id) {
  const uint32_t key = (uint32_t)id + 1u;
  uint32_t h = (key * 2654435761u) >> (32 - 13);
  for (;;) {
    const uint32_t old = atomicCAS(&tab[h], 0u, key);
    if (old == 0u) return true;
    if (old == key) return false;
    h = (h + 1u) & (kHashSlots - 1u);
  }
}

constexpr int kFinalRowBytes = 48 * 1024;  // key rows staged for scoring

struct FinalShared {
  union {
    unsigned long long bk[kBndLds];  // boundary keys (selection phase)
    uint32_t rows[kFinalRowBytes / 4];  // key rows (scoring phase)
  };
  union {
    uint32_t hash[kHashSlots];  // rerank-list membership (selection phase)
    uint32_t seen[2048];        // selected pages (page walk)
  };
  unsigned long long skey[kMaxCand];  // rank keys
  int32_t sid[kMaxCand];
  int32_t spg[kMaxCand];
  uint32_t cnt[256];
  float qkv[128];
  int32_t lcs[512];
  uint32_t cc[32], nb[32], need[32], boff[33], extra[32];
  uint32_t nu;
  uint32_t rr;
  unsigned long long res;
};

template <int DT>
__device__ void final_add(FinalShared &sh, const Dev &dv, int s, int l, int32_t id) {
  dv.cand[((int64_t)s * dv.L + l) * dv.k0 + sh.cc[l] + atomicAdd(&sh.extra[l], 1u)] = id;
  if (hash_insert(sh.hash, id)) sh.sid[atomicAdd(&sh.nu, 1u)] = id;  // scored in phase C
}

template <int DT>
__global__ __launch_bounds__(kFinalThreads) void k_qfinal(Dev dv, int64_t n, int32_t *page_ids,
                                                          int32_t *n_pages, int32_t *topk_ids) {
  __shared__ FinalShared sh;
  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int L = dv.L, k0 = dv.k0;
  const uint32_t k0e = (uint32_t)min((int64_t)k0, n);

  // A. counts, thresholds, the query
  for (int x = tid; x < kHashSlots; x += kFinalThreads) sh.hash[x] = 0;
  if (tid < dv.d) sh.qkv[tid] = dv.qkv[(int64_t)s * dv.d + tid];
  if (tid < L) {
    sh.cc[tid] = dv.cand_count[s * L + tid];
    sh.nb[tid] = dv.bnd_count[s * L + tid];
    sh.extra[tid] = 0;
    sh.need[tid] = 0;
  }
  if (tid == 0) sh.nu = 0;
  if (k0e > 0) {
    for (int l = w; l < L; l += kFinalThreads / 64) {
      uint32_t b, bl;
      wave_find_bin(dv.hist + ((int64_t)s * L + l) * kHistBins, k0e, b, bl);
      if (lane == 0) sh.need[l] = k0e - bl;
    }
  }
  const uint32_t nrr = k0e > 0 ? dv.rr_count[s] : 0u;
  __syncthreads();
  if (tid == 0) {
    uint32_t o = 0;
    for (int l = 0; l < L; ++l) {
      sh.boff[l] = o;
      o += (k0e > 0) ? sh.nb[l] : 0u;
    }
    sh.boff[L] = o;
    sh.nu = nrr;
  }
  // B1. the scored candidates below the boundary bins
  for (uint32_t x = tid; x < nrr; x += kFinalThreads) {
    const int64_t o = (int64_t)s * L * k0 + x;
    const int32_t id = dv.rr_id[o];
    hash_insert(sh.hash, id);
    sh.sid[x] = id;
    sh.skey[x] = dv.rr_key[o];
    sh.spg[x] = dv.rr_pg[o];
  }
  __syncthreads();
  // B2. the need_l smallest (M, i) of each composite's boundary bin
  const uint32_t nbt = sh.boff[L];
  if (nbt > 0) {
    if (nbt <= (uint32_t)kBndLds) {
      for (uint32_t x = tid; x < nbt; x += kFinalThreads) {
        int l = 0;
        while (x >= sh.boff[l + 1]) ++l;
        sh.bk[x] = dv.bnd[((int64_t)s * L + l) * dv.ncap + (x - sh.boff[l])];
      }
      __syncthreads();
      for (uint32_t x = tid; x < nbt; x += kFinalThreads) {
        int l = 0;
        while (x >= sh.boff[l + 1]) ++l;
        const unsigned long long key = sh.bk[x];
        uint32_t rank = 0;
        for (uint32_t y = sh.boff[l]; y < sh.boff[l + 1]; ++y) rank += sh.bk[y] < key;
        if (rank < sh.need[l]) final_add<DT>(sh, dv, s, l, (int32_t)(key & 0xffffffffull));
      }
    } else {
      for (int l = 0; l < L; ++l) {
        const unsigned long long *bk = dv.bnd + ((int64_t)s * L + l) * dv.ncap;
        const uint32_t nbl = sh.nb[l], nd = sh.need[l];
        const unsigned long long thr =
            nd >= nbl ? ~0ull : block_select(bk, nbl, nd, sh.cnt, &sh.res, &sh.rr);
        for (uint32_t x = tid; x < nbl; x += kFinalThreads) {
          const unsigned long long key = bk[x];
          if (key <= thr) final_add<DT>(sh, dv, s, l, (int32_t)(key & 0xffffffffull));
        }
        __syncthreads();
      }
    }
  }
  __syncthreads();
  if (tid < L && k0e > 0) dv.cand_count[s * L + tid] = sh.cc[tid] + sh.extra[tid];

  // C. score the boundary picks (positions nrr .. nu-1); pad for the sort
  const uint32_t nu = sh.nu;
  uint32_t npad = 1;
  while (npad < nu) npad <<= 1;
  {
    unsigned long long *sk = sh.skey + nrr;
    int32_t *sp = sh.spg + nrr;
    const int p = dv.p;
    block_score<DT, kFinalThreads, kFinalRowBytes>(dv, s, sh.sid + nrr, nu - nrr, sh.qkv, sh.lcs,
                                                   sh.rows,
                                   [sk, sp, p](uint32_t x, int32_t, int32_t lc, double sc) {
                                     sk[x] = score_rank_key(sc);
                                     sp[x] = lc / p;
                                   });
  }
  for (uint32_t x = nu + tid; x < npad; x += kFinalThreads) {
    sh.skey[x] = ~0ull;
    sh.sid[x] = 0x7fffffff;
    sh.spg[x] = 0;
  }
  __syncthreads();

  // D. sort by (rank key, token): register bitonic, npad <= 4096
  if (npad <= (uint32_t)kFinalThreads)
    sort_rank_arrays<kFinalThreads, 1>(sh.skey, sh.sid, sh.spg, npad);
  else if (npad <= 2u * kFinalThreads)
    sort_rank_arrays<kFinalThreads, 2>(sh.skey, sh.sid, sh.spg, npad);
  else
    sort_rank_arrays<kFinalThreads, 4>(sh.skey, sh.sid, sh.spg, npad);
  for (int x = tid; x < 2048; x += kFinalThreads) sh.seen[x] = 0;  // the hash is done
  __syncthreads();

  // E. top-k tokens, then pages in rank order
  if (topk_ids)
    for (int x = tid; x < dv.k; x += kFinalThreads)
      topk_ids[(int64_t)s * dv.k + x] = (uint32_t)x < nu ? sh.sid[x] : -1;
  if (w == 0) {
    int pbits = 1;
    while ((1ll << pbits) < dv.pcap) ++pbits;
    int nsel = 0;
    const unsigned long long lt = lanemask_lt();
    for (uint32_t x0 = 0; x0 < nu && nsel < dv.P; x0 += 64) {
      const uint32_t x = x0 + lane;
      const bool valid = x < nu;
      const int32_t pg = valid ? sh.spg[x] : 0;
      const bool fresh = valid && ((sh.seen[pg >> 5] >> (pg & 31)) & 1u) == 0u;
      const unsigned long long act = __ballot(fresh);
      const unsigned long long mt = match_bits((uint32_t)pg, pbits, act);
      const bool firstocc = fresh && (mt & lt) == 0ull;
      const unsigned long long fm = __ballot(firstocc);
      const int pos = nsel + popc64(fm & lt);
      if (firstocc && pos < dv.P) {
        page_ids[(int64_t)s * dv.P + pos] = pg;
        atomicOr(&sh.seen[pg >> 5], 1u << (pg & 31));
      }
      nsel = min(dv.P, nsel + popc64(fm));
      __builtin_amdgcn_wave_barrier();
    }
    for (int x = nsel + lane; x < dv.P; x += 64) page_ids[(int64_t)s * dv.P + x] = -1;
    if (lane == 0) n_pages[s] = nsel;
  }
}

// ---------------------------------------------------------------- launcher

template <int DT>
static hipError_t query_impl(const Dev &dv, int64_t n, const void *q, int32_t *page_ids,
                             int32_t *n_pages, int32_t *topk_ids, hipStream_t st, Timer *tm) {
  const unsigned nblk = (unsigned)((n + kScanTpb - 1) / kScanTpb);  // scan and collect blocks match
  timer_begin(tm, st);
  hipLaunchKernelGGL(k_qprep<DT>, dim3(dv.S), dim3(256), 0, st, dv, q);
  timer_mark(tm, KID_QPREP, st);
  if (n > 0) {
    if (dv.L <= 6)
      hipLaunchKernelGGL((k_qscan<true>), dim3(nblk, dv.S), dim3(512), 0, st, dv, n);
    else
      hipLaunchKernelGGL((k_qscan<false>), dim3(nblk, dv.S), dim3(512), 0, st, dv, n);
    timer_mark(tm, KID_QSCAN, st);
    hipLaunchKernelGGL(k_qcollect<DT>, dim3(nblk, dv.S), dim3(512), 0, st, dv, n);
    timer_mark(tm, KID_QCOLLECT, st);
  }
  hipLaunchKernelGGL(k_qfinal<DT>, dim3(dv.S), dim3(kFinalThreads), 0, st, dv, n, page_ids,
                     n_pages, topk_ids);
  timer_mark(tm, KID_QFINAL, st);
  return hipGetLastError();
}

hipError_t launch_query(const Dev &dv, int64_t n, const void *q, int32_t *page_ids,
                        int32_t *n_pages, int32_t *topk_ids, hipStream_t st, Timer *tm) {
  return dv.dtype == 0 ? query_impl<0>(dv, n, q, page_ids, n_pages, topk_ids, st, tm)
                       : query_impl<1>(dv, n, q, page_ids, n_pages, topk_ids, st, tm);
}

}  // namespace ice
