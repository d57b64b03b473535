// Decode-time query (IceCache paper page, Figure 2 steps (2)-(3); blog page,
// technical details: one prioritized-DCI search per head).
//
// Prioritized DCI visits the entries of a composite's m sorted lists in
// ascending |code - qcode| order and returns tokens in the order their m-th
// entry is visited; with exact integer distances that order is ascending
// (M_i, i) with M_i = max_j |code_ij - qcode_j|, so the k0 candidates of a
// composite are the k0 smallest (M_i, i).  On the GPU the walk becomes one
// coalesced pass over the token-major codes (measured visit fractions on the
// synthetic caches are 60-85% of all list entries, so a walk would touch most
// of them anyway) and an exact selection:
//
//   k_qscan     query prep (fp32 GQA mean, fp64 projection to codes), M_i for
//               every token and composite, a histogram of M_i's top bits;
//   k_qcollect  tokens in bins below the k0-th smallest bin are candidates;
//               each new candidate is scored exactly (fp64, ascending order)
//               and appended to the stream's rerank set; boundary-bin tokens
//               are parked;
//   k_qfinal    (one block per stream) exact selection inside the boundary
//               bins, rank by (score desc, token asc), top-k, page walk.
#include "ice_device.h"

namespace ice {

// ---------------------------------------------------------------- helpers

// Block-wide inclusive scan of one value per thread (256 threads); also
// returns the block total.
__device__ __forceinline__ uint32_t block_incl_scan256(uint32_t v, uint32_t *wsum,
                                                       uint32_t &total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t incl = v;
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  uint32_t pre = 0;
  for (int k = 0; k < w; ++k) pre += wsum[k];
  total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  return pre + incl;
}

// Smallest bin b of h[0..kHistBins) whose inclusive prefix reaches `target`
// (>= 1), and the count below it.  All 256 threads call; results via LDS.
__device__ void find_bin(const uint32_t *h, uint32_t target, uint32_t *wsum, uint32_t *out_bin,
                         uint32_t *out_below) {
  constexpr int per = kHistBins / 256;
  uint32_t loc[per];
  uint32_t sum = 0;
#pragma unroll
  for (int k = 0; k < per; ++k) {
    loc[k] = h[threadIdx.x * per + k];
    sum += loc[k];
  }
  uint32_t total;
  const uint32_t incl = block_incl_scan256(sum, wsum, total);
  const uint32_t excl = incl - sum;
  if (excl < target && incl >= target) {
    uint32_t run = excl;
#pragma unroll
    for (int k = 0; k < per; ++k) {
      if (run < target && run + loc[k] >= target) {
        *out_bin = threadIdx.x * per + k;
        *out_below = run;
      }
      run += loc[k];
    }
  }
  __syncthreads();
}

// Exact fp64 score <qkv, k> in ascending element order (each product of an
// fp32 and a key element is exact in fp64).
template <int DT>
__device__ __forceinline__ double exact_score(const float *qkv, const void *pool, int64_t row,
                                              int d) {
  double acc = 0.0;
  for (int e0 = 0; e0 < d; e0 += 8) {
    float x[8];
    load8<DT>(pool, row + e0, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fma((double)qkv[e0 + j], (double)x[j], acc);
  }
  return acc;
}

// Record token i as a candidate of composite l; the first composite to claim
// it in this query (epoch) scores it and appends it to the rerank set.
template <int DT>
__device__ __forceinline__ void add_candidate(const Dev &dv, int s, int l, int32_t i,
                                              uint32_t epoch, const float *qkv) {
  const uint32_t pos = atomicAdd(&dv.cand_count[s * dv.L + l], 1u);
  dv.cand[((int64_t)s * dv.L + l) * dv.k0 + pos] = i;
  const uint32_t old = atomicMax(&dv.mark[(int64_t)s * dv.ncap + i], epoch);
  if (old < epoch) {
    const int64_t lc = dv.loc[(int64_t)s * dv.ncap + i];
    const double sc = exact_score<DT>(qkv, dv.pool_k, ((int64_t)s * dv.pcap * dv.p + lc) * dv.d,
                                      dv.d);
    const uint32_t cp = atomicAdd(&dv.c_count[s], 1u);
    const int64_t o = (int64_t)s * dv.L * dv.k0 + cp;
    dv.cs_key[o] = score_rank_key(sc);
    dv.cs_id[o] = i;
  }
}

// ---------------------------------------------------------------- scan

// Query prep of stream s into LDS: q_kv = fp32 mean of the g heads (left
// fold, then times fp32(1/g)); qcode_t = code(<q_kv, u_t[:d]> / |q_kv|) in
// fp64.  Needs zs[kMaxMl + 1].
template <int DT>
__device__ void query_prep(const Dev &dv, int s, const void *q, float *qkv, int32_t *qc,
                           double *zs) {
  const int tid = threadIdx.x, d = dv.d, mL = dv.mL, g = dv.g;
  if (tid < d) {
    const float inv_g = (float)__ddiv_rn(1.0, (double)g);
    float acc = load_elem<DT>(q, (int64_t)s * g * d + tid);
    for (int h = 1; h < g; ++h) acc = __fadd_rn(acc, load_elem<DT>(q, ((int64_t)s * g + h) * d + tid));
    qkv[tid] = __fmul_rn(acc, inv_g);
  }
  __syncthreads();
  if (tid < mL) {
    const double *dir = dv.dirs + (size_t)(tid / kDirChunk) * (d + 1) * kDirChunk + (tid % kDirChunk);
    double z = 0.0;
    for (int e = 0; e < d; ++e) z = fma((double)qkv[e], dir[(size_t)e * kDirChunk], z);
    zs[tid] = z;
  } else if (tid == 255) {
    double a = 0.0;
    for (int e = 0; e < d; ++e) a = fma((double)qkv[e], (double)qkv[e], a);
    zs[kMaxMl] = a;
  }
  __syncthreads();
  if (tid < mL) {
    const double qn = __dsqrt_rn(zs[kMaxMl]);
    const double qb = qn > 0.0 ? __ddiv_rn(zs[tid], qn) : 0.0;
    qc[tid] = to_code(qb);
  }
  __syncthreads();
}

// Grid (blocks, S); each block covers `tpb` tokens.  LDS histogram when
// L <= 8, global atomics otherwise.
template <int DT, bool LDS_HIST>
__global__ __launch_bounds__(256) void k_qscan(Dev dv, int64_t n, const void *q, int tpb) {
  const int s = blockIdx.y;
  const int tid = threadIdx.x;
  const int mL = dv.mL, m = dv.m, L = dv.L;
  __shared__ float qkv[128];
  __shared__ int32_t qc[kMaxMl];
  __shared__ double zs[kMaxMl + 1];
  __shared__ uint32_t hist[LDS_HIST ? 8 * kHistBins : 1];
  if (LDS_HIST)
    for (int x = tid; x < L * kHistBins; x += 256) hist[x] = 0;
  query_prep<DT>(dv, s, q, qkv, qc, zs);
  if (blockIdx.x == 0) {
    if (tid < dv.d) dv.qkv[(int64_t)s * dv.d + tid] = qkv[tid];
    if (tid < mL) dv.qcode[(int64_t)s * mL + tid] = qc[tid];
    if (tid < L) {
      dv.cand_count[s * L + tid] = 0;
      dv.bnd_count[s * L + tid] = 0;
    }
    if (tid == 0) dv.c_count[s] = 0;
  }
  uint32_t *ghist = dv.hist + (int64_t)s * L * kHistBins;
  const int64_t i0 = (int64_t)blockIdx.x * tpb;
  const int64_t i1 = min(i0 + tpb, n);
  const bool vec = (mL & 3) == 0;
  for (int64_t i = i0 + tid; i < i1; i += 256) {
    const int32_t *row = dv.codes + ((int64_t)s * dv.ncap + i) * mL;
    int l = 0, j = 0;
    uint32_t M = 0;
    auto take = [&](int32_t code, int t) {
      const uint32_t dd = absdiff(code, qc[t]);
      M = dd > M ? dd : M;
      if (++j == m) {
        dv.mbuf[((int64_t)s * L + l) * dv.ncap + i] = M;
        if (LDS_HIST)
          atomicAdd(&hist[l * kHistBins + (M >> kHistShift)], 1u);
        else
          atomicAdd(&ghist[l * kHistBins + (M >> kHistShift)], 1u);
        ++l;
        j = 0;
        M = 0;
      }
    };
    if (vec) {
      const int4 *r4 = reinterpret_cast<const int4 *>(row);
      for (int x = 0; x < (mL >> 2); ++x) {
        const int4 v = r4[x];
        take(v.x, 4 * x);
        take(v.y, 4 * x + 1);
        take(v.z, 4 * x + 2);
        take(v.w, 4 * x + 3);
      }
    } else {
      for (int t = 0; t < mL; ++t) take(row[t], t);
    }
  }
  if (LDS_HIST) {
    __syncthreads();
    for (int x = tid; x < L * kHistBins; x += 256) {
      const uint32_t h = hist[x];
      if (h) atomicAdd(&ghist[x], h);
    }
  }
}

// ---------------------------------------------------------------- collect

template <int DT>
__global__ __launch_bounds__(256) void k_qcollect(Dev dv, int64_t n, int tpb, uint32_t epoch) {
  const int s = blockIdx.y;
  const int tid = threadIdx.x;
  const int L = dv.L;
  __shared__ float qkv[128];
  __shared__ uint32_t bstar[kMaxMl];
  __shared__ uint32_t below[kMaxMl];
  __shared__ uint32_t wsum[4];
  if (tid < dv.d) qkv[tid] = dv.qkv[(int64_t)s * dv.d + tid];
  const uint32_t k0e = (uint32_t)min((int64_t)dv.k0, n);
  for (int l = 0; l < L; ++l) {
    if (tid == 0) {
      bstar[l] = 0;
      below[l] = 0;
    }
    __syncthreads();
    if (k0e > 0)
      find_bin(dv.hist + ((int64_t)s * L + l) * kHistBins, k0e, wsum, &bstar[l], &below[l]);
    else if (tid == 0)
      bstar[l] = 0;  // no bin below 0: nothing is a candidate
    __syncthreads();
  }
  if (k0e == 0) return;
  const int64_t i0 = (int64_t)blockIdx.x * tpb;
  const int64_t i1 = min(i0 + tpb, n);
  for (int64_t i = i0 + tid; i < i1; i += 256) {
    for (int l = 0; l < L; ++l) {
      const uint32_t M = dv.mbuf[((int64_t)s * L + l) * dv.ncap + i];
      const uint32_t b = M >> kHistShift;
      if (b < bstar[l]) {
        add_candidate<DT>(dv, s, l, (int32_t)i, epoch, qkv);
      } else if (b == bstar[l]) {
        const uint32_t pos = atomicAdd(&dv.bnd_count[s * L + l], 1u);
        dv.bnd[((int64_t)s * L + l) * dv.ncap + pos] = ((unsigned long long)M << 32) | (uint32_t)i;
      }
    }
  }
}

// ---------------------------------------------------------------- final

// r-th smallest (1-based) of n distinct keys in global memory: eight 8-bit
// MSB-first digit passes.  All 256 threads call; returns the key to all.
__device__ unsigned long long block_select(const unsigned long long *keys, uint32_t n,
                                           uint32_t r, uint32_t *cnt, uint32_t *wsum,
                                           unsigned long long *res, uint32_t *rr) {
  const int tid = threadIdx.x;
  unsigned long long prefix = 0, himask = 0;
  if (tid == 0) *rr = r;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    cnt[tid] = 0;
    __syncthreads();
    for (uint32_t x = tid; x < n; x += 256) {
      const unsigned long long k = keys[x];
      if ((k & himask) == prefix) atomicAdd(&cnt[(k >> shift) & 255ull], 1u);
    }
    __syncthreads();
    const uint32_t c = cnt[tid];
    uint32_t total;
    const uint32_t incl = block_incl_scan256(c, wsum, total);
    const uint32_t want = *rr;
    __syncthreads();
    if (incl - c < want && incl >= want) {
      *res = prefix | ((unsigned long long)tid << shift);
      *rr = want - (incl - c);
    }
    __syncthreads();
    prefix = *res;
    himask |= 0xffull << shift;
    __syncthreads();
  }
  return prefix;
}

template <int DT>
__global__ __launch_bounds__(256) void k_qfinal(Dev dv, int64_t n, uint32_t epoch,
                                                int32_t *page_ids, int32_t *n_pages,
                                                int32_t *topk_ids) {
  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int L = dv.L;
  __shared__ float qkv[128];
  __shared__ uint32_t wsum[4];
  __shared__ uint32_t cnt[256];
  __shared__ uint32_t bstar, below, rr;
  __shared__ unsigned long long res;
  __shared__ unsigned long long skey[kMaxCand];
  __shared__ int32_t sid[kMaxCand];
  __shared__ uint32_t seen[2048];  // page bitmap, up to 65536 pages
  if (tid < dv.d) qkv[tid] = dv.qkv[(int64_t)s * dv.d + tid];
  const uint32_t k0e = (uint32_t)min((int64_t)dv.k0, n);

  // 1. exact selection inside each composite's boundary bin
  for (int l = 0; l < L && k0e > 0; ++l) {
    __syncthreads();
    find_bin(dv.hist + ((int64_t)s * L + l) * kHistBins, k0e, wsum, &bstar, &below);
    const uint32_t need = k0e - below;
    const uint32_t nb = dv.bnd_count[s * L + l];
    const unsigned long long *bk = dv.bnd + ((int64_t)s * L + l) * dv.ncap;
    const unsigned long long thr =
        need >= nb ? ~0ull : block_select(bk, nb, need, cnt, wsum, &res, &rr);
    for (uint32_t x = tid; x < nb; x += 256) {
      const unsigned long long key = bk[x];
      if (key <= thr) add_candidate<DT>(dv, s, l, (int32_t)(key & 0xffffffffull), epoch, qkv);
    }
  }
  __syncthreads();
  // the histogram is cleared for the next query
  for (int x = tid; x < L * kHistBins; x += 256) dv.hist[(int64_t)s * L * kHistBins + x] = 0;
  for (int x = tid; x < 2048; x += 256) seen[x] = 0;
  __threadfence_block();
  __syncthreads();

  // 2. rank the candidates by (score desc, token asc): bitonic sort in LDS
  const uint32_t nC = __atomic_load_n(&dv.c_count[s], __ATOMIC_RELAXED);
  uint32_t npad = 1;
  while (npad < nC) npad <<= 1;
  for (uint32_t x = tid; x < npad; x += 256) {
    if (x < nC) {
      skey[x] = dv.cs_key[(int64_t)s * L * dv.k0 + x];
      sid[x] = dv.cs_id[(int64_t)s * L * dv.k0 + x];
    } else {
      skey[x] = ~0ull;
      sid[x] = 0x7fffffff;
    }
  }
  __syncthreads();
  for (uint32_t kk = 2; kk <= npad; kk <<= 1) {
    for (uint32_t jj = kk >> 1; jj > 0; jj >>= 1) {
      for (uint32_t x = tid; x < npad; x += 256) {
        const uint32_t y = x ^ jj;
        if (y > x) {
          const bool up = (x & kk) == 0;
          const unsigned long long a = skey[x], b = skey[y];
          const int32_t ia = sid[x], ib = sid[y];
          const bool gt = a > b || (a == b && ia > ib);
          if (gt == up) {
            skey[x] = b;
            skey[y] = a;
            sid[x] = ib;
            sid[y] = ia;
          }
        }
      }
      __syncthreads();
    }
  }

  // 3. top-k tokens
  if (topk_ids)
    for (int x = tid; x < dv.k; x += 256)
      topk_ids[(int64_t)s * dv.k + x] = (uint32_t)x < nC ? sid[x] : -1;

  // 4. pages in rank order, each the first time one of its tokens appears
  if (tid < 64) {
    int pbits = 1;
    while ((1ll << pbits) < dv.pcap) ++pbits;
    int nsel = 0;
    const unsigned long long lt = lanemask_lt();
    for (uint32_t x0 = 0; x0 < nC && nsel < dv.P; x0 += 64) {
      const uint32_t x = x0 + lane;
      const bool valid = x < nC;
      const int32_t pg = valid ? dv.loc[(int64_t)s * dv.ncap + sid[x]] / dv.p : 0;
      const bool fresh = valid && ((seen[pg >> 5] >> (pg & 31)) & 1u) == 0u;
      const unsigned long long act = __ballot(fresh);
      const unsigned long long mt = match_bits((uint32_t)pg, pbits, act);
      const bool firstocc = fresh && (mt & lt) == 0ull;
      const unsigned long long fm = __ballot(firstocc);
      const int pos = nsel + popc64(fm & lt);
      if (firstocc && pos < dv.P) {
        page_ids[(int64_t)s * dv.P + pos] = pg;
        atomicOr(&seen[pg >> 5], 1u << (pg & 31));
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
static hipError_t query_impl(const Dev &dv, int64_t n, const void *q, uint32_t epoch,
                             int32_t *page_ids, int32_t *n_pages, int32_t *topk_ids,
                             hipStream_t st, Timer *tm) {
  const int tpb = 1024;
  const unsigned nblk = (unsigned)((n + tpb - 1) / tpb);
  timer_begin(tm, st);
  if (n > 0) {
    if (dv.L <= 8)
      hipLaunchKernelGGL((k_qscan<DT, true>), dim3(nblk, dv.S), dim3(256), 0, st, dv, n, q, tpb);
    else
      hipLaunchKernelGGL((k_qscan<DT, false>), dim3(nblk, dv.S), dim3(256), 0, st, dv, n, q, tpb);
    timer_mark(tm, KID_QSCAN, st);
    hipLaunchKernelGGL(k_qcollect<DT>, dim3(nblk, dv.S), dim3(256), 0, st, dv, n, tpb, epoch);
    timer_mark(tm, KID_QCOLLECT, st);
  } else {
    // empty index: still record the query codes and clear the counters
    hipLaunchKernelGGL((k_qscan<DT, false>), dim3(1, dv.S), dim3(256), 0, st, dv, n, q, tpb);
    timer_mark(tm, KID_QSCAN, st);
  }
  hipLaunchKernelGGL(k_qfinal<DT>, dim3(dv.S), dim3(256), 0, st, dv, n, epoch, page_ids, n_pages,
                     topk_ids);
  timer_mark(tm, KID_QFINAL, st);
  return hipGetLastError();
}

hipError_t launch_query(const Dev &dv, int64_t n, const void *q, uint32_t epoch,
                        int32_t *page_ids, int32_t *n_pages, int32_t *topk_ids,
                        hipStream_t st, Timer *tm) {
  return dv.dtype == 0 ? query_impl<0>(dv, n, q, epoch, page_ids, n_pages, topk_ids, st, tm)
                       : query_impl<1>(dv, n, q, epoch, page_ids, n_pages, topk_ids, st, tm);
}

}  // namespace ice
