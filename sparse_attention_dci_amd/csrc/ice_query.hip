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
//   k_qscan     (ice_scan_dev.h) the query codes (fp32 GQA mean, fp64
//               projection; in a decode step also the new token's insert),
//               then M_i for every token and walk and a histogram of the top
//               11 bits of M_i;
//   k_qcollect  tokens in bins below the k0-th smallest bin b* are
//               candidates, tokens in bin b* are parked with their (M_i, i)
//               key; both kinds are scored exactly (fp64, ascending element
//               order) here, many blocks in parallel; the first block of
//               each stream publishes b* and the count below it;
//   k_qfinal    one 1024-thread block per stream: exact selection inside the
//               boundary bins, the union of the composites (LDS hash), a
//               bucket sort by (score desc, token asc), top-k and the page
//               walk; it leaves a clean histogram for the next query (and
//               k_qfinal_big does the same for unions above kMaxCand).
#include <type_traits>

#include "ice_attn_dev.h"
#include "ice_scan_dev.h"

namespace ice {

// Scan and collect blocks: NT threads, 2 * NT tokens (two 64-token tiles per
// wave).  512 by default; when 512-thread blocks would not all get a CU of
// their own, the smallest of 640, 768 and 1024 that does (the 36,864-token
// layer: 232 blocks of 640 instead of 296 of 512, 52.8 instead of 55.5 us
// per step), since a CU holding two blocks finishes last.
constexpr int kFinalThreads = 1024;
static_assert(kFinalThreads == 1 << 10, "the finaliser splits its threads by shifts");
constexpr int kHashSlots = 8192;    // 2 * kMaxCand
constexpr int kBndLds = 2048;       // boundary entries ranked in LDS
constexpr int kBuckets = 2048;
static_assert(kBuckets == kHistBins, "bucket counts are searched as a histogram");
constexpr int kFusedMaxPages = 1024;
constexpr int kFastPages = 32;  // selections every wave walks for itself, at most
constexpr int kMaxTies = 256;  // page budgets up to this take the fused attention

// ---------------------------------------------------------------- helpers

// Exact fp64 scores of cnt tokens by a block of NT threads, in the blocked
// order (ice_step_dev.h): d/16 lanes score each key row, lane j reading
// elements 16j .. 16j+15 straight from the pool (two bf16 or four fp32
// 16-byte requests, in flight together) and summing them in order; the
// lanes' sums are added pairwise.  slot_of(j) gives token j's page slot.
// emit(j, slot, score) receives each result: with nq query vectors (qkv +
// 128 h, the GQA max mode's heads) the largest of the nq scores.  qkv is
// 16-byte aligned.
template <int DT, int NT, typename SlotOf, typename Emit>
__device__ void block_score(const Dev &dv, int s, uint32_t cnt, SlotOf slot_of, const float *qkv,
                            int nq, Emit emit) {
  const int tid = threadIdx.x;
  const int d = dv.d;
  const int64_t row_bytes = (int64_t)d * dv.elem;
  const char *pool =
      reinterpret_cast<const char *>(dv.pool_k) + (int64_t)s * dv.pcap * dv.p * row_bytes;
  const int nbk = d >> 4, lnb = d == 128 ? 3 : 2;
  constexpr int kReq = DT == 0 ? 4 : 2;  // 16-byte requests per lane
  for (uint32_t x = tid; x < cnt * nbk; x += NT) {  // whole lane groups
    const uint32_t r = x >> lnb;
    const int j = x & (nbk - 1);
    const int32_t slot = slot_of(r);
    const uint4 *rp = reinterpret_cast<const uint4 *>(pool + slot * row_bytes) + j * kReq;
    uint4 u[kReq];
#pragma unroll
    for (int i = 0; i < kReq; ++i) u[i] = rp[i];
    double best = 0.0;
    for (int h = 0; h < nq; ++h) {
      // element order within the block of 16
      const float4 *qp = reinterpret_cast<const float4 *>(qkv + 128 * h + 16 * j);
      double z = 0.0;
      if constexpr (DT == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 f = qp[i];
          z = fma((double)f.x, (double)__uint_as_float(u[i].x), z);
          z = fma((double)f.y, (double)__uint_as_float(u[i].y), z);
          z = fma((double)f.z, (double)__uint_as_float(u[i].z), z);
          z = fma((double)f.w, (double)__uint_as_float(u[i].w), z);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float4 f0 = qp[2 * i], f1 = qp[2 * i + 1];
          z = fma((double)f0.x, (double)__uint_as_float(u[i].x << 16), z);
          z = fma((double)f0.y, (double)__uint_as_float(u[i].x & 0xffff0000u), z);
          z = fma((double)f0.z, (double)__uint_as_float(u[i].y << 16), z);
          z = fma((double)f0.w, (double)__uint_as_float(u[i].y & 0xffff0000u), z);
          z = fma((double)f1.x, (double)__uint_as_float(u[i].z << 16), z);
          z = fma((double)f1.y, (double)__uint_as_float(u[i].z & 0xffff0000u), z);
          z = fma((double)f1.z, (double)__uint_as_float(u[i].w << 16), z);
          z = fma((double)f1.w, (double)__uint_as_float(u[i].w & 0xffff0000u), z);
        }
      }
      z = tree_sum(z, nbk);
      best = h == 0 ? z : fmax(best, z);
    }
    if (j == 0) emit(r, slot, best);
  }
}

// ---------------------------------------------------------------- collect

// Blocks of kScanTpb tokens, mapped to streams as in the scan.  Token i is a
// candidate of composite l when its bin is below the k0-th smallest bin b*,
// a boundary entry when its bin is b*.  Every candidate or boundary token of
// the block is scored once; the below-bin ones go to the stream's rerank
// list, the boundary entries carry their score and page to the final
// selection and are also counted in a second-level histogram of bin b* (the
// next 11 bits of M), which lets the finaliser resolve the boundary without
// ranking it.  Appends take one device atomic per block and list, issued
// before the scoring and consumed after it.
constexpr int kSubShift = kHistShift - kHistBits;  // second-level bins: M >> 9 & 2047

// Two shapes: 640-thread blocks (one per CU) have the registers of four
// waves per SIMD; 512-thread blocks (many per CU, the long contexts) those of
// six, so three blocks fit a CU and more of their latency chains overlap.
template <int NT>
struct CollectShape {
  static constexpr int kWavesPerEu = NT == 512 ? 6 : 4;
};

//
// A block serves every walk of its stream: the L composites, or in the GQA
// max mode the g * L (head, composite) walks, head h's walks h * L + l.  A
// token below or at the threshold in several walks is scored once, against
// all g heads in the max mode (read from q, ranked by the largest score),
// and enters the rerank list once.  WIDE (more than 8 walks) keeps M of 16
// walks per token in registers instead of 8.
template <int DT, int NT, bool WIDE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(CollectShape<NT>::kWavesPerEu))) void k_qcollect(
    Dev dv, int64_t n, bool bounded, const void *q) {
  constexpr int kScanThreads = NT, kScanTpb = 2 * NT;
  constexpr int kMw = WIDE ? 16 : 8;  // walks whose M a thread holds in registers
  // grid (S, ranges)
  const int s = (int)blockIdx.x;
  const int64_t rng = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int Lq = dv.Lq, nw = Lq;  // the block's walks: all Lq of the stream
  const int nq = dv.gmax ? dv.g : 1;  // query vectors a candidate is scored against
  __shared__ int32_t bstar[32];  // -1: the composite takes no candidates
  __shared__ uint32_t ccount[32], bcount[32], cbase[32], bbase[32];
  __shared__ uint32_t nc, nrl, rbase;
  // [nq][128] query vectors: dynamic LDS sized at launch (nq * 512 bytes), so
  // the mean mode does not reserve the max mode's 8 KB
  extern __shared__ __attribute__((aligned(16))) float qkv[];
  // the 512-thread shape keeps a token's classification in LDS over the
  // scoring (its 80 registers would spill it to scratch memory)
  constexpr int kKeep = NT == 512 ? 2 * NT : 1;
  __shared__ uint32_t kbelow[kKeep], kbnd[kKeep];
  __shared__ int16_t kslot[kKeep];
  __shared__ int32_t cid[kScanTpb];      // candidate or boundary tokens, as offsets in the block
  __shared__ int32_t lloc[kScanTpb];     // page slots of the block's tokens
  __shared__ unsigned long long skb[kScanTpb];
  __shared__ int32_t spb[kScanTpb];
  const uint32_t k0e = (uint32_t)min((int64_t)dv.k0, n);
  const int64_t i0 = rng * kScanTpb;
  const int64_t i1 = min(i0 + kScanTpb, n);
  const int64_t ii[2] = {i0 + tid, i0 + kScanThreads + tid};
  const bool vv[2] = {ii[0] < i1, ii[1] < i1};

  // 1. loads: the low bins of wave w's threshold histogram first (distances
  // are far below the code range, so the threshold bin is almost always among
  // them; the whole histogram is read when it is not), M of both tokens for
  // the first kMw walks, their page slots, the query (unconditional loads
  // at clamped addresses)
  uint4 hlow = make_uint4(0u, 0u, 0u, 0u);
  uint32_t klw = k0e;
  if (w < nw) {
    hlow = wave_hist_load_low(dv.hist + ((int64_t)s * Lq + w) * kHistBins);
    if (bounded) klw = min(k0e, dv.vcount[s * Lq + w]);
  }
  uint32_t Mv[2][kMw];
  int32_t lc[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t ic = vv[u] ? ii[u] : 0;
#pragma unroll
    for (int l = 0; l < kMw; ++l)
      Mv[u][l] = l < nw ? dv.mbuf[((int64_t)s * Lq + l) * dv.ncap + ic] : 0u;
    lc[u] = dv.loc[(int64_t)s * dv.ncap + ic];
  }
  auto Mof = [&](int u, int l) -> uint32_t {
    uint32_t M = 0;
    if (l < kMw) {
#pragma unroll
      for (int x = 0; x < kMw; ++x)
        if (x == l) M = Mv[u][x];
    } else {
      M = dv.mbuf[((int64_t)s * Lq + l) * dv.ncap + (vv[u] ? ii[u] : 0)];
    }
    return M;
  };
  // the query vectors: q_kv (mean mode), or the g heads as fp32 (max mode)
  float qk[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int x = min(tid + kScanThreads * u, nq * dv.d - 1);
    qk[u] = dv.gmax ? load_elem<DT>(q, (int64_t)s * dv.g * dv.d + x) : dv.qkv[(int64_t)s * dv.d + x];
  }
  if (k0e == 0) return;  // after the loads: the kernel arguments arrive in one round
  for (int l = w; l < nw; l += kScanThreads / 64) {
    const uint32_t *hl = dv.hist + ((int64_t)s * Lq + l) * kHistBins;
    uint32_t kl = klw;
    if (l != w) {  // more composites than waves
      kl = bounded ? min(k0e, dv.vcount[s * Lq + l]) : k0e;
      hlow = wave_hist_load_low(hl);
    }
    uint32_t bb = 0, bl = 0;
    if (kl > 0 && !wave_find_bin_low(hlow, kl, bb, bl)) wave_find_bin_seq(hl, kl, bb, bl);
    if (lane == 0) {
      bstar[l] = kl > 0 ? (int32_t)bb : -1;
      if (rng == 0) {  // for the finaliser: b* and the count below it
        dv.bsel[((int64_t)s * Lq + l) * 2] = bb;
        dv.bsel[((int64_t)s * Lq + l) * 2 + 1] = bl;
      }
    }
  }
  const int ld = dv.d == 128 ? 7 : 6;  // d is 64 or 128
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int x = tid + kScanThreads * u;
    if (x < nq * dv.d) qkv[((x >> ld) << 7) + (x & (dv.d - 1))] = qk[u];
  }
  for (int x = tid + 2 * kScanThreads; x < nq * dv.d; x += kScanThreads)  // g * d > 2 * NT
    qkv[((x >> ld) << 7) + (x & (dv.d - 1))] =
        load_elem<DT>(q, (int64_t)s * dv.g * dv.d + x);
  lloc[tid] = lc[0];
  lloc[kScanThreads + tid] = lc[1];
  if (tid < nw) {
    ccount[tid] = 0;
    bcount[tid] = 0;
  }
  if (tid == 0) {
    nc = 0;
    nrl = 0;
  }
  __syncthreads();

  // 2. classify
  uint32_t below[2], bnd[2];
  int slot[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    below[u] = 0;
    bnd[u] = 0;
    slot[u] = -1;
    if (vv[u]) {
      auto classify = [&](int l, uint32_t M) {
        const int32_t bb = (int32_t)(M >> kHistShift);
        if (bb < bstar[l]) below[u] |= 1u << l;
        if (bb == bstar[l]) {
          bnd[u] |= 1u << l;
          atomicAdd(&dv.hist2[((int64_t)s * Lq + l) * kHistBins +
                              ((M >> kSubShift) & (kHistBins - 1))],
                    1u);
        }
      };
      if constexpr (WIDE) {  // registers by constant index; walks past 16 from memory
#pragma unroll
        for (int l = 0; l < kMw; ++l)
          if (l < nw) classify(l, Mv[u][l]);
        for (int l = kMw; l < nw; ++l)
          classify(l, dv.mbuf[((int64_t)s * Lq + l) * dv.ncap + ii[u]]);
      } else {
        for (int l = 0; l < nw; ++l) classify(l, Mof(u, l));
      }
    }
    if (below[u] | bnd[u]) {  // sparse: a few lanes per block
      slot[u] = (int)atomicAdd(&nc, 1u);
      cid[slot[u]] = (int32_t)(ii[u] - i0);
      if (below[u]) atomicAdd(&nrl, 1u);
      for (int l = 0; l < nw; ++l) {
        if ((below[u] >> l) & 1u) atomicAdd(&ccount[l], 1u);
        if ((bnd[u] >> l) & 1u) atomicAdd(&bcount[l], 1u);
      }
    }
  }
  lds_barrier();

  // 3. one device atomic per list for the block, consumed after the scoring
  uint32_t my_c = 0, my_b = 0, my_r = 0;
  if (tid < nw) {
    my_c = ccount[tid] ? atomicAdd(&dv.cand_count[s * Lq + tid], ccount[tid]) : 0u;
    my_b = bcount[tid] ? atomicAdd(&dv.bnd_count[s * Lq + tid], bcount[tid]) : 0u;
  }
  if (tid == 64) my_r = nrl ? atomicAdd(&dv.rr_count[s], nrl) : 0u;

  // 4. exact scores of the block's candidate and boundary tokens
  const int lp = dv.lp;  // pages are 2^lp slots
  unsigned long long *skbp = skb;
  int32_t *spbp = spb;
  const int32_t *cidp = cid, *llocp = lloc;
  if constexpr (NT == 512) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      kbelow[tid + NT * u] = below[u];
      kbnd[tid + NT * u] = bnd[u];
      kslot[tid + NT * u] = (int16_t)slot[u];
    }
  }
  block_score<DT, kScanThreads>(
      dv, s, nc, [cidp, llocp](uint32_t j) { return llocp[cidp[j]]; }, qkv, nq,
      [skbp, spbp, lp](uint32_t x, int32_t slotx, double sc) {
        skbp[x] = score_rank_key(sc);
        spbp[x] = slotx >> lp;
      });
  if constexpr (NT == 512) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      below[u] = kbelow[tid + NT * u];
      bnd[u] = kbnd[tid + NT * u];
      slot[u] = kslot[tid + NT * u];
    }
  }

  // 5. the appends
  if (tid < nw) {
    cbase[tid] = my_c;
    bbase[tid] = my_b;
    ccount[tid] = 0;
    bcount[tid] = 0;
  }
  if (tid == 64) {
    rbase = my_r;
    nrl = 0;
  }
  lds_barrier();
  const int64_t rr0 = (int64_t)s * Lq * dv.k0;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (slot[u] < 0) continue;
    const int64_t iu = i0 + tid + (int64_t)kScanThreads * u;  // ii[u], recomputed
    const int32_t i = (int32_t)iu;
    const unsigned long long rk = skb[slot[u]];
    const int32_t pg = spb[slot[u]];
    if (below[u]) {
      const int64_t o = rr0 + rbase + atomicAdd(&nrl, 1u);
      dv.rr_key[o] = rk;
      dv.rr_id[o] = i;
      dv.rr_pg[o] = pg;
    }
    for (int l = 0; l < nw; ++l) {
      if ((below[u] >> l) & 1u)
        dv.cand[((int64_t)s * Lq + l) * dv.k0 + cbase[l] + atomicAdd(&ccount[l], 1u)] = i;
      if ((bnd[u] >> l) & 1u) {
        const int64_t o = ((int64_t)s * Lq + l) * dv.ncap + bbase[l] + atomicAdd(&bcount[l], 1u);
        // the 512-thread shape (80 registers) reads M again (L2-hot) rather
        // than keep its registers over the scoring, which would spill them
        uint32_t Mx;
        if constexpr (NT == 512)
          Mx = dv.mbuf[((int64_t)s * Lq + l) * dv.ncap + iu];
        else
          Mx = Mof(u, l);
        dv.bnd[o] = ((unsigned long long)Mx << 32) | (uint32_t)i;
        dv.bnd_rk[o] = rk;
        dv.bnd_pg[o] = pg;
      }
    }
  }
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

// Inserts id into an LDS hash set of 2^BITS slots (linear probing); true when
// it was not there yet.
template <int BITS = 13>
__device__ __forceinline__ bool hash_insert(uint32_t *tab, int32_t id) {
  const uint32_t key = (uint32_t)id + 1u;
  uint32_t h = (key * 2654435761u) >> (32 - BITS);
  for (;;) {
    const uint32_t old = atomicCAS(&tab[h], 0u, key);
    if (old == 0u) return true;
    if (old == key) return false;
    h = (h + 1u) & ((1u << BITS) - 1u);
  }
}

__device__ __forceinline__ bool key_less(unsigned long long ka, int32_t ia, unsigned long long kb,
                                         int32_t ib) {
  return ka < kb || (ka == kb && ia < ib);
}

// Score back from its rank key (the inverse of score_rank_key).
__device__ __forceinline__ double rank_key_score(unsigned long long key) {
  const unsigned long long ord = ~key;
  const unsigned long long b = (ord >> 63) ? (ord & 0x7fffffffffffffffull) : ~ord;
  return __longlong_as_double((long long)b);
}

// The finaliser's part of the query statistics: per composite, the visit
// count's start (0 when the walk completed its k0-th candidate, whose key the
// count pass then ranks among all entries; else every entry the walk may
// visit, vlimit) and that key; the union size and the pages selected.
__device__ __forceinline__ void final_stats(const Dev &dv, int s, int64_t n, uint32_t k0e,
                                            const uint32_t *cc, const uint32_t *extra,
                                            const unsigned long long *klast, uint32_t nu,
                                            uint32_t nsel, ice_query_stats *stats,
                                            unsigned long long vlimit) {
  const int tid = threadIdx.x, L = dv.Lq;
  if (tid < L) {
    const uint32_t kl = k0e > 0 ? cc[tid] + extra[tid] : 0u;
    const bool full = n > 0 && kl == (uint32_t)dv.k0;
    stats[s].visits[tid] = full ? 0 : (n > 0 ? (long long)vlimit : 0);
    dv.vlast[(int64_t)s * L + tid] = full ? klast[tid] : ~0ull;
  }
  if (tid == 0) {
    stats[s].n_cand = (int32_t)nu;
    stats[s].n_pages = (int32_t)nsel;
    stats[s].n_tokens = 0;
    stats[s].reserved = 0;
  }
}

struct FinalShared {
  unsigned long long skey[kMaxCand];  // the rerank list: rank key, token, page
  int32_t sid[kMaxCand];
  int32_t spg[kMaxCand];
  union {
    struct {  // boundary entries (selection phase)
      unsigned long long bk[kBndLds];
      unsigned long long brk[kBndLds];
      int32_t bpg[kBndLds];
    };
    struct {  // bucket sort (sort phase): keys and list positions in bucket order
      unsigned long long tk[kMaxCand];
      int32_t tx[kMaxCand];
    };
  };
  union {
    uint32_t hash[kHashSlots];  // rerank-list membership (selection phase)
    struct __attribute__((aligned(16))) {
      uint32_t bcnt[kBuckets];
      uint32_t bstart[kBuckets];
      uint32_t seen[2048];  // selected pages (page walk)
    };
  };
  uint32_t cnt[256];
  uint32_t cc[32], nb[32], need[32], boff[33], extra[32], b2[32], need2[32];
  unsigned long long klast[32];  // largest (M, token) key picked per composite (statistics)
  uint32_t tie[kMaxTies];  // boundary entries in their composite's second-level bin b2
  uint32_t ntie;
  uint32_t nu;
  uint32_t rr;
  unsigned long long res;
  unsigned long long wlo[16], whi[16];
  uint32_t wsum[16];
  int32_t sel[kFusedMaxPages];  // the selected pages, for the fused attention
  int32_t nsel;
  float wm[16 * 16], wl[16 * 16];
  // past the wave outputs of the fused attention (which overwrite the rank
  // arrays): the pages of the first 64 ranks, and each wave's own copy of the
  // selection when those ranks hold all of it
  int32_t top_pg[64];
  int32_t wsel[16 * kFastPages];
};

// PER = union elements per thread (L * k0 <= PER * kFinalThreads): 1 when the
// union holds at most 1,024 tokens, which keeps the per-element loops (and the
// code the block has to fetch: most of this kernel's time is instruction
// fetch on a cold cache) a quarter of the size.
template <int DT, int D, int PER>
__global__ __launch_bounds__(kFinalThreads) void k_qfinal(Dev dv, int64_t n, bool bounded,
                                                          int32_t *page_ids, int32_t *n_pages,
                                                          int32_t *topk_ids, const void *q,
                                                          float *out, ice_query_stats *stats,
                                                          unsigned long long vlimit) {
  __shared__ FinalShared sh;
  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int L = dv.Lq, k0 = dv.k0;  // the query's walks
  const uint32_t k0e = (uint32_t)min((int64_t)k0, n);

  // A. loads, all issued before any is used (one round trip): the
  // second-level histogram of wave w's composite and the count below its
  // threshold bin b* (the collect pass found b*), the counts; thread tid also
  // owns boundary entry ep of composite lp (for the prefetch below)
  uint32_t h2[kBinsPerLane], bl_ld = 0;  // second-level histogram; count below b*
  if (w < L) {  // wave w's composite
    wave_hist_load(dv.hist2 + ((int64_t)s * L + w) * kHistBins, h2);
    bl_ld = dv.bsel[((int64_t)s * L + w) * 2 + 1];
  }
  const uint32_t kl_ld = bounded && w < L ? dv.vcount[s * L + w] : k0e;
  const uint32_t nrr_ld = dv.rr_count[s];
  // boundary entries prefetched per composite: kFinalThreads / 2^ceil(log2 L),
  // so a thread's composite and entry come by shifts
  const int lgl = L > 1 ? 32 - __builtin_clz((uint32_t)(L - 1)) : 0;
  const int per = kFinalThreads >> lgl;
  const int lp = min(tid >> (10 - lgl), L - 1);
  const uint32_t ep = (uint32_t)(tid - lp * per);
  const uint32_t nbp = dv.bnd_count[s * L + lp];
  uint32_t cc_ld = 0, nb_ld = 0;
  if (tid < L) {
    cc_ld = dv.cand_count[s * L + tid];
    nb_ld = dv.bnd_count[s * L + tid];
  }
  // the rerank list and this thread's boundary entry: their addresses depend
  // on nothing loaded (clamped into the arrays; the counts decide later which
  // values are used), so they are in flight with the histogram, and stay in
  // flight across the barriers up to the attention (which order LDS only)
  constexpr int kPer = PER;
  int32_t pid[kPer], ppg[kPer];
  unsigned long long pkey[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint32_t x = tid + kFinalThreads * j;
    const int64_t o = (int64_t)s * L * k0 + min(x, (uint32_t)(L * k0 - 1));
    pid[j] = dv.rr_id[o];
    pkey[j] = dv.rr_key[o];
    ppg[j] = dv.rr_pg[o];
  }
  const int64_t po = ((int64_t)s * L + lp) * dv.ncap + min((int64_t)ep, dv.ncap - 1);
  const unsigned long long pbk = dv.bnd[po], pbrk = dv.bnd_rk[po];
  const int32_t pbpg = dv.bnd_pg[po];
  // union membership: a bitmap over the tokens when they fit the table (one
  // atomic test-and-set per token), else the LDS hash
  const bool bitmap = n <= (int64_t)32 * kHashSlots;
  const int hwords = bitmap ? (int)((n + 31) >> 5) : kHashSlots;
  for (int x = tid; x < hwords; x += kFinalThreads) sh.hash[x] = 0;
  auto mark = [&](int32_t id) -> bool {  // true when id was not in the union yet
    if (bitmap) {
      const uint32_t bit = 1u << (id & 31);
      return (atomicOr(&sh.hash[id >> 5], bit) & bit) == 0u;
    }
    return hash_insert(sh.hash, id);
  };
  if (tid < L) {
    sh.cc[tid] = cc_ld;
    sh.nb[tid] = nb_ld;
    sh.extra[tid] = 0;
    sh.klast[tid] = 0;
  }
  {  // need, b2, need2 of composite l come from wave l alone (all zero when it takes no
     // candidates: k0e = 0, or a bounded walk that completes no token)
    for (int l = w; l < L; l += kFinalThreads / 64) {
      uint32_t b2, bl2;
      if (l != w)  // more composites than waves
        wave_hist_load(dv.hist2 + ((int64_t)s * L + l) * kHistBins, h2);
      const uint32_t kl = min(k0e, l == w ? kl_ld : (bounded ? dv.vcount[s * L + l] : k0e));
      uint32_t need = 0, need2 = 0;  // picks from the boundary bin (>= 1 when kl > 0) and
      b2 = 0;                        // from its second-level bin b2
      if (kl > 0) {  // the first-level bin b* and the count below it come from the collect pass
        const uint32_t bl = l == w ? bl_ld : dv.bsel[((int64_t)s * L + l) * 2 + 1];
        need = kl - bl;
        wave_find_bin_regs(h2, need, b2, bl2);
        need2 = need - bl2;
      }
      if (lane == 0) {
        sh.need[l] = need;
        sh.b2[l] = b2;
        sh.need2[l] = need2;
      }
    }
  }
  const uint32_t nrr = k0e > 0 ? nrr_ld : 0u;
  const bool pv = tid < L * per && ep < nbp && k0e > 0;
  if (w == 0) {  // the composites' boundary offsets: a prefix of the counts (lanes < L hold them)
    const uint32_t v = k0e > 0 ? nb_ld : 0u;
    const uint32_t incl = wave_incl_scan(v);
    if (lane <= L) sh.boff[lane] = incl - v;
    if (lane == 0) {
      sh.nu = nrr;
      sh.ntie = 0;
    }
  }
  lds_barrier();
  u32x4 qh[D / 32], ql[D / 32];  // needed by the attention only: in flight meanwhile
  attn_load_q<DT, D>(dv, s, q, qh, ql);
  const uint32_t nbt = sh.boff[L];
  const bool bnd_lds = nbt <= (uint32_t)kBndLds;

  // B. the scored below-bin candidates and, when they fit, the boundary
  // entries (a composite's entries past the prefetched ones are loaded here)
  // the rerank list holds every token once: the collect block that holds a
  // token appends it once, in however many walks it is a candidate (the GQA
  // max mode's g * L walks included)
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint32_t x = tid + kFinalThreads * j;
    if (x < nrr) {
      mark(pid[j]);
      sh.sid[x] = pid[j];
      sh.skey[x] = pkey[j];
      sh.spg[x] = ppg[j];
    }
  }
  if (bnd_lds) {
    if (pv) {
      const uint32_t x = sh.boff[lp] + ep;
      sh.bk[x] = pbk;
      sh.brk[x] = pbrk;
      sh.bpg[x] = pbpg;
    }
    for (uint32_t x = tid; x < nbt; x += kFinalThreads) {
      int l = 0;
      while (x >= sh.boff[l + 1]) ++l;
      if (x - sh.boff[l] < (uint32_t)per) continue;
      const int64_t o = ((int64_t)s * L + l) * dv.ncap + (x - sh.boff[l]);
      sh.bk[x] = dv.bnd[o];
      sh.brk[x] = dv.bnd_rk[o];
      sh.bpg[x] = dv.bnd_pg[o];
    }
  }
  {  // a clean histogram for the next query: every read of it is done, and
     // the stores drain while the rest runs (no later barrier waits for them)
    uint4 *hist = reinterpret_cast<uint4 *>(dv.hist + (int64_t)s * L * kHistBins);
    uint4 *hist2 = reinterpret_cast<uint4 *>(dv.hist2 + (int64_t)s * L * kHistBins);
    for (int x = tid; x < L * kHistBins / 4; x += kFinalThreads) {  // 16-byte stores
      hist[x] = make_uint4(0u, 0u, 0u, 0u);
      hist2[x] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  lds_barrier();

  // C. the need_l smallest (M, i) of each composite's boundary bin join the
  // composite's candidates, and the union when not in it yet: every entry in
  // a second-level bin below b2_l, and the need2_l smallest of bin b2_l
  auto add_pick = [&](int l, unsigned long long key, unsigned long long rk, int32_t pg) {
    const int32_t id = (int32_t)(key & 0xffffffffull);
    dv.cand[((int64_t)s * L + l) * k0 + sh.cc[l] + atomicAdd(&sh.extra[l], 1u)] = id;
    if (stats != nullptr) atomicMax(&sh.klast[l], key);
    if (mark(id)) {
      const uint32_t pos = atomicAdd(&sh.nu, 1u);
      sh.sid[pos] = id;
      sh.skey[pos] = rk;
      sh.spg[pos] = pg;
    }
  };
  auto sub_of = [](unsigned long long key) -> uint32_t {
    return (uint32_t)(key >> (32 + kSubShift)) & (kHistBins - 1);
  };
  if (nbt > 0) {
    if (bnd_lds) {
      // entries below second-level bin b2_l are picked outright; the few in
      // bin b2_l go to a tie list and are ranked among themselves
      for (uint32_t x = tid; x < nbt; x += kFinalThreads) {
        int l = 0;
        while (x >= sh.boff[l + 1]) ++l;
        const unsigned long long key = sh.bk[x];
        const uint32_t sb = sub_of(key);
        if (sb < sh.b2[l]) add_pick(l, key, sh.brk[x], sh.bpg[x]);
        if (sb == sh.b2[l]) {
          const uint32_t t = atomicAdd(&sh.ntie, 1u);
          if (t < kMaxTies) sh.tie[t] = x;
        }
      }
      lds_barrier();
      const uint32_t nt = sh.ntie;
      if (nt <= (uint32_t)kMaxTies) {
        for (uint32_t t = tid; t < nt; t += kFinalThreads) {
          const uint32_t x = sh.tie[t];
          int l = 0;
          while (x >= sh.boff[l + 1]) ++l;
          const unsigned long long key = sh.bk[x];
          uint32_t rank = 0;
          for (uint32_t u = 0; u < nt; ++u) {
            const uint32_t y = sh.tie[u];
            rank += (y >= sh.boff[l]) & (y < sh.boff[l + 1]) & (sh.bk[y] < key);
          }
          if (rank < sh.need2[l]) add_pick(l, key, sh.brk[x], sh.bpg[x]);
        }
      } else {  // many equal second-level bins: rank tied entries over their composite
        for (uint32_t x = tid; x < nbt; x += kFinalThreads) {
          int l = 0;
          while (x >= sh.boff[l + 1]) ++l;
          const unsigned long long key = sh.bk[x];
          if (sub_of(key) != sh.b2[l]) continue;
          uint32_t rank = 0;
          for (uint32_t y = sh.boff[l]; y < sh.boff[l + 1]; ++y)
            rank += (sub_of(sh.bk[y]) == sh.b2[l]) & (sh.bk[y] < key);
          if (rank < sh.need2[l]) add_pick(l, key, sh.brk[x], sh.bpg[x]);
        }
      }
    } else {
      for (int l = 0; l < L; ++l) {
        const int64_t o0 = ((int64_t)s * L + l) * dv.ncap;
        const unsigned long long *bk = dv.bnd + o0;
        const uint32_t nbl = sh.nb[l], nd = sh.need[l];
        const unsigned long long thr =
            nd >= nbl ? ~0ull : block_select(bk, nbl, nd, sh.cnt, &sh.res, &sh.rr);
        for (uint32_t x = tid; x < nbl; x += kFinalThreads) {
          const unsigned long long key = bk[x];
          if (key <= thr) add_pick(l, key, dv.bnd_rk[o0 + x], dv.bnd_pg[o0 + x]);
        }
        __syncthreads();
      }
    }
  }
  lds_barrier();
  const uint32_t nu = sh.nu;

  // D. bucket sort by (rank key, token).  Bucket = floor((s_max - score) *
  // (kBuckets-1) / (s_max - s_min)) never decreases along ascending keys, so
  // an element's rank is its bucket's start plus the number of smaller
  // elements inside its bucket.  The count's atomic hands every element its
  // slot inside the bucket; the sorted list ends up rank-ordered (token,
  // page) over the dead key array.
  int32_t* const rsid = reinterpret_cast<int32_t *>(&sh.skey[0]);
  int32_t* const rspg = rsid + kMaxCand;
  {
    constexpr int kPer = PER;
    unsigned long long kx[kPer];
    int32_t ix[kPer], px[kPer];
    uint32_t bkt[kPer], within[kPer], rnk[kPer];
    unsigned long long lo = ~0ull, hi = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t x = tid + kFinalThreads * j;
      kx[j] = ~0ull;
      ix[j] = 0;
      px[j] = 0;
      if (x < nu) {  // whole waves past nu skip
        kx[j] = sh.skey[x];
        ix[j] = sh.sid[x];
        px[j] = sh.spg[x];
        lo = min(lo, kx[j]);
        hi = max(hi, kx[j]);
      }
    }
    lo = wave_minmax_u64<false>(lo);
    hi = wave_minmax_u64<true>(hi);
    if (lane == 0) {
      sh.wlo[w] = lo;
      sh.whi[w] = hi;
    }
    for (int x = tid; x < kBuckets; x += kFinalThreads) sh.bcnt[x] = 0;
    lds_barrier();
    lo = ~0ull;
    hi = 0;
#pragma unroll
    for (int k = 0; k < kFinalThreads / 64; ++k) {
      lo = min(lo, sh.wlo[k]);
      hi = max(hi, sh.whi[k]);
    }
    const double smax = nu ? rank_key_score(lo) : 0.0;
    const double smin = nu ? rank_key_score(hi) : 0.0;
    const double scale = smax > smin ? (double)(kBuckets - 1) / (smax - smin) : 0.0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      bkt[j] = 0;
      within[j] = 0;
      if (tid + kFinalThreads * j < nu) {
        const double t = (smax - rank_key_score(kx[j])) * scale;
        bkt[j] = (uint32_t)min((double)(kBuckets - 1), t);
        within[j] = atomicAdd(&sh.bcnt[bkt[j]], 1u);
      }
    }
    lds_barrier();
    {  // exclusive scan of the bucket counts, two per thread
      const uint32_t c0 = sh.bcnt[2 * tid], c1 = sh.bcnt[2 * tid + 1];
      const uint32_t incl = wave_incl_scan(c0 + c1);
      if (lane == 63) sh.wsum[w] = incl;
      lds_barrier();
      uint32_t pre = 0;
      for (int k = 0; k < w; ++k) pre += sh.wsum[k];
      const uint32_t excl = pre + incl - (c0 + c1);
      sh.bstart[2 * tid] = excl;
      sh.bstart[2 * tid + 1] = excl + c0;
    }
    lds_barrier();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t x = tid + kFinalThreads * j;
      if (x < nu) {
        const uint32_t pos = sh.bstart[bkt[j]] + within[j];
        sh.tk[pos] = kx[j];
        sh.tx[pos] = (int32_t)x;
      }
    }
    lds_barrier();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t x = tid + kFinalThreads * j;
      rnk[j] = 0;
      if (x < nu) {
        const uint32_t b0 = sh.bstart[bkt[j]], b1 = b0 + sh.bcnt[bkt[j]];
        uint32_t r = b0, eq = 0;
        for (uint32_t y = b0; y < b1; ++y) {
          const unsigned long long ky = sh.tk[y];
          r += ky < kx[j];
          eq += ky == kx[j];
        }
        if (eq > 1)  // equal keys (rare): order them by token
          for (uint32_t y = b0; y < b1; ++y)
            r += sh.tk[y] == kx[j] && sh.sid[sh.tx[y]] < ix[j];
        rnk[j] = r;
      }
    }
    lds_barrier();  // every read of the key arrays is done
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (tid + kFinalThreads * j < nu) {
        rsid[rnk[j]] = ix[j];
        rspg[rnk[j]] = px[j];
        if (rnk[j] < 64u) sh.top_pg[rnk[j]] = px[j];
      }
    }
    for (int x = tid; x < 2048; x += kFinalThreads) sh.seen[x] = 0;
    lds_barrier();
  }

  // E. top-k tokens, then pages in rank order
  if (topk_ids)
    for (int x = tid; x < dv.k; x += kFinalThreads)
      topk_ids[(int64_t)s * dv.k + x] = (uint32_t)x < nu ? rsid[x] : -1;
  if (w == 0) {
    int pbits = 1;
    while ((1ll << pbits) < dv.pcap) ++pbits;
    int nsel = 0;
    const unsigned long long lt = lanemask_lt();
    for (uint32_t x0 = 0; x0 < nu && nsel < dv.P; x0 += 64) {
      const uint32_t x = x0 + lane;
      const bool valid = x < nu;
      const int32_t pg = valid ? (x0 == 0 ? sh.top_pg[x] : rspg[x]) : 0;
      const bool fresh = valid && ((sh.seen[pg >> 5] >> (pg & 31)) & 1u) == 0u;
      const unsigned long long act = __ballot(fresh);
      const unsigned long long mt = match_bits((uint32_t)pg, pbits, act);
      const bool firstocc = fresh && (mt & lt) == 0ull;
      const unsigned long long fm = __ballot(firstocc);
      const int pos = nsel + popc64(fm & lt);
      if (firstocc && pos < dv.P) {
        page_ids[(int64_t)s * dv.P + pos] = pg;
        if (pos < kFusedMaxPages) sh.sel[pos] = pg;
        atomicOr(&sh.seen[pg >> 5], 1u << (pg & 31));
      }
      nsel = min(dv.P, nsel + popc64(fm));
      __builtin_amdgcn_wave_barrier();
    }
    for (int x = nsel + lane; x < dv.P; x += 64) page_ids[(int64_t)s * dv.P + x] = -1;
    if (lane == 0) {
      n_pages[s] = nsel;
      sh.nsel = nsel;
    }
  }
  // F. the candidate counts, for inspection, and the statistics
  if (tid < L && k0e > 0) dv.cand_count[s * L + tid] = sh.cc[tid] + sh.extra[tid];
  if (stats != nullptr) {
    lds_barrier();  // the page walk's count
    final_stats(dv, s, n, k0e, sh.cc, sh.extra, sh.klast, nu, sh.nsel, stats, vlimit);
  }
  if (out == nullptr) return;

  // G. the fused sparse attention over the selected pages: 16 waves, one
  // 16-token chunk at a time each (keys and values requested together),
  // merged at the end (LDS of the dead selection arrays holds the wave
  // outputs)
  constexpr int NW = kFinalThreads / 64;
  static_assert(sizeof(FinalShared) >= (size_t)NW * kMaxGroup * D * 4 + 0, "wave outputs fit");
  static_assert(offsetof(FinalShared, sel) >= (size_t)NW * kMaxGroup * D * 4,
                "the wave outputs leave the selection, its copies and the top ranks' pages");
  AttnWave<D> st;
  attn_init(st);
  // When the first 64 ranks hold the whole selection (and no top-k is
  // written, whose reads of the rank arrays the wave outputs would race),
  // every wave walks them for itself, as wave 0 did, and starts its chunk at
  // once; else all wait for wave 0's walk.
  int np;
  const int32_t *selp;
  bool fast = topk_ids == nullptr && dv.P <= kFastPages;
  {
    int pbits = 1;
    while ((1ll << pbits) < dv.pcap) ++pbits;
    const bool valid = (uint32_t)lane < nu;
    const int32_t pg = valid ? sh.top_pg[lane] : 0;
    const unsigned long long act = __ballot(valid);
    const unsigned long long mt = match_bits((uint32_t)pg, pbits, act);
    const unsigned long long lt = lanemask_lt();
    const bool firstocc = valid && (mt & lt) == 0ull;
    const unsigned long long fm = __ballot(firstocc);
    const int nf = popc64(fm);
    fast = fast && (nf >= dv.P || nu <= 64u);
    np = min(dv.P, nf);
    selp = sh.wsel + w * kFastPages;
    const int pos = popc64(fm & lt);
    if (fast && firstocc && pos < dv.P) sh.wsel[w * kFastPages + pos] = pg;
    __builtin_amdgcn_wave_barrier();
  }
  if (!fast) {  // uniform: every wave decides on the same ranks
    lds_barrier();
    np = sh.nsel;
    selp = sh.sel;
  }
  for (int T0 = w * kAttnChunk; T0 < np * dv.p; T0 += NW * kAttnChunk)
    attn_chunk<DT, D, DT == 0, kAttnChunk / 16>(dv, s, T0, selp, np, qh, ql, st);
  float *red = reinterpret_cast<float *>(&sh.skey[0]);
  attn_publish(st, w, NW, dv.g, sh.wm, sh.wl, red);
  lds_barrier();
  for (int x = tid; x < dv.g * D; x += kFinalThreads) {
    float M, num, den;
    attn_merge<D>(NW, dv.g, x, sh.wm, sh.wl, red, M, num, den);
    out[(int64_t)s * dv.g * D + x] = den > 0.0f ? num / den : 0.0f;
  }
}

// ---------------------------------------------------------------- final, large unions

// For L*k0 above kMaxCand (the 262k-token configuration: 6 x 2048): the union
// of the candidates stays in global memory (the rerank list, followed by the
// boundary picks that are new to it) and, for the ranking, in registers
// (kPerBig elements per thread).  Duplicates are caught by a bitmap over the
// tokens (one test-and-set per token) when the stream has at most kBitTokens
// tokens, else by an LDS hash of 2^14 slots.  The ranking uses the small
// path's score buckets and proceeds in windows of consecutive buckets holding
// at most kWin elements, each ranked in LDS, until the page walk has P pages
// and the top-k (when asked for) is written.  A bucket of more than kWin elements (near equal scores) is ranked
// by counting over the union in global memory.  The attention runs in its own
// kernel.
constexpr int kBigHashBits = 14;
constexpr int64_t kBitTokens = (int64_t)32 << kBigHashBits;  // bitmap of the hash's words
constexpr int kWin = 4096;
constexpr int kWinWalk = 1024;  // window of the page walk alone (no top-k asked)
constexpr int kBndBig = 5120;  // boundary keys held in LDS (their rank keys and pages stay global)
constexpr int kPerBig = kMaxCandBig / kFinalThreads;
constexpr int kPerBnd = kBndBig / kFinalThreads;
static_assert(kPerBig * kFinalThreads == kMaxCandBig && kPerBnd * kFinalThreads == kBndBig, "");

struct BigShared {
  union {
    uint32_t hash[1 << kBigHashBits];  // union membership: bitmap or hash (selection phase)
    struct {                           // one window of the ranking, in bucket order
      unsigned long long wk[kWin];     // keys; later the rank-ordered tokens and pages
      int32_t wid[kWin];               // tokens
      int32_t wpg[kWin];               // pages
    };
  };
  union {
    unsigned long long bk[kBndBig];  // boundary keys (selection phase)
    struct {                         // bucket counts (ranking phase)
      uint32_t bcnt[kBuckets];
      uint32_t bstart[kBuckets + 1];
    };
  };
  uint32_t seen[2048];
  uint32_t cnt[256];
  uint32_t cc[32], nb[32], need[32], boff[33], extra[32], b2[32], need2[32];
  unsigned long long klast[32];
  uint32_t tie[kMaxTies];
  uint32_t ntie, nux, rr, nsel, win_end;
  unsigned long long res;
  unsigned long long wlo[16], whi[16];
  uint32_t wsum[16];
};

template <int DT>
__global__ __launch_bounds__(kFinalThreads) void k_qfinal_big(Dev dv, int64_t n, bool bounded,
                                                              int32_t *page_ids, int32_t *n_pages,
                                                              int32_t *topk_ids,
                                                              ice_query_stats *stats,
                                                              unsigned long long vlimit) {
  __shared__ BigShared sh;
  constexpr int NT = kFinalThreads;
  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int L = dv.Lq, k0 = dv.k0;  // the query's walks
  const uint32_t k0e = (uint32_t)min((int64_t)k0, n);
  const int64_t o0 = (int64_t)s * L * k0;  // the stream's union arrays (rerank list first)
  unsigned long long *ukey = dv.rr_key + o0;
  int32_t *uid = dv.rr_id + o0, *upg = dv.rr_pg + o0;

  // A. counts and the two threshold levels of every composite, all loads
  // issued before any is used
  uint32_t h2[kBinsPerLane], bl_ld = 0;  // second-level histogram; count below b*
  if (w < L) {  // wave w's composite
    wave_hist_load(dv.hist2 + ((int64_t)s * L + w) * kHistBins, h2);
    bl_ld = dv.bsel[((int64_t)s * L + w) * 2 + 1];
  }
  const uint32_t kl_ld = bounded && w < L ? dv.vcount[s * L + w] : k0e;
  const uint32_t nrr_ld = dv.rr_count[s];
  uint32_t cc_ld = 0, nb_ld = 0;
  if (tid < L) {
    cc_ld = dv.cand_count[s * L + tid];
    nb_ld = dv.bnd_count[s * L + tid];
  }
  const bool bitmap = n <= kBitTokens;
  const int hwords = bitmap ? (int)((n + 31) >> 5) : (1 << kBigHashBits);
  for (int x = tid; x < hwords; x += NT) sh.hash[x] = 0;
  // true when the token was not in the union yet
  auto mark = [&](int32_t id) -> bool {
    if (bitmap) {
      const uint32_t bit = 1u << (id & 31);
      return (atomicOr(&sh.hash[id >> 5], bit) & bit) == 0u;
    }
    return hash_insert<kBigHashBits>(sh.hash, id);
  };
  if (tid < L) {
    sh.cc[tid] = cc_ld;
    sh.nb[tid] = nb_ld;
    sh.extra[tid] = 0;
    sh.klast[tid] = 0;
  }
  {  // need, b2, need2 of composite l come from wave l alone (all zero when it takes no
     // candidates: k0e = 0, or a bounded walk that completes no token)
    for (int l = w; l < L; l += NT / 64) {
      uint32_t b2, bl2;
      if (l != w)  // more composites than waves
        wave_hist_load(dv.hist2 + ((int64_t)s * L + l) * kHistBins, h2);
      const uint32_t kl = min(k0e, l == w ? kl_ld : (bounded ? dv.vcount[s * L + l] : k0e));
      uint32_t need = 0, need2 = 0;  // picks from the boundary bin (>= 1 when kl > 0) and
      b2 = 0;                        // from its second-level bin b2
      if (kl > 0) {  // the first-level bin b* and the count below it come from the collect pass
        const uint32_t bl = l == w ? bl_ld : dv.bsel[((int64_t)s * L + l) * 2 + 1];
        need = kl - bl;
        wave_find_bin_regs(h2, need, b2, bl2);
        need2 = need - bl2;
      }
      if (lane == 0) {
        sh.need[l] = need;
        sh.b2[l] = b2;
        sh.need2[l] = need2;
      }
    }
  }
  __syncthreads();
  const uint32_t nrr = k0e > 0 ? nrr_ld : 0u;
  if (tid == 0) {
    uint32_t o = 0;
    for (int l = 0; l < L; ++l) {
      sh.boff[l] = o;
      o += (k0e > 0) ? sh.nb[l] : 0u;
    }
    sh.boff[L] = o;
    sh.ntie = 0;
    sh.nux = 0;
    sh.nsel = 0;
  }
  __syncthreads();
  const uint32_t nbt = sh.boff[L];
  const bool bnd_lds = nbt <= (uint32_t)kBndBig;
  auto comp_of = [&](uint32_t x) {
    int l = 0;
    while (x >= sh.boff[l + 1]) ++l;
    return l;
  };
  auto bnd_off = [&](int l, uint32_t x) {
    return ((int64_t)s * L + l) * dv.ncap + (x - sh.boff[l]);
  };

  // B. the rerank list's tokens into the hash; the boundary keys into LDS
  // (each thread's loads issued together)
  {
    int32_t ids[kPerBig];
#pragma unroll
    for (int j = 0; j < kPerBig; ++j) {
      const uint32_t x = tid + NT * j;
      ids[j] = x < nrr ? uid[x] : -1;
    }
    if (bnd_lds) {
      int64_t bo[kPerBnd];
#pragma unroll
      for (int j = 0; j < kPerBnd; ++j) {
        const uint32_t x = tid + NT * j;
        bo[j] = x < nbt ? bnd_off(comp_of(x), x) : -1;
      }
      unsigned long long bv[kPerBnd];
#pragma unroll
      for (int j = 0; j < kPerBnd; ++j) bv[j] = bo[j] >= 0 ? dv.bnd[bo[j]] : 0ull;
#pragma unroll
      for (int j = 0; j < kPerBnd; ++j)
        if (bo[j] >= 0) sh.bk[tid + NT * j] = bv[j];
    }
#pragma unroll
    for (int j = 0; j < kPerBig; ++j)
      if (ids[j] >= 0) mark(ids[j]);
  }
  __syncthreads();

  // C. boundary picks, as in the small path; new tokens are appended to the
  // union after the rerank list
  auto add_pick = [&](int l, unsigned long long key, unsigned long long rk, int32_t pg) {
    const int32_t id = (int32_t)(key & 0xffffffffull);
    dv.cand[((int64_t)s * L + l) * k0 + sh.cc[l] + atomicAdd(&sh.extra[l], 1u)] = id;
    if (stats != nullptr) atomicMax(&sh.klast[l], key);
    if (mark(id)) {
      const uint32_t pos = nrr + atomicAdd(&sh.nux, 1u);
      ukey[pos] = rk;
      uid[pos] = id;
      upg[pos] = pg;
    }
  };
  auto add_pick_x = [&](int l, unsigned long long key, uint32_t x) {
    const int64_t o = bnd_off(l, x);
    add_pick(l, key, dv.bnd_rk[o], dv.bnd_pg[o]);
  };
  auto sub_of = [](unsigned long long key) -> uint32_t {
    return (uint32_t)(key >> (32 + kSubShift)) & (kHistBins - 1);
  };
  if (nbt > 0) {
    if (bnd_lds) {
      // entries below second-level bin b2_l: picked outright (their rank
      // keys and pages loaded together); bin b2_l: the tie list
      int64_t po[kPerBnd];
      unsigned long long pk[kPerBnd];
      int pl[kPerBnd];
#pragma unroll
      for (int j = 0; j < kPerBnd; ++j) {
        const uint32_t x = tid + NT * j;
        po[j] = -1;
        pk[j] = 0;
        pl[j] = 0;
        if (x < nbt) {
          const int l = comp_of(x);
          const unsigned long long key = sh.bk[x];
          const uint32_t sb = sub_of(key);
          if (sb < sh.b2[l]) {
            po[j] = bnd_off(l, x);
            pk[j] = key;
            pl[j] = l;
          }
          if (sb == sh.b2[l]) {
            const uint32_t t = atomicAdd(&sh.ntie, 1u);
            if (t < kMaxTies) sh.tie[t] = x;
          }
        }
      }
      unsigned long long prk[kPerBnd];
      int32_t ppg[kPerBnd];
#pragma unroll
      for (int j = 0; j < kPerBnd; ++j) {
        prk[j] = po[j] >= 0 ? dv.bnd_rk[po[j]] : 0ull;
        ppg[j] = po[j] >= 0 ? dv.bnd_pg[po[j]] : 0;
      }
#pragma unroll
      for (int j = 0; j < kPerBnd; ++j)
        if (po[j] >= 0) add_pick(pl[j], pk[j], prk[j], ppg[j]);
      __syncthreads();
      const uint32_t nt = sh.ntie;
      if (nt <= (uint32_t)kMaxTies) {
        for (uint32_t t = tid; t < nt; t += NT) {
          const uint32_t x = sh.tie[t];
          const int l = comp_of(x);
          const unsigned long long key = sh.bk[x];
          uint32_t rank = 0;
          for (uint32_t u = 0; u < nt; ++u) {
            const uint32_t y = sh.tie[u];
            rank += (y >= sh.boff[l]) & (y < sh.boff[l + 1]) & (sh.bk[y] < key);
          }
          if (rank < sh.need2[l]) add_pick_x(l, key, x);
        }
      } else {
        for (uint32_t x = tid; x < nbt; x += NT) {
          const int l = comp_of(x);
          const unsigned long long key = sh.bk[x];
          if (sub_of(key) != sh.b2[l]) continue;
          uint32_t rank = 0;
          for (uint32_t y = sh.boff[l]; y < sh.boff[l + 1]; ++y)
            rank += (sub_of(sh.bk[y]) == sh.b2[l]) & (sh.bk[y] < key);
          if (rank < sh.need2[l]) add_pick_x(l, key, x);
        }
      }
    } else {
      for (int l = 0; l < L; ++l) {
        const int64_t ob = ((int64_t)s * L + l) * dv.ncap;
        const unsigned long long *bk = dv.bnd + ob;
        const uint32_t nbl = sh.nb[l], nd = sh.need[l];
        const unsigned long long thr =
            nd >= nbl ? ~0ull : block_select(bk, nbl, nd, sh.cnt, &sh.res, &sh.rr);
        for (uint32_t x = tid; x < nbl; x += NT) {
          const unsigned long long key = bk[x];
          if (key <= thr) add_pick(l, key, dv.bnd_rk[ob + x], dv.bnd_pg[ob + x]);
        }
        __syncthreads();
      }
    }
  }
  __syncthreads();  // the union is complete (and its global writes visible to the block)
  const uint32_t nu = nrr + sh.nux;

  // D. ranking in windows of score buckets, the union in registers
  unsigned long long kx[kPerBig];
  int32_t ix[kPerBig], px[kPerBig];
  uint32_t bw[kPerBig];  // bucket | slot inside the bucket << 12
  auto bkt_of = [](uint32_t v) { return v & 0xfffu; };
  auto within_of = [](uint32_t v) { return v >> 12; };
#pragma unroll
  for (int j = 0; j < kPerBig; ++j) {
    const uint32_t x = tid + NT * j;
    kx[j] = x < nu ? ukey[x] : ~0ull;
    ix[j] = x < nu ? uid[x] : 0;
    px[j] = x < nu ? upg[x] : 0;
  }
  unsigned long long lo = ~0ull, hi = 0;
#pragma unroll
  for (int j = 0; j < kPerBig; ++j)
    if (tid + NT * j < nu) {
      lo = min(lo, kx[j]);
      hi = max(hi, kx[j]);
    }
  lo = wave_minmax_u64<false>(lo);
  hi = wave_minmax_u64<true>(hi);
  if (lane == 0) {
    sh.wlo[w] = lo;
    sh.whi[w] = hi;
  }
  for (int x = tid; x < kBuckets; x += NT) sh.bcnt[x] = 0;
  for (int x = tid; x < 2048; x += NT) sh.seen[x] = 0;
  if (tid == 0) sh.win_end = 0;
  __syncthreads();
  lo = ~0ull;
  hi = 0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    lo = min(lo, sh.wlo[k]);
    hi = max(hi, sh.whi[k]);
  }
  const double smax = nu ? rank_key_score(lo) : 0.0;
  const double smin = nu ? rank_key_score(hi) : 0.0;
  const double scale = smax > smin ? (double)(kBuckets - 1) / (smax - smin) : 0.0;
#pragma unroll
  for (int j = 0; j < kPerBig; ++j) {
    bw[j] = kBuckets;  // past every window
    if (tid + NT * j < nu) {
      const double t = (smax - rank_key_score(kx[j])) * scale;
      const uint32_t b = (uint32_t)min((double)(kBuckets - 1), t);
      bw[j] = b | (atomicAdd(&sh.bcnt[b], 1u) << 12);
    }
  }
  __syncthreads();
  {  // exclusive scan of the bucket counts, two per thread
    const uint32_t c0 = sh.bcnt[2 * tid], c1 = sh.bcnt[2 * tid + 1];
    const uint32_t incl = wave_incl_scan(c0 + c1);
    if (lane == 63) sh.wsum[w] = incl;
    __syncthreads();
    uint32_t pre = 0;
    for (int k = 0; k < w; ++k) pre += sh.wsum[k];
    const uint32_t excl = pre + incl - (c0 + c1);
    sh.bstart[2 * tid] = excl;
    sh.bstart[2 * tid + 1] = excl + c0;
    if (tid == 0) sh.bstart[kBuckets] = nu;
  }
  __syncthreads();

  const int P = dv.P;
  const uint32_t want_top = topk_ids ? min((uint32_t)dv.k, nu) : 0u;
  int pbits = 1;
  while ((1ll << pbits) < dv.pcap) ++pbits;
  int32_t *const rsid = reinterpret_cast<int32_t *>(&sh.wk[0]);  // over the dead keys
  int32_t *const rspg = rsid + kWin;
  uint32_t B0 = 0, rank_base = 0;
  while (B0 < (uint32_t)kBuckets && rank_base < nu &&
         ((int)sh.nsel < P || rank_base < want_top)) {
    // the window: buckets [B0, B1), the largest B1 whose buckets hold at most
    // lim elements (one bucket at least).  The page walk alone needs the
    // first ranks only, so its windows hold at most kWinWalk elements, unless
    // bucket B0 alone holds more (then up to kWin).  Bucket starts grow with
    // b, so the buckets that fit are a run from B0 + 1: each wave finds its
    // last one by a ballot and takes the largest with one LDS atomic.
    const uint32_t base = sh.bstart[B0];
    const uint32_t lim = want_top == 0u && sh.bstart[B0 + 1] - base <= (uint32_t)kWinWalk
                             ? (uint32_t)kWinWalk : (uint32_t)kWin;
    if (tid == 0) atomicMax(&sh.win_end, B0 + 1);
    for (uint32_t b0 = B0 + 1; b0 <= (uint32_t)kBuckets; b0 += NT) {  // uniform bound
      const uint32_t b = b0 + tid;
      const bool fits = b <= (uint32_t)kBuckets && sh.bstart[b] - base <= lim;
      const unsigned long long bal = __ballot(fits);
      if (lane == 0 && bal)
        atomicMax(&sh.win_end, b0 + 64 * w + 63 - (uint32_t)__builtin_clzll(bal));
    }
    __syncthreads();
    const uint32_t B1 = sh.win_end;
    const uint32_t cntw = sh.bstart[B1] - base;
    if (cntw <= (uint32_t)kWin) {
      // scatter the window's elements in bucket order, rank each by position
      // (kWin / NT per thread), then write tokens and pages in rank order
#pragma unroll
      for (int j = 0; j < kPerBig; ++j)
        if (bkt_of(bw[j]) >= B0 && bkt_of(bw[j]) < B1) {
          const uint32_t pos = sh.bstart[bkt_of(bw[j])] - base + within_of(bw[j]);
          sh.wk[pos] = kx[j];
          sh.wid[pos] = ix[j];
          sh.wpg[pos] = px[j];
        }
      __syncthreads();
      constexpr int kPerWin = kWin / NT;
      uint32_t rr[kPerWin];
      int32_t ri[kPerWin], rp[kPerWin];
#pragma unroll
      for (int j = 0; j < kPerWin; ++j) {
        const uint32_t x = tid + NT * j;
        rr[j] = ~0u;
        ri[j] = 0;
        rp[j] = 0;
        if (x < cntw) {
          const unsigned long long kk = sh.wk[x];
          const int32_t id = sh.wid[x];
          const double t = (smax - rank_key_score(kk)) * scale;
          const uint32_t b = (uint32_t)min((double)(kBuckets - 1), t);
          const uint32_t b0 = sh.bstart[b] - base, b1 = b0 + sh.bcnt[b];
          uint32_t r = b0, eq = 0;
          for (uint32_t y = b0; y < b1; ++y) {
            const unsigned long long ky = sh.wk[y];
            r += ky < kk;
            eq += ky == kk;
          }
          if (eq > 1)  // equal keys (rare): order them by token
            for (uint32_t y = b0; y < b1; ++y) r += sh.wk[y] == kk && sh.wid[y] < id;
          rr[j] = r;
          ri[j] = id;
          rp[j] = sh.wpg[x];
        }
      }
      __syncthreads();  // every read of the window is done
#pragma unroll
      for (int j = 0; j < kPerWin; ++j)
        if (rr[j] != ~0u) {
          rsid[rr[j]] = ri[j];
          rspg[rr[j]] = rp[j];
        }
    } else {
      // one bucket above the window size: rank its elements by counting
      // over the union (slow; only near-equal scores get here), written out
      // in chunks of kWin ranks below
#pragma unroll
      for (int j = 0; j < kPerBig; ++j) {
        if (bkt_of(bw[j]) != B0) continue;
        uint32_t r = 0;
        for (uint32_t y = 0; y < nu; ++y) {
          const unsigned long long ky = ukey[y];
          if (ky < kx[j] || (ky == kx[j] && uid[y] < ix[j])) {
            const double t = (smax - rank_key_score(ky)) * scale;
            r += (uint32_t)min((double)(kBuckets - 1), t) == B0;
          }
        }
        bw[j] = (bw[j] & 0xfffu) | (r << 12);  // the rank replaces the slot (bucket B0 is done after)
      }
    }
    // walk the window's ranks in chunks of kWin (one chunk unless one bucket
    // holds more)
    for (uint32_t c0 = 0; c0 < cntw; c0 += kWin) {
      const uint32_t cw = min((uint32_t)kWin, cntw - c0);
      if (cntw > (uint32_t)kWin) {
#pragma unroll
        for (int j = 0; j < kPerBig; ++j) {
          const uint32_t r = within_of(bw[j]);
          if (bkt_of(bw[j]) == B0 && r >= c0 && r < c0 + cw) {
            rsid[r - c0] = ix[j];
            rspg[r - c0] = px[j];
          }
        }
      }
      __syncthreads();
      const uint32_t rb = rank_base + c0;
      if (topk_ids)
        for (uint32_t r = tid; r < cw; r += NT)
          if (rb + r < want_top) topk_ids[(int64_t)s * dv.k + rb + r] = rsid[r];
      if (w == 0 && (int)sh.nsel < P) {
        int nsel = sh.nsel;
        const unsigned long long lt = lanemask_lt();
        for (uint32_t x0 = 0; x0 < cw && nsel < P; x0 += 64) {
          const uint32_t x = x0 + lane;
          const bool valid = x < cw;
          const int32_t pg = valid ? rspg[x] : 0;
          const bool fresh = valid && ((sh.seen[pg >> 5] >> (pg & 31)) & 1u) == 0u;
          const unsigned long long act = __ballot(fresh);
          const unsigned long long mt = match_bits((uint32_t)pg, pbits, act);
          const bool firstocc = fresh && (mt & lt) == 0ull;
          const unsigned long long fm = __ballot(firstocc);
          const int pos = nsel + popc64(fm & lt);
          if (firstocc && pos < P) {
            page_ids[(int64_t)s * P + pos] = pg;
            atomicOr(&sh.seen[pg >> 5], 1u << (pg & 31));
          }
          nsel = min(P, nsel + popc64(fm));
          __builtin_amdgcn_wave_barrier();
        }
        if (lane == 0) sh.nsel = nsel;
      }
      __syncthreads();
    }
    rank_base += cntw;
    B0 = B1;
  }

  // E. padding and counts
  const int nsel = sh.nsel;
  for (int x = nsel + tid; x < P; x += NT) page_ids[(int64_t)s * P + x] = -1;
  if (tid == 0) n_pages[s] = nsel;
  if (topk_ids)
    for (uint32_t x = want_top + tid; x < (uint32_t)dv.k; x += NT)
      topk_ids[(int64_t)s * dv.k + x] = -1;
  if (tid < L && k0e > 0) dv.cand_count[s * L + tid] = sh.cc[tid] + sh.extra[tid];
  if (stats != nullptr)
    final_stats(dv, s, n, k0e, sh.cc, sh.extra, sh.klast, nu, (uint32_t)nsel, stats, vlimit);
  uint4 *hist = reinterpret_cast<uint4 *>(dv.hist + (int64_t)s * L * kHistBins);
  uint4 *hist2 = reinterpret_cast<uint4 *>(dv.hist2 + (int64_t)s * L * kHistBins);
  for (int x = tid; x < L * kHistBins / 4; x += NT) {  // 16-byte stores
    hist[x] = make_uint4(0u, 0u, 0u, 0u);
    hist2[x] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// ---------------------------------------------------------------- launcher

template <int DT, bool LH, int R, int NT>
static void launch_scan(const Dev &dv, int64_t n, dim3 grid, const void *q, const void *k_new,
                        const void *v_new, hipStream_t st) {
  if (dv.Gq > 1)
    hipLaunchKernelGGL((k_qscan<DT, LH, R, NT, true, 1>), grid, dim3(NT), 0, st, dv, n, q, k_new,
                       v_new, dv.Gq);
  else
    hipLaunchKernelGGL((k_qscan<DT, LH, R, NT, false, 1>), grid, dim3(NT), 0, st, dv, n, q, k_new,
                       v_new, 1);
}

template <int DT, bool LH, int NT>
static void launch_scan_r(const Dev &dv, int64_t n, dim3 grid, const void *q,
                          const void *k_new, const void *v_new, hipStream_t st) {
  switch ((dv.mL + kPipe - 1) / kPipe) {
    case 1: launch_scan<DT, LH, 1, NT>(dv, n, grid, q, k_new, v_new, st); break;
    case 2: launch_scan<DT, LH, 2, NT>(dv, n, grid, q, k_new, v_new, st); break;
    case 3: launch_scan<DT, LH, 3, NT>(dv, n, grid, q, k_new, v_new, st); break;
    case 4: launch_scan<DT, LH, 4, NT>(dv, n, grid, q, k_new, v_new, st); break;
    case 5: launch_scan<DT, LH, 5, NT>(dv, n, grid, q, k_new, v_new, st); break;
    case 6: launch_scan<DT, LH, 6, NT>(dv, n, grid, q, k_new, v_new, st); break;
    case 7: launch_scan<DT, LH, 7, NT>(dv, n, grid, q, k_new, v_new, st); break;
    default: launch_scan<DT, LH, 8, NT>(dv, n, grid, q, k_new, v_new, st); break;  // mL <= 128
  }
}

// Grid of the scan and the collect: x streams (consecutive blocks take
// different streams, so with S a multiple of 8 a stream's blocks share an
// XCD), y token ranges of 2 * NT (at most 2^22 tokens per stream under the
// page-capacity limit: 4,096 ranges), z the scan's passes.
template <int NT>
static dim3 range_grid(const Dev &dv, int64_t n, int passes) {
  const int64_t nrange = (n + 2 * NT - 1) / (2 * NT);
  return dim3((unsigned)dv.S, (unsigned)max(nrange, (int64_t)1), (unsigned)passes);
}

// The scan in NT-thread blocks of 2 * NT tokens, one pass per head in the
// GQA max mode (the mean mode has one).
template <int DT, int NT>
static void launch_scan_nt(const Dev &dv, int64_t n, const void *q, const void *k_new,
                           const void *v_new, hipStream_t st) {
  const dim3 grid = range_grid<NT>(dv, n, dv.Gq);
  if (dv.L <= 6)
    launch_scan_r<DT, true, NT>(dv, n, grid, q, k_new, v_new, st);
  else
    launch_scan_r<DT, false, NT>(dv, n, grid, q, k_new, v_new, st);
}

// The collect in NT-thread blocks of 2 * NT tokens, every walk of a stream
// in each block.
template <int DT, int NT>
static void launch_collect(const Dev &dv, int64_t n, bool bounded, const void *q,
                           hipStream_t st) {
  const dim3 grid = range_grid<NT>(dv, n, 1);
  const size_t qbytes = (size_t)(dv.gmax ? dv.g : 1) * 128 * sizeof(float);
  if (dv.Lq > 8)
    hipLaunchKernelGGL((k_qcollect<DT, NT, true>), grid, dim3(NT), qbytes, st, dv, n, bounded, q);
  else
    hipLaunchKernelGGL((k_qcollect<DT, NT, false>), grid, dim3(NT), qbytes, st, dv, n, bounded, q);
}

// Block shape for `blocks(nt)` blocks of nt threads: 512 by default; when
// 512-thread blocks would not all get a CU of their own, the smallest of 640,
// 768 and 1024 that does.
template <typename Blocks, typename Launch>
static void by_shape(int64_t cus, Blocks blocks, Launch launch) {
  auto fits = [&](int nt) { return blocks(nt) <= cus; };
  if (fits(512) || !fits(1024))
    launch(std::integral_constant<int, 512>());
  else if (fits(640))
    launch(std::integral_constant<int, 640>());
  else if (fits(768))
    launch(std::integral_constant<int, 768>());
  else
    launch(std::integral_constant<int, 1024>());
}

// The query over n tokens (token n - 1 inserted by the scan when k_new is
// given): scan, the visit-budget passes when the walk is bounded (k1 < m * n),
// collect, final.
template <int DT, int PER>
static void launch_final(const Dev &dv, int64_t n, bool bounded, int32_t *page_ids,
                         int32_t *n_pages, int32_t *topk_ids, const void *q, float *out,
                         ice_query_stats *stats, unsigned long long vlimit, hipStream_t st) {
  static_assert(PER * kFinalThreads <= kMaxCand, "union arrays");
  if (dv.d == 128)
    hipLaunchKernelGGL((k_qfinal<DT, 128, PER>), dim3(dv.S), dim3(kFinalThreads), 0, st, dv, n,
                       bounded, page_ids, n_pages, topk_ids, q, out, stats, vlimit);
  else
    hipLaunchKernelGGL((k_qfinal<DT, 64, PER>), dim3(dv.S), dim3(kFinalThreads), 0, st, dv, n,
                       bounded, page_ids, n_pages, topk_ids, q, out, stats, vlimit);
}

template <int DT>
static void query_tail(const Dev &dv, int64_t n, int64_t k1, int32_t *page_ids,
                       int32_t *n_pages, int32_t *topk_ids, const void *q, const void *k_new,
                       const void *v_new, float *out, ice_query_stats *stats, hipStream_t st,
                       Timer *tm) {
  const bool bounded = n > 0 && k1 > 0 && k1 < (int64_t)dv.m * n;
  // the entries a walk may visit: its budget, else all m * n
  const unsigned long long vlimit = bounded ? (unsigned long long)k1 : (unsigned long long)dv.m * n;
  const int64_t cus = dv.ncu;
  auto ranges = [&](int nt) { return (int64_t)dv.S * ((n + 2 * nt - 1) / (2 * nt)); };
  // the scan: the GQA max mode's heads in one block when the group allows
  // it, else one pass per head
  if (!launch_scan_heads(dv, n, q, k_new, v_new, st))
    by_shape(cus, [&](int nt) { return ranges(nt) * dv.Gq; }, [&](auto nt) {
      launch_scan_nt<DT, decltype(nt)::value>(dv, n, q, k_new, v_new, st);
    });
  timer_mark(tm, KID_QSCAN, st);
  if (bounded) {
    for (int head = 0; head < dv.Gq; ++head)
      (void)launch_visit_budget(dv, n, (uint32_t)k1, head, st);  // a launch error stays for the caller's check
    timer_mark(tm, KID_VISIT, st);
  }
  if (n > 0) {
    by_shape(cus, ranges, [&](auto nt) {
      launch_collect<DT, decltype(nt)::value>(dv, n, bounded, q, st);
    });
    timer_mark(tm, KID_QCOLLECT, st);
  }
  if (dv.Lq * dv.k0 > kMaxCand)
    hipLaunchKernelGGL(k_qfinal_big<DT>, dim3(dv.S), dim3(kFinalThreads), 0, st, dv, n, bounded,
                       page_ids, n_pages, topk_ids, stats, vlimit);
  else if (dv.Lq * dv.k0 <= kFinalThreads)
    launch_final<DT, 1>(dv, n, bounded, page_ids, n_pages, topk_ids, q, out, stats, vlimit, st);
  else
    launch_final<DT, kMaxCand / kFinalThreads>(dv, n, bounded, page_ids, n_pages, topk_ids, q,
                                               out, stats, vlimit, st);
  timer_mark(tm, KID_QFINAL, st);
}

hipError_t launch_query(const Dev &dv, int64_t n, int64_t k1, const void *q, int32_t *page_ids,
                        int32_t *n_pages, int32_t *topk_ids, ice_query_stats *stats,
                        hipStream_t st, Timer *tm) {
  timer_begin(tm, st);
  if (dv.dtype == 0)
    query_tail<0>(dv, n, k1, page_ids, n_pages, topk_ids, q, nullptr, nullptr, nullptr, stats, st,
                  tm);
  else
    query_tail<1>(dv, n, k1, page_ids, n_pages, topk_ids, q, nullptr, nullptr, nullptr, stats, st,
                  tm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || stats == nullptr) return e;
  return launch_stats(dv, n, stats, page_ids, n_pages, st);
}

hipError_t launch_decode(const Dev &dv, int64_t n, int64_t k1, const void *k_new,
                         const void *v_new, const void *q, int32_t *page_ids, int32_t *n_pages,
                         int32_t *topk_ids, float *out, ice_query_stats *stats, hipStream_t st,
                         Timer *tm) {
  // the new token is token n (inserted by the scan); the query sees n + 1
  // tokens.  Budgets of one attention split (kAttnTpb tokens) and unions that
  // fit LDS: the finaliser runs the attention itself, with the standalone
  // kernel's arithmetic (16 waves of one chunk, merged by their maxima).
  // Larger budgets take the standalone kernels, whose per-split partials and
  // merge fix the summation order, so the step equals the separate calls; so
  // does a host-offloaded pool (its selected pages are staged first).
  timer_begin(tm, st);
  const bool fused = dv.attn_nsplit == 1 && dv.Lq * dv.k0 <= kMaxCand && !dv.offload;
  float *fo = fused ? out : nullptr;
  if (dv.dtype == 0)
    query_tail<0>(dv, n + 1, k1, page_ids, n_pages, topk_ids, q, k_new, v_new, fo, stats, st, tm);
  else
    query_tail<1>(dv, n + 1, k1, page_ids, n_pages, topk_ids, q, k_new, v_new, fo, stats, st, tm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!fused && (e = launch_attn(dv, q, page_ids, n_pages, out, st, tm)) != hipSuccess) return e;
  return stats != nullptr ? launch_stats(dv, n + 1, stats, page_ids, n_pages, st) : hipSuccess;
}

}  // namespace ice
