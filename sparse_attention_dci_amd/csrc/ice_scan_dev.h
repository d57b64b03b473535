// The query's code scan (IceCache paper page, Figure 2 step (2); blog page,
// technical details: one prioritized-DCI search per head): the query codes,
// then M_i = max_j |code_ij - qcode_j| for every token and composite and a
// histogram of the top 11 bits of M_i.  A template shared by the mean mode's
// and the GQA max mode's launches (one head per block, or every head of the
// group in one block over a single read of the codes).
#pragma once

#include "ice_step_dev.h"

namespace ice {

// Buffer resource over a byte range: loads past its end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_range(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Codes are read once per query: non-temporal (nt), so the stream does not
// push the rest of the step's working set (and the kernels' code) out of L2.
__device__ __forceinline__ int32_t ld_code(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, /*nt*/ 2);
}

// Grid (S, max(1, ceil(n / kScanTpb)), passes) of NT-thread blocks.  Block
// (s, r, h) serves stream s (consecutive blocks take different streams, so
// with S a multiple of 8 all blocks of a stream land on one XCD and share its
// L2), the r-th range of kScanTpb = 2 * NT tokens and the GQA max mode's
// pass h (the mean mode has one): wave w takes tiles 2w and
// 2w+1 of the range, lane j token j of a tile, and reads code t of its 64
// tokens as one contiguous 256-byte load.  kPipe codes of each tile are in
// flight at a time: every code slot is refilled with the code kPipe places
// later right after it is used.  R = ceil(mL / kPipe) is a template
// parameter, so the walk over code positions is straight-line code and every
// wait covers exactly the loads it needs.  The histogram lives in LDS when
// L <= 6, and only the bins at or below the block's own k0-th bin (its
// largest bin when it counted fewer than k0 tokens) are added to the global
// one; with L > 6 every count goes straight to global.
//
// Every block first derives the query codes itself (the directions staged in
// LDS, the arithmetic of ice_step_dev.h), so no prep kernel sits on the
// query's critical path; the blocks of range 0 publish q_kv and the codes for
// the later kernels and clear the query's counters.  In a decode step (k_new
// given) token n - 1 is the new token: the block whose range holds it leaves
// it out of its code walk, and the block of range 0 (dispatched first, so the
// insert is off the critical path of the last blocks) projects it on the
// same staged directions, adds its M values to its own histogram and writes
// its codes, list entries, page and pool rows at the end.
constexpr int kPipe = 16;

// Histograms a block of GH heads holds in LDS (8 KB each): GH * L of them.
template <int GH>
struct ScanWalks {
  static constexpr int kLds = GH == 1 ? 6 : (GH == 2 ? 12 : 16);
};

//
// GQA max mode, two layouts.  One head per block (GH = 1, MULTI): the blocks
// of pass `head` (the grid holds every head's pass) walk the L composites
// with that head's own query (its row of q alone) and fill walks
// head * L .. head * L + L - 1 of the stream's query arrays.  Every head in
// one block (GH = g, a grid of one pass): the block derives the GH heads'
// query codes, reads each code once and keeps GH running maxima per token,
// filling walk h * L + l for head h; its LDS holds the GH * L histograms, so
// one block fits a CU.  The mean mode has one pass, head 0.  In a decode step
// the range-0 block of every pass projects the new token for its M values;
// pass 0's also stores it.
template <int DT, bool LDS_HIST, int R, int NT, bool MULTI, int GH>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(GH == 1 ? 6 : NT / 256))) void k_qscan(
    Dev dv, int64_t n, const void *q, const void *k_new, const void *v_new, int npass) {
  static_assert(GH == 1 || (!MULTI && LDS_HIST), "a block of several heads is the only pass");
  static_assert(GH <= 4 && GH * 128 <= NT, "one thread per (head, direction) slot");
  constexpr int kScanTpb = 2 * NT;
  constexpr int W = R * kPipe;  // staged direction columns (>= mL, <= the stored row width)
  constexpr int W4 = W / 4;
  constexpr int kStage = (129 * W4 + NT - 1) / NT;
  constexpr int kWalks = ScanWalks<GH>::kLds;
  // grid (S, ranges, passes): the GQA max mode's passes share the launch
  // (MULTI; else one pass, head 0 at compile time)
  const int head = MULTI ? (int)blockIdx.z : 0;
  const int s = (int)blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int mL = dv.mL, m = dv.m, L = dv.L, d = dv.d, g = dv.g;
  const int64_t r = blockIdx.y;
  const int64_t nold = k_new != nullptr ? n - 1 : n;  // tokens already in the index
  // the blocks of range 0, dispatched first, insert token nold, which keeps
  // the insert off the last blocks' critical path (no short circuit: no
  // branch before the kernel arguments are all requested)
  const bool proj = (k_new != nullptr) & (r == 0);  // every pass's range-0 block projects it
  const bool ins = proj & (head == 0);                // pass 0's stores it
  // directions: element e < d of direction t at dl[((e / 16) * W + t) * 16 + e % 16]
  // (each lane of a query lane group reads its 16 elements as four 16-byte
  // runs), u_t[d] at ud[t]
  union __attribute__((aligned(16))) ScanShared {
    uint32_t hist[LDS_HIST ? kWalks * kHistBins : 1];
    float dl[128 * W];
  };
  __shared__ ScanShared sm;
  __shared__ float ud[W];
  __shared__ int32_t qc[GH * kMaxMl], nc[kMaxMl];
  __shared__ int32_t blim[kWalks];
  __shared__ __attribute__((aligned(16))) float qkv[GH * 128], kv[128];
  __shared__ double zs[GH * kMaxMl], rs[kMaxMl];
  __shared__ double qsq_s[GH], ksq_s;
  __shared__ uint32_t cell_s;
  __shared__ int32_t loc_s;
  const int lo = head * L;                          // this pass's first walk
  const int nw = GH * L;                            // this block's walks
  const int gq = dv.gmax ? 1 : g;                     // heads folded into one query
  const int nh = GH > 1 ? GH : gq;                   // rows of q the prep reads
  const int64_t qr0 = (int64_t)s * g + (dv.gmax ? head : 0);  // its first row of q
  uint32_t *ghist = dv.hist + ((int64_t)s * dv.Lq + lo) * kHistBins;

  // 1. the prep's loads, every one issued before any is used (clamped
  // addresses, no branches): the directions, heads 0..3 of element tid, the
  // new key (any valid address when there is none), the insert's scalars
  const int tot4 = (d + 1) * W4;
  float4 st4[kStage];
#pragma unroll
  for (int k = 0; k < kStage; ++k) {
    const int x = min(tid + NT * k, tot4 - 1);
    st4[k] = *reinterpret_cast<const float4 *>(dv.dirs32 + (int64_t)(x / W4) * dv.mLp +
                                               (x % W4) * 4);
  }
  const int te = min(tid & 127, d - 1);
  float hv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) hv[j] = load_elem<DT>(q, (qr0 + min(j, nh - 1)) * d + te);
  const float kx = load_elem<DT>(k_new != nullptr ? k_new : q, (int64_t)s * d + te);
  const int32_t np0 = dv.npages[s];
  const double ic = dv.inv_c[s], ic2 = dv.inv_c2[s];
#pragma unroll
  for (int k = 0; k < kStage; ++k) {
    const int x = tid + NT * k;
    const int e = x / W4, t0 = (x % W4) * 4;
    const float c4[4] = {st4[k].x, st4[k].y, st4[k].z, st4[k].w};
    if (e < d) {
#pragma unroll
      for (int c = 0; c < 4; ++c) sm.dl[((((e >> 4) * W) + t0 + c) << 4) + (e & 15)] = c4[c];
    } else if (e == d) {
#pragma unroll
      for (int c = 0; c < 4; ++c) ud[t0 + c] = c4[c];
    }
  }
  if constexpr (GH == 1) {
    float acc = hv[0];  // left fold of the heads
#pragma unroll
    for (int j = 1; j < 4; ++j) acc = j < gq ? __fadd_rn(acc, hv[j]) : acc;
    for (int h0 = 4; h0 < gq; h0 += 4) {  // groups above 4
#pragma unroll
      for (int j = 0; j < 4; ++j) hv[j] = load_elem<DT>(q, (qr0 + min(h0 + j, gq - 1)) * d + te);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = h0 + j < gq ? __fadd_rn(acc, hv[j]) : acc;
    }
    if (tid < d) qkv[tid] = __fmul_rn(acc, group_inv(gq));
  } else {  // each head is its own query (a group of one)
    if (tid < d) {
#pragma unroll
      for (int h = 0; h < GH; ++h) qkv[h * 128 + tid] = __fmul_rn(hv[h], group_inv(1));
    }
  }
  if (proj && tid >= 256 && tid < 256 + d) kv[tid - 256] = kx;
  lds_barrier();

  // the first kEarly codes of both tiles go out before the chains
  constexpr int kEarly = 8;
  const uint32_t tile_bytes = (uint32_t)mL * kCodeTile * 4;
  const __amdgpu_buffer_rsrc_t rc =
      byte_range(dv.codes + (int64_t)s * dv.ntile * mL * kCodeTile, (uint32_t)dv.ntile * tile_bytes);
  const uint32_t oa = (uint32_t)(r * (kScanTpb / 64) + 2 * w) * tile_bytes + lane * 4;
  int32_t a[kPipe], b[kPipe];
#pragma unroll
  for (int x = 0; x < kEarly; ++x) {
    a[x] = ld_code(rc, oa + x * 256);
    b[x] = ld_code(rc, oa + tile_bytes + x * 256);
  }

  // the query's dot products in the blocked order: lane group t (d/16 lanes)
  // of head h is direction t, group mL the norm (head h's groups follow head
  // h - 1's); the insert's element-order chains run on the top threads,
  // it = NT-1-tid (r_t for it < mL, |k|^2 for it = mL)
  {
    const int nbk = d >> 4, lnb = d == 128 ? 3 : 2, mL1 = mL + 1;
    for (int x = tid; x < GH * mL1 * nbk; x += NT) {  // whole lane groups
      const int t2 = x >> lnb, j = x & (nbk - 1);
      int h = 0;
#pragma unroll
      for (int c = 1; c < GH; ++c) h += t2 >= c * mL1 ? 1 : 0;
      const int t = t2 - h * mL1;
      const float *qrow = qkv + 128 * h;
      const float *b = t < mL ? sm.dl + ((j * W + t) << 4) : qrow + 16 * j;
      double z = fma16(qrow + 16 * j, b, 0.0);
      z = tree_sum(z, nbk);
      if (j == 0) {
        if (t < mL)
          zs[h * kMaxMl + t] = z;
        else
          qsq_s[h] = z;
      }
    }
  }
  const int it = NT - 1 - tid;
  if (proj && it <= mL) {  // element order: one chain through the blocks
    double z = 0.0;
    for (int j = 0; j < (d >> 4); ++j)
      z = fma16(kv + 16 * j, it < mL ? sm.dl + ((j * W + it) << 4) : kv + 16 * j, z);
    if (it < mL)
      rs[it] = z;
    else
      ksq_s = z;
  }
  lds_barrier();
  // the rest of the first kPipe codes of both tiles (the chains needed the
  // registers)
#pragma unroll
  for (int x = kEarly; x < kPipe; ++x) {
    a[x] = ld_code(rc, oa + x * 256);
    b[x] = ld_code(rc, oa + tile_bytes + x * 256);
  }

  const int qh = tid >> 7, qt = tid & 127;  // (head, direction) slot of thread tid
  if (qh < GH && qt < mL) qc[qh * kMaxMl + qt] = query_code(zs[qh * kMaxMl + qt], qsq_s[qh]);
  if (proj) {
    if (it < mL) nc[it] = insert_code(rs[it], (double)ud[it], ksq_s, ic, ic2);
    if (w == 4) {  // the new token's cell: sign bits of r on the first D directions
      const unsigned long long bal = __ballot(lane < dv.D && rs[lane < mL ? lane : 0] >= 0.0);
      if (lane == 0) cell_s = (uint32_t)bal & ((1u << dv.D) - 1u);
    }
  }
  lds_barrier();
  if (r == 0) {  // publication and the query's counters (the rerank list's: first pass only)
    const int64_t hq = (int64_t)s * dv.Gq + (dv.gmax ? head : 0);
    if (qh < GH && qt < mL) dv.qcode[(hq + qh) * mL + qt] = qc[qh * kMaxMl + qt];
    if (qh < GH && qt < d) dv.qkv[(hq + qh) * d + qt] = qkv[qh * 128 + qt];
    if (tid < nw) {
      dv.cand_count[s * dv.Lq + lo + tid] = 0;
      dv.bnd_count[s * dv.Lq + lo + tid] = 0;
    }
    if (tid == 0 && head == 0) dv.rr_count[s] = 0;
  }
  if (LDS_HIST) {  // 16-byte stores (the union is 16-byte aligned: float4 staging)
    uint4 *h4 = reinterpret_cast<uint4 *>(sm.hist);
    for (int x = tid; x < nw * kHistBins / 4; x += NT) h4[x] = make_uint4(0u, 0u, 0u, 0u);
    lds_barrier();
  }
  uint32_t *hist = sm.hist;

  // 2. M per token and walk.  Composite boundaries depend on the code
  // position only, so every branch but the ragged tail's is uniform.
  const int64_t i0 = r * kScanTpb, i1 = min(i0 + kScanTpb, n);
  const int64_t ia = i0 + 128 * w + lane, ib = ia + 64;
  const int64_t iv = min(i1, nold);  // the new token is added after the walk
  const bool va = ia < iv, vb = ib < iv;
  // the tokens each of the block's histograms counts: its range's indexed
  // tokens, and in the block of range 0 the new token
  const uint32_t ncount = (uint32_t)(iv > i0 ? iv - i0 : 0) + (proj ? 1u : 0u);
  int32_t Ma[GH], Mb[GH];
#pragma unroll
  for (int h = 0; h < GH; ++h) Ma[h] = Mb[h] = 0;
  int l = 0, tend = m - 1;
  // this round's query codes, uniform (scalar registers): kQw positions of
  // every head at a time (fewer with more heads, so they stay in registers)
  constexpr int kQw = GH > 2 ? kPipe / 2 : kPipe;
  int32_t qround[GH][kQw];
#pragma unroll
  for (int t = 0; t < R * kPipe; ++t) {
    const int x = t % kPipe;
    if (t % kQw == 0) {
#pragma unroll
      for (int h = 0; h < GH; ++h)
#pragma unroll
        for (int y = 0; y < kQw; ++y)
          qround[h][y] = __builtin_amdgcn_readfirstlane(qc[h * kMaxMl + min(t + y, kMaxMl - 1)]);
    }
    if (t < mL) {
#pragma unroll
      for (int h = 0; h < GH; ++h) {
        const int32_t qv = qround[h][t % kQw];
        const int32_t da = a[x] - qv, db = b[x] - qv;  // |da| < 2^31: no overflow
        Ma[h] = max(Ma[h], max(da, -da));
        Mb[h] = max(Mb[h], max(db, -db));
      }
    }
    if (t + kPipe < R * kPipe) {
      a[x] = ld_code(rc, oa + (t + kPipe) * 256);
      b[x] = ld_code(rc, oa + tile_bytes + (t + kPipe) * 256);
    }
    if (t < mL && t == tend) {  // composite l complete (placeholders never are)
#pragma unroll
      for (int h = 0; h < GH; ++h) {
        const int wk = h * L + l;
        uint32_t *mrow = dv.mbuf + ((int64_t)s * dv.Lq + lo + wk) * dv.ncap;
        if (va) {
          mrow[ia] = (uint32_t)Ma[h];
          if (LDS_HIST)
            atomicAdd(&hist[wk * kHistBins + (Ma[h] >> kHistShift)], 1u);
          else
            atomicAdd(&ghist[wk * kHistBins + (Ma[h] >> kHistShift)], 1u);
        }
        if (vb) {
          mrow[ib] = (uint32_t)Mb[h];
          if (LDS_HIST)
            atomicAdd(&hist[wk * kHistBins + (Mb[h] >> kHistShift)], 1u);
          else
            atomicAdd(&ghist[wk * kHistBins + (Mb[h] >> kHistShift)], 1u);
        }
        Ma[h] = 0;
        Mb[h] = 0;
      }
      ++l;
      tend += m;
    }
  }

  if (proj && tid < GH) {  // the new token's M of every composite, thread h for head h
    const int h = tid;
    for (int l2 = 0; l2 < L; ++l2) {
      int32_t M = 0;
      for (int j = 0; j < m; ++j) {
        const int32_t dd = nc[l2 * m + j] - qc[h * kMaxMl + l2 * m + j];
        M = max(M, max(dd, -dd));
      }
      const int wk = h * L + l2;
      dv.mbuf[((int64_t)s * dv.Lq + lo + wk) * dv.ncap + nold] = (uint32_t)M;
      if (LDS_HIST)
        atomicAdd(&hist[wk * kHistBins + (M >> kHistShift)], 1u);
      else
        atomicAdd(&ghist[wk * kHistBins + (M >> kHistShift)], 1u);
    }
  }

  // 3. flush the block's histogram.  The k0-th smallest M of the stream is
  // never in a higher bin than the k0-th smallest of a block that counted at
  // least k0 tokens, so every bin up to the global threshold bin still
  // receives every block's count; a block that counted fewer adds its bins up
  // to its largest M's (all it holds).
  if (LDS_HIST) {
    lds_barrier();
    const uint32_t tgt = min(ncount, (uint32_t)max(dv.k0, 0));
    for (int l2 = w; l2 < nw; l2 += NT / 64) {
      int32_t lim = -1;  // no count to add
      if (tgt > 0) {  // the low bins first (almost always there)
        uint32_t bb, bl;
        const uint4 v = reinterpret_cast<const uint4 *>(hist + l2 * kHistBins)[lane];
        if (!wave_find_bin_low(v, tgt, bb, bl)) wave_find_bin(hist + l2 * kHistBins, tgt, bb, bl);
        lim = (int32_t)bb;
      }
      if (lane == 0) blim[l2] = lim;
    }
    lds_barrier();
    if constexpr (GH == 1) {  // every thread takes bin tid of each walk in turn
      for (int l2 = 0; l2 < nw; ++l2) {
        const int lim = (int)blim[l2];
        for (int b = tid; b <= lim; b += NT) {
          const uint32_t h = hist[l2 * kHistBins + b];
          if (h) atomicAdd(&ghist[l2 * kHistBins + b], h);
        }
      }
    } else {  // GH * L walks: wave w takes walks w, w + NT/64, ..., a lane per bin
      for (int l2 = w; l2 < nw; l2 += NT / 64) {
        const int lim = (int)blim[l2];
        for (int b = lane; b <= lim; b += 64) {
          const uint32_t h = hist[l2 * kHistBins + b];
          if (h) atomicAdd(&ghist[l2 * kHistBins + b], h);
        }
      }
    }
  }

  // 4. the insert's stores: codes and list entries, the page rule, the pool
  if (ins) {
    if (tid < mL) insert_code_store(dv, s, nold, tid, nc[tid]);
    if (tid == 0) loc_s = insert_page_rule(dv, s, nold, cell_s, np0);
    __syncthreads();
    if (tid < d) insert_pool_store<DT>(dv, s, loc_s, tid, k_new, v_new);
  }
}

// Launches of the scan with every head of the GQA max mode's group in one
// block (ice_scan_heads.hip).  Returns false, launching nothing, when the
// group does not fit that layout (g not 2 or 4, g * L histograms beyond the
// block's LDS, more than 64 directions): the caller then runs one pass per
// head.
bool launch_scan_heads(const Dev &dv, int64_t n, const void *q, const void *k_new,
                       const void *v_new, hipStream_t st);

}  // namespace ice
