// Standalone sparse attention over every token of the selected pages
// (IceCache paper page, Figure 2 step (3)), for callers that pass their own
// page lists; a decode step runs the same wave routine (ice_attn_dev.h) inside
// the query finaliser instead.
//
// The tokens of a stream's selected pages, taken page after page, are cut
// into blocks of kAttnTpb = 256; a block is 16 waves of one 16-token chunk
// each (keys and values requested together), merged in LDS by their softmax
// maxima.  Blocks of one stream are merged by a second kernel when the
// budget spans several.  With one block per stream the arithmetic is the
// fused finaliser's, so both give identical outputs.
#include "ice_attn_dev.h"
#include "ice_step_dev.h"

namespace ice {

constexpr int kAttnWaves = kAttnTpb / kAttnChunk;
constexpr int kAttnThreads = kAttnWaves * 64;

// Grid (attn_nsplit, S), 1024 threads.  Block b covers tokens b*256 .. +255 of
// the stream's selection, one 16-token chunk per wave; its page numbers are
// staged in LDS first.  With one block per stream the block writes the
// output, else a partial (max, sum, values) per head for k_attn_merge.
// With `staged` (a host-offloaded pool) dv describes the staging area, in
// which the stream's selected pages sit in selection order: page j of the
// selection is staged page j.
template <int DT, int D>
__global__ __launch_bounds__(kAttnThreads) void k_attn(Dev dv, const void *q,
                                                       const int32_t *page_ids,
                                                       const int32_t *n_pages, float *out,
                                                       bool staged) {
  const int s = blockIdx.y, sp = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6;
  const int g = dv.g, p = dv.p, P = dv.P;
  constexpr int kWin = kAttnTpb / 8;  // pages of the block's window (p >= 8)
  __shared__ int32_t sel[kWin];
  __shared__ float wm[kAttnWaves * 16], wl[kAttnWaves * 16];
  __shared__ float red[kAttnWaves * kMaxGroup * D];
  const int pbase = sp * kAttnTpb / p;  // p divides kAttnTpb
  const int np = min(min(n_pages[s], P) - pbase, kAttnTpb / p);
  if (tid < kAttnTpb / p)
    sel[tid] = staged ? min(pbase + tid, P - 1) : page_ids[(int64_t)s * P + min(pbase + tid, P - 1)];
  u32x4 qh[D / 32], ql[D / 32];
  attn_load_q<DT, D>(dv, s, q, qh, ql);
  AttnWave<D> st;
  attn_init(st);
  __syncthreads();
  if (w * kAttnChunk < np * p)
    attn_chunk<DT, D, false, kAttnChunk / 16>(dv, s, w * kAttnChunk, sel, np, qh, ql, st);
  attn_publish(st, w, kAttnWaves, g, wm, wl, red);
  __syncthreads();
  const int ns = dv.attn_nsplit;
  for (int x = tid; x < g * D; x += kAttnThreads) {
    float M, num, den;
    attn_merge<D>(kAttnWaves, g, x, wm, wl, red, M, num, den);
    const int h = x / D, e = x % D;
    if (ns == 1) {
      out[(int64_t)s * g * D + x] = den > 0.0f ? num / den : 0.0f;
    } else {
      float *pp = dv.attn_part + (((int64_t)s * ns + sp) * g + h) * (D + 2);
      pp[e] = num;
      if (e == 0) {
        pp[D] = M;
        pp[D + 1] = den;
      }
    }
  }
}

// Merges the blocks of each stream: one block per stream.  The blocks'
// maxima and sums go to LDS first (one load per pair, all in flight), each
// head's weights are computed once, and the value loads of eight blocks are
// issued together; the sums run over the blocks in order.
constexpr int kMergeMaxSplit = kMaxBudget / kAttnTpb;

template <int D>
__global__ __launch_bounds__(256) void k_attn_merge(Dev dv, float *out) {
  const int s = blockIdx.x, g = dv.g, ns = dv.attn_nsplit;
  __shared__ float wgt[kMergeMaxSplit * kMaxGroup];  // the blocks' maxima, then weights
  __shared__ float sum[kMergeMaxSplit * kMaxGroup];  // the blocks' softmax sums
  __shared__ float den_s[kMaxGroup];
  const float *base = dv.attn_part + (int64_t)s * ns * g * (D + 2);
  for (int x = threadIdx.x; x < ns * g; x += 256) {  // x = k * g + h
    wgt[x] = base[(int64_t)x * (D + 2) + D];
    sum[x] = base[(int64_t)x * (D + 2) + D + 1];
  }
  __syncthreads();
  // per head: the common max, the weights exp(m_k - M), the weighted sum
  float mk_h = 0.0f;
  if (threadIdx.x < g) {
    const int h = threadIdx.x;
    float M = -INFINITY;
    for (int k = 0; k < ns; ++k) M = fmaxf(M, wgt[k * g + h]);
    float den = 0.0f;
    for (int k = 0; k < ns; ++k) {
      const float mk = wgt[k * g + h];
      const float wk = (M == -INFINITY || mk == -INFINITY) ? 0.0f : __expf(mk - M);
      den = fmaf(wk, sum[k * g + h], den);
    }
    den_s[h] = den;
    mk_h = M;
  }
  __syncthreads();
  if (threadIdx.x < g) {  // weights replace the maxima (every read of the maxima is done)
    const int h = threadIdx.x;
    for (int k = 0; k < ns; ++k) {
      const float mk = wgt[k * g + h];
      wgt[k * g + h] = (mk_h == -INFINITY || mk == -INFINITY) ? 0.0f : __expf(mk - mk_h);
    }
  }
  __syncthreads();
  for (int x = threadIdx.x; x < g * D; x += 256) {
    const int h = x / D, e = x % D;
    float num = 0.0f;
    for (int k0 = 0; k0 < ns; k0 += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = base[((int64_t)min(k0 + j, ns - 1) * g + h) * (D + 2) + e];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (k0 + j < ns) num = fmaf(wgt[(k0 + j) * g + h], v[j], num);
    }
    const float den = den_s[h];
    out[((int64_t)s * g + h) * D + e] = den > 0.0f ? num / den : 0.0f;
  }
}

// The selected pages of a host-offloaded pool into the staging area: block
// (j, s) copies page j of stream s's selection (its keys, then its values,
// each p*d contiguous elements) with 16-byte loads over the host link, and its
// valid-slot count (0 past the selection or for a page number outside the
// pool, whose tokens the attention then masks, as it does on the pool).
__global__ __launch_bounds__(256) void k_fetch_pages(Dev dv, const int32_t *page_ids,
                                                     const int32_t *n_pages) {
  const int j = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const int64_t P = dv.P;
  const int np = min(n_pages[s], dv.P);
  const int32_t pg = page_ids[(int64_t)s * P + j];
  const bool ok = j < np && pg >= 0 && pg < dv.pcap;
  if (tid == 0) dv.stage_len[(int64_t)s * P + j] = ok ? dv.page_len[(int64_t)s * dv.pcap + pg] : 0;
  if (!ok) return;
  const int64_t chunks = (int64_t)dv.p * dv.d * dv.elem / 16;  // per page, K or V
  const uint4 *srck = reinterpret_cast<const uint4 *>(dv.pool_k) + ((int64_t)s * dv.pcap + pg) * chunks;
  const uint4 *srcv = reinterpret_cast<const uint4 *>(dv.pool_v) + ((int64_t)s * dv.pcap + pg) * chunks;
  uint4 *dk = reinterpret_cast<uint4 *>(dv.stage_k) + ((int64_t)s * P + j) * chunks;
  uint4 *dvv = reinterpret_cast<uint4 *>(dv.stage_v) + ((int64_t)s * P + j) * chunks;
  for (int64_t x = tid; x < chunks; x += 256) {
    const uint4 a = srck[x], b = srcv[x];
    dk[x] = a;
    dvv[x] = b;
  }
}

template <int DT, int D>
static hipError_t attn_impl(const Dev &dv, const void *q, const int32_t *page_ids,
                            const int32_t *n_pages, float *out, hipStream_t st, Timer *tm) {
  timer_begin(tm, st);
  Dev da = dv;  // the pool the attention reads: the resident one, or the staged pages
  if (dv.offload) {
    hipLaunchKernelGGL(k_fetch_pages, dim3(dv.P, dv.S), dim3(256), 0, st, dv, page_ids, n_pages);
    timer_mark(tm, KID_FETCH, st);
    da.pool_k = dv.stage_k;
    da.pool_v = dv.stage_v;
    da.page_len = dv.stage_len;
    da.pcap = dv.P;
  }
  hipLaunchKernelGGL((k_attn<DT, D>), dim3(dv.attn_nsplit, dv.S), dim3(kAttnThreads), 0, st, da,
                     q, page_ids, n_pages, out, dv.offload != 0);
  timer_mark(tm, KID_ATTN, st);
  if (dv.attn_nsplit > 1) {
    hipLaunchKernelGGL(k_attn_merge<D>, dim3(dv.S), dim3(256), 0, st, dv, out);
    timer_mark(tm, KID_AMERGE, st);
  }
  return hipGetLastError();
}

// A decode step that reuses an earlier selection, in one kernel: one block of
// 16 waves per stream.  Wave 0 inserts the new token n (its projections, as
// k_insert computes them, the codes and list entries, and the page rule's
// decision), while waves 1-15 attend over the selected pages as they stand
// before the insert (the 16 chunks of a 256-token budget).  After a block
// barrier, past every attention load, wave 0 commits the page tables and the
// pool row; when the new token's page is among the selected ones, its logit
// and value enter each head's softmax with the waves' partial results.
// Results: the index as ice_insert leaves it; the attention as ice_insert +
// ice_sparse_attn give it up to the fp32 rounding of the added token (its
// logit summed in element order instead of the matrix cores' order).
template <int DT, int D>
__global__ __launch_bounds__(kAttnThreads) void k_reuse(Dev dv, int64_t n, const void *k_new,
                                                        const void *v_new, const void *q,
                                                        const int32_t *page_ids,
                                                        const int32_t *n_pages, float *out) {
  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = dv.g, p = dv.p, P = dv.P, mL = dv.mL, mLp = dv.mLp;
  constexpr int kWin = kAttnTpb / 8;
  __shared__ int32_t sel[kWin];
  __shared__ float wm[kAttnWaves * 16], wl[kAttnWaves * 16];
  union ReuseShared {
    float red[kAttnWaves * kMaxGroup * D];  // the waves' outputs (after the barrier)
    float dl[129 * kMaxMl];                 // directions [e][mLp] (before it)
  };
  __shared__ __attribute__((aligned(16))) ReuseShared u;
  __shared__ float kv[128];
  __shared__ double rs[kMaxMl + 1];  // r_t, then |k|^2 at mL
  __shared__ float zq[kMaxGroup];    // the new token's logit per head
  __shared__ int32_t incl_s;

  // loads of every wave before the first barrier: the window's pages, the
  // directions (all mL at once), the new key; wave 0 also the stream's scalars
  const int np = min(min(n_pages[s], P), kAttnTpb / p);
  if (tid < kAttnTpb / p) sel[tid] = page_ids[(int64_t)s * P + min(tid, P - 1)];
  const int tot4 = (D + 1) * (mLp / 4);
  for (int x = tid; x < tot4; x += kAttnThreads)
    reinterpret_cast<float4 *>(u.dl)[x] = reinterpret_cast<const float4 *>(dv.dirs32)[x];
  if (tid < D) kv[tid] = load_elem<DT>(k_new, (int64_t)s * D + tid);
  int32_t np0 = 0;
  double ic = 0.0, ic2 = 0.0;
  if (w == 0) {
    np0 = dv.npages[s];
    ic = dv.inv_c[s];
    ic2 = dv.inv_c2[s];
  }
  u32x4 qh[D / 32], ql[D / 32];
  attn_load_q<DT, D>(dv, s, q, qh, ql);
  AttnWave<D> st;
  attn_init(st);
  lds_barrier();

  uint32_t cell = 0;
  PagePick pk{0, 0, 0};
  if (w == 0) {
    // the projections in element order (as the build's and the insert's)
    for (int t = lane; t <= mL; t += 64)
      rs[t] = t < mL ? dot_chain(kv, u.dl + t, mLp, D) : dot_chain(kv, kv, 1, D);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    for (int t = lane; t < mL; t += 64)
      insert_code_store(dv, s, n, t, insert_code(rs[t], (double)u.dl[D * mLp + t], rs[mL], ic, ic2));
    const unsigned long long bal = __ballot(lane < dv.D && rs[lane < mL ? lane : 0] >= 0.0);
    cell = (uint32_t)bal & ((1u << dv.D) - 1u);
    if (lane == 0) pk = insert_page_decide(dv, s, cell, np0);
    // the new token's logit per head (element order, fp32), when it lands in a selected page
    // (as many times as the selection lists its page, as the separate calls attend it)
    const int32_t npg = __builtin_amdgcn_readfirstlane(pk.pid);
    const int cnt = popc64(__ballot(lane < np && sel[min(lane, kWin - 1)] == npg));
    if (lane == 0) incl_s = cnt;
    if (cnt > 0)
      for (int h = 0; h < g; ++h) {
        float z = 0.0f;
        for (int e = lane; e < D; e += 64)
          z = fmaf(load_elem<DT>(q, ((int64_t)s * g + h) * D + e), kv[e], z);
        for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
        if (lane == 0) zq[h] = z * (1.0f / sqrtf((float)D));
      }
  } else {
    for (int T0 = (w - 1) * kAttnChunk; T0 < np * p; T0 += (kAttnWaves - 1) * kAttnChunk)
      attn_chunk<DT, D, DT == 0, kAttnChunk / 16>(dv, s, T0, sel, np, qh, ql, st);
  }
  lds_barrier();  // every attention load is done and the directions are dead
  if (w == 0) {  // the insert's pool row and page tables
    if (lane == 0) insert_page_commit(dv, s, n, cell, pk);
    const int32_t lc = __builtin_amdgcn_readfirstlane(pk.pid * p + pk.slot);
    for (int e = lane; e < D; e += 64) insert_pool_store<DT>(dv, s, lc, e, k_new, v_new);
  }
  attn_publish(st, w, kAttnWaves, g, wm, wl, u.red);
  lds_barrier();
  const int cnt = incl_s;
  for (int x = tid; x < g * D; x += kAttnThreads) {
    float M, num, den;
    attn_merge<D>(kAttnWaves, g, x, wm, wl, u.red, M, num, den);
    const int h = x / D, e = x % D;
    if (cnt > 0) {  // the new token joins with weight exp(z - M'), M' the new common max
      const float z = zq[h];
      const float Mn = fmaxf(M, z);
      const float r = M == -INFINITY ? 0.0f : __expf(M - Mn);
      const float wn = (float)cnt * __expf(z - Mn);
      num = fmaf(wn, load_elem<DT>(v_new, (int64_t)s * D + e), num * r);
      den = fmaf(wn, 1.0f, den * r);
    }
    out[(int64_t)s * g * D + x] = den > 0.0f ? num / den : 0.0f;
  }
}

hipError_t launch_reuse(const Dev &dv, int64_t n, const void *k_new, const void *v_new,
                        const void *q, const int32_t *page_ids, const int32_t *n_pages,
                        float *out, hipStream_t st, Timer *tm) {
  timer_begin(tm, st);
  if (dv.dtype == 0) {
    if (dv.d == 128)
      hipLaunchKernelGGL((k_reuse<0, 128>), dim3(dv.S), dim3(kAttnThreads), 0, st, dv, n, k_new,
                         v_new, q, page_ids, n_pages, out);
    else
      hipLaunchKernelGGL((k_reuse<0, 64>), dim3(dv.S), dim3(kAttnThreads), 0, st, dv, n, k_new,
                         v_new, q, page_ids, n_pages, out);
  } else {
    if (dv.d == 128)
      hipLaunchKernelGGL((k_reuse<1, 128>), dim3(dv.S), dim3(kAttnThreads), 0, st, dv, n, k_new,
                         v_new, q, page_ids, n_pages, out);
    else
      hipLaunchKernelGGL((k_reuse<1, 64>), dim3(dv.S), dim3(kAttnThreads), 0, st, dv, n, k_new,
                         v_new, q, page_ids, n_pages, out);
  }
  timer_mark(tm, KID_REUSE, st);
  return hipGetLastError();
}

hipError_t launch_attn(const Dev &dv, const void *q, const int32_t *page_ids,
                       const int32_t *n_pages, float *out, hipStream_t st, Timer *tm) {
  if (dv.dtype == 0)
    return dv.d == 128 ? attn_impl<0, 128>(dv, q, page_ids, n_pages, out, st, tm)
                       : attn_impl<0, 64>(dv, q, page_ids, n_pages, out, st, tm);
  return dv.d == 128 ? attn_impl<1, 128>(dv, q, page_ids, n_pages, out, st, tm)
                     : attn_impl<1, 64>(dv, q, page_ids, n_pages, out, st, tm);
}

}  // namespace ice
