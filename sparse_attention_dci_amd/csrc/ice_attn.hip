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

hipError_t launch_attn(const Dev &dv, const void *q, const int32_t *page_ids,
                       const int32_t *n_pages, float *out, hipStream_t st, Timer *tm) {
  if (dv.dtype == 0)
    return dv.d == 128 ? attn_impl<0, 128>(dv, q, page_ids, n_pages, out, st, tm)
                       : attn_impl<0, 64>(dv, q, page_ids, n_pages, out, st, tm);
  return dv.d == 128 ? attn_impl<1, 128>(dv, q, page_ids, n_pages, out, st, tm)
                     : attn_impl<1, 64>(dv, q, page_ids, n_pages, out, st, tm);
}

}  // namespace ice
