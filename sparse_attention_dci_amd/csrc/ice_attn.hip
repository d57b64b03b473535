// Sparse attention over every token of the selected pages (IceCache paper
// page, Figure 2 step (3)).
//
// The tokens of a stream's selected pages, taken page after page, are split
// into chunks of `tps` tokens; one block per (chunk, stream) stages the
// chunk's K and V rows in LDS (each page is p contiguous rows, so the copy is
// a run of 16-byte loads), forms the
// logits of all g query heads of the stream, and writes an fp32 softmax
// partial (max, sum, sum of weighted values).  A second kernel merges the
// partials of each head.
#include "ice_device.h"

namespace ice {

constexpr int kAttnMaxTps = 32;

template <int DT>
__global__ __launch_bounds__(256) void k_attn_part(Dev dv, const void *q,
                                                   const int32_t *page_ids,
                                                   const int32_t *n_pages) {
  const int s = blockIdx.y, sp = blockIdx.x;
  const int tid = threadIdx.x;
  const int d = dv.d, g = dv.g, p = dv.p, tps = dv.attn_tps;
  __shared__ float qs[kMaxGroup * 128];
  __shared__ float kt[kAttnMaxTps * 129];
  __shared__ float vt[kAttnMaxTps * 128];
  __shared__ float z[kMaxGroup * kAttnMaxTps];
  __shared__ float hm[kMaxGroup], hl[kMaxGroup];
  __shared__ int32_t rowpage[kAttnMaxTps];
  __shared__ int32_t rowok[kAttnMaxTps];

  const int np = min(n_pages[s], dv.P);
  for (int x = tid; x < g * d; x += 256)
    qs[x] = load_elem<DT>(q, (int64_t)s * g * d + x);
  if (tid < tps) {
    const int gt = sp * tps + tid;  // token of the concatenated selected pages
    const int pi = gt / p;
    const int slot = gt % p;
    int pg = -1, ok = 0;
    if (pi < np) {
      pg = page_ids[(int64_t)s * dv.P + pi];
      ok = (pg >= 0 && pg < dv.pcap) ? (slot < dv.page_len[(int64_t)s * dv.pcap + pg]) : 0;
    }
    rowpage[tid] = pg;
    rowok[tid] = ok;
  }
  __syncthreads();
  // stage rows (fp32 in LDS; K rows padded to 129 floats against bank conflicts)
  for (int x = tid; x < tps * (d / 8); x += 256) {
    const int r = x / (d / 8), c8 = (x % (d / 8)) * 8;
    float kx[8], vx[8];
    if (rowok[r]) {
      const int64_t row = ((int64_t)s * dv.pcap + rowpage[r]) * p + ((sp * tps + r) % p);
      load8<DT>(dv.pool_k, row * d + c8, kx);
      load8<DT>(dv.pool_v, row * d + c8, vx);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) kx[j] = vx[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      kt[r * 129 + c8 + j] = kx[j];
      vt[r * 128 + c8 + j] = vx[j];
    }
  }
  __syncthreads();
  const float scale = 1.0f / sqrtf((float)d);
  for (int x = tid; x < g * tps; x += 256) {
    const int h = x / tps, r = x % tps;
    float acc = 0.0f;
    const float *qh = qs + h * d;
    const float *kr = kt + r * 129;
    for (int e = 0; e < d; ++e) acc = fmaf(qh[e], kr[e], acc);
    z[h * tps + r] = rowok[r] ? acc * scale : -INFINITY;
  }
  __syncthreads();
  if (tid < g) {
    float mx = -INFINITY;
    for (int r = 0; r < tps; ++r) mx = fmaxf(mx, z[tid * tps + r]);
    float sum = 0.0f;
    for (int r = 0; r < tps; ++r) {
      const float w = mx == -INFINITY ? 0.0f : __expf(z[tid * tps + r] - mx);
      z[tid * tps + r] = w;
      sum += w;
    }
    hm[tid] = mx;
    hl[tid] = sum;
  }
  __syncthreads();
  float *part = dv.attn_part + ((int64_t)s * dv.attn_nsplit + sp) * g * (d + 2);
  for (int x = tid; x < g * d; x += 256) {
    const int h = x / d, e = x % d;
    float acc = 0.0f;
    for (int r = 0; r < tps; ++r) acc = fmaf(z[h * tps + r], vt[r * 128 + e], acc);
    part[h * (d + 2) + e] = acc;
  }
  if (tid < g) {
    part[tid * (d + 2) + d] = hm[tid];
    part[tid * (d + 2) + d + 1] = hl[tid];
  }
}

// One block per query head: merge the split partials.
__global__ __launch_bounds__(128) void k_attn_combine(Dev dv, float *out) {
  const int hq = blockIdx.x;  // s * g + h
  const int s = hq / dv.g, h = hq % dv.g;
  const int d = dv.d;
  const float *base = dv.attn_part + (int64_t)s * dv.attn_nsplit * dv.g * (d + 2);
  float M = -INFINITY;
  for (int sp = 0; sp < dv.attn_nsplit; ++sp)
    M = fmaxf(M, base[((int64_t)sp * dv.g + h) * (d + 2) + d]);
  for (int e = threadIdx.x; e < d; e += blockDim.x) {
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
      for (int sp = 0; sp < dv.attn_nsplit; ++sp) {
        const float *pp = base + ((int64_t)sp * dv.g + h) * (d + 2);
        const float mk = pp[d];
        if (mk == -INFINITY) continue;
        const float wgt = __expf(mk - M);
        num = fmaf(wgt, pp[e], num);
        den = fmaf(wgt, pp[d + 1], den);
      }
    }
    out[(int64_t)hq * d + e] = den > 0.0f ? num / den : 0.0f;
  }
}

template <int DT>
static hipError_t attn_impl(const Dev &dv, const void *q, const int32_t *page_ids,
                            const int32_t *n_pages, float *out, hipStream_t st, Timer *tm) {
  timer_begin(tm, st);
  hipLaunchKernelGGL(k_attn_part<DT>, dim3(dv.attn_nsplit, dv.S), dim3(256), 0, st, dv, q,
                     page_ids, n_pages);
  timer_mark(tm, KID_ATTN_PART, st);
  hipLaunchKernelGGL(k_attn_combine, dim3(dv.S * dv.g), dim3(128), 0, st, dv, out);
  timer_mark(tm, KID_ATTN_COMBINE, st);
  return hipGetLastError();
}

hipError_t launch_attn(const Dev &dv, const void *q, const int32_t *page_ids,
                       const int32_t *n_pages, float *out, hipStream_t st, Timer *tm) {
  return dv.dtype == 0 ? attn_impl<0>(dv, q, page_ids, n_pages, out, st, tm)
                       : attn_impl<1>(dv, q, page_ids, n_pages, out, st, tm);
}

}  // namespace ice
