// Sparse attention over every token of the selected pages (IceCache paper
// page, Figure 2 step (3)).
//
// The tokens of a stream's selected pages, taken page after page, are split
// into chunks of kTps tokens; one block per (chunk, stream) stages the
// chunk's K and V rows in LDS (each page is p contiguous rows, so the copy is
// a run of 16-byte loads), forms the logits of all g query heads of the
// stream (each dot product split over up to 8 lanes), takes a half-wave
// softmax per head, and writes an fp32 partial (max, sum, weighted values).
// The last block of a stream to finish (a device-scope ticket taken after a
// release fence) merges the partials.
#include "ice_device.h"

namespace ice {

constexpr int kTps = 32;  // tokens per block

template <int DT>
__global__ __launch_bounds__(256) void k_attn(Dev dv, const void *q, const int32_t *page_ids,
                                              const int32_t *n_pages, float *out) {
  const int s = blockIdx.y, sp = blockIdx.x;
  const int tid = threadIdx.x;
  const int d = dv.d, g = dv.g, p = dv.p;
  __shared__ float qs[kMaxGroup * 128];
  __shared__ float kt[kTps * 129];
  __shared__ float vt[kTps * 128];
  __shared__ float z[kMaxGroup * kTps];
  __shared__ float hm[kMaxGroup], hl[kMaxGroup];
  __shared__ int32_t rowpage[kTps];
  __shared__ int32_t rowok[kTps];
  __shared__ uint32_t ticket;

  if (tid < kTps) {
    const int gt = sp * kTps + tid;  // token of the concatenated selected pages
    const int pi = gt / p;
    // the page id and the page count are loaded together
    const int32_t pg = page_ids[(int64_t)s * dv.P + min(pi, dv.P - 1)];
    const int np = min(n_pages[s], dv.P);
    rowpage[tid] = (pi < np && pg >= 0 && pg < dv.pcap) ? pg : -1;
  }
  for (int x = tid; x < g * d; x += 256) qs[x] = load_elem<DT>(q, (int64_t)s * g * d + x);
  __syncthreads();
  // stage rows (fp32 in LDS; K rows padded to 129 floats against bank conflicts);
  // the page length is loaded together with the row chunks
  for (int x = tid; x < kTps * (d / 8); x += 256) {
    const int r = x / (d / 8), c8 = (x % (d / 8)) * 8;
    const int pg = rowpage[r];
    const int pgc = pg >= 0 ? pg : 0;  // clamped: the loads are unconditional
    const int slot = (sp * kTps + r) % p;
    float kx[8], vx[8];
    const int64_t row = ((int64_t)s * dv.pcap + pgc) * p + slot;
    load8<DT>(dv.pool_k, row * d + c8, kx);
    load8<DT>(dv.pool_v, row * d + c8, vx);
    const bool ok = pg >= 0 && slot < dv.page_len[(int64_t)s * dv.pcap + pgc];
    if (!ok) {  // empty slots hold no token (and arbitrary bytes): zero them
#pragma unroll
      for (int j = 0; j < 8; ++j) kx[j] = vx[j] = 0.0f;
    }
    if (c8 == 0) rowok[r] = ok;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      kt[r * 129 + c8 + j] = kx[j];
      vt[r * 128 + c8 + j] = vx[j];
    }
  }
  __syncthreads();
  // logits: tp lanes per (head, token) pair
  const float scale = 1.0f / sqrtf((float)d);
  const int npair = g * kTps;
  int tp = 1;
  while (tp < 8 && tp * 2 * npair <= 256) tp *= 2;
  for (int x = tid; x < npair * tp; x += 256) {
    const int pair = x / tp, part = x % tp;
    const int h = pair / kTps, r = pair % kTps;
    const int chunk = d / tp, e0 = part * chunk;
    const float *qh = qs + h * d + e0;
    const float *kr = kt + r * 129 + e0;
    float acc = 0.0f;
#pragma unroll 16
    for (int e = 0; e < chunk; ++e) acc = fmaf(qh[e], kr[e], acc);
    for (int o = tp >> 1; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (part == 0) z[h * kTps + r] = rowok[r] ? acc * scale : -INFINITY;
  }
  __syncthreads();
  // softmax pieces per head, one half-wave per head
  for (int h0 = 0; h0 < g; h0 += 8) {
    const int h = h0 + (tid >> 5), r = tid & 31;
    if (h < g) {
      const float v = z[h * kTps + r];
      float mx = v;
      for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 32));
      const float e = mx == -INFINITY ? 0.0f : __expf(v - mx);
      float sum = e;
      for (int o = 16; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 32);
      z[h * kTps + r] = e;
      if (r == 0) {
        hm[h] = mx;
        hl[h] = sum;
      }
    }
  }
  __syncthreads();
  float *part = dv.attn_part + ((int64_t)s * dv.attn_nsplit + sp) * g * (d + 2);
  for (int x = tid; x < g * d; x += 256) {
    const int h = x / d, e = x % d;
    float acc = 0.0f;
#pragma unroll
    for (int r = 0; r < kTps; ++r) acc = fmaf(z[h * kTps + r], vt[r * 128 + e], acc);
    part[h * (d + 2) + e] = acc;
  }
  if (tid < g) {
    part[tid * (d + 2) + d] = hm[tid];
    part[tid * (d + 2) + d + 1] = hl[tid];
  }

  // The last split of the stream to finish merges every split's partial.
  __threadfence();
  __syncthreads();
  if (tid == 0) ticket = atomicAdd(&dv.attn_done[s], 1u);
  __syncthreads();
  if (ticket != (uint32_t)dv.attn_nsplit - 1u) return;
  __threadfence();
  const float *base = dv.attn_part + (int64_t)s * dv.attn_nsplit * g * (d + 2);
  const int ns = dv.attn_nsplit;
  for (int x = tid; x < g * d; x += 256) {
    const int h = x / d, e = x % d;
    float M = -INFINITY;
#pragma unroll 8
    for (int k = 0; k < ns; ++k) M = fmaxf(M, base[((int64_t)k * g + h) * (d + 2) + d]);
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
#pragma unroll 8
      for (int k = 0; k < ns; ++k) {
        const float *pp = base + ((int64_t)k * g + h) * (d + 2);
        const float mk = pp[d];
        const float wgt = mk == -INFINITY ? 0.0f : __expf(mk - M);
        num = fmaf(wgt, pp[e], num);
        den = fmaf(wgt, pp[d + 1], den);
      }
    }
    out[((int64_t)s * g + h) * d + e] = den > 0.0f ? num / den : 0.0f;
  }
  if (tid == 0) dv.attn_done[s] = 0;
}

template <int DT>
static hipError_t attn_impl(const Dev &dv, const void *q, const int32_t *page_ids,
                            const int32_t *n_pages, float *out, hipStream_t st, Timer *tm) {
  timer_begin(tm, st);
  hipLaunchKernelGGL(k_attn<DT>, dim3(dv.attn_nsplit, dv.S), dim3(256), 0, st, dv, q, page_ids,
                     n_pages, out);
  timer_mark(tm, KID_ATTN, st);
  return hipGetLastError();
}

hipError_t launch_attn(const Dev &dv, const void *q, const int32_t *page_ids,
                       const int32_t *n_pages, float *out, hipStream_t st, Timer *tm) {
  return dv.dtype == 0 ? attn_impl<0>(dv, q, page_ids, n_pages, out, st, tm)
                       : attn_impl<1>(dv, q, page_ids, n_pages, out, st, tm);
}

}  // namespace ice
