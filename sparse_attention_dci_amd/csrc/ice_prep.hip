// Per-stream work at the head of a decode step: the dynamic insert of the new
// token (IceCache blog page, technical details: the tree takes new tokens
// with no rebuild) and the query's projection codes (IceCache paper page,
// Figure 2 step (2)).  Both project a vector on the same m*L directions, so
// one block per stream stages each round of 32 directions in LDS once and
// runs both sets of fp64 chains side by side:
//   wave 0  r_t = <k, u_t[:d]>      wave 1  z_t = <q_kv, u_t[:d]>
//   wave 2  |k|^2                   wave 3  |q_kv|^2
// every chain in ascending element order (each product of two values that
// fp32 holds exactly is exact in fp64).
//   insert  x_t = r_t / c + sqrt(max(0, 1 - |k|^2 / c^2)) u_t[d] with the
//           stored c; code = round(x_t * 2^29) saturated; the token enters
//           every list after all equal codes (position n of the insert
//           region); its cell is the sign pattern of r on the first D
//           directions; it joins the last page of its cell while that page
//           has room, else opens page number n_pages;
//   query   q_kv = fp32 mean of the g heads (left fold, then times
//           fp32(1/g)); qcode_t = code(z_t / |q_kv|); the query's counters
//           are cleared for the scan.
#include "ice_device.h"

namespace ice {

constexpr int kPrepThreads = 256;
constexpr int kPrepIns = 1, kPrepQry = 2;

template <int DT>
__global__ __launch_bounds__(kPrepThreads) void k_prep(Dev dv, int64_t n, const void *k_new,
                                                       const void *v_new, const void *q,
                                                       int mode) {
  constexpr int NT = kPrepThreads;
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int d = dv.d, mL = dv.mL, p = dv.p, g = dv.g, L = dv.L;
  const bool ins = (mode & kPrepIns) != 0, qry = (mode & kPrepQry) != 0;
  __shared__ float kv[128];
  __shared__ float qs[kMaxGroup * 128];
  __shared__ float qkv[128];
  __shared__ float dl[129 * 32];  // directions t0 .. t0+31 as [e][32]; row d is u_t[d]
  __shared__ double rs[kMaxMl], ud[kMaxMl], zs[kMaxMl];
  __shared__ double nsq_s, qsq_s;
  __shared__ uint32_t cell_s;
  __shared__ int32_t loc_s;

  // 1. loads, all issued before any is used: the page count (for the
  // insert's page rule), the key, the heads, directions 0..31
  const int32_t np0 = dv.npages[s];
  float kx = 0.0f;
  if (ins) kx = load_elem<DT>(k_new, (int64_t)s * d + min(tid, d - 1));
  constexpr int kHeadIters = kMaxGroup * 128 / NT;
  float hv[kHeadIters];
  const int gd = g * d;
  if (qry) {
#pragma unroll
    for (int k = 0; k < kHeadIters; ++k)
      hv[k] = load_elem<DT>(q, (int64_t)s * gd + min(tid + NT * k, gd - 1));
  }
  auto stage = [&](int t0) {
    constexpr int kIters = (129 * 8 + NT - 1) / NT;
    const int tot = (d + 1) * 8;  // float4 units
    float4 v[kIters];
#pragma unroll
    for (int k = 0; k < kIters; ++k) {
      const int x = min(tid + NT * k, tot - 1);
      v[k] = *reinterpret_cast<const float4 *>(dv.dirs32 + (int64_t)(x >> 3) * dv.mLp + t0 +
                                               (x & 7) * 4);
    }
#pragma unroll
    for (int k = 0; k < kIters; ++k) {
      const int x = tid + NT * k;
      if (x < tot) *reinterpret_cast<float4 *>(dl + (x >> 3) * 32 + (x & 7) * 4) = v[k];
    }
  };
  stage(0);
  if (ins && tid < d) kv[tid] = kx;
  if (qry) {
#pragma unroll
    for (int k = 0; k < kHeadIters; ++k)
      if (tid + NT * k < gd) qs[tid + NT * k] = hv[k];
  }
  __syncthreads();
  if (qry && tid < d) {
    const float inv_g = (float)__ddiv_rn(1.0, (double)g);
    float acc = qs[tid];
    for (int h = 1; h < g; ++h) acc = __fadd_rn(acc, qs[h * d + tid]);
    qkv[tid] = __fmul_rn(acc, inv_g);
  }
  __syncthreads();

  // 2. the chains
  if (ins && tid == 128) {
    double a = 0.0;
#pragma unroll 8
    for (int e = 0; e < d; ++e) a = fma((double)kv[e], (double)kv[e], a);
    nsq_s = a;
  }
  if (qry && tid == 192) {
    double a = 0.0;
#pragma unroll 8
    for (int e = 0; e < d; ++e) a = fma((double)qkv[e], (double)qkv[e], a);
    qsq_s = a;
  }
  for (int t0 = 0; t0 < mL; t0 += 32) {
    if (t0 > 0) {
      __syncthreads();
      stage(t0);
      __syncthreads();
    }
    if (ins && tid < 32 && t0 + tid < mL) {
      double r = 0.0;
#pragma unroll 8
      for (int e = 0; e < d; ++e) r = fma((double)kv[e], (double)dl[e * 32 + tid], r);
      rs[t0 + tid] = r;
      ud[t0 + tid] = (double)dl[d * 32 + tid];
    }
    if (qry && tid >= 64 && tid < 96 && t0 + tid - 64 < mL) {
      const int j = tid - 64;
      double z = 0.0;
#pragma unroll 8
      for (int e = 0; e < d; ++e) z = fma((double)qkv[e], (double)dl[e * 32 + j], z);
      zs[t0 + j] = z;
    }
  }
  __syncthreads();

  // 3. the query's codes and counters
  if (qry) {
    if (tid < mL) {
      const double qn = __dsqrt_rn(qsq_s);
      const double qb = qn > 0.0 ? __ddiv_rn(zs[tid], qn) : 0.0;
      dv.qcode[(int64_t)s * mL + tid] = to_code(qb);
    }
    if (tid < d) dv.qkv[(int64_t)s * d + tid] = qkv[tid];
    if (tid < L) {
      dv.cand_count[s * L + tid] = 0;
      dv.bnd_count[s * L + tid] = 0;
    }
    if (tid == 0) dv.rr_count[s] = 0;
  }
  if (!ins) return;

  // 4. the insert: codes and list entries, the page rule, the pool
  if (tid < 64) {  // cell = sign bits of r on the first D directions (D <= 13)
    const unsigned long long bal = __ballot(tid < dv.D && rs[tid < mL ? tid : 0] >= 0.0);
    if (tid == 0) cell_s = (uint32_t)bal & ((1u << dv.D) - 1u);
  }
  if (tid < mL) {
    double b = __dsub_rn(1.0, __dmul_rn(nsq_s, dv.inv_c2[s]));
    if (b < 0.0) b = 0.0;
    const double sv = __dsqrt_rn(b);
    const double x = __dadd_rn(__dmul_rn(rs[tid], dv.inv_c[s]), __dmul_rn(sv, ud[tid]));
    const int32_t code = to_code(x);
    dv.codes[code_index(dv.ntile, mL, s, n, tid)] = code;
    dv.list_code[((int64_t)s * mL + tid) * dv.ncap + n] = code;
    dv.list_id[((int64_t)s * mL + tid) * dv.ncap + n] = (int32_t)n;
  }
  __syncthreads();
  if (tid == 0) {
    const uint32_t c = cell_s;
    const int64_t ci = (int64_t)s * dv.ncell + c;
    const int32_t cntc = dv.cell_count[ci], last = dv.cell_last[ci];  // loaded together
    const int32_t slot = cntc & (p - 1);
    int32_t pid = last;
    if (slot == 0) {
      pid = np0;
      dv.npages[s] = np0 + 1;
      dv.cell_last[ci] = pid;
      dv.page_cell[(int64_t)s * dv.pcap + pid] = (int32_t)c;
    }
    dv.cell_count[ci] = cntc + 1;
    dv.page_tokens[((int64_t)s * dv.pcap + pid) * p + slot] = (int32_t)n;
    dv.page_len[(int64_t)s * dv.pcap + pid] = slot + 1;
    const int32_t lc = pid * p + slot;
    dv.loc[(int64_t)s * dv.ncap + n] = lc;
    loc_s = lc;
  }
  __syncthreads();
  // key row at its slot; value element e at [page][e][slot]
  const int64_t row = ((int64_t)s * dv.pcap * p + loc_s) * d;
  const int64_t vcol = ((int64_t)s * dv.pcap + loc_s / p) * d * p + (loc_s % p);
  if (tid < d) {
    if constexpr (DT == 0) {
      reinterpret_cast<float *>(dv.pool_k)[row + tid] = kv[tid];
      reinterpret_cast<float *>(dv.pool_v)[vcol + (int64_t)tid * p] =
          reinterpret_cast<const float *>(v_new)[(int64_t)s * d + tid];
    } else {
      reinterpret_cast<uint16_t *>(dv.pool_k)[row + tid] =
          reinterpret_cast<const uint16_t *>(k_new)[(int64_t)s * d + tid];
      reinterpret_cast<uint16_t *>(dv.pool_v)[vcol + (int64_t)tid * p] =
          reinterpret_cast<const uint16_t *>(v_new)[(int64_t)s * d + tid];
    }
  }
}

hipError_t launch_prep(const Dev &dv, int64_t n, const void *k_new, const void *v_new,
                       const void *q, int mode, hipStream_t st) {
  if (dv.dtype == 0)
    hipLaunchKernelGGL(k_prep<0>, dim3(dv.S), dim3(kPrepThreads), 0, st, dv, n, k_new, v_new, q,
                       mode);
  else
    hipLaunchKernelGGL(k_prep<1>, dim3(dv.S), dim3(kPrepThreads), 0, st, dv, n, k_new, v_new, q,
                       mode);
  return hipGetLastError();
}

hipError_t launch_insert(const Dev &dv, int64_t n, const void *k_new, const void *v_new,
                         hipStream_t st, Timer *tm) {
  timer_begin(tm, st);
  hipError_t e = launch_prep(dv, n, k_new, v_new, nullptr, kPrepIns, st);
  timer_mark(tm, KID_PREP, st);
  return e;
}

}  // namespace ice
