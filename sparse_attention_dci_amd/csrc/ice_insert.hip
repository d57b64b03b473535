// The standalone dynamic insert (ice_insert): one block per stream projects
// the new key on the m*L directions and enters it in the lists, the tree's
// pages and the pool (the arithmetic is in ice_step_dev.h).  A decode step
// runs the same insert inside its scan kernel instead.  The directions are
// staged in LDS 32 at a time; wave 0 runs the 32 fp64 chains r_t, thread 128
// the chain |k|^2.
#include "ice_step_dev.h"

namespace ice {

constexpr int kInsThreads = 256;

template <int DT>
__global__ __launch_bounds__(kInsThreads) void k_insert(Dev dv, int64_t n, const void *k_new,
                                                        const void *v_new) {
  constexpr int NT = kInsThreads;
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int d = dv.d, mL = dv.mL;
  __shared__ float kv[128];
  __shared__ float dl[129 * 32];  // directions t0 .. t0+31 as [e][32]; row d is u_t[d]
  __shared__ double rs[kMaxMl], ud[kMaxMl];
  __shared__ double nsq_s;
  __shared__ int32_t loc_s;

  const int32_t np0 = dv.npages[s];
  const double ic = dv.inv_c[s], ic2 = dv.inv_c2[s];
  const float kx = load_elem<DT>(k_new, (int64_t)s * d + min(tid, d - 1));
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
  if (tid < d) kv[tid] = kx;
  __syncthreads();
  if (tid == 128) nsq_s = dot_chain(kv, kv, 1, d);
  for (int t0 = 0; t0 < mL; t0 += 32) {
    if (t0 > 0) {
      __syncthreads();
      stage(t0);
      __syncthreads();
    }
    if (tid < 32 && t0 + tid < mL) {
      rs[t0 + tid] = dot_chain(kv, dl + tid, 32, d);
      ud[t0 + tid] = (double)dl[d * 32 + tid];
    }
  }
  __syncthreads();

  __shared__ uint32_t cell_s;
  if (tid < 64) {  // cell = sign bits of r on the first D directions (D <= 13)
    const unsigned long long bal = __ballot(tid < dv.D && rs[tid < mL ? tid : 0] >= 0.0);
    if (tid == 0) cell_s = (uint32_t)bal & ((1u << dv.D) - 1u);
  }
  if (tid < mL)
    insert_code_store(dv, s, n, tid, insert_code(rs[tid], ud[tid], nsq_s, ic, ic2));
  __syncthreads();
  if (tid == 0) loc_s = insert_page_rule(dv, s, n, cell_s, np0);
  __syncthreads();
  if (tid < d) insert_pool_store<DT>(dv, s, loc_s, tid, k_new, v_new);
}

hipError_t launch_insert(const Dev &dv, int64_t n, const void *k_new, const void *v_new,
                         hipStream_t st, Timer *tm) {
  timer_begin(tm, st);
  if (dv.dtype == 0)
    hipLaunchKernelGGL(k_insert<0>, dim3(dv.S), dim3(kInsThreads), 0, st, dv, n, k_new, v_new);
  else
    hipLaunchKernelGGL(k_insert<1>, dim3(dv.S), dim3(kInsThreads), 0, st, dv, n, k_new, v_new);
  timer_mark(tm, KID_INSERT, st);
  return hipGetLastError();
}

}  // namespace ice
