// The GQA max mode's code scan with every head of the group in one block
// (IceCache blog page, technical details: one prioritized-DCI search per
// head; the heads share each read of the codes).  Its own translation unit:
// these instantiations compile beside the query kernels.
#include "ice_scan_dev.h"

namespace ice {

template <int DT, int R, int NT, int GH>
static void launch_heads(const Dev &dv, int64_t n, const void *q, const void *k_new,
                         const void *v_new, hipStream_t st) {
  const int64_t nrange = (n + 2 * NT - 1) / (2 * NT);
  const dim3 grid((unsigned)dv.S, (unsigned)max(nrange, (int64_t)1), 1u);
  hipLaunchKernelGGL((k_qscan<DT, true, R, NT, false, GH>), grid, dim3(NT), 0, st, dv, n, q,
                     k_new, v_new, 1);
}

template <int DT, int NT, int GH>
static void launch_heads_r(const Dev &dv, int64_t n, const void *q, const void *k_new,
                           const void *v_new, hipStream_t st) {
  switch ((dv.mL + kPipe - 1) / kPipe) {
    case 1: launch_heads<DT, 1, NT, GH>(dv, n, q, k_new, v_new, st); break;
    case 2: launch_heads<DT, 2, NT, GH>(dv, n, q, k_new, v_new, st); break;
    case 3: launch_heads<DT, 3, NT, GH>(dv, n, q, k_new, v_new, st); break;
    default: launch_heads<DT, 4, NT, GH>(dv, n, q, k_new, v_new, st); break;  // mL <= 64
  }
}

template <int DT, int GH>
static void launch_heads_nt(const Dev &dv, int64_t n, const void *q, const void *k_new,
                            const void *v_new, hipStream_t st) {
  // one block per CU (its LDS holds g * L histograms): the smallest block
  // that gives every block a CU of its own, else the largest (the most waves
  // per CU)
  auto fits = [&](int nt) { return (int64_t)dv.S * ((n + 2 * nt - 1) / (2 * nt)) <= dv.ncu; };
  if (fits(512))
    launch_heads_r<DT, 512, GH>(dv, n, q, k_new, v_new, st);
  else if (fits(640))
    launch_heads_r<DT, 640, GH>(dv, n, q, k_new, v_new, st);
  else if (fits(768))
    launch_heads_r<DT, 768, GH>(dv, n, q, k_new, v_new, st);
  else
    launch_heads_r<DT, 1024, GH>(dv, n, q, k_new, v_new, st);
}

bool launch_scan_heads(const Dev &dv, int64_t n, const void *q, const void *k_new,
                       const void *v_new, hipStream_t st) {
  if (!dv.gmax || dv.mL > 64) return false;
  if (dv.g == 2 && dv.g * dv.L <= ScanWalks<2>::kLds) {
    if (dv.dtype == 0)
      launch_heads_nt<0, 2>(dv, n, q, k_new, v_new, st);
    else
      launch_heads_nt<1, 2>(dv, n, q, k_new, v_new, st);
    return true;
  }
  if (dv.g == 4 && dv.g * dv.L <= ScanWalks<4>::kLds) {
    if (dv.dtype == 0)
      launch_heads_nt<0, 4>(dv, n, q, k_new, v_new, st);
    else
      launch_heads_nt<1, 4>(dv, n, q, k_new, v_new, st);
    return true;
  }
  return false;
}

}  // namespace ice
