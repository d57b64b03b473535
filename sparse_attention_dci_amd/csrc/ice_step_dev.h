// Per-token arithmetic of a decode step shared by the standalone insert kernel
// and the scan kernel that runs the step's insert and query prep at its head.
//
// Query prep (IceCache paper page, Figure 2 step (2)): the query direction is
// q_kv = fp32 mean of the g heads (left fold, then times fp32(1/g)), and
// qcode_t = code(<q_kv, u_t[:d]> / |q_kv|), the dot product and the norm in
// fp64 in the blocked order below.  The new token's projections (key side)
// take element order, as the build's do.
//
// Insert (IceCache blog page, technical details: new tokens enter the tree
// with no rebuild): r_t = <k, u_t[:d]> in fp64, x_t = r_t / c +
// sqrt(max(0, 1 - |k|^2 / c^2)) u_t[d] with the stored c, code = code(x_t);
// the token enters every list after all equal codes (position n of the insert
// region); its cell is the sign pattern of r on the first D directions; it
// joins the last page of its cell while that page has room, else opens page
// number n_pages.
#pragma once

#include "ice_device.h"

namespace ice {

// fp64 chain sum_e a[e] * b[e * stride] over e < d (a multiple of 16), in
// ascending e, a and b in LDS.  A rolled loop over pairs of 8-element
// batches held in two register sets: each batch's reads are issued while the
// other batch is summed (the last read repeats the last batch), so the
// dependent fma chain rarely waits on LDS and few registers are used.
__device__ __forceinline__ double dot_chain(const float *a, const float *b, int stride, int d) {
  constexpr int B = 8;
  float a0[B], b0[B], a1[B], b1[B];
  auto rd = [&](float (&x)[B], float (&y)[B], int e) {
#pragma unroll
    for (int j = 0; j < B; ++j) {
      x[j] = a[e + j];
      y[j] = b[(e + j) * stride];
    }
  };
  auto sum = [](double z, const float (&x)[B], const float (&y)[B]) {
#pragma unroll
    for (int j = 0; j < B; ++j) z = fma((double)x[j], (double)y[j], z);
    return z;
  };
  rd(a0, b0, 0);
  double z = 0.0;
#pragma unroll 1
  for (int e0 = 0; e0 < d; e0 += 2 * B) {
    rd(a1, b1, e0 + B);
    z = sum(z, a0, b0);
    rd(a0, b0, min(e0 + 2 * B, d - B));
    z = sum(z, a1, b1);
  }
  return z;
}

// The query side's dot products (its projections and norm, and the rerank
// scores) take a fixed blocked order: elements in blocks of 16, each block
// summed in element order, then the block sums added pairwise, neighbours
// first.  A group of d/16 consecutive lanes computes one: lane j sums block j
// (the products are exact in fp64, so each fma rounds once, as an addition
// would), then xor-1, xor-2 and xor-4 exchanges add the pairs level by level.
// fp64 addition commutes, so every lane of the group ends with the same total.
__device__ __forceinline__ double tree_sum(double z, int nbk) {
  z += __shfl_xor(z, 1);
  if (nbk > 2) z += __shfl_xor(z, 2);
  if (nbk > 4) z += __shfl_xor(z, 4);
  return z;
}

// z + a[0] b[0] + ... + a[15] b[15], added in element order; a and b are
// 16-byte aligned runs of 16 floats (four vector reads each).  A query lane
// computes its block with z = 0; element-order chains continue z block by
// block.
__device__ __forceinline__ double fma16(const float *a, const float *b, double z) {
  float x[16], y[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 fa = reinterpret_cast<const float4 *>(a)[i];
    const float4 fb = reinterpret_cast<const float4 *>(b)[i];
    x[4 * i] = fa.x;
    x[4 * i + 1] = fa.y;
    x[4 * i + 2] = fa.z;
    x[4 * i + 3] = fa.w;
    y[4 * i] = fb.x;
    y[4 * i + 1] = fb.y;
    y[4 * i + 2] = fb.z;
    y[4 * i + 3] = fb.w;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) z = fma((double)x[i], (double)y[i], z);
  return z;
}

__device__ __forceinline__ float group_inv(int g) { return (float)__ddiv_rn(1.0, (double)g); }

__device__ __forceinline__ int32_t query_code(double z, double qsq) {
  const double qn = __dsqrt_rn(qsq);
  return to_code(qn > 0.0 ? __ddiv_rn(z, qn) : 0.0);
}

// inv_c = 1 / c and inv_c2 = 1 / c^2 of the stream, as stored at build.
__device__ __forceinline__ int32_t insert_code(double r, double ud, double nsq, double inv_c,
                                               double inv_c2) {
  double b = __dsub_rn(1.0, __dmul_rn(nsq, inv_c2));
  if (b < 0.0) b = 0.0;
  const double sv = __dsqrt_rn(b);
  return to_code(__dadd_rn(__dmul_rn(r, inv_c), __dmul_rn(sv, ud)));
}

// Code t of the new token n into the tiled codes and the tail of list t.
__device__ __forceinline__ void insert_code_store(const Dev &dv, int s, int64_t n, int t,
                                                  int32_t code) {
  dv.codes[code_index(dv.ntile, dv.mL, s, n, t)] = code;
  dv.list_code[((int64_t)s * dv.mL + t) * dv.ncap + n] = code;
  dv.list_id[((int64_t)s * dv.mL + t) * dv.ncap + n] = (int32_t)n;
}

// The page rule for token n in cell c, split in two so that a caller can
// decide first and write later (one thread).  np0 is npages[s] as loaded
// before.  The token's slot in the pool is pid * p + slot.
struct PagePick {
  int32_t cntc, pid, slot;
};

__device__ __forceinline__ PagePick insert_page_decide(const Dev &dv, int s, uint32_t c,
                                                       int32_t np0) {
  const int64_t ci = (int64_t)s * dv.ncell + c;
  const int32_t cntc = dv.cell_count[ci], last = dv.cell_last[ci];  // loaded together
  const int32_t slot = cntc & (dv.p - 1);
  return PagePick{cntc, slot == 0 ? np0 : last, slot};
}

__device__ __forceinline__ void insert_page_commit(const Dev &dv, int s, int64_t n, uint32_t c,
                                                   PagePick pk) {
  const int p = dv.p;
  const int64_t ci = (int64_t)s * dv.ncell + c;
  if (pk.slot == 0) {
    dv.npages[s] = pk.pid + 1;
    dv.cell_last[ci] = pk.pid;
    dv.page_cell[(int64_t)s * dv.pcap + pk.pid] = (int32_t)c;
  }
  dv.cell_count[ci] = pk.cntc + 1;
  dv.page_tokens[((int64_t)s * dv.pcap + pk.pid) * p + pk.slot] = (int32_t)n;
  dv.page_len[(int64_t)s * dv.pcap + pk.pid] = pk.slot + 1;
  dv.loc[(int64_t)s * dv.ncap + n] = pk.pid * p + pk.slot;
}

// Both at once; returns the token's slot in the pool (page * p + slot).
__device__ __forceinline__ int32_t insert_page_rule(const Dev &dv, int s, int64_t n, uint32_t c,
                                                    int32_t np0) {
  const PagePick pk = insert_page_decide(dv, s, c, np0);
  insert_page_commit(dv, s, n, c, pk);
  return pk.pid * dv.p + pk.slot;
}

// Element e of the new token's key row (at its slot) and value column
// ([page][e][slot]), copied from the caller's k_new and v_new.
template <int DT>
__device__ __forceinline__ void insert_pool_store(const Dev &dv, int s, int32_t lc, int e,
                                                  const void *k_new, const void *v_new) {
  const int d = dv.d, p = dv.p;
  const int64_t row = ((int64_t)s * dv.pcap * p + lc) * d;
  const int64_t vcol = ((int64_t)s * dv.pcap + lc / p) * d * p + (lc % p);
  if constexpr (DT == 0) {
    reinterpret_cast<float *>(dv.pool_k)[row + e] =
        reinterpret_cast<const float *>(k_new)[(int64_t)s * d + e];
    reinterpret_cast<float *>(dv.pool_v)[vcol + (int64_t)e * p] =
        reinterpret_cast<const float *>(v_new)[(int64_t)s * d + e];
  } else {
    reinterpret_cast<uint16_t *>(dv.pool_k)[row + e] =
        reinterpret_cast<const uint16_t *>(k_new)[(int64_t)s * d + e];
    reinterpret_cast<uint16_t *>(dv.pool_v)[vcol + (int64_t)e * p] =
        reinterpret_cast<const uint16_t *>(v_new)[(int64_t)s * d + e];
  }
}

}  // namespace ice
