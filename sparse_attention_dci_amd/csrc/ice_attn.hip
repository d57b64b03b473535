// Sparse attention over every token of the selected pages (IceCache paper
// page, Figure 2 step (3)).
//
// The tokens of a stream's selected pages, taken page after page, are cut
// into blocks of kAttnTpb = 256; a block is 8 waves of 32 tokens.  Both
// products run on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16, fp32
// accumulation), 16 query heads wide (heads past g are zero):
//   logits  S^T[token][head] = K rows x q^T: a lane feeds 8 consecutive key
//           elements of one token, read straight from the key pool;
//   values  O[head][e] = P x V: a lane feeds the probabilities of 8 tokens
//           for one head and the values of the same 8 tokens for one
//           element.  Those 8 tokens are two runs of 4 consecutive page
//           slots, which is why values are stored element-major inside a
//           page: each run is one 8-byte (bf16) or 16-byte (fp32) load.
// fp32 keys, values and queries enter as a bf16 pair hi + lo and take three
// products (hi*hi, hi*lo, lo*hi); probabilities always do, so the only
// precision loss against fp32 arithmetic is the dropped lo*lo term (relative
// 2^-16).  The softmax is exact per block (block-wide max); blocks of one
// stream are merged by a second kernel when the budget spans several.
#include "ice_device.h"

namespace ice {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAttnWaves = kAttnTpb / 32;
constexpr int kAttnThreads = kAttnWaves * 64;

__device__ __forceinline__ floatx4 mfma(u32x4 a, u32x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Round to nearest even bf16 (finite inputs), as the high 16 bits.
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Two floats -> packed bf16 pairs hi (x ~ hi) and lo (x - hi ~ lo).
__device__ __forceinline__ void split2(float x0, float x1, uint32_t &hi, uint32_t &lo) {
  const uint32_t h0 = bf16_rne(x0), h1 = bf16_rne(x1);
  const uint32_t l0 = bf16_rne(x0 - __uint_as_float(h0 << 16));
  const uint32_t l1 = bf16_rne(x1 - __uint_as_float(h1 << 16));
  hi = h0 | (h1 << 16);
  lo = l0 | (l1 << 16);
}

// Eight fp32 values -> bf16x8 hi and lo operands.
__device__ __forceinline__ void split8(const float (&x)[8], u32x4 &hi, u32x4 &lo) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t h, l;
    split2(x[2 * j], x[2 * j + 1], h, l);
    hi[j] = h;
    lo[j] = l;
  }
}

__device__ __forceinline__ u32x4 ld16(const void *p) {
  const uint4 v = *reinterpret_cast<const uint4 *>(p);
  return u32x4{v.x, v.y, v.z, v.w};
}

// Grid (attn_nsplit, S), 512 threads.  Wave w of block b takes tokens
// b*256 + w*32 .. +31 of the stream's selection.  Lane (G, c) = (lane / 16,
// lane % 16).
template <int DT, int D>
__global__ __launch_bounds__(kAttnThreads) void k_attn(Dev dv, const void *q,
                                                       const int32_t *page_ids,
                                                       const int32_t *n_pages, float *out) {
  constexpr int KK = D / 32;  // 32-element chunks of a key row
  constexpr int EB = D / 16;  // 16-element blocks of the output
  const int s = blockIdx.y, sp = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = lane >> 4, c = lane & 15;
  const int g = dv.g, p = dv.p, P = dv.P;
  const int64_t pcap = dv.pcap;
  __shared__ float smax[kAttnWaves][16], ssum[kAttnWaves][16];
  __shared__ float red[kAttnWaves][kMaxGroup * D];

  // 1. pages: the token this lane feeds to the logits (T0 + 16a + c) and the
  // slot runs it feeds to the values (T0 + 16a + 4G .. +3), a = 0, 1.  All
  // loads are unconditional; invalid pages read page 0 and are masked.
  const int T0 = sp * kAttnTpb + w * 32;
  const int np = min(n_pages[s], P);
  int32_t pgk[2], pgv[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    pgk[a] = page_ids[(int64_t)s * P + min((T0 + 16 * a + c) / p, P - 1)];
    pgv[a] = page_ids[(int64_t)s * P + min((T0 + 16 * a + 4 * G) / p, P - 1)];
  }
  bool okv[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const bool okk = (T0 + 16 * a + c) / p < np && pgk[a] >= 0 && pgk[a] < pcap;
    okv[a] = (T0 + 16 * a + 4 * G) / p < np && pgv[a] >= 0 && pgv[a] < pcap;
    pgk[a] = okk ? pgk[a] : 0;
    pgv[a] = okv[a] ? pgv[a] : 0;
  }
  int32_t plen[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) plen[a] = dv.page_len[(int64_t)s * pcap + pgv[a]];

  // 2. loads: key chunks, value runs, the query heads (zero past g)
  u32x4 kr[2][KK][DT == 0 ? 2 : 1];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int64_t row = ((int64_t)s * pcap + pgk[a]) * p + (T0 + 16 * a + c) % p;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int e0 = 32 * kk + 8 * G;
      if constexpr (DT == 0) {
        const float *kp = reinterpret_cast<const float *>(dv.pool_k) + row * D + e0;
        kr[a][kk][0] = ld16(kp);
        kr[a][kk][1] = ld16(kp + 4);
      } else {
        kr[a][kk][0] = ld16(reinterpret_cast<const uint16_t *>(dv.pool_k) + row * D + e0);
      }
    }
  }
  // value run of group a, output block eb: elements (16eb + c) of slots
  // (T0 + 16a + 4G) % p .. +3
  u32x4 vr[EB][DT == 0 ? 2 : 1];
#pragma unroll
  for (int eb = 0; eb < EB; ++eb) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int64_t col = (((int64_t)s * pcap + pgv[a]) * D + 16 * eb + c) * p +
                          (T0 + 16 * a + 4 * G) % p;
      if constexpr (DT == 0) {
        vr[eb][a] = ld16(reinterpret_cast<const float *>(dv.pool_v) + col);
      } else {
        const uint2 v2 = *reinterpret_cast<const uint2 *>(
            reinterpret_cast<const uint16_t *>(dv.pool_v) + col);
        vr[eb][0][2 * a] = v2.x;
        vr[eb][0][2 * a + 1] = v2.y;
      }
    }
  }
  const int hq = c < g ? c : 0;
  u32x4 qh[KK], ql[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int64_t o = ((int64_t)s * g + hq) * D + 32 * kk + 8 * G;
    if constexpr (DT == 0) {
      const float *qp = reinterpret_cast<const float *>(q) + o;
      const u32x4 x0 = ld16(qp), x1 = ld16(qp + 4);
      float f[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[j] = __uint_as_float(x0[j]);
        f[4 + j] = __uint_as_float(x1[j]);
      }
      split8(f, qh[kk], ql[kk]);
    } else {
      qh[kk] = ld16(reinterpret_cast<const uint16_t *>(q) + o);
      ql[kk] = u32x4{0u, 0u, 0u, 0u};
    }
    if (c >= g) qh[kk] = ql[kk] = u32x4{0u, 0u, 0u, 0u};
  }

  // 3. logits: lane (G, c) gets token T0 + 16a + 4G + i, head c, in z[a][i]
  const float scale = 1.0f / sqrtf((float)D);
  float z[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if constexpr (DT == 0) {
        float f[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f[j] = __uint_as_float(kr[a][kk][0][j]);
          f[4 + j] = __uint_as_float(kr[a][kk][1][j]);
        }
        u32x4 kh, kl;
        split8(f, kh, kl);
        acc = mfma(kh, qh[kk], acc);
        acc = mfma(kh, ql[kk], acc);
        acc = mfma(kl, qh[kk], acc);
      } else {
        acc = mfma(kr[a][kk][0], qh[kk], acc);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = (T0 + 16 * a + 4 * G + i) % p;
      z[a][i] = (okv[a] && slot < plen[a]) ? acc[i] * scale : -INFINITY;
    }
  }

  // 4. block-wide softmax pieces per head
  float mx = -INFINITY;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, z[a][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (lane < 16) smax[w][lane] = mx;
  lds_barrier();
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < kAttnWaves; ++k) M = fmaxf(M, smax[k][c]);
  float pr[2][4], lsum = 0.0f;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[a][i] = z[a][i] == -INFINITY ? 0.0f : __expf(z[a][i] - M);
      lsum += pr[a][i];
    }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (lane < 16) ssum[w][lane] = lsum;

  // 5. values: A = probabilities (head c; tokens of run 0 then run 1), B =
  // value runs (element 16eb + c; same tokens), output lane (G, c) holds
  // head 4G + i, element 16eb + c
  u32x4 ph, pl;
  {
    const float f[8] = {pr[0][0], pr[0][1], pr[0][2], pr[0][3],
                        pr[1][0], pr[1][1], pr[1][2], pr[1][3]};
    split8(f, ph, pl);
  }
  floatx4 o[EB];
#pragma unroll
  for (int eb = 0; eb < EB; ++eb) {
    floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float f[8];
    if constexpr (DT == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[j] = __uint_as_float(vr[eb][0][j]);
        f[4 + j] = __uint_as_float(vr[eb][1][j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[2 * j] = __uint_as_float(vr[eb][0][j] << 16);
        f[2 * j + 1] = __uint_as_float(vr[eb][0][j] & 0xffff0000u);
      }
    }
    // slots holding no token may hold any bytes (zero times NaN is NaN):
    // the token's logit is -inf exactly there, for every head
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (z[j >> 2][j & 3] == -INFINITY) f[j] = 0.0f;
    u32x4 vh, vl;
    split8(f, vh, vl);
    acc = mfma(ph, vh, acc);
    acc = mfma(pl, vh, acc);
    if constexpr (DT == 0) acc = mfma(ph, vl, acc);
    o[eb] = acc;
  }

  // 6. sum the waves (in wave order), normalise or leave a partial
#pragma unroll
  for (int eb = 0; eb < EB; ++eb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * G + i < g) red[w][(4 * G + i) * D + 16 * eb + c] = o[eb][i];
  lds_barrier();
  const int ns = dv.attn_nsplit;
  for (int x = tid; x < g * D; x += kAttnThreads) {
    const int h = x / D, e = x % D;
    float num = 0.0f, den = 0.0f, bm = -INFINITY;
#pragma unroll
    for (int k = 0; k < kAttnWaves; ++k) {
      num += red[k][x];
      den += ssum[k][h];
      bm = fmaxf(bm, smax[k][h]);
    }
    if (ns == 1) {
      out[((int64_t)s * g + h) * D + e] = den > 0.0f ? num / den : 0.0f;
    } else {
      float *pp = dv.attn_part + (((int64_t)s * ns + sp) * g + h) * (D + 2);
      pp[e] = num;
      if (e == 0) {
        pp[D] = bm;
        pp[D + 1] = den;
      }
    }
  }
}

// Merges the blocks of each stream: one block per stream.
template <int D>
__global__ __launch_bounds__(256) void k_attn_merge(Dev dv, float *out) {
  const int s = blockIdx.x, g = dv.g, ns = dv.attn_nsplit;
  const float *base = dv.attn_part + (int64_t)s * ns * g * (D + 2);
  for (int x = threadIdx.x; x < g * D; x += 256) {
    const int h = x / D, e = x % D;
    float M = -INFINITY;
    for (int k = 0; k < ns; ++k) M = fmaxf(M, base[((int64_t)k * g + h) * (D + 2) + D]);
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
      for (int k = 0; k < ns; ++k) {
        const float *pp = base + ((int64_t)k * g + h) * (D + 2);
        const float mk = pp[D];
        const float wgt = mk == -INFINITY ? 0.0f : __expf(mk - M);
        num = fmaf(wgt, pp[e], num);
        den = fmaf(wgt, pp[D + 1], den);
      }
    }
    out[((int64_t)s * g + h) * D + e] = den > 0.0f ? num / den : 0.0f;
  }
}

template <int DT, int D>
static hipError_t attn_impl(const Dev &dv, const void *q, const int32_t *page_ids,
                            const int32_t *n_pages, float *out, hipStream_t st, Timer *tm) {
  timer_begin(tm, st);
  hipLaunchKernelGGL((k_attn<DT, D>), dim3(dv.attn_nsplit, dv.S), dim3(kAttnThreads), 0, st, dv,
                     q, page_ids, n_pages, out);
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
