// Wave-level sparse attention over 32-token chunks of a stream's selected
// pages (IceCache paper page, Figure 2 step (3)), shared by the standalone
// attention kernel and the fused query finaliser.
//
// Both products run on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16, fp32
// accumulation), 16 query heads wide (heads past g are zero).  Lane (G, c) =
// (lane / 16, lane % 16):
//   logits  S^T[token][head] = K rows x q^T: the lane feeds 8 consecutive key
//           elements of token T0 + 16a + c (a = 0, 1) and receives the logits
//           of tokens T0 + 16a + 4G + i (i = 0..3) for head c;
//   values  O[head][e] = P x V: the lane feeds the probabilities of those 8
//           tokens for head c and the values of the same 8 tokens for
//           element 16eb + c; they are two runs of 4 consecutive page slots,
//           which is why values are stored element-major inside a page (one
//           8-byte or 16-byte load per run).  The lane accumulates head
//           4G + i, element 16eb + c.
// fp32 keys, values and queries enter as a bf16 pair hi + lo and take three
// products (hi*hi, hi*lo, lo*hi); probabilities always do, so the only loss
// against fp32 arithmetic is the dropped lo*lo term (relative 2^-16).  The
// softmax is online per wave (running max and sum per head); waves are
// merged at the end with their maxima.
#pragma once

#include "ice_device.h"

namespace ice {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma_bf16(u32x4 a, u32x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Round to nearest even bf16 (finite inputs), as the high 16 bits.
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Eight fp32 values -> bf16x8 operands hi (x ~ hi) and lo (x - hi ~ lo).
__device__ __forceinline__ void split8(const float (&x)[8], u32x4 &hi, u32x4 &lo) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t h0 = bf16_rne(x[2 * j]), h1 = bf16_rne(x[2 * j + 1]);
    const uint32_t l0 = bf16_rne(x[2 * j] - __uint_as_float(h0 << 16));
    const uint32_t l1 = bf16_rne(x[2 * j + 1] - __uint_as_float(h1 << 16));
    hi[j] = h0 | (h1 << 16);
    lo[j] = l0 | (l1 << 16);
  }
}

__device__ __forceinline__ u32x4 ld16(const void *p) {
  const uint4 v = *reinterpret_cast<const uint4 *>(p);
  return u32x4{v.x, v.y, v.z, v.w};
}

// Running state of one wave: softmax max and sum of head c (lane % 16) and
// the unnormalised output rows 4G + i, elements 16eb + c.
template <int D>
struct AttnWave {
  float m, l;
  floatx4 o[D / 16];
};

// The query operands of head c (zero past g), hi and lo (lo is zero for bf16).
template <int DT, int D>
__device__ __forceinline__ void attn_load_q(const Dev &dv, int s, const void *q, u32x4 (&qh)[D / 32],
                                            u32x4 (&ql)[D / 32]) {
  const int lane = __lane_id(), G = lane >> 4, c = lane & 15, g = dv.g;
  const int hq = c < g ? c : 0;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
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
}

template <int D>
__device__ __forceinline__ void attn_init(AttnWave<D> &st) {
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int eb = 0; eb < D / 16; ++eb) st.o[eb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
}

// Tokens T0 .. T0+16*NA-1 of the stream's selection (pages sel[0..np), p
// tokens each, page after page): NA = 2 for 32-token chunks, 1 for 16-token
// chunks (the second half of the values product is then zero).  Every load is
// unconditional: tokens past the selection, on invalid page numbers or in
// empty slots read page 0 and are masked (their logit is -inf and their
// values are zeroed, since empty slots may hold any bytes).  LATE_V issues
// the value loads after the logits (one more round trip, about 30 fewer
// registers).
template <int DT, int D, bool LATE_V = false, int NA = 2>
__device__ __forceinline__ void attn_chunk(const Dev &dv, int s, int T0, const int32_t *sel,
                                           int np, const u32x4 (&qh)[D / 32],
                                           const u32x4 (&ql)[D / 32], AttnWave<D> &st) {
  constexpr int KK = D / 32, EB = D / 16;
  const int lane = __lane_id(), G = lane >> 4, c = lane & 15;
  const int p = dv.p, lp = dv.lp, pm = dv.p - 1;  // p is a power of two
  const int64_t pcap = dv.pcap;
  int32_t pgk[2], pgv[2];
  bool okv[2] = {false, false};
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    const int pik = (T0 + 16 * a + c) >> lp, piv = (T0 + 16 * a + 4 * G) >> lp;
    const int32_t pk = sel[min(pik, np - 1)], pv = sel[min(piv, np - 1)];
    const bool okk = pik < np && pk >= 0 && pk < pcap;
    okv[a] = piv < np && pv >= 0 && pv < pcap;
    pgk[a] = okk ? pk : 0;
    pgv[a] = okv[a] ? pv : 0;
  }
  int32_t plen[2] = {0, 0};
  u32x4 kr[NA][KK][DT == 0 ? 2 : 1];
  u32x4 vr[EB][DT == 0 ? 2 : 1];
#pragma unroll
  for (int eb = 0; eb < EB; ++eb)
#pragma unroll
    for (int x = 0; x < (DT == 0 ? 2 : 1); ++x) vr[eb][x] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int a = 0; a < NA; ++a) plen[a] = dv.page_len[(int64_t)s * pcap + pgv[a]];
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    const int64_t row = ((int64_t)s * pcap + pgk[a]) * p + ((T0 + 16 * a + c) & pm);
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
  auto load_v = [&]() {
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) {
#pragma unroll
      for (int a = 0; a < NA; ++a) {
        const int64_t col =
            (((int64_t)s * pcap + pgv[a]) * D + 16 * eb + c) * p + ((T0 + 16 * a + 4 * G) & pm);
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
  };
  if (!LATE_V) load_v();

  // logits of tokens T0 + 16a + 4G + i, head c
  const float scale = 1.0f / sqrtf((float)D);
  float z[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) z[1][i] = -INFINITY;
#pragma unroll
  for (int a = 0; a < NA; ++a) {
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
        acc = mfma_bf16(kh, qh[kk], acc);
        acc = mfma_bf16(kh, ql[kk], acc);
        acc = mfma_bf16(kl, qh[kk], acc);
      } else {
        acc = mfma_bf16(kr[a][kk][0], qh[kk], acc);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = (T0 + 16 * a + 4 * G + i) & pm;
      z[a][i] = (okv[a] && slot < plen[a]) ? acc[i] * scale : -INFINITY;
    }
  }

  if (LATE_V) load_v();

  // online softmax of head c
  float cm = -INFINITY;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) cm = fmaxf(cm, z[a][i]);
  cm = fmaxf(cm, __shfl_xor(cm, 16));
  cm = fmaxf(cm, __shfl_xor(cm, 32));
  const float mnew = fmaxf(st.m, cm);
  const float rescale = mnew == -INFINITY ? 1.0f : __expf(st.m - mnew);
  float pr[2][4], ls = 0.0f;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[a][i] = z[a][i] == -INFINITY ? 0.0f : __expf(z[a][i] - mnew);
      ls += pr[a][i];
    }
  ls += __shfl_xor(ls, 16);
  ls += __shfl_xor(ls, 32);
  st.l = st.l * rescale + ls;
  st.m = mnew;
  float rs_row[4];  // the rescale of the rows this lane accumulates (heads 4G + i)
#pragma unroll
  for (int i = 0; i < 4; ++i) rs_row[i] = __shfl(rescale, 4 * G + i);

  // values
  u32x4 ph, pl;
  {
    const float f[8] = {pr[0][0], pr[0][1], pr[0][2], pr[0][3],
                        pr[1][0], pr[1][1], pr[1][2], pr[1][3]};
    split8(f, ph, pl);
  }
  // a token's logit is -inf exactly where it is masked, for every head; bf16
  // values are already the operand, so masking their packed words is all
  uint32_t vmask[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    vmask[j] = (z[(2 * j) >> 2][(2 * j) & 3] == -INFINITY ? 0u : 0x0000ffffu) |
               (z[(2 * j + 1) >> 2][(2 * j + 1) & 3] == -INFINITY ? 0u : 0xffff0000u);
#pragma unroll
  for (int eb = 0; eb < EB; ++eb) {
    u32x4 vh, vl;
    if constexpr (DT == 0) {
      float f[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[j] = __uint_as_float(vr[eb][0][j]);
        f[4 + j] = __uint_as_float(vr[eb][1][j]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (z[j >> 2][j & 3] == -INFINITY) f[j] = 0.0f;
      split8(f, vh, vl);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) vh[j] = vr[eb][0][j] & vmask[j];
    }
    floatx4 acc = st.o[eb];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= rs_row[i];
    acc = mfma_bf16(ph, vh, acc);
    acc = mfma_bf16(pl, vh, acc);
    if constexpr (DT == 0) acc = mfma_bf16(ph, vl, acc);
    st.o[eb] = acc;
  }
}

// Publishes a wave's state to LDS: wm/wl [nw][16], red [nw][g][D] (then the
// rows of heads g..15 of every wave, which nothing reads: red holds
// nw * 16 * D floats, and the stores need no per-head branch).
template <int D>
__device__ __forceinline__ void attn_publish(const AttnWave<D> &st, int w, int nw, int g, float *wm,
                                             float *wl, float *red) {
  const int lane = __lane_id(), G = lane >> 4, c = lane & 15;
  if (lane < 16) {
    wm[w * 16 + lane] = st.m;
    wl[w * 16 + lane] = st.l;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * G + i;
    const int64_t row = r < g ? (int64_t)w * g + r : (int64_t)nw * g + (int64_t)w * (16 - g) + (r - g);
#pragma unroll
    for (int eb = 0; eb < D / 16; ++eb) red[row * D + 16 * eb + c] = st.o[eb][i];
  }
}

// Merge of nw published waves for output element x = h * D + e: the common
// max M, the numerator and the softmax sum relative to M.
template <int D>
__device__ __forceinline__ void attn_merge(int nw, int g, int x, const float *wm, const float *wl,
                                           const float *red, float &M, float &num, float &den) {
  const int h = x / D;
  M = -INFINITY;
  for (int k = 0; k < nw; ++k) M = fmaxf(M, wm[k * 16 + h]);
  num = 0.0f;
  den = 0.0f;
  if (M == -INFINITY) return;
  for (int k = 0; k < nw; ++k) {
    const float mk = wm[k * 16 + h];
    const float wgt = mk == -INFINITY ? 0.0f : __expf(mk - M);
    num = fmaf(wgt, red[(int64_t)k * g * D + x], num);
    den = fmaf(wgt, wl[k * 16 + h], den);
  }
}

}  // namespace ice
