// Prefill indexing and the per-token insert (IceCache paper page, Figure 2
// step (1); blog page, technical details: the tree takes new tokens without
// a rebuild).
//
// Build = directions to fp64 -> key norms (max -> c) -> projection codes and
// tree cells -> per-direction LSD radix sort -> pages in token order -> pool
// scatter.  Every floating-point step reproduces a fixed fp64 evaluation
// order (products of key and direction elements are exact in fp64), so the
// codes, lists, cells and pages are bit-identical to a sequential CPU
// evaluation of the same definitions.
#include "ice_device.h"

namespace ice {

// ---------------------------------------------------------------- fills

__global__ void k_fill_i32(int32_t *p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void k_fill_u64(unsigned long long *p, int64_t n, unsigned long long v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

static hipError_t fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

// ---------------------------------------------------------------- directions

// dirs [mL][d+1] (dtype) -> [nchunk][d+1][16] fp64, zero past mL.
template <int DT>
__global__ void k_dirs(Dev dv, const void *dirs) {
  const int64_t total = (int64_t)dv.nchunk * (dv.d + 1) * kDirChunk;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < total;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(x % kDirChunk);
    const int64_t r = x / kDirChunk;
    const int e = (int)(r % (dv.d + 1));
    const int ch = (int)(r / (dv.d + 1));
    const int t = ch * kDirChunk + j;
    dv.dirs[x] = t < dv.mL ? (double)load_elem<DT>(dirs, (int64_t)t * (dv.d + 1) + e) : 0.0;
  }
  // fp32 copy, element-major (every value is exact in fp32)
  const int64_t total32 = (int64_t)(dv.d + 1) * dv.mLp;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < total32;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int e = (int)(x / dv.mLp), t = (int)(x % dv.mLp);
    dv.dirs32[x] = t < dv.mL ? load_elem<DT>(dirs, (int64_t)t * (dv.d + 1) + e) : 0.0f;
  }
}

// ---------------------------------------------------------------- norms

// |k|^2 of every key row (fp64, ascending element order), kept for the
// projection, and the largest per stream, as the bit pattern of a
// non-negative double (order-preserving as an integer).  A block
// stages kNormRows consecutive key rows in LDS with coalesced 16-byte loads
// (word-major, odd stride: the chain reads of one row per lane fall in
// distinct banks), then one thread per row runs the chain, its reads a batch
// ahead of the dependent fma.
template <int DT>
struct NormRows {
  static constexpr int kRows = DT == 0 ? 128 : 256;  // rows staged per block
  static constexpr int kMaxWords = DT == 0 ? 128 : 64;  // words of a d = 128 row
  static constexpr int kStride = kRows + 1;            // odd
};

// Stages key rows r0 .. r0 + kRows - 1 of stream s (clamped to n - 1) in LDS,
// word w of row r at w * kStride + r, with coalesced 16-byte loads.
template <int DT>
__device__ __forceinline__ void stage_rows(const Dev &dv, const void *K, int s, int64_t n,
                                           int64_t r0, uint32_t *rows) {
  constexpr int R = NormRows<DT>::kRows, ST = NormRows<DT>::kStride;
  const int tid = threadIdx.x;
  const int words = dv.d * (DT == 0 ? 4 : 2) / 4;
  const int cpr = words / 4;  // 16-byte chunks per row
  const char *kb = reinterpret_cast<const char *>(K) + (int64_t)s * n * words * 4;
  constexpr int kIter = R * NormRows<DT>::kMaxWords / 4 / 256;
  uint4 v[kIter];
#pragma unroll
  for (int k = 0; k < kIter; ++k) {  // clamped, unconditional loads
    const int x = tid + 256 * k;
    const int r = x / cpr, c = x % cpr;
    const int64_t row = min(r0 + (r < R ? r : R - 1), n - 1);
    v[k] = reinterpret_cast<const uint4 *>(kb + row * words * 4)[c];
  }
#pragma unroll
  for (int k = 0; k < kIter; ++k) {
    const int x = tid + 256 * k;
    const int r = x / cpr, c = x % cpr;
    if (r < R) {
      uint32_t *dst = rows + (4 * c) * ST + r;
      dst[0] = v[k].x;
      dst[ST] = v[k].y;
      dst[2 * ST] = v[k].z;
      dst[3 * ST] = v[k].w;
    }
  }
}

// fp64 sum of squares of a staged row (ascending element order), the reads
// a batch ahead of the dependent fma.
template <int DT>
__device__ __forceinline__ double row_norm2(const uint32_t *rw, int words) {
  constexpr int B = 8, ST = NormRows<DT>::kStride;
  uint32_t a0[B], a1[B];
  auto rd = [&](uint32_t (&x)[B], int w0) {
#pragma unroll
    for (int j = 0; j < B; ++j) x[j] = rw[(w0 + j) * ST];
  };
  auto sum = [](double acc, const uint32_t (&x)[B]) {
#pragma unroll
    for (int j = 0; j < B; ++j) {
      if constexpr (DT == 0) {
        const double f = (double)__uint_as_float(x[j]);
        acc = fma(f, f, acc);  // f*f is exact
      } else {
        const double lo = (double)__uint_as_float(x[j] << 16);
        const double hi = (double)__uint_as_float(x[j] & 0xffff0000u);
        acc = fma(lo, lo, acc);
        acc = fma(hi, hi, acc);
      }
    }
    return acc;
  };
  double nsq = 0.0;
  rd(a0, 0);
#pragma unroll 1
  for (int w0 = 0; w0 < words; w0 += 2 * B) {
    rd(a1, w0 + B);
    nsq = sum(nsq, a0);
    rd(a0, min(w0 + 2 * B, words - B));
    nsq = sum(nsq, a1);
  }
  return nsq;
}

template <int DT>
__global__ __launch_bounds__(256) void k_norms(Dev dv, BuildScratch bs, const void *K, int64_t n) {
  constexpr int R = NormRows<DT>::kRows;
  __shared__ uint32_t rows[NormRows<DT>::kMaxWords * NormRows<DT>::kStride];
  __shared__ unsigned long long wmax[4];
  const int s = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * R;
  stage_rows<DT>(dv, K, s, n, r0, rows);
  __syncthreads();
  double nsq = 0.0;
  if (tid < R && r0 + tid < n) {
    nsq = row_norm2<DT>(rows + tid, dv.d * (DT == 0 ? 4 : 2) / 4);
    bs.nsq[(int64_t)s * n + r0 + tid] = nsq;
  }
  unsigned long long b = (unsigned long long)__double_as_longlong(nsq);
  for (int off = 32; off >= 1; off >>= 1) {
    unsigned long long o = __shfl_xor(b, off);
    b = o > b ? o : b;
  }
  if (lane == 0) wmax[w] = b;
  __syncthreads();
  if (tid == 0) {
    unsigned long long m = wmax[0];
    for (int k = 1; k < 4; ++k) m = wmax[k] > m ? wmax[k] : m;
    atomicMax(&dv.maxnsq[s], m);
  }
}

// ---------------------------------------------------------------- projection

// c, 1/c and 1/c^2 of stream s: the fixed bound, or the largest key norm
// rounded to fp32 (1 when every key is zero).
__device__ __forceinline__ float stream_bound(const Dev &dv, int s, float c_fixed) {
  if (c_fixed > 0.0f) return c_fixed;
  const double mx = __longlong_as_double((long long)dv.maxnsq[s]);
  const float c = (float)__dsqrt_rn(mx);
  return c > 0.0f ? c : 1.0f;
}

// Projection on the fp64 matrix cores.  v_mfma_f64_16x16x4f64 adds the four
// products of its k-slice to the accumulator one after another, in k order,
// each addition rounded (checked on gfx950 against sequential fma chains, also
// with operands spread over 2^-40 .. 2^12), so a chain of HD/4 of them over
// k = 0 .. HD-1 is the chain r_t = fma(k_e, u_te, r_t), ascending e, bit for
// bit.  Every product of a key element and a direction element is exact in
// fp64.  Then
//   x_t = r_t * (1/c) + sqrt(max(0, 1 - |k|^2 (1/c)^2)) * u_td
//   code_t = round(x_t * 2^29), saturated; cell = sign bits of r_t, t < D.
//
// A wave takes 16 tokens and every one of the NC chunks of 16 directions
// (the keys are read once).  Lane (q, j) = (lane / 16, lane % 16):
//   A  keys: lane (q, j) supplies element 4kk + q of token t0 + j; it loads
//      the whole row in 16-byte pieces (the four lanes of a token share the
//      addresses) and picks the elements of its residue q;
//   B  directions, staged in LDS once per block as [NC][HD][16]: lane (q, j)
//      supplies u_{16ct + j, 4kk + q}, 512 contiguous bytes per wave;
//   D  lane (q, j), register r: token t0 + q + 4r, direction 16ct + j.
// The waves of a block take consecutive tiles, so a block writes 64
// consecutive tokens of every direction.  |k|^2 comes from k_norms.  (More
// tiles per wave, for more independent chains, measured slower.)
template <int DT, int HD>
struct ProjRow {
  static constexpr int kChunks = HD * (DT == 0 ? 4 : 2) / 16;  // 16-byte pieces per key row
};

template <int DT, int HD>
__device__ __forceinline__ void proj_load_row(const char *kb, int64_t row, uint4 (&v)[ProjRow<DT, HD>::kChunks]) {
  constexpr int CH = ProjRow<DT, HD>::kChunks;
  const uint4 *rp = reinterpret_cast<const uint4 *>(kb + row * (int64_t)CH * 16);
#pragma unroll
  for (int c = 0; c < CH; ++c) v[c] = rp[c];
}

// Element 4kk + q of the row held in v, as a double (q = lane / 16).
template <int DT, int HD>
__device__ __forceinline__ double proj_elem(const uint4 (&v)[ProjRow<DT, HD>::kChunks], int kk,
                                            int q) {
  if constexpr (DT == 0) {  // piece kk holds elements 4kk .. 4kk+3
    const uint4 x = v[kk];
    const uint32_t lo = (q & 1) ? x.y : x.x, hi = (q & 1) ? x.w : x.z;
    return (double)__uint_as_float((q & 2) ? hi : lo);
  } else {  // piece kk/2 holds elements 8(kk/2) .. +7; ours is 4(kk&1) + q in it
    const uint4 x = v[kk >> 1];
    const uint32_t wd = (kk & 1) ? ((q & 2) ? x.w : x.z) : ((q & 2) ? x.y : x.x);
    return (double)__uint_as_float((q & 1) ? (wd & 0xffff0000u) : (wd << 16));
  }
}

typedef double doublex4 __attribute__((ext_vector_type(4)));

template <int DT, int HD, int NC>
__global__ __launch_bounds__(256) void k_project(Dev dv, BuildScratch bs,
                                                 const void *__restrict__ K, int64_t n,
                                                 float c_fixed) {
  constexpr int CH = ProjRow<DT, HD>::kChunks;
  __shared__ double su[NC * HD * kDirChunk];
  const int s = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q = lane >> 4, j = lane & 15;
  const int mL = dv.mL;
  const float c = stream_bound(dv, s, c_fixed);
  const double inv_c = __ddiv_rn(1.0, (double)c);
  const double inv_c2 = __dmul_rn(inv_c, inv_c);
  if (blockIdx.x == 0 && tid == 0) {
    dv.norm_c[s] = c;
    dv.inv_c[s] = inv_c;
    dv.inv_c2[s] = inv_c2;
  }
  if (n == 0) return;
  for (int x = tid; x < NC * HD * kDirChunk; x += 256) {  // rows e < HD of every chunk
    const int ct = x / (HD * kDirChunk), r = x % (HD * kDirChunk);
    su[x] = dv.dirs[(int64_t)ct * (HD + 1) * kDirChunk + r];
  }
  double ud[NC];  // u_{16ct + j, HD}
#pragma unroll
  for (int ct = 0; ct < NC; ++ct) ud[ct] = dv.dirs[((int64_t)ct * (HD + 1) + HD) * kDirChunk + j];
  __syncthreads();

  const char *kb = reinterpret_cast<const char *>(K) + (int64_t)s * n * CH * 16;
  const int64_t ntiles = (n + 15) / 16, stride = (int64_t)gridDim.x * 4;
  for (int64_t tile = (int64_t)blockIdx.x * 4 + w; tile < ntiles; tile += stride) {
    const int64_t t0 = tile * 16;
    uint4 cur[CH];
    proj_load_row<DT, HD>(kb, min(t0 + j, n - 1), cur);
    double nsq[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) nsq[r] = bs.nsq[(int64_t)s * n + min(t0 + q + 4 * r, n - 1)];
    doublex4 acc[NC];
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) acc[ct] = doublex4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kk = 0; kk < HD / 4; ++kk) {
      const double a = proj_elem<DT, HD>(cur, kk, q);
#pragma unroll
      for (int ct = 0; ct < NC; ++ct)
        acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(
            a, su[(ct * HD + 4 * kk + q) * kDirChunk + j], acc[ct], 0, 0, 0);
      // keeps the direction reads from being hoisted all at once (registers)
      if ((kk & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t tok = t0 + q + 4 * r;
      double bb = __dsub_rn(1.0, __dmul_rn(nsq[r], inv_c2));
      if (bb < 0.0) bb = 0.0;
      const double sv = __dsqrt_rn(bb);
      // cell: sign bits of the first D directions (D <= 16: chunk 0)
      const unsigned long long nonneg = __ballot(j < dv.D && acc[0][r] >= 0.0);
      if (j == 0 && tok < n)
        bs.cell[(int64_t)s * n + tok] = (uint32_t)(nonneg >> (16 * q)) & 0xffffu;
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        const int t = ct * kDirChunk + j;
        const double x = __dadd_rn(__dmul_rn(acc[ct][r], inv_c), __dmul_rn(sv, ud[ct]));
        if (t < mL && tok < n) {
          const int32_t code = to_code(x);
          dv.codes[code_index(dv.ntile, mL, s, tok, t)] = code;
          bs.codes_dm[((int64_t)s * mL + t) * n + tok] = code;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- list sort

// Exclusive scan over the 256 digits: thread tid < 256 holds digit tid's
// value (the rest pass 0 and ignore the result).  Every thread of the block
// calls it (two barriers inside).
template <int NT>
__device__ __forceinline__ uint32_t digit_excl_scan(uint32_t v, uint32_t *wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63 && w < 4) wsum[w] = incl;
  __syncthreads();
  uint32_t pre = 0;
  for (int k = 0; k < w && k < 4; ++k) pre += wsum[k];
  __syncthreads();
  return pre + incl - v;
}

// One block sorts one (stream, direction) list ascending by (code, token):
// four stable LSD passes of 8 bits over the order-preserving unsigned image
// of the code.  Pass 0 reads the direction-major codes with implicit tokens;
// passes alternate between the scratch pair and the index lists, ending in
// the index lists.  The four digit histograms come from one initial pass (a
// pass never changes the multiset of keys).  A pass walks the list in tiles
// of NT x ITEMS entries; wave w owns the tile's w-th part (64 x ITEMS
// consecutive entries), row j of it being 64 consecutive entries:
//   ranks  row by row, lanes with equal digits are matched with ballots and
//          ranked after the wave's running count of that digit (LDS, updated
//          by each digit's last lane); per digit (one thread each) the waves'
//          counts, prefix-summed over the waves, and the digits' starts in
//          the tile complete every entry's stable rank within the tile;
//   stage  the tile is written to LDS in digit order;
//   write  consecutive threads copy consecutive staged entries to their
//          digit's running position in the output, so each digit's run goes
//          out as one coalesced stretch instead of one scattered word per
//          entry.
// Larger blocks mean fewer tiles per pass, and each tile pays the same chain
// of round trips and barriers: 1024 x 12 sorts the 36k layer's lists in
// 188 us and the 262k layer's in 4.2 ms (256 x 16: 310 us and 5.1 ms; a sweep
// of 512-1024 threads x 8-24 items put 1024 x 12 first for both).
constexpr int kSortThreads = 1024, kSortItems = 12;

template <int NT, int ITEMS>
__global__ __launch_bounds__(NT) void k_sort_lists(Dev dv, BuildScratch bs, int64_t n) {
  constexpr int NW = NT / 64, TILE = NT * ITEMS, PART = TILE / NW;
  static_assert(NT >= 256, "one thread per digit");
  const int lst = blockIdx.x;  // s * mL + t
  const int s = lst / dv.mL, t = lst % dv.mL;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool digit = tid < 256;  // this thread owns digit tid
  const int32_t *in0 = bs.codes_dm + (int64_t)lst * n;
  int32_t *tc = bs.tmp_code + (int64_t)lst * n;
  int32_t *ti = bs.tmp_id + (int64_t)lst * n;
  int32_t *oc = dv.list_code + ((int64_t)s * dv.mL + t) * dv.ncap;
  int32_t *oi = dv.list_id + ((int64_t)s * dv.mL + t) * dv.ncap;

  __shared__ uint32_t ghist[4][256];
  __shared__ uint32_t gbase[256], ls[256];
  __shared__ uint32_t cntw[NW][256];
  __shared__ uint32_t skey[TILE];
  __shared__ int32_t sval[TILE];
  __shared__ uint32_t wsum[4];

  for (int x = tid; x < 4 * 256; x += NT) ghist[x >> 8][x & 255] = 0;
  __syncthreads();
  for (int64_t x = tid; x < n; x += NT) {
    const uint32_t key = (uint32_t)in0[x] ^ 0x80000000u;
#pragma unroll
    for (int k = 0; k < 4; ++k) atomicAdd(&ghist[k][(key >> (8 * k)) & 255u], 1u);
  }
  __syncthreads();
  const unsigned long long lt = lanemask_lt();

  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 8 * pass;
    const int32_t *sc = pass == 0 ? in0 : ((pass & 1) ? tc : oc);
    const int32_t *si = pass == 0 ? nullptr : ((pass & 1) ? ti : oi);
    int32_t *dc = (pass & 1) ? oc : tc;
    int32_t *di = (pass & 1) ? oi : ti;
    {
      const uint32_t gb = digit_excl_scan<NT>(digit ? ghist[pass][tid] : 0u, wsum);
      if (digit) gbase[tid] = gb;
    }

    for (int64_t t0 = 0; t0 < n; t0 += TILE) {
      const int nv = (int)min((int64_t)TILE, n - t0);
      uint32_t key[ITEMS];
      int32_t val[ITEMS];
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {  // clamped, unconditional loads
        const int64_t x = t0 + w * PART + j * 64 + lane;
        const int64_t xc = x < n ? x : n - 1;
        key[j] = (uint32_t)sc[xc] ^ 0x80000000u;
        val[j] = si ? si[xc] : (int32_t)x;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) cntw[w][q * 64 + lane] = 0;
      __builtin_amdgcn_wave_barrier();
      // ranks inside the wave's part, row by row
      uint32_t rank[ITEMS];
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        const bool valid = w * PART + j * 64 + lane < nv;
        const uint32_t dig = (key[j] >> shift) & 255u;
        const unsigned long long mt = match_bits(dig, 8, __ballot(valid));
        const uint32_t before = valid ? cntw[w][dig] : 0u;
        rank[j] = before + (uint32_t)popc64(mt & lt);
        __builtin_amdgcn_wave_barrier();
        if (valid && ((mt >> lane) >> 1) == 0ull) cntw[w][dig] = before + (uint32_t)popc64(mt);
        __builtin_amdgcn_wave_barrier();
      }
      __syncthreads();
      // per digit: the waves' offsets, the tile count and the digit's start
      uint32_t run = 0;
      if (digit) {
#pragma unroll
        for (int k = 0; k < NW; ++k) {
          const uint32_t c = cntw[k][tid];
          cntw[k][tid] = run;
          run += c;
        }
      }
      {
        const uint32_t st = digit_excl_scan<NT>(run, wsum);  // (barriers inside)
        if (digit) ls[tid] = st;
      }
      __syncthreads();
      // stage in digit order
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        if (w * PART + j * 64 + lane < nv) {
          const uint32_t dig = (key[j] >> shift) & 255u;
          const uint32_t pos = ls[dig] + cntw[w][dig] + rank[j];
          skey[pos] = key[j];
          sval[pos] = val[j];
        }
      }
      __syncthreads();
      // write each digit's run out contiguously
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        const int x = j * NT + tid;
        if (x < nv) {
          const uint32_t k2 = skey[x];
          const uint32_t dig = (k2 >> shift) & 255u;
          const uint32_t gpos = gbase[dig] + (uint32_t)x - ls[dig];
          dc[gpos] = (int32_t)(k2 ^ 0x80000000u);
          di[gpos] = sval[x];
        }
      }
      __syncthreads();
      if (digit) gbase[tid] += run;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- pages

// The tree's leaves as pages: each cell's tokens, in token order, cut into
// pages of p, pages numbered by their first token (which is what inserting
// the tokens one by one gives).  In parallel over chunks of kPageChunk tokens:
//   k_cell_count   per chunk, the tokens of each cell (LDS histogram);
//   k_cell_scan    per cell (a lane) and stream, the count of the cell in all
//                  earlier chunks (four waves split the chunks, then pass the
//                  carry), the cell totals and page counts, and per chunk the
//                  pages its tokens open (the ranks that are multiples of p);
//   k_page_prefix  per stream, the prefix sums of those: every chunk's first
//                  page id, every cell's first entry in the page_of table;
//   k_cell_rank    one wave per chunk walks it 64 tokens at a time: a token's
//                  rank in its cell = its cell's count before the chunk + the
//                  same-cell tokens before it in the chunk (ballots); openers
//                  (rank a multiple of p) number their pages;
//   k_page_fill    every token's page and slot from its rank.

__global__ __launch_bounds__(256) void k_cell_count(Dev dv, BuildScratch bs, int64_t n, int cmax) {
  extern __shared__ int32_t hc[];
  const int s = blockIdx.y;
  const int64_t k = blockIdx.x, nchunk = gridDim.x;
  const int ncell = (int)dv.ncell;
  for (int c = threadIdx.x; c < ncell; c += 256) hc[c] = 0;
  __syncthreads();
  const uint32_t *cells = bs.cell + (int64_t)s * n;
  const int64_t i0 = k * kPageChunk;
  for (int64_t i = i0 + threadIdx.x; i < min(i0 + kPageChunk, n); i += 256)
    atomicAdd(&hc[cells[i]], 1);
  __syncthreads();
  int32_t *out = bs.chunk_cnt + ((int64_t)s * nchunk + k) * cmax;
  for (int c = threadIdx.x; c < ncell; c += 256) out[c] = hc[c];
}

// grid (ceil(ncell / 64), S), 256 threads; LDS: nchunk counters
__global__ __launch_bounds__(256) void k_cell_scan(Dev dv, BuildScratch bs, int64_t nchunk,
                                                   int cmax) {
  extern __shared__ int32_t opk[];
  __shared__ int32_t qsum[4][64];
  constexpr int B = 16;
  const int s = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ncell = (int)dv.ncell, p = dv.p;
  const int c = blockIdx.x * 64 + lane;
  const bool cv = c < ncell;
  const int cl = cv ? c : 0;
  int32_t *cc = bs.chunk_cnt + (int64_t)s * nchunk * cmax;
  for (int64_t k = tid; k < nchunk; k += 256) opk[k] = 0;
  const int64_t q0 = nchunk * w / 4, q1 = nchunk * (w + 1) / 4;
  int32_t sum = 0;
  for (int64_t k0 = q0; k0 < q1; k0 += B) {  // this wave's quarter: its sum
    int32_t x[B];
#pragma unroll
    for (int j = 0; j < B; ++j) x[j] = cc[min(k0 + j, q1 - 1) * cmax + cl];
#pragma unroll
    for (int j = 0; j < B; ++j) sum += k0 + j < q1 ? x[j] : 0;
  }
  qsum[w][lane] = sum;
  __syncthreads();
  int32_t tot = 0;
  for (int u = 0; u < w; ++u) tot += qsum[u][lane];
  for (int64_t k0 = q0; k0 < q1; k0 += B) {  // counts before each chunk; pages opened
    int32_t x[B];
#pragma unroll
    for (int j = 0; j < B; ++j) x[j] = cc[min(k0 + j, q1 - 1) * cmax + cl];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      if (k0 + j < q1 && cv) {
        cc[(k0 + j) * cmax + c] = tot;
        const int32_t opened = (tot + x[j] + p - 1) / p - (tot + p - 1) / p;
        if (opened) atomicAdd(&opk[k0 + j], opened);
        tot += x[j];
      }
    }
  }
  __syncthreads();
  for (int64_t k = tid; k < nchunk; k += 256)
    if (opk[k]) atomicAdd(&bs.chunk_pg[(int64_t)s * (nchunk + 1) + k], opk[k]);
  if (w == 0 && cv) {
    const int32_t total = qsum[0][lane] + qsum[1][lane] + qsum[2][lane] + qsum[3][lane];
    dv.cell_count[(int64_t)s * ncell + c] = total;
    if (total == 0) dv.cell_last[(int64_t)s * ncell + c] = -1;
    bs.cell_pg[(int64_t)s * (cmax + 1) + c] = (total + p - 1) / p;
  }
}

// Exclusive prefix of x[0..m) in place (one 1024-thread block); returns the total.
__device__ int32_t block_prefix_1024(int32_t *x, int64_t m, int32_t *wsum) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t per = (m + 1023) / 1024;
  const int64_t b = tid * per, e = min(b + per, m);
  int32_t loc = 0;
  for (int64_t i = b; i < e; ++i) loc += x[i];
  int32_t incl = loc;
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int32_t pre = 0, tot = 0;
  for (int u = 0; u < 16; ++u) {
    if (u < w) pre += wsum[u];
    tot += wsum[u];
  }
  int32_t run = pre + incl - loc;
  for (int64_t i = b; i < e; ++i) {
    const int32_t v = x[i];
    x[i] = run;
    run += v;
  }
  __syncthreads();
  return tot;
}

__global__ __launch_bounds__(1024) void k_page_prefix(Dev dv, BuildScratch bs, int64_t nchunk,
                                                      int cmax) {
  __shared__ int32_t wsum[16];
  const int s = blockIdx.x;
  int32_t *cpg = bs.cell_pg + (int64_t)s * (cmax + 1);
  const int32_t tc = block_prefix_1024(cpg, dv.ncell, wsum);
  if (threadIdx.x == 0) cpg[dv.ncell] = tc;
  int32_t *kpg = bs.chunk_pg + (int64_t)s * (nchunk + 1);
  const int32_t tk = block_prefix_1024(kpg, nchunk, wsum);
  if (threadIdx.x == 0) {
    kpg[nchunk] = tk;
    dv.npages[s] = tk;
  }
}

// grid (nchunk, S), one wave; LDS: ncell counters
__global__ __launch_bounds__(64) void k_cell_rank(Dev dv, BuildScratch bs, int64_t n, int cmax) {
  extern __shared__ int32_t cnt[];
  constexpr int kSteps = kPageChunk / 64;
  const int s = blockIdx.y;
  const int64_t k = blockIdx.x, nchunk = gridDim.x;
  const int lane = threadIdx.x;
  const int ncell = (int)dv.ncell, p = dv.p;
  const int32_t *cpg = bs.cell_pg + (int64_t)s * (cmax + 1);
  const uint32_t *cells = bs.cell + (int64_t)s * n;
  const int64_t i0 = k * kPageChunk, i1 = min(i0 + kPageChunk, n);
  // loads first: the chunk's cells, their page_of offsets, the counts before the chunk
  uint32_t cv[kSteps];
  int32_t po[kSteps];
#pragma unroll
  for (int j = 0; j < kSteps; ++j) cv[j] = cells[min(i0 + 64 * j + lane, n - 1)];
#pragma unroll
  for (int j = 0; j < kSteps; ++j) po[j] = cpg[cv[j]];
  const int32_t *base = bs.chunk_cnt + ((int64_t)s * nchunk + k) * cmax;
  for (int c = lane; c < ncell; c += 64) cnt[c] = base[c];
  const int32_t pg0 = bs.chunk_pg[(int64_t)s * (nchunk + 1) + k];
  int32_t *pof = bs.page_of + (int64_t)s * (n / 8 + cmax + 1);
  __syncthreads();
  const unsigned long long lt = lanemask_lt();
  int32_t opened = 0;
#pragma unroll
  for (int j = 0; j < kSteps; ++j) {
    const int64_t i = i0 + 64 * j + lane;
    const bool valid = i < i1;
    const uint32_t c = cv[j];
    const unsigned long long mt = match_bits(c, dv.D, __ballot(valid));
    const int32_t rank = valid ? cnt[c] + popc64(mt & lt) : 0;
    const bool first = valid && rank % p == 0;
    const unsigned long long fm = __ballot(first);
    if (first) {
      const int32_t pid = pg0 + opened + popc64(fm & lt);
      pof[po[j] + rank / p] = pid;
      dv.page_cell[(int64_t)s * dv.pcap + pid] = (int32_t)c;
    }
    if (valid) bs.rank[(int64_t)s * n + i] = rank;
    __builtin_amdgcn_wave_barrier();
    if (valid && ((mt >> lane) >> 1) == 0ull) cnt[c] = rank + 1;  // the cell's last lane
    opened += popc64(fm);
    __builtin_amdgcn_wave_barrier();
  }
}

__global__ __launch_bounds__(256) void k_page_fill(Dev dv, BuildScratch bs, int64_t n, int cmax) {
  const int s = blockIdx.y;
  const int p = dv.p, ncell = (int)dv.ncell;
  const int32_t *cpg = bs.cell_pg + (int64_t)s * (cmax + 1);
  const int32_t *pof = bs.page_of + (int64_t)s * (n / 8 + cmax + 1);
  const int32_t *ccount = dv.cell_count + (int64_t)s * ncell;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const uint32_t c = bs.cell[(int64_t)s * n + i];
    const int32_t rank = bs.rank[(int64_t)s * n + i];
    const int32_t pid = pof[cpg[c] + rank / p], slot = rank % p;
    dv.loc[(int64_t)s * dv.ncap + i] = pid * p + slot;
    dv.page_tokens[((int64_t)s * dv.pcap + pid) * p + slot] = (int32_t)i;
    if (slot == 0) dv.page_len[(int64_t)s * dv.pcap + pid] = min(p, ccount[c] - rank);
  }
  // each non-empty cell's last page
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < ncell;
       c += (int64_t)gridDim.x * 256) {
    const int32_t cnt = ccount[c];
    if (cnt > 0) dv.cell_last[(int64_t)s * ncell + c] = pof[cpg[c] + (cnt - 1) / p];
  }
}

// Copy every key row to its page slot (16 bytes per thread).
__global__ __launch_bounds__(256) void k_scatter(Dev dv, const void *K, int64_t n) {
  const int64_t row_bytes = (int64_t)dv.d * dv.elem;
  const int64_t cpr = row_bytes / 16;
  const int64_t total = (int64_t)dv.S * n * cpr;
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < total;
       x += (int64_t)gridDim.x * 256) {
    const int64_t row = x / cpr;
    const int64_t cc = x % cpr;
    const int64_t s = row / n, i = row % n;
    const int64_t lc = dv.loc[s * dv.ncap + i];
    const int64_t dst = ((s * dv.pcap * dv.p) + lc) * row_bytes + cc * 16;
    const int64_t src = row * row_bytes + cc * 16;
    *reinterpret_cast<uint4 *>((char *)dv.pool_k + dst) =
        *reinterpret_cast<const uint4 *>((const char *)K + src);
  }
}

// Values into the element-major page layout ([e][slot] inside a page): a block
// transposes whole pages through LDS, rows in and element columns out, both
// as 16-byte accesses.  Empty slots are written as zeros.
constexpr int kScatterTile = 32 * 1024;

__global__ __launch_bounds__(256) void k_scatter_v(Dev dv, const void *V, int64_t n) {
  const int s = blockIdx.y;
  const int p = dv.p, d = dv.d, elem = dv.elem;
  const int row_bytes = d * elem;
  const int pb = max(1, kScatterTile / (p * row_bytes));  // pages per round
  const int cpr = row_bytes / 16;                          // 16-byte chunks per row
  const int epc = 16 / elem;                               // elements per 16 bytes
  const int cpe = p / epc;                                 // 16-byte chunks per column
  // every size above is a power of two: index arithmetic by shifts
  const int lp = dv.lp, lcpr = __builtin_ctz((unsigned)cpr), lcpe = __builtin_ctz((unsigned)cpe),
            ld = __builtin_ctz((unsigned)d);
  __shared__ uint4 tile[kScatterTile / 16];
  const int64_t npg = dv.npages[s];
  for (int64_t pg0 = (int64_t)blockIdx.x * pb; pg0 < npg; pg0 += (int64_t)gridDim.x * pb) {
    const int np = (int)min((int64_t)pb, npg - pg0);
    for (int x = threadIdx.x; x < np * p * cpr; x += 256) {
      const int j = x >> (lp + lcpr), slot = (x >> lcpr) & (p - 1), ch = x & (cpr - 1);
      const int32_t tok = dv.page_tokens[((int64_t)s * dv.pcap + pg0 + j) * p + slot];
      uint4 v = {0u, 0u, 0u, 0u};
      if (tok >= 0 && tok < n)
        v = reinterpret_cast<const uint4 *>(V)[((int64_t)s * n + tok) * cpr + ch];
      tile[(j * p + slot) * cpr + ch] = v;
    }
    __syncthreads();
    for (int x = threadIdx.x; x < np * d * cpe; x += 256) {
      const int j = x >> (ld + lcpe), e = (x >> lcpe) & (d - 1), c = x & (cpe - 1);
      uint32_t wds[4];
      if (elem == 2) {
        const uint16_t *t16 = reinterpret_cast<const uint16_t *>(tile);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int s0 = c * 8 + 2 * u;
          wds[u] = (uint32_t)t16[(j * p + s0) * d + e] |
                   ((uint32_t)t16[(j * p + s0 + 1) * d + e] << 16);
        }
      } else {
        const uint32_t *t32 = reinterpret_cast<const uint32_t *>(tile);
#pragma unroll
        for (int u = 0; u < 4; ++u) wds[u] = t32[(j * p + c * 4 + u) * d + e];
      }
      const int64_t dst = (((int64_t)s * dv.pcap + pg0 + j) * d + e) * p + c * epc;
      *reinterpret_cast<uint4 *>((char *)dv.pool_v + dst * elem) =
          make_uint4(wds[0], wds[1], wds[2], wds[3]);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- launchers

// Blocks per stream: enough tiles per block to amortise its direction
// staging, about eight blocks per CU over all streams (a sweep of 512 to 4096
// blocks put the best at 2048 for both the 36k and the 262k layers).
template <int DT, int HD, int NC>
static hipError_t launch_project_nc(const Dev &dv, const BuildScratch &bs, const void *K,
                                    int64_t n, float c_fixed, hipStream_t st) {
  const int64_t ntiles = (n + 15) / 16;
  int64_t nb = (ntiles + 3) / 4;
  const int64_t cap = 2048 / dv.S > 0 ? 2048 / dv.S : 1;
  if (nb > cap) nb = cap;
  if (nb < 1) nb = 1;
  hipLaunchKernelGGL((k_project<DT, HD, NC>), dim3((unsigned)nb, dv.S), dim3(256), 0, st, dv, bs,
                     K, n, c_fixed);
  return hipGetLastError();
}

template <int DT, int HD>
static hipError_t launch_project_hd(const Dev &dv, const BuildScratch &bs, const void *K,
                                    int64_t n, float c_fixed, hipStream_t st) {
  switch (dv.nchunk) {
    case 1: return launch_project_nc<DT, HD, 1>(dv, bs, K, n, c_fixed, st);
    case 2: return launch_project_nc<DT, HD, 2>(dv, bs, K, n, c_fixed, st);
    case 3: return launch_project_nc<DT, HD, 3>(dv, bs, K, n, c_fixed, st);
    case 4: return launch_project_nc<DT, HD, 4>(dv, bs, K, n, c_fixed, st);
    case 5: return launch_project_nc<DT, HD, 5>(dv, bs, K, n, c_fixed, st);
    case 6: return launch_project_nc<DT, HD, 6>(dv, bs, K, n, c_fixed, st);
    case 7: return launch_project_nc<DT, HD, 7>(dv, bs, K, n, c_fixed, st);
    case 8: return launch_project_nc<DT, HD, 8>(dv, bs, K, n, c_fixed, st);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
static hipError_t launch_project(const Dev &dv, const BuildScratch &bs, const void *K, int64_t n,
                                 float c_fixed, hipStream_t st) {
  static_assert(kMaxMl <= 8 * kDirChunk && kMaxTreeDepth <= kDirChunk, "chunks");
  return dv.d == 64 ? launch_project_hd<DT, 64>(dv, bs, K, n, c_fixed, st)
                    : launch_project_hd<DT, 128>(dv, bs, K, n, c_fixed, st);
}

template <int DT>
static hipError_t build_impl(const Dev &dv, const BuildScratch &bs, int64_t n, const void *K,
                             const void *V, const void *dirs, float c_fixed, hipStream_t st) {
  hipError_t e;
  // index state
  if ((e = fill_i32(dv.page_tokens, (int64_t)dv.S * dv.pcap * dv.p, -1, st))) return e;
  if ((e = fill_i32(dv.page_len, (int64_t)dv.S * dv.pcap, 0, st))) return e;
  if ((e = fill_i32(dv.page_cell, (int64_t)dv.S * dv.pcap, -1, st))) return e;
  if ((e = fill_i32((int32_t *)dv.hist, (int64_t)dv.S * dv.Lq * kHistBins, 0, st))) return e;
  if ((e = fill_i32((int32_t *)dv.hist2, (int64_t)dv.S * dv.Lq * kHistBins, 0, st))) return e;
  if ((e = fill_i32((int32_t *)dv.vhist, (int64_t)dv.S * dv.Lq * kHistBins, 0, st))) return e;
  if ((e = fill_i32((int32_t *)dv.cand_count, (int64_t)dv.S * dv.Lq, 0, st))) return e;
  hipLaunchKernelGGL(k_fill_u64, dim3(1), dim3(256), 0, st, dv.maxnsq, (int64_t)dv.S, 0ull);
  {
    const int64_t total = (int64_t)dv.nchunk * (dv.d + 1) * kDirChunk;
    hipLaunchKernelGGL(k_dirs<DT>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, dv,
                       dirs);
  }
  if (n > 0)  // every row's |k|^2 (the projection needs them), and c when not fixed
    hipLaunchKernelGGL(k_norms<DT>,
                       dim3((unsigned)((n + NormRows<DT>::kRows - 1) / NormRows<DT>::kRows), dv.S),
                       dim3(256), 0, st, dv, bs, K, n);
  // (an empty build still fixes c, 1/c and 1/c^2)
  if ((e = launch_project<DT>(dv, bs, K, n, c_fixed, st))) return e;
  if (n > 0)
    hipLaunchKernelGGL((k_sort_lists<kSortThreads, kSortItems>), dim3(dv.S * dv.mL),
                       dim3(kSortThreads), 0, st, dv, bs, n);
  if (n > 0) {
    const int64_t nchunk = (n + kPageChunk - 1) / kPageChunk;
    const int cmax = 1 << min(dv.mL, kMaxTreeDepth);
    const size_t lds = (size_t)dv.ncell * sizeof(int32_t);
    hipLaunchKernelGGL(k_cell_count, dim3((unsigned)nchunk, dv.S), dim3(256), lds, st, dv, bs, n,
                       cmax);
    if ((e = fill_i32(bs.chunk_pg, (int64_t)dv.S * (nchunk + 1), 0, st))) return e;
    hipLaunchKernelGGL(k_cell_scan, dim3((unsigned)((dv.ncell + 63) / 64), dv.S), dim3(256),
                       (size_t)nchunk * sizeof(int32_t), st, dv, bs, nchunk, cmax);
    hipLaunchKernelGGL(k_page_prefix, dim3(dv.S), dim3(1024), 0, st, dv, bs, nchunk, cmax);
    hipLaunchKernelGGL(k_cell_rank, dim3((unsigned)nchunk, dv.S), dim3(64), lds, st, dv, bs, n,
                       cmax);
    int64_t fb = (n + 255) / 256;
    if (fb > 4096) fb = 4096;
    hipLaunchKernelGGL(k_page_fill, dim3((unsigned)fb, dv.S), dim3(256), 0, st, dv, bs, n, cmax);
  } else {  // no tokens: no pages, empty cells
    if ((e = fill_i32(dv.npages, dv.S, 0, st))) return e;
    if ((e = fill_i32(dv.cell_count, (int64_t)dv.S * dv.ncell, 0, st))) return e;
    if ((e = fill_i32(dv.cell_last, (int64_t)dv.S * dv.ncell, -1, st))) return e;
  }
  if (n > 0) {
    const int64_t total = (int64_t)dv.S * n * ((int64_t)dv.d * dv.elem / 16);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_scatter, dim3((unsigned)blocks), dim3(256), 0, st, dv, K, n);
    const int pb = (kScatterTile / (dv.p * dv.d * dv.elem)) > 0 ? kScatterTile / (dv.p * dv.d * dv.elem) : 1;
    int64_t vb = (dv.pcap + pb - 1) / pb;
    if (vb > 256) vb = 256;
    hipLaunchKernelGGL(k_scatter_v, dim3((unsigned)vb, dv.S), dim3(256), 0, st, dv, V, n);
  }
  return hipGetLastError();
}

hipError_t launch_build(const Dev &dv, const BuildScratch &bs, int64_t n, const void *K,
                        const void *V, const void *dirs, float c_fixed, hipStream_t st) {
  return dv.dtype == 0 ? build_impl<0>(dv, bs, n, K, V, dirs, c_fixed, st)
                       : build_impl<1>(dv, bs, n, K, V, dirs, c_fixed, st);
}

}  // namespace ice
