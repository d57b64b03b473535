// Host side of the C ABI declared in include/ice.h: argument checks (all
// before any HIP call), the workspace layout, and kernel launches on the
// caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "ice.h"
#include "ice_common.h"

using ice::Dev;

// Build scratch of ice_build_index_noalloc: one fixed array per GPU.  In host
// code its name stands for a host-side shadow, never a device address: only
// the address hipGetSymbolAddress returns for the current device is used.
static __device__ __align__(256) unsigned char scratch[ICE_NOALLOC_SCRATCH_BYTES];

namespace ice {

// Per-kernel event timing of the decode-time calls (off unless enabled).
struct Timer {
  hipEvent_t last = nullptr;
  struct Rec {
    int kid;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> events;
  hipEvent_t make() {
    hipEvent_t e = nullptr;
    // timestamps only: no system-scope release/acquire around each record,
    // which would add its cache work to every timed kernel
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    events.push_back(e);
    return e;
  }
  void clear() {
    for (hipEvent_t e : events) hipEventDestroy(e);
    events.clear();
    recs.clear();
    last = nullptr;
  }
};

void timer_begin(Timer *tm, hipStream_t st) {
  if (!tm) return;
  tm->last = tm->make();
  if (tm->last) hipEventRecord(tm->last, st);
}

void timer_mark(Timer *tm, int kid, hipStream_t st) {
  if (!tm) return;
  hipEvent_t e = tm->make();
  if (!e) return;
  hipEventRecord(e, st);
  if (tm->last) tm->recs.push_back({kid, tm->last, e});
  tm->last = e;
}

}  // namespace ice

namespace {

constexpr int64_t kAlign = 256;
constexpr int64_t kMaxPages = 65536;

int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// D = round(log2(n / (4p))) clamped to [1, min(mL, 13)]; round(log2 x) >= t
// exactly when 2^(2t-1) <= x^2, evaluated in integers.
int derive_depth(int64_t n, int p, int mL) {
  int t = 0;
  const unsigned __int128 n2 = (unsigned __int128)n * (unsigned __int128)n;
  const unsigned __int128 q2 = (unsigned __int128)(4 * p) * (unsigned __int128)(4 * p);
  for (int cand = 1; cand < 40; ++cand) {  // n < 2^31 ends the loop long before overflow
    const unsigned __int128 lhs = ((unsigned __int128)1 << (2 * cand - 1)) * q2;
    if (lhs > n2) break;
    t = cand;
  }
  int cap = mL < ice::kMaxTreeDepth ? mL : ice::kMaxTreeDepth;
  if (t > cap) t = cap;
  if (t < 1) t = 1;
  return t;
}

struct Layout {
  int D, nchunk, k0, elem, attn_nsplit;
  int64_t ncell, pcap;
  int64_t dirs, dirs32, norm_c, inv_c, inv_c2, maxnsq, codes, list_code, list_id, loc, page_tokens,
      page_len, page_cell, npages, cell_count, cell_last, pool_k, pool_v, qkv, qcode, mbuf,
      hist, hist2, cand, cand_count, bnd, bnd_rk, bnd_pg, bnd_count, rr_key, rr_id, rr_pg, rr_count,
      attn_part, vhist, vstate, vtie, vcount, bsel, vlast, stage_k, stage_v, stage_len;
  int64_t nvrange;
  int64_t total;
};

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// Parameter checks shared by every entry point that takes ice_params.
ice_status check_params(const ice_params *prm, int32_t S, int64_t n, int64_t ncap) {
  if (!prm) return ICE_ERR_INVALID_ARG;
  if (prm->head_dim != 64 && prm->head_dim != 128) return ICE_ERR_INVALID_ARG;
  const int p = prm->page_size;
  if (!(p == 8 || p == 16 || p == 32 || p == 64)) return ICE_ERR_INVALID_ARG;
  if (prm->budget_k <= 0 || prm->budget_k % p != 0) return ICE_ERR_INVALID_ARG;
  if (prm->m < 1 || prm->L < 1 || (int64_t)prm->m * prm->L > ice::kMaxMl)
    return ICE_ERR_INVALID_ARG;
  if (prm->gqa_group < 1 || prm->gqa_group > ice::kMaxGroup) return ICE_ERR_INVALID_ARG;
  if (prm->k0 < 0 || prm->k1 < 0) return ICE_ERR_INVALID_ARG;
  if (prm->tree_depth < 0 || prm->tree_depth > ice::kMaxTreeDepth ||
      prm->tree_depth > prm->m * prm->L)
    return ICE_ERR_INVALID_ARG;
  if (!(prm->c >= 0.0f) || std::isinf(prm->c)) return ICE_ERR_INVALID_ARG;
  if (prm->dtype != ICE_F32 && prm->dtype != ICE_BF16) return ICE_ERR_INVALID_ARG;
  if (prm->gqa_mode != ICE_GQA_MEAN && prm->gqa_mode != ICE_GQA_MAX) return ICE_ERR_INVALID_ARG;
  if (prm->offload < 0 || prm->offload > 2) return ICE_ERR_INVALID_ARG;
  if (S < 1 || n < 0 || ncap < n || ncap < 1 || ncap > 0x7fffffffLL - 1)
    return ICE_ERR_INVALID_ARG;
  if (prm->L > 32) return ICE_ERR_UNSUPPORTED;
  const int64_t k0 = prm->k0 > 0 ? prm->k0 : prm->budget_k;
  if (k0 * prm->L > ice::kMaxCandBig) return ICE_ERR_UNSUPPORTED;
  if (prm->budget_k > ice::kMaxBudget) return ICE_ERR_UNSUPPORTED;
  if (n > (int64_t)ice::kPageChunk * 16384) return ICE_ERR_UNSUPPORTED;  // build's chunk counters
  if (prm->gqa_mode == ICE_GQA_MAX &&
      ((int64_t)prm->gqa_group * prm->L > 32 || (int64_t)prm->gqa_group * prm->L * k0 > ice::kMaxCand))
    return ICE_ERR_UNSUPPORTED;  // the pooled walks' candidates stay in the finaliser's LDS
  return ICE_OK;
}

ice_status make_layout(const ice_params *prm, int32_t S, int64_t n, int64_t ncap, Layout *L) {
  ice_status st = check_params(prm, S, n, ncap);
  if (st != ICE_OK) return st;
  const int d = prm->head_dim, p = prm->page_size, mL = prm->m * prm->L;
  Layout y;
  std::memset(&y, 0, sizeof(y));
  y.D = prm->tree_depth > 0 ? prm->tree_depth : derive_depth(n, p, mL);
  y.ncell = (int64_t)1 << y.D;
  y.pcap = (ncap + p - 1) / p + y.ncell;
  // this limit also keeps m * ncap below 2^29, so a bounded walk's entry
  // counts fit in 32 bits
  if (y.pcap > kMaxPages) return ICE_ERR_UNSUPPORTED;
  y.nchunk = (mL + ice::kDirChunk - 1) / ice::kDirChunk;
  y.k0 = prm->k0 > 0 ? prm->k0 : prm->budget_k;
  y.elem = prm->dtype == ICE_F32 ? 4 : 2;
  y.attn_nsplit = (prm->budget_k + ice::kAttnTpb - 1) / ice::kAttnTpb;
  const int64_t Sl = S, g = prm->gqa_group;
  const int64_t Gq = prm->gqa_mode == ICE_GQA_MAX ? g : 1;
  const int64_t Ll = prm->L * Gq;  // all walks of a query
  int64_t o = 0;
  auto seg = [&](int64_t bytes) {
    int64_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  y.dirs = seg((int64_t)y.nchunk * (d + 1) * ice::kDirChunk * 8);
  y.dirs32 = seg((int64_t)(d + 1) * ((mL + 31) / 32 * 32) * 4);
  y.norm_c = seg(Sl * 4);
  y.inv_c = seg(Sl * 8);
  y.inv_c2 = seg(Sl * 8);
  y.maxnsq = seg(Sl * 8);
  y.codes = seg(Sl * ((ncap + ice::kCodeTile - 1) / ice::kCodeTile) * ice::kCodeTile * mL * 4);
  y.list_code = seg(Sl * mL * ncap * 4);
  y.list_id = seg(Sl * mL * ncap * 4);
  y.loc = seg(Sl * ncap * 4);
  y.page_tokens = seg(Sl * y.pcap * p * 4);
  y.page_len = seg(Sl * y.pcap * 4);
  y.page_cell = seg(Sl * y.pcap * 4);
  y.npages = seg(Sl * 4);
  y.cell_count = seg(Sl * y.ncell * 4);
  y.cell_last = seg(Sl * y.ncell * 4);
  if (prm->offload) {  // the pool is in host memory; P staged pages per stream here
    // (offload 2: the keys stay here, only the values are in host memory)
    y.pool_k = prm->offload == 2 ? seg(Sl * y.pcap * p * d * y.elem) : -1;
    y.pool_v = -1;
    const int64_t P = prm->budget_k / p;
    y.stage_k = seg(Sl * P * p * d * y.elem);
    y.stage_v = seg(Sl * P * p * d * y.elem);
    y.stage_len = seg(Sl * P * 4);
  } else {
    y.pool_k = seg(Sl * y.pcap * p * d * y.elem);
    y.pool_v = seg(Sl * y.pcap * p * d * y.elem);
    y.stage_k = y.stage_v = y.stage_len = -1;
  }
  y.qkv = seg(Sl * Gq * d * 4);
  y.qcode = seg(Sl * Gq * mL * 4);
  y.mbuf = seg(Sl * Ll * ncap * 4);
  y.hist = seg(Sl * Ll * ice::kHistBins * 4);
  y.hist2 = seg(Sl * Ll * ice::kHistBins * 4);
  y.cand = seg(Sl * Ll * y.k0 * 4);
  y.cand_count = seg(Sl * Ll * 4);
  y.bnd = seg(Sl * Ll * ncap * 8);
  y.bnd_rk = seg(Sl * Ll * ncap * 8);
  y.bnd_pg = seg(Sl * Ll * ncap * 4);
  y.bnd_count = seg(Sl * Ll * 4);
  y.rr_key = seg(Sl * Ll * y.k0 * 8);
  y.rr_id = seg(Sl * Ll * y.k0 * 4);
  y.rr_pg = seg(Sl * Ll * y.k0 * 4);
  y.rr_count = seg(Sl * 4);
  y.attn_part = seg(Sl * y.attn_nsplit * g * (d + 2) * 4);
  y.nvrange = (ncap + ice::kVisitRange - 1) / ice::kVisitRange;
  y.vhist = seg(Sl * Ll * ice::kHistBins * 4);
  y.vstate = seg(Sl * Ll * 4 * 4);
  y.vtie = seg(Sl * Ll * y.nvrange * 4);
  y.vcount = seg(Sl * Ll * 4);
  y.bsel = seg(Sl * Ll * 2 * 4);
  y.vlast = seg(Sl * Ll * 8);
  y.total = o;
  *L = y;
  return ICE_OK;
}

// Offsets of the build scratch arrays (ice::BuildScratch order); returns the total.
int64_t scratch_offsets(const ice_params *prm, int32_t S, int64_t n, int64_t off[10]) {
  const int64_t mL = (int64_t)prm->m * prm->L;
  const int64_t cmax = (int64_t)1 << (mL < ice::kMaxTreeDepth ? mL : ice::kMaxTreeDepth);
  const int64_t nchunk = (n + ice::kPageChunk - 1) / ice::kPageChunk;
  const int64_t sz[10] = {S * mL * n * 4,         S * mL * n * 4,          S * mL * n * 4,
                          S * n * 4,              S * nchunk * cmax * 4,   S * n * 4,
                          S * (nchunk + 1) * 4,   S * (cmax + 1) * 4,      S * (n / 8 + cmax + 1) * 4,
                          S * n * 8};
  int64_t o = 0;
  for (int i = 0; i < 10; ++i) {
    off[i] = o;
    o = align_up(o + sz[i]);
  }
  return o;
}

// The offloaded pool in host memory: pool_k at 0, pool_v at *off_v (offload 1),
// or pool_v alone at 0 (offload 2: the keys stay in the workspace); returns the
// total.
int64_t host_pool_layout(const Layout &y, const ice_params *prm, int32_t S, int64_t *off_v) {
  const int64_t one = (int64_t)S * y.pcap * prm->page_size * prm->head_dim * y.elem;
  if (prm->offload == 2) {
    *off_v = 0;
    return align_up(one);
  }
  *off_v = align_up(one);
  return align_up(*off_v + one);
}

int64_t scratch_size(const ice_params *prm, int32_t S, int64_t n) {
  int64_t off[10];
  return scratch_offsets(prm, S, n, off);
}

bool aligned(const void *ptr, uintptr_t a) { return ((uintptr_t)ptr % a) == 0; }

// Device address of the fixed build scratch on the current device, resolved
// once per device (nullptr when HIP cannot resolve it).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices];

void *noalloc_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_dev[dev] = ptr;
  }
  return g_scratch_dev[dev];
}

}  // namespace

struct ice_index {
  ice_params prm;
  int32_t S;
  int64_t n, nbuild, ncap;
  Layout lay;
  char *ws;
  Dev dv;
  ice::Timer *timer;
};

extern "C" {

size_t ice_workspace_bytes(const ice_params *prm, int32_t n_streams, int64_t n_tokens,
                           int64_t capacity_tokens) {
  Layout y;
  if (make_layout(prm, n_streams, n_tokens, capacity_tokens, &y) != ICE_OK) return 0;
  return (size_t)y.total;
}

size_t ice_build_scratch_bytes(const ice_params *prm, int32_t n_streams, int64_t n_tokens) {
  if (check_params(prm, n_streams, n_tokens, n_tokens > 0 ? n_tokens : 1) != ICE_OK) return 0;
  const int64_t s = scratch_size(prm, n_streams, n_tokens);
  return (size_t)(s > 0 ? s : kAlign);
}

}  // extern "C"

namespace {

// The build behind ice_build_index and ice_build_index_offload; pool_dev is
// the device address of the host pool (offload), else null.
ice_status build_common(const ice_params *prm, int32_t n_streams, int64_t n_tokens,
                        int64_t capacity_tokens, const void *K, const void *V, const void *dirs,
                        void *workspace, size_t workspace_bytes, void *build_scratch,
                        size_t scratch_bytes, char *pool_dev, void *stream, ice_index **out) {
  Layout y;
  ice_status st = make_layout(prm, n_streams, n_tokens, capacity_tokens, &y);
  if (st != ICE_OK) return st;
  if (!dirs || !aligned(dirs, 4)) return ICE_ERR_INVALID_ARG;
  if (n_tokens > 0 && (!K || !V || !aligned(K, 16) || !aligned(V, 16)))
    return ICE_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, kAlign) || workspace_bytes < (size_t)y.total)
    return ICE_ERR_WORKSPACE;
  const int64_t need_scratch = scratch_size(prm, n_streams, n_tokens);
  if (n_tokens > 0 &&
      (!build_scratch || !aligned(build_scratch, kAlign) || scratch_bytes < (size_t)need_scratch))
    return ICE_ERR_WORKSPACE;

  ice_index *idx = new (std::nothrow) ice_index;
  if (!idx) return ICE_ERR_INVALID_ARG;
  idx->prm = *prm;
  idx->S = n_streams;
  idx->n = n_tokens;
  idx->nbuild = n_tokens;
  idx->ncap = capacity_tokens;
  idx->lay = y;
  idx->ws = (char *)workspace;
  idx->timer = nullptr;
  Dev &dv = idx->dv;
  std::memset(&dv, 0, sizeof(dv));
  char *w = (char *)workspace;
  dv.S = n_streams;
  dv.d = prm->head_dim;
  dv.p = prm->page_size;
  dv.m = prm->m;
  dv.L = prm->L;
  dv.mL = prm->m * prm->L;
  dv.g = prm->gqa_group;
  dv.gmax = prm->gqa_mode == ICE_GQA_MAX ? 1 : 0;
  dv.Gq = dv.gmax ? dv.g : 1;
  dv.Lq = dv.L * dv.Gq;
  dv.D = y.D;
  dv.k = prm->budget_k;
  dv.P = prm->budget_k / prm->page_size;
  dv.k0 = y.k0;
  dv.dtype = prm->dtype;
  dv.elem = y.elem;
  dv.ncap = capacity_tokens;
  dv.pcap = y.pcap;
  dv.ncell = y.ncell;
  dv.nbuild = n_tokens;
  dv.nchunk = y.nchunk;
  dv.attn_nsplit = y.attn_nsplit;
  dv.lp = 0;
  while ((1 << dv.lp) < dv.p) ++dv.lp;
  {  // sizes the scan's blocks (256 on a whole MI355X; fewer on a partition)
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        ncu <= 0)
      ncu = 256;
    dv.ncu = ncu;
  }
  dv.dirs = (double *)(w + y.dirs);
  dv.dirs32 = (float *)(w + y.dirs32);
  dv.mLp = (dv.mL + 31) / 32 * 32;
  dv.norm_c = (float *)(w + y.norm_c);
  dv.inv_c = (double *)(w + y.inv_c);
  dv.inv_c2 = (double *)(w + y.inv_c2);
  dv.maxnsq = (unsigned long long *)(w + y.maxnsq);
  dv.codes = (int32_t *)(w + y.codes);
  dv.ntile = (capacity_tokens + ice::kCodeTile - 1) / ice::kCodeTile;
  dv.list_code = (int32_t *)(w + y.list_code);
  dv.list_id = (int32_t *)(w + y.list_id);
  dv.loc = (int32_t *)(w + y.loc);
  dv.page_tokens = (int32_t *)(w + y.page_tokens);
  dv.page_len = (int32_t *)(w + y.page_len);
  dv.page_cell = (int32_t *)(w + y.page_cell);
  dv.npages = (int32_t *)(w + y.npages);
  dv.cell_count = (int32_t *)(w + y.cell_count);
  dv.cell_last = (int32_t *)(w + y.cell_last);
  dv.offload = prm->offload;
  if (prm->offload) {
    int64_t off_v = 0;
    host_pool_layout(y, prm, n_streams, &off_v);
    dv.pool_k = prm->offload == 2 ? w + y.pool_k : pool_dev;
    dv.pool_v = pool_dev + off_v;
    dv.stage_k = w + y.stage_k;
    dv.stage_v = w + y.stage_v;
    dv.stage_len = (int32_t *)(w + y.stage_len);
  } else {
    dv.pool_k = w + y.pool_k;
    dv.pool_v = w + y.pool_v;
  }
  dv.qkv = (float *)(w + y.qkv);
  dv.qcode = (int32_t *)(w + y.qcode);
  dv.mbuf = (uint32_t *)(w + y.mbuf);
  dv.hist = (uint32_t *)(w + y.hist);
  dv.hist2 = (uint32_t *)(w + y.hist2);
  dv.cand = (int32_t *)(w + y.cand);
  dv.cand_count = (uint32_t *)(w + y.cand_count);
  dv.bnd = (unsigned long long *)(w + y.bnd);
  dv.bnd_rk = (unsigned long long *)(w + y.bnd_rk);
  dv.bnd_pg = (int32_t *)(w + y.bnd_pg);
  dv.bnd_count = (uint32_t *)(w + y.bnd_count);
  dv.rr_key = (unsigned long long *)(w + y.rr_key);
  dv.rr_id = (int32_t *)(w + y.rr_id);
  dv.rr_pg = (int32_t *)(w + y.rr_pg);
  dv.rr_count = (uint32_t *)(w + y.rr_count);
  dv.attn_part = (float *)(w + y.attn_part);
  dv.nvrange = y.nvrange;
  dv.vhist = (uint32_t *)(w + y.vhist);
  dv.vstate = (uint32_t *)(w + y.vstate);
  dv.vtie = (uint32_t *)(w + y.vtie);
  dv.vcount = (uint32_t *)(w + y.vcount);
  dv.bsel = (uint32_t *)(w + y.bsel);
  dv.vlast = (unsigned long long *)(w + y.vlast);

  ice::BuildScratch bs;
  std::memset(&bs, 0, sizeof(bs));
  if (n_tokens > 0) {
    char *sc = (char *)build_scratch;
    int64_t off[10];
    scratch_offsets(prm, n_streams, n_tokens, off);
    bs.codes_dm = (int32_t *)(sc + off[0]);
    bs.tmp_code = (int32_t *)(sc + off[1]);
    bs.tmp_id = (int32_t *)(sc + off[2]);
    bs.cell = (uint32_t *)(sc + off[3]);
    bs.chunk_cnt = (int32_t *)(sc + off[4]);
    bs.rank = (int32_t *)(sc + off[5]);
    bs.chunk_pg = (int32_t *)(sc + off[6]);
    bs.cell_pg = (int32_t *)(sc + off[7]);
    bs.page_of = (int32_t *)(sc + off[8]);
    bs.nsq = (double *)(sc + off[9]);
  }
  hipError_t e = ice::launch_build(dv, bs, n_tokens, K, V, dirs, prm->c, (hipStream_t)stream);
  if (e != hipSuccess) {
    delete idx;
    return ICE_ERR_HIP;
  }
  *out = idx;
  return ICE_OK;
}

}  // namespace

extern "C" {

ice_status ice_build_index(const ice_params *prm, int32_t n_streams, int64_t n_tokens,
                           int64_t capacity_tokens, const void *K, const void *V,
                           const void *dirs, void *workspace, size_t workspace_bytes,
                           void *build_scratch, size_t scratch_bytes, void *stream,
                           ice_index **out) {
  if (!out) return ICE_ERR_INVALID_ARG;
  *out = nullptr;
  if (prm && prm->offload) return ICE_ERR_INVALID_ARG;  // ice_build_index_offload
  return build_common(prm, n_streams, n_tokens, capacity_tokens, K, V, dirs, workspace,
                      workspace_bytes, build_scratch, scratch_bytes, nullptr, stream, out);
}

size_t ice_host_pool_bytes(const ice_params *prm, int32_t n_streams, int64_t n_tokens,
                           int64_t capacity_tokens) {
  Layout y;
  if (!prm || !prm->offload ||
      make_layout(prm, n_streams, n_tokens, capacity_tokens, &y) != ICE_OK)
    return 0;
  int64_t off_v = 0;
  return (size_t)host_pool_layout(y, prm, n_streams, &off_v);
}

ice_status ice_build_index_offload(const ice_params *prm, int32_t n_streams, int64_t n_tokens,
                                   int64_t capacity_tokens, const void *K, const void *V,
                                   const void *dirs, void *workspace, size_t workspace_bytes,
                                   void *build_scratch, size_t scratch_bytes, void *host_pool,
                                   size_t host_pool_bytes, void *stream, ice_index **out) {
  if (!out) return ICE_ERR_INVALID_ARG;
  *out = nullptr;
  if (!prm || !prm->offload) return ICE_ERR_INVALID_ARG;  // ice_build_index
  Layout y;
  ice_status st = make_layout(prm, n_streams, n_tokens, capacity_tokens, &y);
  if (st != ICE_OK) return st;
  int64_t off_v = 0;
  const int64_t need = host_pool_layout(y, prm, n_streams, &off_v);
  if (!host_pool || !aligned(host_pool, kAlign) || host_pool_bytes < (size_t)need)
    return ICE_ERR_WORKSPACE;
  if (!workspace || !aligned(workspace, kAlign) || workspace_bytes < (size_t)y.total)
    return ICE_ERR_WORKSPACE;
  void *dev = nullptr;  // pinned, device-mapped host memory only
  if (hipHostGetDevicePointer(&dev, host_pool, 0) != hipSuccess || !dev) {
    (void)hipGetLastError();
    return ICE_ERR_INVALID_ARG;
  }
  return build_common(prm, n_streams, n_tokens, capacity_tokens, K, V, dirs, workspace,
                      workspace_bytes, build_scratch, scratch_bytes, (char *)dev, stream, out);
}

ice_status ice_build_index_noalloc(const ice_params *prm, int32_t n_streams, int64_t n_tokens,
                                   int64_t capacity_tokens, const void *K, const void *V,
                                   const void *dirs, void *workspace, size_t workspace_bytes,
                                   void *stream, ice_index **out) {
  if (!out) return ICE_ERR_INVALID_ARG;
  *out = nullptr;
  Layout y;
  ice_status st = make_layout(prm, n_streams, n_tokens, capacity_tokens, &y);
  if (st != ICE_OK) return st;
  if (scratch_size(prm, n_streams, n_tokens) > (int64_t)ICE_NOALLOC_SCRATCH_BYTES)
    return ICE_ERR_SCRATCH_LIMIT;
  void *dev_scratch = noalloc_scratch();
  if (!dev_scratch) return ICE_ERR_HIP;
  return ice_build_index(prm, n_streams, n_tokens, capacity_tokens, K, V, dirs, workspace,
                         workspace_bytes, dev_scratch, ICE_NOALLOC_SCRATCH_BYTES, stream, out);
}

ice_status ice_insert(ice_index *idx, const void *k_new, const void *v_new, void *stream) {
  if (!idx || !k_new || !v_new || !aligned(k_new, 4) || !aligned(v_new, 4))
    return ICE_ERR_INVALID_ARG;
  if (idx->n >= idx->ncap) return ICE_ERR_CAPACITY;
  hipError_t e = ice::launch_insert(idx->dv, idx->n, k_new, v_new, (hipStream_t)stream,
                                    idx->timer);
  if (e != hipSuccess) return ICE_ERR_HIP;
  idx->n += 1;
  return ICE_OK;
}

size_t ice_merge_scratch_bytes(const ice_index *idx) {
  if (!idx) return 0;
  const int64_t b = ice::merge_scratch_bytes(idx->dv, idx->n);
  return (size_t)(b > 0 ? align_up(b) : kAlign);
}

ice_status ice_merge_lists(ice_index *idx, void *scratch, size_t scratch_bytes, void *stream) {
  if (!idx) return ICE_ERR_INVALID_ARG;
  const int64_t t = idx->n - idx->nbuild;
  if (t <= 0) return ICE_OK;
  if (t > ice::kMaxMergeTail) return ICE_ERR_UNSUPPORTED;
  if (!scratch || !aligned(scratch, kAlign) ||
      scratch_bytes < (size_t)ice::merge_scratch_bytes(idx->dv, idx->n))
    return ICE_ERR_WORKSPACE;
  hipError_t e = ice::launch_merge(idx->dv, idx->nbuild, idx->n, scratch, (hipStream_t)stream);
  if (e != hipSuccess) return ICE_ERR_HIP;
  idx->nbuild = idx->n;
  idx->dv.nbuild = idx->n;
  return ICE_OK;
}

ice_status ice_query_pages(ice_index *idx, const void *q, int32_t *page_ids, int32_t *n_pages,
                           int32_t *topk_ids, ice_query_stats *stats, void *stream) {
  if (!idx || !q || !page_ids || !n_pages || !aligned(q, 16) || !aligned(page_ids, 4) ||
      !aligned(n_pages, 4) || (topk_ids && !aligned(topk_ids, 4)) || (stats && !aligned(stats, 8)))
    return ICE_ERR_INVALID_ARG;
  hipError_t e = ice::launch_query(idx->dv, idx->n, idx->prm.k1, q, page_ids, n_pages, topk_ids,
                                   stats, (hipStream_t)stream, idx->timer);
  return e == hipSuccess ? ICE_OK : ICE_ERR_HIP;
}

ice_status ice_sparse_attn(const ice_index *idx, const void *q, const int32_t *page_ids,
                           const int32_t *n_pages, float *out, void *stream) {
  if (!idx || !q || !page_ids || !n_pages || !out || !aligned(q, 16) || !aligned(page_ids, 4) ||
      !aligned(n_pages, 4) || !aligned(out, 4))
    return ICE_ERR_INVALID_ARG;
  hipError_t e = ice::launch_attn(idx->dv, q, page_ids, n_pages, out, (hipStream_t)stream,
                                  idx->timer);
  return e == hipSuccess ? ICE_OK : ICE_ERR_HIP;
}

ice_status ice_decode_step(ice_index *idx, const void *k_new, const void *v_new, const void *q,
                           int32_t *page_ids, int32_t *n_pages, int32_t *topk_ids, float *out,
                           ice_query_stats *stats, void *stream) {
  if (!idx || !k_new || !v_new || !q || !page_ids || !n_pages || !out || !aligned(k_new, 4) ||
      !aligned(v_new, 4) || !aligned(q, 16) || !aligned(page_ids, 4) || !aligned(n_pages, 4) ||
      !aligned(out, 4) || (topk_ids && !aligned(topk_ids, 4)) || (stats && !aligned(stats, 8)))
    return ICE_ERR_INVALID_ARG;
  if (idx->n >= idx->ncap) return ICE_ERR_CAPACITY;
  hipError_t e = ice::launch_decode(idx->dv, idx->n, idx->prm.k1, k_new, v_new, q, page_ids,
                                    n_pages, topk_ids, out, stats, (hipStream_t)stream,
                                    idx->timer);
  if (e != hipSuccess) return ICE_ERR_HIP;
  idx->n += 1;
  return ICE_OK;
}

ice_status ice_decode_step_reuse(ice_index *idx, const void *k_new, const void *v_new,
                                 const void *q, const int32_t *page_ids, const int32_t *n_pages,
                                 float *out, void *stream) {
  if (!idx || !k_new || !v_new || !q || !page_ids || !n_pages || !out || !aligned(k_new, 4) ||
      !aligned(v_new, 4) || !aligned(q, 16) || !aligned(page_ids, 4) || !aligned(n_pages, 4) ||
      !aligned(out, 4))
    return ICE_ERR_INVALID_ARG;
  if (idx->n >= idx->ncap) return ICE_ERR_CAPACITY;
  if (idx->dv.attn_nsplit == 1 && !idx->dv.offload) {  // one kernel
    const hipError_t e = ice::launch_reuse(idx->dv, idx->n, k_new, v_new, q, page_ids, n_pages,
                                           out, (hipStream_t)stream, idx->timer);
    if (e != hipSuccess) return ICE_ERR_HIP;
    idx->n += 1;
    return ICE_OK;
  }
  hipError_t e = ice::launch_insert(idx->dv, idx->n, k_new, v_new, (hipStream_t)stream,
                                    idx->timer);
  if (e != hipSuccess) return ICE_ERR_HIP;
  idx->n += 1;
  e = ice::launch_attn(idx->dv, q, page_ids, n_pages, out, (hipStream_t)stream, idx->timer);
  return e == hipSuccess ? ICE_OK : ICE_ERR_HIP;
}

void ice_destroy_index(ice_index *idx) {
  if (!idx) return;
  if (idx->timer) {
    idx->timer->clear();
    delete idx->timer;
  }
  delete idx;
}

ice_status ice_timing_enable(ice_index *idx, int enable) {
  if (!idx) return ICE_ERR_INVALID_ARG;
  if (enable && !idx->timer) {
    idx->timer = new (std::nothrow) ice::Timer;
    if (!idx->timer) return ICE_ERR_INVALID_ARG;
  } else if (!enable && idx->timer) {
    idx->timer->clear();
    delete idx->timer;
    idx->timer = nullptr;
  }
  return ICE_OK;
}

ice_status ice_timing_read(ice_index *idx, double *total_ms, int64_t *launches) {
  if (!idx || !total_ms || !launches) return ICE_ERR_INVALID_ARG;
  for (int k = 0; k < ICE_TIMED_KERNELS; ++k) {
    total_ms[k] = 0.0;
    launches[k] = 0;
  }
  if (!idx->timer) return ICE_OK;
  for (const auto &r : idx->timer->recs) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess) return ICE_ERR_HIP;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return ICE_ERR_HIP;
    total_ms[r.kid] += ms;
    launches[r.kid] += 1;
  }
  idx->timer->clear();
  return ICE_OK;
}

const char *ice_timing_name(int kernel) {
  static const char *names[ICE_TIMED_KERNELS] = {"insert", "qscan",  "qcollect", "qfinal", "attn",
                                                 "amerge", "visit",  "fetch",    "reuse"};
  return (kernel >= 0 && kernel < ICE_TIMED_KERNELS) ? names[kernel] : "";
}

const char *ice_status_string(ice_status s) {
  switch (s) {
    case ICE_OK: return "ok";
    case ICE_ERR_INVALID_ARG: return "invalid argument";
    case ICE_ERR_CAPACITY: return "index capacity exhausted";
    case ICE_ERR_UNSUPPORTED: return "unsupported setting";
    case ICE_ERR_WORKSPACE: return "workspace or scratch too small or misaligned";
    case ICE_ERR_HIP: return "HIP launch error";
    case ICE_ERR_SCRATCH_LIMIT:
      return "the build needs more scratch than the no-allocation build's fixed array";
  }
  return "unknown status";
}

ice_status ice_index_layout(const ice_index *idx, ice_layout *out) {
  if (!idx || !out) return ICE_ERR_INVALID_ARG;
  const Layout &y = idx->lay;
  std::memset(out, 0, sizeof(*out));
  out->n_streams = idx->S;
  out->n_tokens = idx->n;
  out->n_build = idx->nbuild;
  out->capacity_tokens = idx->ncap;
  out->page_capacity = y.pcap;
  out->n_cells = y.ncell;
  out->tree_depth = y.D;
  out->mL = idx->prm.m * idx->prm.L;
  out->k0 = y.k0;
  out->elem_bytes = y.elem;
  out->Lq = idx->prm.L * (idx->prm.gqa_mode == ICE_GQA_MAX ? idx->prm.gqa_group : 1);
  out->Gq = idx->prm.gqa_mode == ICE_GQA_MAX ? idx->prm.gqa_group : 1;
  out->norm_c = y.norm_c;
  out->codes = y.codes;
  out->list_code = y.list_code;
  out->list_id = y.list_id;
  out->loc = y.loc;
  out->page_tokens = y.page_tokens;
  out->page_len = y.page_len;
  out->page_cell = y.page_cell;
  out->npages = y.npages;
  out->cell_count = y.cell_count;
  if (idx->prm.offload) {  // offsets into the host pool (offload 2: pool_k in the workspace)
    int64_t off_v = 0;
    host_pool_layout(y, &idx->prm, idx->S, &off_v);
    out->pool_k = idx->prm.offload == 2 ? y.pool_k : 0;
    out->pool_v = off_v;
  } else {
    out->pool_k = y.pool_k;
    out->pool_v = y.pool_v;
  }
  out->offload = idx->prm.offload;
  out->qcode = y.qcode;
  out->cand = y.cand;
  out->cand_count = y.cand_count;
  out->workspace_bytes = y.total;
  return ICE_OK;
}

}  // extern "C"
