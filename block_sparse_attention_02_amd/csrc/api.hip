// C-ABI entry points of libbsa: argument validation on the host, then
// stream-ordered kernel launches.  The contract is documented in include/bsa.h.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "bsa.h"
#include "bsa_internal.hpp"

namespace bsa {
// Defined beside the KV-outer kernels, which own the workspace layout.
void kvouter_index_layout(const KvOuterParams& p, bsa_kvouter_layout* out);
}  // namespace bsa

namespace {

thread_local std::string g_err;

bsa_status fail(bsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

bsa_status ok() {
  g_err.clear();
  return BSA_OK;
}

bsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(BSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates a strided [B,N,H,D] view.  `vec` elements per 16-byte vector must
// divide every stride (and D) when `need_vec` is set.
bsa_status check_desc(const bsa_tdesc& d, const char* name, int vec, bool need_vec) {
  if (d.B < 1 || d.N < 1 || d.H < 1 || d.D < 1)
    return fail(BSA_ERR_SHAPE, "%s: sizes must be positive (B=%lld N=%lld H=%lld D=%lld)", name,
                (long long)d.B, (long long)d.N, (long long)d.H, (long long)d.D);
  if (d.sB < 0 || d.sN < 0 || d.sH < 0) return fail(BSA_ERR_SHAPE, "%s: negative stride", name);
  if (need_vec && (d.D % vec || d.sB % vec || d.sN % vec || d.sH % vec))
    return fail(BSA_ERR_SHAPE, "%s: D and strides must be multiples of %d elements", name, vec);
  if (d.N >= (int64_t)1 << 31) return fail(BSA_ERR_UNSUPPORTED, "%s: N must be below 2^31", name);
  return BSA_OK;
}

int elem_bytes(bsa_dtype dt) { return dt == BSA_F32 ? 4 : 2; }

// Sticky index-error flag, one per device: kernels that meet a block id
// outside their table skip it and set the flag; bsa_check reads and clears it.
// Host code reaches each device's copy only through the address that
// hipGetSymbolAddress returns for that device.
constexpr int kMaxDevices = 64;
std::mutex g_dev_mutex;
uint32_t* g_err_flag[kMaxDevices] = {nullptr};

}  // namespace

static __device__ uint32_t index_error_flag;

namespace {

// The current device's flag (nullptr if the device cannot be queried).
uint32_t* device_error_flag() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  if (!g_err_flag[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(index_error_flag)) != hipSuccess) return nullptr;
    g_err_flag[dev] = static_cast<uint32_t*>(ptr);
  }
  return g_err_flag[dev];
}

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

const char* bsa_last_error(void) { return g_err.c_str(); }

const char* bsa_version(void) { return "libbsa 0.1 (gfx950)"; }

bsa_status bsa_check(void* stream) {
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "stream synchronize");
  e = hipGetLastError();
  if (e != hipSuccess) return hip_status(e, "asynchronous error");
  uint32_t* flag = device_error_flag();
  if (!flag) return fail(BSA_ERR_HIP, "bsa_check: the device's index-error flag is not reachable");
  uint32_t v = 0;
  e = hipMemcpy(&v, flag, sizeof v, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_status(e, "index-error flag read");
  if (v == 0) return ok();
  const uint32_t zero = 0;
  e = hipMemcpy(flag, &zero, sizeof zero, hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_status(e, "index-error flag clear");
  return fail(BSA_ERR_INDEX, "a kernel met a block id at or beyond the number of blocks; the entry was skipped");
}

// ---------------------------------------------------------------------------- tiling
bsa_status bsa_tile_dims(int T, int H, int W, int bT, int bH, int bW, int* J, int* M) {
  if (!J || !M) return fail(BSA_ERR_ARG, "bsa_tile_dims: null output pointer");
  if (T < 1 || H < 1 || W < 1 || bT < 1 || bH < 1 || bW < 1)
    return fail(BSA_ERR_SHAPE, "bsa_tile_dims: grid and block sizes must be positive");
  const int64_t n = (int64_t)T * H * W;
  const int64_t jt = (T + bT - 1) / bT, jh = (H + bH - 1) / bH, jw = (W + bW - 1) / bW;
  const int64_t jj = jt * jh * jw, mm = (int64_t)bT * bH * bW;
  if (n >= (int64_t)1 << 31 || jj * mm >= (int64_t)1 << 31)
    return fail(BSA_ERR_UNSUPPORTED, "bsa_tile_dims: grid too large for int32 tables");
  *J = (int)jj;
  *M = (int)mm;
  return ok();
}

bsa_status vsa_tile_index(int T, int H, int W, int bT, int bH, int bW, int32_t* perm, int32_t* block_len,
                          int32_t* inv, void* stream) {
  int J = 0, M = 0;
  bsa_status st = bsa_tile_dims(T, H, W, bT, bH, bW, &J, &M);
  if (st != BSA_OK) return st;
  if (!perm || !block_len) return fail(BSA_ERR_ARG, "vsa_tile_index: perm and block_len are required");
  return hip_status(bsa::launch_tile_index(T, H, W, bT, bH, bW, J, M, perm, block_len, inv, (hipStream_t)stream),
                    "vsa_tile_index launch");
}

int vsa_budget(double drop_ratio, int J) {
  if (J < 1 || !(drop_ratio >= 0.0 && drop_ratio <= 1.0)) return -1;
  const double keep = std::ceil((1.0 - drop_ratio) * J - 1e-9);
  int r = (int)keep;
  if (r > J) r = J;
  if (r < 1) r = 1;
  return r;
}

// ------------------------------------------------------------------ pool / route / TopK
static bsa_status check_route(const vsa_route_args* a) {
  if (!a) return fail(BSA_ERR_ARG, "vsa_pool_route_topk: null args");
  if (!a->q || !a->k || !a->perm || !a->block_len || !a->q2k_idx || !a->q2k_num)
    return fail(BSA_ERR_ARG, "vsa_pool_route_topk: q, k, perm, block_len, q2k_idx and q2k_num are required");
  if (a->dt != BSA_BF16 && a->dt != BSA_F32) return fail(BSA_ERR_ARG, "vsa_pool_route_topk: bad dtype");
  bsa_status st = check_desc(a->d, "q/k", 1, false);
  if (st != BSA_OK) return st;
  if (a->d.D > 256) return fail(BSA_ERR_UNSUPPORTED, "vsa_pool_route_topk: D must be <= 256");
  if ((a->qbar && !aligned16(a->qbar)) || (a->kbar && !aligned16(a->kbar)))
    return fail(BSA_ERR_ARG, "vsa_pool_route_topk: qbar and kbar must be 16-byte aligned");
  if (a->J < 1 || a->M < 1) return fail(BSA_ERR_SHAPE, "vsa_pool_route_topk: J and M must be positive");
  if (a->J > bsa::kRouteMaxJ)
    return fail(BSA_ERR_UNSUPPORTED, "vsa_pool_route_topk: J=%d exceeds %d blocks", a->J, bsa::kRouteMaxJ);
  if (a->R < 1 || a->R > a->J) return fail(BSA_ERR_SHAPE, "vsa_pool_route_topk: R must lie in [1, J]");
  if (a->kmax < a->R) return fail(BSA_ERR_SHAPE, "vsa_pool_route_topk: kmax must be >= R");
  if (!std::isfinite(a->scale)) return fail(BSA_ERR_ARG, "vsa_pool_route_topk: scale must be finite");
  if ((int64_t)a->d.B * a->d.H > 65535)
    return fail(BSA_ERR_UNSUPPORTED, "vsa_pool_route_topk: B*H must be <= 65535");
  if (a->perm_bh_stride < 0 || (a->perm_bh_stride > 0 && a->perm_bh_stride < (int64_t)a->J * a->M))
    return fail(BSA_ERR_SHAPE, "vsa_pool_route_topk: perm_bh_stride must be 0 or >= J*M");
  return BSA_OK;
}

bsa_status vsa_pool_route_topk_ws(const vsa_route_args* a, size_t* bytes) {
  if (!bytes) return fail(BSA_ERR_ARG, "vsa_pool_route_topk_ws: null output");
  bsa_status st = check_route(a);
  if (st != BSA_OK) return st;
  const size_t one = round_up((size_t)a->d.B * a->d.H * a->J * a->d.D * sizeof(float));
  *bytes = (a->qbar ? 0 : one) + (a->kbar ? 0 : one) +
           round_up(bsa::route_planes_bytes((int)(a->d.B * a->d.H), a->J, (int)a->d.D));
  return ok();
}

bsa_status vsa_pool_route_topk(const vsa_route_args* a, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  bsa_status st = vsa_pool_route_topk_ws(a, &need);
  if (st != BSA_OK) return st;
  if (need && (!ws || ws_bytes < need))
    return fail(BSA_ERR_WORKSPACE, "vsa_pool_route_topk: workspace of %zu bytes required", need);
  if (need && !aligned16(ws)) return fail(BSA_ERR_WORKSPACE, "vsa_pool_route_topk: workspace must be 16-byte aligned");
  const size_t one = round_up((size_t)a->d.B * a->d.H * a->J * a->d.D * sizeof(float));
  char* w = static_cast<char*>(ws);
  float* qbar = a->qbar;
  float* kbar = a->kbar;
  if (!qbar) { qbar = reinterpret_cast<float*>(w); w += one; }
  if (!kbar) { kbar = reinterpret_cast<float*>(w); w += one; }
  __bf16* kplanes = reinterpret_cast<__bf16*>(w);
  const int vec = 16 / elem_bytes(a->dt);
  const bool vec_ok = a->d.D % vec == 0 && a->d.sB % vec == 0 && a->d.sN % vec == 0 && a->d.sH % vec == 0 &&
                      aligned16(a->q) && aligned16(a->k);
  bsa::PoolParams pp{a->q, a->k, a->d.sB, a->d.sN, a->d.sH, (int)a->d.B, (int)a->d.H, (int)a->d.D, a->J, a->M,
                     a->perm, a->block_len, qbar, kbar, a->perm_bh_stride};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = bsa::launch_pool(pp, a->dt == BSA_F32, vec_ok, s);
  if (e != hipSuccess) return hip_status(e, "pool launch");
  bsa::RouteParams rp{qbar, kbar, (int)a->d.B, (int)a->d.H, a->J, (int)a->d.D, a->R, a->kmax, a->scale,
                      a->q2k_idx, a->q2k_num, a->E, 0, a->J, 0, a->J, 0, 1, kplanes};
  e = bsa::launch_route_topk(rp, s);
  if (e != hipSuccess || !a->item_order) return hip_status(e, "route/topk launch");
  return hip_status(bsa::launch_item_order(a->q2k_idx, a->q2k_num, (int)(a->d.B * a->d.H), a->J, a->kmax, 0,
                                           a->item_order, s),
                    "item order launch");
}

// ------------------------------------------------------------------ H3 multi-region layout
// Builds the layout parts (dense chunks first, then the videos) of a segment
// list, with the totals.
static bsa_status h3_build(const bsa_segment* seg, int nseg, int bT, int bH, int bW, bsa::H3Layout* L, int* J,
                           int* N, int* num_prefix, int* nreg, int* spans) {
  if (!seg) return fail(BSA_ERR_ARG, "h3 layout: null segment list");
  if (nseg < 1 || nseg > BSA_H3_MAX_SEGMENTS)
    return fail(BSA_ERR_UNSUPPORTED, "h3 layout: 1 to %d segments", BSA_H3_MAX_SEGMENTS);
  if (bT < 1 || bH < 1 || bW < 1) return fail(BSA_ERR_SHAPE, "h3 layout: block sizes must be positive");
  const int64_t M = (int64_t)bT * bH * bW;
  if (M >= (int64_t)1 << 20) return fail(BSA_ERR_UNSUPPORTED, "h3 layout: block capacity too large");
  int64_t tok0[BSA_H3_MAX_SEGMENTS];
  int64_t off = 0;
  for (int k = 0; k < nseg; ++k) {
    const bsa_segment& g = seg[k];
    tok0[k] = off;
    if (g.video == 0) {
      if (g.T < 0) return fail(BSA_ERR_SHAPE, "h3 layout: segment %d has a negative token count", k);
      off += g.T;
    } else if (g.video == 1) {
      if (g.T < 1 || g.H < 1 || g.W < 1) return fail(BSA_ERR_SHAPE, "h3 layout: video segment %d is empty", k);
      off += (int64_t)g.T * g.H * g.W;
    } else {
      return fail(BSA_ERR_ARG, "h3 layout: segment %d: video must be 0 or 1", k);
    }
    if (off >= (int64_t)1 << 31) return fail(BSA_ERR_UNSUPPORTED, "h3 layout: too many tokens");
  }
  L->nparts = 0;
  L->M = (int)M;
  L->bT = bT, L->bH = bH, L->bW = bW;
  int64_t b = 0;
  int np = 0, nr = 0;
  for (int pass = 0; pass < 2; ++pass)
    for (int k = 0; k < nseg; ++k) {
      const bsa_segment& g = seg[k];
      if (g.video != pass || (pass == 0 && g.T == 0)) continue;
      bsa::H3Part P{};
      P.video = pass;
      P.tok0 = (int)tok0[k];
      P.b0 = (int)b;
      int64_t nb;
      if (pass == 0) {
        P.n = g.T;
        nb = (g.T + M - 1) / M;
      } else {
        P.T = g.T, P.H = g.H, P.W = g.W;
        P.JH = (g.H + bH - 1) / bH, P.JW = (g.W + bW - 1) / bW;
        nb = (int64_t)((g.T + bT - 1) / bT) * P.JH * P.JW;
      }
      b += nb;
      if (b * M >= (int64_t)1 << 31) return fail(BSA_ERR_UNSUPPORTED, "h3 layout: grid too large for int32 tables");
      P.b1 = (int)b;
      L->part[L->nparts++] = P;
      if (pass == 0) {
        np = (int)b;
      } else {
        if (spans) spans[2 * nr] = P.b0, spans[2 * nr + 1] = P.b1;
        ++nr;
      }
    }
  if (b < 1) return fail(BSA_ERR_SHAPE, "h3 layout: no tokens");
  *J = (int)b;
  *N = (int)off;
  *num_prefix = np;
  *nreg = nr;
  return BSA_OK;
}

bsa_status h3_tile_dims(const bsa_segment* seg, int nseg, int bT, int bH, int bW, int* J, int* M, int* N,
                        int* num_prefix, int* nregions, int* spans) {
  if (!J || !M || !N || !num_prefix || !nregions) return fail(BSA_ERR_ARG, "h3_tile_dims: null output pointer");
  bsa::H3Layout L;
  bsa_status st = h3_build(seg, nseg, bT, bH, bW, &L, J, N, num_prefix, nregions, spans);
  if (st != BSA_OK) return st;
  *M = L.M;
  return ok();
}

bsa_status h3_tile_index(const bsa_segment* seg, int nseg, int bT, int bH, int bW, int32_t* perm,
                         int32_t* block_len, int32_t* inv, void* stream) {
  bsa::H3Layout L;
  int J = 0, N = 0, np = 0, nr = 0;
  bsa_status st = h3_build(seg, nseg, bT, bH, bW, &L, &J, &N, &np, &nr, nullptr);
  if (st != BSA_OK) return st;
  if (!perm || !block_len) return fail(BSA_ERR_ARG, "h3_tile_index: perm and block_len are required");
  return hip_status(bsa::launch_h3_tile_index(L, J, perm, block_len, inv, (hipStream_t)stream),
                    "h3 tile index launch");
}

static bsa_status check_h3_route(const h3_route_args* a, int* nsel) {
  if (!a) return fail(BSA_ERR_ARG, "h3_pool_route_topk: null args");
  if (!a->q || !a->k || !a->perm || !a->block_len || !a->q2k_idx || !a->q2k_num)
    return fail(BSA_ERR_ARG, "h3_pool_route_topk: q, k, perm, block_len, q2k_idx and q2k_num are required");
  if (a->dt != BSA_BF16 && a->dt != BSA_F32) return fail(BSA_ERR_ARG, "h3_pool_route_topk: bad dtype");
  bsa_status st = check_desc(a->d, "q/k", 1, false);
  if (st != BSA_OK) return st;
  if (a->d.D > 256) return fail(BSA_ERR_UNSUPPORTED, "h3_pool_route_topk: D must be <= 256");
  if ((a->qbar && !aligned16(a->qbar)) || (a->kbar && !aligned16(a->kbar)))
    return fail(BSA_ERR_ARG, "h3_pool_route_topk: qbar and kbar must be 16-byte aligned");
  if (a->J < 1 || a->M < 1) return fail(BSA_ERR_SHAPE, "h3_pool_route_topk: J and M must be positive");
  if (a->J > bsa::kRouteMaxJ)
    return fail(BSA_ERR_UNSUPPORTED, "h3_pool_route_topk: J=%d exceeds %d blocks", a->J, bsa::kRouteMaxJ);
  if (!std::isfinite(a->scale)) return fail(BSA_ERR_ARG, "h3_pool_route_topk: scale must be finite");
  if ((int64_t)a->d.B * a->d.H > 65535) return fail(BSA_ERR_UNSUPPORTED, "h3_pool_route_topk: B*H must be <= 65535");
  if (a->num_prefix < 0 || a->num_prefix > a->J)
    return fail(BSA_ERR_SHAPE, "h3_pool_route_topk: num_prefix must lie in [0, J]");
  if (a->nregions < 0 || a->nregions > BSA_H3_MAX_SEGMENTS)
    return fail(BSA_ERR_UNSUPPORTED, "h3_pool_route_topk: 0 to %d regions", BSA_H3_MAX_SEGMENTS);
  if ((a->nregions == 0) != (a->num_prefix == a->J))
    return fail(BSA_ERR_SHAPE, "h3_pool_route_topk: the regions must cover blocks [num_prefix, J)");
  if (a->nregions > 0 && (!a->spans || !a->budgets))
    return fail(BSA_ERR_ARG, "h3_pool_route_topk: spans and budgets are required");
  int at = a->num_prefix, sel = a->num_prefix;
  for (int r = 0; r < a->nregions; ++r) {
    const int b0 = a->spans[2 * r], b1 = a->spans[2 * r + 1];
    if (b0 != at || b1 <= b0 || b1 > a->J)
      return fail(BSA_ERR_SHAPE, "h3_pool_route_topk: region %d [%d, %d) does not continue the tiling at %d", r, b0,
                  b1, at);
    if (a->budgets[r] < 1 || a->budgets[r] > b1 - b0)
      return fail(BSA_ERR_SHAPE, "h3_pool_route_topk: budget of region %d must lie in [1, %d]", r, b1 - b0);
    at = b1;
    sel += a->budgets[r];
  }
  if (at != a->J) return fail(BSA_ERR_SHAPE, "h3_pool_route_topk: the regions must end at J");
  if (a->kmax < sel || (a->num_prefix > 0 && a->kmax < a->J))
    return fail(BSA_ERR_SHAPE, "h3_pool_route_topk: kmax must be >= %d", a->num_prefix > 0 ? a->J : sel);
  *nsel = sel;
  return BSA_OK;
}

// Pooled means (unless the caller takes them) and the key planes of the widest
// region; the arguments are already checked.
static size_t h3_route_ws_bytes(const h3_route_args* a) {
  const size_t one = round_up((size_t)a->d.B * a->d.H * a->J * a->d.D * sizeof(float));
  size_t planes = 0;
  for (int r = 0; r < a->nregions; ++r)
    planes = std::max(planes, bsa::route_planes_bytes((int)(a->d.B * a->d.H), a->spans[2 * r + 1] - a->spans[2 * r],
                                                      (int)a->d.D));
  return (a->qbar ? 0 : one) + (a->kbar ? 0 : one) + round_up(planes);
}

bsa_status h3_pool_route_topk_ws(const h3_route_args* a, size_t* bytes) {
  if (!bytes) return fail(BSA_ERR_ARG, "h3_pool_route_topk_ws: null output");
  int nsel = 0;
  bsa_status st = check_h3_route(a, &nsel);
  if (st != BSA_OK) return st;
  *bytes = h3_route_ws_bytes(a);
  return ok();
}

bsa_status h3_pool_route_topk(const h3_route_args* a, void* ws, size_t ws_bytes, void* stream) {
  int nsel = 0;
  bsa_status st = check_h3_route(a, &nsel);
  if (st != BSA_OK) return st;
  const size_t one = round_up((size_t)a->d.B * a->d.H * a->J * a->d.D * sizeof(float));
  const size_t need = h3_route_ws_bytes(a);
  if (need && (!ws || ws_bytes < need))
    return fail(BSA_ERR_WORKSPACE, "h3_pool_route_topk: workspace of %zu bytes required", need);
  if (need && !aligned16(ws)) return fail(BSA_ERR_WORKSPACE, "h3_pool_route_topk: workspace must be 16-byte aligned");
  char* w = static_cast<char*>(ws);
  float* qbar = a->qbar;
  float* kbar = a->kbar;
  if (!qbar) { qbar = reinterpret_cast<float*>(w); w += one; }
  if (!kbar) { kbar = reinterpret_cast<float*>(w); w += one; }
  __bf16* kplanes = reinterpret_cast<__bf16*>(w);  // shared by the regions' launches, in stream order
  const int vec = 16 / elem_bytes(a->dt);
  const bool vec_ok = a->d.D % vec == 0 && a->d.sB % vec == 0 && a->d.sN % vec == 0 && a->d.sH % vec == 0 &&
                      aligned16(a->q) && aligned16(a->k);
  const int B = (int)a->d.B, H = (int)a->d.H, D = (int)a->d.D, J = a->J, P = a->num_prefix;
  bsa::PoolParams pp{a->q, a->k, a->d.sB, a->d.sN, a->d.sH, B, H, D, J, a->M, a->perm, a->block_len, qbar, kbar, 0};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = bsa::launch_pool(pp, a->dt == BSA_F32, vec_ok, s);
  if (e != hipSuccess) return hip_status(e, "pool launch");
  int out_off = P;
  for (int r = 0; r < a->nregions; ++r) {
    const int b0 = a->spans[2 * r], b1 = a->spans[2 * r + 1];
    bsa::RouteParams rp{qbar, kbar, B, H, J, D, a->budgets[r], a->kmax, a->scale, a->q2k_idx, a->q2k_num, nullptr,
                        P, J - P, b0, b1 - b0, out_off, 0, kplanes};
    e = bsa::launch_route_topk(rp, s);
    if (e != hipSuccess) return hip_status(e, "grouped route/topk launch");
    out_off += a->budgets[r];
  }
  e = bsa::launch_h3_fill(a->q2k_idx, a->q2k_num, B * H, J, a->kmax, P, nsel, !a->no_fill, s);
  if (e != hipSuccess || !a->item_order) return hip_status(e, "grouped index fill launch");
  return hip_status(bsa::launch_item_order(a->q2k_idx, a->q2k_num, B * H, J, a->kmax, P, a->item_order, s),
                    "item order launch");
}

// ------------------------------------------------------------------- query-outer attention
static bsa_status check_attn_common(const bsa_qouter_args* a) {
  if (!a) return fail(BSA_ERR_ARG, "bsa_forward_qouter: null args");
  if (!a->q || !a->k || !a->v || !a->out) return fail(BSA_ERR_ARG, "bsa_forward_qouter: q, k, v, out are required");
  if (a->dt != BSA_BF16 && a->dt != BSA_F32) return fail(BSA_ERR_ARG, "bsa_forward_qouter: bad dtype");
  const int vec = 16 / elem_bytes(a->dt);
  bsa_status st = check_desc(a->dq, "q", vec, true);
  if (st != BSA_OK) return st;
  if ((st = check_desc(a->dkv, "k/v", vec, true)) != BSA_OK) return st;
  if ((st = check_desc(a->dout, "out", vec, true)) != BSA_OK) return st;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->out))
    return fail(BSA_ERR_SHAPE, "bsa_forward_qouter: q, k, v, out must be 16-byte aligned");
  if (a->dq.D != a->dkv.D || a->dq.D != a->dout.D) return fail(BSA_ERR_SHAPE, "bsa_forward_qouter: D mismatch");
  if (a->dq.D != 64 && a->dq.D != 128) return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_qouter: D must be 64 or 128");
  if (a->dq.B != a->dkv.B || a->dq.B != a->dout.B) return fail(BSA_ERR_SHAPE, "bsa_forward_qouter: B mismatch");
  if (a->dq.N != a->dkv.N || a->dq.N != a->dout.N) return fail(BSA_ERR_SHAPE, "bsa_forward_qouter: N mismatch");
  if (a->dq.H != a->dout.H) return fail(BSA_ERR_SHAPE, "bsa_forward_qouter: q and out heads differ");
  if (a->dq.H % a->dkv.H) return fail(BSA_ERR_SHAPE, "bsa_forward_qouter: Hq must be a multiple of Hkv");
  if (!std::isfinite(a->scale)) return fail(BSA_ERR_ARG, "bsa_forward_qouter: scale must be finite");
  return BSA_OK;
}

// Every host-side check of a query-outer call (common and per mode).
static bsa_status check_qouter(const bsa_qouter_args* a) {
  bsa_status st = check_attn_common(a);
  if (st != BSA_OK) return st;
  if (a->mode == BSA_SEL_BLOCK) {
    if (a->dq.H != a->dkv.H) return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_qouter: block mode needs Hq == Hkv");
    if (!a->perm || !a->block_len || !a->q2k_idx || !a->q2k_num)
      return fail(BSA_ERR_ARG, "bsa_forward_qouter: perm, block_len, q2k_idx, q2k_num are required");
    if (a->J < 1 || a->kmax < 1) return fail(BSA_ERR_SHAPE, "bsa_forward_qouter: J and kmax must be positive");
    if (a->M != 16 && a->M != 32 && a->M != 64 && a->M != 128)
      return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_qouter: block capacity M must be 16, 32, 64 or 128");
    // capacity 128 runs as 64-token halves: twice the query blocks and kept entries
    const int64_t halves = a->M == 128 ? 2 : 1;
    if ((int64_t)a->dq.B * a->dq.H * a->J * halves >= (int64_t)1 << 31 || a->kmax * halves >= (int64_t)1 << 30)
      return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_qouter: too many query blocks or kept entries");
    if (a->M == 128 && (a->coarse || a->gate))
      return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_qouter: the coarse branch needs block capacity <= 64");
    if (a->M == 128 && (int64_t)a->dq.B * a->dq.H * 2 * a->J * 2 * a->kmax >= (int64_t)1 << 37)
      return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_qouter: the half tables of capacity 128 would be too large");
    if (a->dt == BSA_BF16) {  // the kernels address one (batch, head) K/V slice with 32-bit offsets
      const int64_t slice = (a->dkv.N - 1) * a->dkv.sN * 2 + a->dkv.D * 2;
      if (slice >= (int64_t)1 << 32 || a->dkv.N >= (int64_t)1 << 24 || a->dkv.sN * 2 >= (int64_t)1 << 24)
        return fail(BSA_ERR_UNSUPPORTED,
                    "bsa_forward_qouter: block mode needs N < 2^24, a token stride below 2^24 bytes and one "
                    "(batch, head) K/V slice below 4 GiB");
    }
    if (a->k_sum || a->v_sum || a->b_sum) {
      if (!a->k_sum || !a->v_sum || !a->b_sum)
        return fail(BSA_ERR_ARG, "bsa_forward_qouter: k_sum, v_sum and b_sum go together");
      if (a->dt != BSA_BF16 || a->M != 64)
        return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_qouter: summaries need bf16 and block capacity 64");
      if (a->J > 4096) return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_qouter: summaries need J <= 4096");
      if (!aligned16(a->k_sum) || !aligned16(a->v_sum) || (reinterpret_cast<uintptr_t>(a->b_sum) & 3))
        return fail(BSA_ERR_SHAPE, "bsa_forward_qouter: k_sum/v_sum must be 16-byte and b_sum 4-byte aligned");
    }
    if (a->perm_bh_stride < 0 || (a->perm_bh_stride > 0 && a->perm_bh_stride < (int64_t)a->J * a->M))
      return fail(BSA_ERR_SHAPE, "bsa_forward_qouter: perm_bh_stride must be 0 or >= J*M");
    if (a->order_long < 0 || a->order_long > a->J)
      return fail(BSA_ERR_ARG, "bsa_forward_qouter: order_long must lie in [0, J]");
    if (a->perm_bh_stride && a->k_sum)
      return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_qouter: summaries need one shared perm table");
    if (a->coarse || a->gate) {
      if (!a->coarse || !a->gate) return fail(BSA_ERR_ARG, "bsa_forward_qouter: coarse and gate go together");
      if (!aligned16(a->coarse) || !aligned16(a->gate))
        return fail(BSA_ERR_SHAPE, "bsa_forward_qouter: coarse and gate must be 16-byte aligned");
    }
    return BSA_OK;
  }
  if (a->mode == BSA_SEL_TOKEN) {
    if (a->dt != BSA_BF16) return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_qouter: token mode needs bf16");
    if (!a->blk_idx) return fail(BSA_ERR_ARG, "bsa_forward_qouter: blk_idx is required");
    if (a->S < 1 || a->S > 64) return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_qouter: S must lie in [1, 64]");
    if (a->BS != 16 && a->BS != 32 && a->BS != 64 && a->BS != 128)
      return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_qouter: block size BS must be 16, 32, 64 or 128");
    const int64_t G = a->dq.H / a->dkv.H;
    const int64_t items = a->dq.B * a->dq.N * a->dkv.H * ((G + 15) / 16);
    if (items >= (int64_t)1 << 31) return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_qouter: too many tokens");
    return BSA_OK;
  }
  return fail(BSA_ERR_ARG, "bsa_forward_qouter: unknown mode %d", a->mode);
}

// Index tables of a capacity-128 call rewritten for 64-token halves:
// kept lists, counts, half lengths and (when given) the processing order.
struct HalfTables {
  size_t idx, num, len, order;
  size_t total() const { return idx + num + len + order; }
};
static HalfTables half_tables(const bsa_qouter_args* a) {
  HalfTables t{0, 0, 0, 0};
  if (a->mode != BSA_SEL_BLOCK || a->M != 128) return t;
  const size_t rows = (size_t)a->dq.B * a->dq.H * 2 * a->J;
  t.idx = round_up(rows * 2 * a->kmax * sizeof(int32_t));
  t.num = round_up(rows * sizeof(int32_t));
  t.len = round_up((size_t)2 * a->J * sizeof(int32_t));
  t.order = a->item_order ? round_up(rows * sizeof(int32_t)) : 0;
  return t;
}

// Workspace of bsa_forward_qouter: the scheduler state of the block-mode
// persistent grid (bf16; none for the fp32 and token modes), then the half
// tables of a capacity-128 call.
static size_t qouter_sched_need(const bsa_qouter_args* a) {
  return (a->mode == BSA_SEL_BLOCK && a->dt == BSA_BF16) ? bsa::qouter_sched_bytes() : 0;
}
static size_t qouter_ws_need(const bsa_qouter_args* a) { return qouter_sched_need(a) + half_tables(a).total(); }

// Launches a validated call with `sched` as the scheduler state (nullptr when
// the mode needs none).
static bsa_status launch_qouter(const bsa_qouter_args* a, void* sched, void* stream) {
  const float scale_log2 = a->scale * 1.4426950408889634f;
  hipStream_t s = (hipStream_t)stream;
  if (a->mode == BSA_SEL_BLOCK && a->M == 128) {
    // the same attention over 64-token halves: rewrite the tables behind the
    // scheduler state, then run the capacity-64 kernels on them
    const HalfTables t = half_tables(a);
    char* w = static_cast<char*>(sched) + qouter_sched_need(a);
    int32_t* idx2 = reinterpret_cast<int32_t*>(w);
    int32_t* num2 = reinterpret_cast<int32_t*>(w + t.idx);
    int32_t* len2 = reinterpret_cast<int32_t*>(w + t.idx + t.num);
    int32_t* ord2 = a->item_order ? reinterpret_cast<int32_t*>(w + t.idx + t.num + t.len) : nullptr;
    hipError_t e = bsa::launch_expand_halves(a->q2k_idx, a->q2k_num, a->block_len, a->item_order,
                                             (int)(a->dq.B * a->dq.H), a->J, a->kmax, idx2, num2, len2, ord2, s);
    if (e != hipSuccess) return hip_status(e, "half-block tables launch");
    bsa_qouter_args h = *a;
    h.M = 64;
    h.J = 2 * a->J;
    h.kmax = 2 * a->kmax;
    h.q2k_idx = idx2;
    h.q2k_num = num2;
    h.block_len = len2;
    h.item_order = ord2;
    h.order_long = 2 * a->order_long;
    return launch_qouter(&h, qouter_sched_need(a) ? sched : nullptr, stream);
  }
  if (a->mode == BSA_SEL_BLOCK) {
    bsa::VsaAttnParams p{a->q, a->k, a->v, a->out,
                         a->dq.sB, a->dq.sN, a->dq.sH, a->dkv.sB, a->dkv.sN, a->dkv.sH,
                         a->dout.sB, a->dout.sN, a->dout.sH,
                         a->perm, a->block_len, a->q2k_idx, a->q2k_num,
                         (int)a->dq.B, (int)a->dq.H, a->J, a->M, a->kmax, (int)a->dq.D, a->dq.N,
                         scale_log2, a->lse, a->item_order, a->k_sum, a->v_sum, a->b_sum,
                         a->coarse, a->gate, a->perm_bh_stride, sched, device_error_flag(), a->order_long};
    return hip_status(bsa::launch_vsa_attention(p, a->dt == BSA_F32, s), "vsa attention launch");
  }
  bsa::NsaAttnParams p{a->q, a->k, a->v, a->out,
                       a->dq.sB, a->dq.sN, a->dq.sH, a->dkv.sB, a->dkv.sN, a->dkv.sH,
                       a->dout.sB, a->dout.sN, a->dout.sH,
                       a->blk_idx, a->blk_cnt,
                       (int)a->dq.B, (int)a->dq.H, (int)a->dkv.H, a->S, a->BS, a->causal ? 1 : 0,
                       (int)a->dq.D, a->dq.N, scale_log2, a->lse, device_error_flag()};
  return hip_status(bsa::launch_nsa_attention(p, false, s), "nsa attention launch");
}

bsa_status bsa_qouter_ws(const bsa_qouter_args* a, size_t* bytes) {
  if (!bytes) return fail(BSA_ERR_ARG, "bsa_qouter_ws: null output");
  bsa_status st = check_qouter(a);
  if (st != BSA_OK) return st;
  *bytes = qouter_ws_need(a);
  return ok();
}

bsa_status bsa_forward_qouter(const bsa_qouter_args* a, void* ws, size_t ws_bytes, void* stream) {
  bsa_status st = check_qouter(a);
  if (st != BSA_OK) return st;
  const size_t need = qouter_ws_need(a);
  if (need && (!ws || ws_bytes < need))
    return fail(BSA_ERR_WORKSPACE, "bsa_forward_qouter: workspace of %zu bytes required", need);
  if (need && (reinterpret_cast<uintptr_t>(ws) & 255u))
    return fail(BSA_ERR_WORKSPACE, "bsa_forward_qouter: workspace must be 256-byte aligned");
  return launch_qouter(a, need ? ws : nullptr, stream);
}

// ---------------------------------------------- query-outer attention, no allocation
// Scratch of bsa_forward_qouter_static: the scheduler state that
// bsa_forward_qouter keeps in the caller's workspace.  One copy per device,
// held until the process ends; host code reaches a device's copy only through
// the address hipGetSymbolAddress returns for it (kept in g_scratch_ptr).
constexpr size_t kQouterScratchBytes = 256 * 1024;
}  // extern "C"

static __device__ __align__(256) unsigned char scratch[kQouterScratchBytes];

namespace {
void* g_scratch_ptr[kMaxDevices] = {nullptr};

// The current device's scratch address, looked up once per device with that
// device current; nullptr (and the HIP error in *e) if the lookup fails.
void* device_scratch(hipError_t* e) {
  int dev = 0;
  *e = hipGetDevice(&dev);
  if (*e != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *e = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    *e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (*e != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

bsa_status bsa_forward_qouter_static(const bsa_qouter_args* a, void* stream) {
  bsa_status st = check_qouter(a);
  if (st != BSA_OK) return st;
  const size_t need = qouter_ws_need(a);
  if (need > kQouterScratchBytes)
    return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_qouter_static: %zu bytes of scratch needed, the static limit is %zu",
                need, kQouterScratchBytes);
  void* sched = nullptr;
  if (need) {
    hipError_t e = hipSuccess;
    sched = device_scratch(&e);
    if (!sched) return hip_status(e, "bsa_forward_qouter_static: scratch address");
  }
  return launch_qouter(a, sched, stream);
}

// ------------------------------------------------------------------ coarse branch
static bsa_status check_coarse(const vsa_coarse_args* a) {
  if (!a) return fail(BSA_ERR_ARG, "vsa_coarse: null args");
  if (!a->v || !a->perm || !a->block_len || !a->E || !a->C)
    return fail(BSA_ERR_ARG, "vsa_coarse: v, perm, block_len, E and C are required");
  if (a->dt != BSA_BF16 && a->dt != BSA_F32) return fail(BSA_ERR_ARG, "vsa_coarse: bad dtype");
  bsa_status st = check_desc(a->d, "v", 1, false);
  if (st != BSA_OK) return st;
  if (a->d.D != 64 && a->d.D != 128) return fail(BSA_ERR_UNSUPPORTED, "vsa_coarse: D must be 64 or 128");
  if (a->J < 1 || a->M < 1) return fail(BSA_ERR_SHAPE, "vsa_coarse: J and M must be positive");
  if ((int64_t)a->d.B * a->d.H > 65535) return fail(BSA_ERR_UNSUPPORTED, "vsa_coarse: B*H must be <= 65535");
  if (!aligned16(a->C) || (a->vbar && !aligned16(a->vbar)))
    return fail(BSA_ERR_SHAPE, "vsa_coarse: C and vbar must be 16-byte aligned");
  return BSA_OK;
}

bsa_status vsa_coarse_ws(const vsa_coarse_args* a, size_t* bytes) {
  if (!bytes) return fail(BSA_ERR_ARG, "vsa_coarse_ws: null output");
  bsa_status st = check_coarse(a);
  if (st != BSA_OK) return st;
  const size_t BH = (size_t)a->d.B * a->d.H;
  *bytes = (a->vbar ? 0 : round_up(BH * a->J * a->d.D * sizeof(float))) +
           round_up(2 * BH * a->d.D * bsa::coarse_jpad(a->J) * sizeof(__bf16));
  return ok();
}

bsa_status vsa_coarse(const vsa_coarse_args* a, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  bsa_status st = vsa_coarse_ws(a, &need);
  if (st != BSA_OK) return st;
  if (need && (!ws || ws_bytes < need))
    return fail(BSA_ERR_WORKSPACE, "vsa_coarse: workspace of %zu bytes required", need);
  if (!aligned16(ws)) return fail(BSA_ERR_WORKSPACE, "vsa_coarse: workspace must be 16-byte aligned");
  const size_t BH = (size_t)a->d.B * a->d.H;
  const size_t vbar_ws = a->vbar ? 0 : round_up(BH * a->J * a->d.D * sizeof(float));
  float* vbar = a->vbar ? a->vbar : static_cast<float*>(ws);
  __bf16* vt = reinterpret_cast<__bf16*>(static_cast<char*>(ws) + vbar_ws);
  const int vec = 16 / elem_bytes(a->dt);
  const bool vec_ok = a->d.D % vec == 0 && a->d.sB % vec == 0 && a->d.sN % vec == 0 && a->d.sH % vec == 0 &&
                      aligned16(a->v);
  // the pooling kernel of the routing step, run on V alone
  bsa::PoolParams pp{a->v, a->v, a->d.sB, a->d.sN, a->d.sH, (int)a->d.B, (int)a->d.H, (int)a->d.D, a->J, a->M,
                     a->perm, a->block_len, vbar, vbar, 0};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = bsa::launch_pool(pp, a->dt == BSA_F32, vec_ok, s, 1);
  if (e != hipSuccess) return hip_status(e, "pool launch");
  bsa::CoarseParams cp{a->E, vbar, a->C, (int)(a->d.B * a->d.H), a->J, (int)a->d.D, vt};
  return hip_status(bsa::launch_coarse(cp, s), "coarse launch");
}

// ------------------------------------------------------------ Spark-Reweight summaries
static bsa_status check_summaries(const spark_summary_args* a) {
  if (!a) return fail(BSA_ERR_ARG, "spark_summaries: null args");
  if (!a->k || !a->v || !a->perm || !a->block_len || !a->k_sum || !a->v_sum || !a->b_sum)
    return fail(BSA_ERR_ARG, "spark_summaries: k, v, perm, block_len, k_sum, v_sum and b_sum are required");
  if (!a->anchor && !a->q) return fail(BSA_ERR_ARG, "spark_summaries: q is required when anchor is NULL");
  if (a->dt != BSA_BF16) return fail(BSA_ERR_UNSUPPORTED, "spark_summaries: bf16 only");
  bsa_status st = check_desc(a->d, "q/k/v", 8, true);
  if (st != BSA_OK) return st;
  if (a->d.D != 64 && a->d.D != 128) return fail(BSA_ERR_UNSUPPORTED, "spark_summaries: D must be 64 or 128");
  if (a->J < 1 || a->M < 1 || a->M > 64)
    return fail(BSA_ERR_SHAPE, "spark_summaries: J must be positive and M in [1, 64]");
  if ((int64_t)a->d.B * a->d.H * a->J >= (int64_t)1 << 31)
    return fail(BSA_ERR_UNSUPPORTED, "spark_summaries: too many blocks");
  if (a->d.N >= (int64_t)1 << 31) return fail(BSA_ERR_UNSUPPORTED, "spark_summaries: N must be below 2^31");
  if (!std::isfinite(a->scale)) return fail(BSA_ERR_ARG, "spark_summaries: scale must be finite");
  if (!aligned16(a->k) || !aligned16(a->v) || (a->q && !aligned16(a->q)) || !aligned16(a->k_sum) ||
      !aligned16(a->v_sum))
    return fail(BSA_ERR_SHAPE, "spark_summaries: q, k, v, k_sum, v_sum must be 16-byte aligned");
  return BSA_OK;
}

bsa_status spark_summaries_ws(const spark_summary_args* a, size_t* bytes) {
  if (!bytes) return fail(BSA_ERR_ARG, "spark_summaries_ws: null output");
  bsa_status st = check_summaries(a);
  if (st != BSA_OK) return st;
  *bytes = 0;
  if (!a->anchor) {
    *bytes += round_up(bsa::anchor_workspace_bytes((int)a->d.B, (int)a->d.N, (int)a->d.H, (int)a->d.D));
    if (!a->anchor_out) *bytes += round_up((size_t)a->d.B * a->d.H * a->d.D * sizeof(float));
  }
  return ok();
}

bsa_status spark_summaries(const spark_summary_args* a, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  bsa_status st = spark_summaries_ws(a, &need);
  if (st != BSA_OK) return st;
  if (need && (!ws || ws_bytes < need))
    return fail(BSA_ERR_WORKSPACE, "spark_summaries: workspace of %zu bytes required", need);
  hipStream_t s = (hipStream_t)stream;
  const int B = (int)a->d.B, N = (int)a->d.N, H = (int)a->d.H, D = (int)a->d.D;
  const float* anchor = a->anchor;
  if (!anchor) {
    char* w = static_cast<char*>(ws);
    float* part = reinterpret_cast<float*>(w);
    w += round_up(bsa::anchor_workspace_bytes(B, N, H, D));
    float* anc = a->anchor_out ? a->anchor_out : reinterpret_cast<float*>(w);
    hipError_t e = bsa::launch_anchor(a->q, a->d.sB, a->d.sN, a->d.sH, B, N, H, D, part, anc, s);
    if (e != hipSuccess) return hip_status(e, "anchor launch");
    anchor = anc;
  } else if (a->anchor_out) {
    hipError_t e = hipMemcpyAsync(a->anchor_out, a->anchor, (size_t)B * H * D * sizeof(float),
                                  hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_status(e, "anchor copy");
  }
  bsa::SummaryParams sp{a->k, a->v, a->d.sB, a->d.sN, a->d.sH, B, H, D, a->J, a->M,
                        a->perm, a->block_len, anchor, a->scale, a->k_sum, a->v_sum, a->b_sum};
  return hip_status(bsa::launch_summaries(sp, s), "summary launch");
}

// ------------------------------------------------------------------------ Spark-Reblock
bsa_status spark_reblock_dims(int N, int M, int* J, int* nlevels) {
  if (!J || !nlevels) return fail(BSA_ERR_ARG, "spark_reblock_dims: null output pointer");
  if (N < 1 || M < 1) return fail(BSA_ERR_SHAPE, "spark_reblock_dims: N and M must be positive");
  const int64_t jj = ((int64_t)N + M - 1) / M;
  if (jj > 65536 || jj * M >= (int64_t)1 << 31)
    return fail(BSA_ERR_UNSUPPORTED, "spark_reblock_dims: at most 65536 leaves");
  *J = (int)jj;
  *nlevels = bsa::reblock_levels(N, M);
  return ok();
}

namespace {
struct ReblockWs {
  size_t part, moment, factor, features, dirs, keys, order, total;
};

ReblockWs reblock_ws_layout(const spark_reblock_args* a) {
  const int64_t BH = a->d.B * a->d.H, N = a->d.N, D = a->d.D;
  const int64_t nc = (N + 2047) / 2048;
  const int nlev = bsa::reblock_levels((int)N, a->M);
  const int64_t slots = (int64_t)1 << (nlev > 1 ? nlev - 2 : 0);
  ReblockWs w{};
  w.part = round_up((size_t)(nc * BH * D * D * 4));
  w.moment = a->moment ? 0 : round_up((size_t)(BH * D * D * 4));
  w.factor = a->factor ? 0 : round_up((size_t)(BH * D * D * 4));
  w.features = round_up((size_t)(BH * N * D * 2));  // fp16 features (the debug output is a copy)
  w.dirs = round_up((size_t)(BH * slots * D * 4));
  w.keys = round_up((size_t)(BH * N * 8));
  w.order = round_up((size_t)(BH * N * 4));
  w.total = w.part + w.moment + w.factor + w.features + w.dirs + 2 * w.keys + 2 * w.order;
  return w;
}
}  // namespace

static bsa_status check_reblock(const spark_reblock_args* a) {
  if (!a) return fail(BSA_ERR_ARG, "spark_reblock: null args");
  if (!a->q || !a->k || !a->perm || !a->block_len)
    return fail(BSA_ERR_ARG, "spark_reblock: q, k, perm and block_len are required");
  if (a->dt != BSA_BF16) return fail(BSA_ERR_UNSUPPORTED, "spark_reblock: bf16 only");
  bsa_status st = check_desc(a->d, "q/k", 8, true);
  if (st != BSA_OK) return st;
  if (a->d.D != 64 && a->d.D != 128) return fail(BSA_ERR_UNSUPPORTED, "spark_reblock: D must be 64 or 128");
  if (a->M != 16 && a->M != 32 && a->M != 64) return fail(BSA_ERR_UNSUPPORTED, "spark_reblock: M must be 16, 32 or 64");
  if (a->d.B * a->d.H > 65535) return fail(BSA_ERR_UNSUPPORTED, "spark_reblock: B*H must be <= 65535");
  if (a->d.B * a->d.H * a->d.N >= (int64_t)1 << 31)
    return fail(BSA_ERR_UNSUPPORTED, "spark_reblock: B*H*N must be below 2^31");
  int J = 0, nl = 0;
  if ((st = spark_reblock_dims((int)a->d.N, a->M, &J, &nl)) != BSA_OK) return st;
  if (!(a->ridge > 0.f) || !std::isfinite(a->ridge)) return fail(BSA_ERR_ARG, "spark_reblock: ridge must be > 0");
  if (!aligned16(a->q) || !aligned16(a->k) || (a->factor && !aligned16(a->factor)) ||
      (a->features && !aligned16(a->features)) || (a->dirs && !aligned16(a->dirs)))
    return fail(BSA_ERR_SHAPE, "spark_reblock: q, k, factor, features and dirs must be 16-byte aligned");
  return BSA_OK;
}

bsa_status spark_reblock_ws(const spark_reblock_args* a, size_t* bytes) {
  if (!bytes) return fail(BSA_ERR_ARG, "spark_reblock_ws: null output");
  bsa_status st = check_reblock(a);
  if (st != BSA_OK) return st;
  *bytes = reblock_ws_layout(a).total;
  return ok();
}

bsa_status spark_reblock(const spark_reblock_args* a, void* ws, size_t ws_bytes, void* stream) {
  bsa_status st = check_reblock(a);
  if (st != BSA_OK) return st;
  const ReblockWs w = reblock_ws_layout(a);
  if (!ws || ws_bytes < w.total) return fail(BSA_ERR_WORKSPACE, "spark_reblock: workspace of %zu bytes required", w.total);
  if (reinterpret_cast<uintptr_t>(ws) & 255u)
    return fail(BSA_ERR_WORKSPACE, "spark_reblock: workspace must be 256-byte aligned");
  char* p = static_cast<char*>(ws);
  auto take = [&](size_t n) { char* r = p; p += n; return r; };
  bsa::ReblockParams rp{};
  rp.q = a->q, rp.k = a->k, rp.sB = a->d.sB, rp.sN = a->d.sN, rp.sH = a->d.sH;
  rp.B = (int)a->d.B, rp.H = (int)a->d.H, rp.N = (int)a->d.N, rp.D = (int)a->d.D, rp.M = a->M;
  rp.ridge = a->ridge;
  rp.part = reinterpret_cast<float*>(take(w.part));
  rp.moment = a->moment ? a->moment : reinterpret_cast<float*>(take(w.moment));
  rp.factor = a->factor ? a->factor : reinterpret_cast<float*>(take(w.factor));
  rp.features = reinterpret_cast<_Float16*>(take(w.features));
  rp.features32 = a->features;
  rp.dirs = reinterpret_cast<float*>(take(w.dirs));
  rp.keys0 = reinterpret_cast<uint64_t*>(take(w.keys));
  rp.keys1 = reinterpret_cast<uint64_t*>(take(w.keys));
  rp.order0 = reinterpret_cast<int32_t*>(take(w.order));
  rp.order1 = reinterpret_cast<int32_t*>(take(w.order));
  rp.levels = a->levels, rp.perm = a->perm, rp.block_len = a->block_len;
  rp.dirs_out = a->dirs;
  return hip_status(bsa::launch_reblock(rp, (hipStream_t)stream), "reblock launch");
}

// ------------------------------------------------------------------------ KV-outer
static bsa_status check_kvouter(const bsa_kvouter_args* a, bsa::KvOuterParams* out) {
  if (!a) return fail(BSA_ERR_ARG, "bsa_forward_kvouter: null args");
  if (!a->q || !a->k || !a->v || !a->q2k || !a->o_buf || !a->lse_buf || !a->nslot)
    return fail(BSA_ERR_ARG, "bsa_forward_kvouter: q, k, v, q2k, o_buf, lse_buf and nslot are required");
  if (a->dt != BSA_BF16) return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_kvouter: bf16 only");
  bsa_status st = check_desc(a->dq, "q", 8, true);
  if (st != BSA_OK) return st;
  if ((st = check_desc(a->dkv, "k/v", 8, true)) != BSA_OK) return st;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o_buf))
    return fail(BSA_ERR_SHAPE, "bsa_forward_kvouter: q, k, v, o_buf must be 16-byte aligned");
  if (a->dq.D != a->dkv.D || (a->dq.D != 64 && a->dq.D != 128))
    return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_kvouter: D must be 64 or 128 for q and k/v");
  if (a->dq.B != a->dkv.B || a->dq.N != a->dkv.N) return fail(BSA_ERR_SHAPE, "bsa_forward_kvouter: B/N mismatch");
  if (a->dq.H % a->dkv.H) return fail(BSA_ERR_SHAPE, "bsa_forward_kvouter: Hq must be a multiple of Hkv");
  if (a->BK != 16 && a->BK != 32 && a->BK != 64 && a->BK != 128)
    return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_kvouter: BK must be 16, 32, 64 or 128");
  if (a->k_sel < 1 || a->k_sel > 64) return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_kvouter: k_sel must lie in [1, 64]");
  if (a->chunk_cap < 0) return fail(BSA_ERR_ARG, "bsa_forward_kvouter: chunk_cap must be >= 0");
  if (!std::isfinite(a->scale)) return fail(BSA_ERR_ARG, "bsa_forward_kvouter: scale must be finite");
  const int64_t threads = a->dq.B * a->dq.N * a->dkv.H;
  if (threads * a->k_sel >= (int64_t)1 << 31)
    return fail(BSA_ERR_UNSUPPORTED, "bsa_forward_kvouter: B*N*Hkv*k_sel must be below 2^31");
  *out = bsa::KvOuterParams{a->q, a->k, a->v, a->dq.sB, a->dq.sN, a->dq.sH, a->dkv.sB, a->dkv.sN, a->dkv.sH,
                            a->q2k, a->q2k_cnt, (int)a->dq.B, (int)a->dq.H, (int)a->dkv.H, a->k_sel, a->BK,
                            (int)a->dq.D, a->causal ? 1 : 0, a->chunk_cap, a->dq.N,
                            a->scale * 1.4426950408889634f, reinterpret_cast<__bf16*>(a->o_buf), a->lse_buf,
                            a->nslot, device_error_flag()};
  return BSA_OK;
}

bsa_status bsa_kvouter_ws(const bsa_kvouter_args* a, size_t* bytes) {
  if (!bytes) return fail(BSA_ERR_ARG, "bsa_kvouter_ws: null output");
  bsa::KvOuterParams p{};
  bsa_status st = check_kvouter(a, &p);
  if (st != BSA_OK) return st;
  *bytes = bsa::kvouter_ws_bytes(p);
  return ok();
}

bsa_status bsa_kvouter_index_layout(const bsa_kvouter_args* a, bsa_kvouter_layout* out) {
  if (!out) return fail(BSA_ERR_ARG, "bsa_kvouter_index_layout: null output");
  bsa::KvOuterParams p{};
  bsa_status st = check_kvouter(a, &p);
  if (st != BSA_OK) return st;
  bsa::kvouter_index_layout(p, out);
  return ok();
}

bsa_status bsa_forward_kvouter(const bsa_kvouter_args* a, void* ws, size_t ws_bytes, void* stream) {
  bsa::KvOuterParams p{};
  bsa_status st = check_kvouter(a, &p);
  if (st != BSA_OK) return st;
  const size_t need = bsa::kvouter_ws_bytes(p);
  if (!ws || ws_bytes < need)
    return fail(BSA_ERR_WORKSPACE, "bsa_forward_kvouter: workspace of %zu bytes required", need);
  if (reinterpret_cast<uintptr_t>(ws) & 255u)
    return fail(BSA_ERR_WORKSPACE, "bsa_forward_kvouter: workspace must be 256-byte aligned");
  return hip_status(bsa::launch_kvouter(p, ws, (hipStream_t)stream), "kv-outer launch");
}

bsa_status bsa_combine(const bsa_combine_args* a, void* stream) {
  if (!a) return fail(BSA_ERR_ARG, "bsa_combine: null args");
  if (!a->o_buf || !a->lse_buf || !a->nslot || !a->out)
    return fail(BSA_ERR_ARG, "bsa_combine: o_buf, lse_buf, nslot and out are required");
  bsa_status st = check_desc(a->dout, "out", 8, true);
  if (st != BSA_OK) return st;
  if (!aligned16(a->o_buf) || !aligned16(a->out))
    return fail(BSA_ERR_SHAPE, "bsa_combine: o_buf and out must be 16-byte aligned");
  if (a->Hkv < 1 || a->dout.H % a->Hkv) return fail(BSA_ERR_SHAPE, "bsa_combine: Hq must be a multiple of Hkv");
  if (a->k_sel < 1 || a->k_sel > 64) return fail(BSA_ERR_UNSUPPORTED, "bsa_combine: k_sel must lie in [1, 64]");
  if (a->dout.D > 256) return fail(BSA_ERR_UNSUPPORTED, "bsa_combine: D must be <= 256");
  if (a->dout.B * a->dout.N >= (int64_t)1 << 31) return fail(BSA_ERR_UNSUPPORTED, "bsa_combine: too many positions");
  bsa::CombineParams p{reinterpret_cast<const __bf16*>(a->o_buf), a->lse_buf, a->nslot, (int)a->dout.B,
                       (int)a->dout.H, a->Hkv, a->k_sel, (int)a->dout.D, a->dout.N,
                       reinterpret_cast<__bf16*>(a->out), a->dout.sB, a->dout.sN, a->dout.sH, a->lse};
  return hip_status(bsa::launch_combine(p, (hipStream_t)stream), "combine launch");
}

}  // extern "C"
