// Host side of the gnf4 C ABI: argument validation, path dispatch, error text.
// Every check runs before any HIP call, so invalid arguments are rejected
// identically on machines without a GPU.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "common.h"

#ifndef GNF4_REVISION
#define GNF4_REVISION "unknown"
#endif

namespace gnf4 {

static thread_local char g_err[512] = "";

static gnf4_status fail(gnf4_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

static gnf4_status ok() {
  g_err[0] = '\0';
  return GNF4_OK;
}

static gnf4_status device_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(GNF4_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// The route's workspace: at least route_workspace_bytes(T*k, E) bytes,
// 16-byte aligned (NULL allowed when none is needed).
static gnf4_status check_route_workspace(int32_t T, int32_t k, int32_t E, const void *workspace,
                                         size_t workspace_bytes) {
  const size_t need = route_workspace_bytes((int64_t)T * k, E);
  if (need == 0) return ok();
  if (workspace_bytes < need)
    return fail(GNF4_ERR_WORKSPACE, "route workspace of %zu bytes given, %zu needed for T*k = %lld, "
                "E = %d", workspace_bytes, need, (long long)T * k, E);
  if (!workspace || !aligned16(workspace))
    return fail(GNF4_ERR_INVALID_ARG, "route workspace must be a 16-byte aligned device pointer");
  return ok();
}

int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

static gnf4_status check_weights(const gnf4_weights *w) {
  if (!w) return fail(GNF4_ERR_INVALID_ARG, "weights descriptor is NULL");
  if (w->format < GNF4_NF4 || w->format > GNF4_MXFP4)
    return fail(GNF4_ERR_INVALID_ARG, "unknown format %d", w->format);
  if (w->E < 1 || w->E > GNF4_MAX_EXPERTS)
    return fail(GNF4_ERR_INVALID_ARG, "E = %d outside [1, %d]", w->E, GNF4_MAX_EXPERTS);
  if (w->N < 1 || w->N > GNF4_MAX_N)
    return fail(GNF4_ERR_INVALID_ARG, "N = %d outside [1, %d]", w->N, GNF4_MAX_N);
  const int blk = w->format == GNF4_MXFP4 ? 32 : 64;
  if (w->K < blk || w->K > GNF4_MAX_K || w->K % blk)
    return fail(GNF4_ERR_INVALID_ARG, "K = %d must be a positive multiple of %d up to %d", w->K,
                blk, GNF4_MAX_K);
  if (!w->codes || !w->scales) return fail(GNF4_ERR_INVALID_ARG, "codes or scales is NULL");
  if (!aligned16(w->codes)) return fail(GNF4_ERR_INVALID_ARG, "codes must be 16-byte aligned");
  if (w->format == GNF4_NF4 && ((uintptr_t)w->scales & 3u))
    return fail(GNF4_ERR_INVALID_ARG, "float32 scales must be 4-byte aligned");
  if (w->format == GNF4_NF4_DQ && !w->scales2)
    return fail(GNF4_ERR_INVALID_ARG, "NF4_DQ needs scales2");
  if (w->format == GNF4_NF4_DQ && ((uintptr_t)w->scales2 & 3u))
    return fail(GNF4_ERR_INVALID_ARG, "scales2 must be 4-byte aligned");
  if ((int64_t)w->E * w->N * (w->K / 2) > (int64_t)1 << 40)
    return fail(GNF4_ERR_UNSUPPORTED, "weight tensor too large");
  if ((int64_t)w->N * (w->K / 2) >= (int64_t)1 << 32)
    return fail(GNF4_ERR_UNSUPPORTED, "one expert's packed codes must be below 4 GiB");
  return ok();
}

static Weights to_kernel(const gnf4_weights *w) {
  Weights k;
  k.format = w->format;
  k.E = w->E;
  k.N = w->N;
  k.K = w->K;
  k.codes = w->codes;
  k.scales = w->scales;
  k.scales2 = w->scales2;
  return k;
}

// Decode path for T*k routed rows at or below this count, and the largest K
// its register-resident token slices cover.
constexpr int kGemvMaxRows = 64;
constexpr int kGemvMaxK = 8192;

}  // namespace gnf4

using namespace gnf4;

extern "C" {

size_t gnf4_route_workspace_bytes(int32_t T, int32_t k, int32_t E) {
  if (T < 0 || k < 1 || k > 64 || E < 1 || E > GNF4_MAX_EXPERTS ||
      (int64_t)T * k >= ((int64_t)1 << 31) - 1024)
    return 0;
  return route_workspace_bytes((int64_t)T * k, E);
}

gnf4_status gnf4_route(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E, int32_t *counts,
                       int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *active,
                       int32_t *n_active, int32_t *bad_id_flag, void *workspace,
                       size_t workspace_bytes, gnf4_stream_t stream) {
  if (E < 1 || E > GNF4_MAX_EXPERTS)
    return fail(GNF4_ERR_INVALID_ARG, "E = %d outside [1, %d]", E, GNF4_MAX_EXPERTS);
  if (k < 1 || k > 64) return fail(GNF4_ERR_INVALID_ARG, "k = %d outside [1, 64]", k);
  if (T < 0) return fail(GNF4_ERR_INVALID_ARG, "T = %d is negative", T);
  if ((int64_t)T * k >= ((int64_t)1 << 31) - 1024)
    return fail(GNF4_ERR_INVALID_ARG, "T*k too large");
  if (!counts || !offsets || !active || !n_active || !bad_id_flag)
    return fail(GNF4_ERR_INVALID_ARG, "an output pointer is NULL");
  if (T > 0 && (!topk_ids || !perm || !inv))
    return fail(GNF4_ERR_INVALID_ARG, "topk_ids, perm or inv is NULL");
  gnf4_status st = check_route_workspace(T, k, E, workspace, workspace_bytes);
  if (st != GNF4_OK) return st;
  return device_status(launch_route(topk_ids, T, k, E, counts, offsets, perm, inv, active,
                                    n_active, bad_id_flag, workspace, (hipStream_t)stream),
                       "route launch");
}

gnf4_status gnf4_route_noalloc(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E,
                               int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv,
                               int32_t *active, int32_t *n_active, int32_t *bad_id_flag,
                               gnf4_stream_t stream) {
  if (E < 1 || E > GNF4_MAX_EXPERTS)
    return fail(GNF4_ERR_INVALID_ARG, "E = %d outside [1, %d]", E, GNF4_MAX_EXPERTS);
  if (k < 1 || k > 64) return fail(GNF4_ERR_INVALID_ARG, "k = %d outside [1, 64]", k);
  if (T < 0) return fail(GNF4_ERR_INVALID_ARG, "T = %d is negative", T);
  if ((int64_t)T * k >= ((int64_t)1 << 31) - 1024)
    return fail(GNF4_ERR_INVALID_ARG, "T*k too large");
  if (!counts || !offsets || !active || !n_active || !bad_id_flag)
    return fail(GNF4_ERR_INVALID_ARG, "an output pointer is NULL");
  if (T > 0 && (!topk_ids || !perm || !inv))
    return fail(GNF4_ERR_INVALID_ARG, "topk_ids, perm or inv is NULL");
  const size_t need = route_workspace_bytes((int64_t)T * k, E);
  if (need > route_scratch_bytes())
    return fail(GNF4_ERR_WORKSPACE, "T*k = %lld over E = %d needs %zu bytes of route workspace, "
                "more than the %zu-byte static one (use gnf4_route with a workspace)",
                (long long)T * k, E, need, route_scratch_bytes());
  void *ws = nullptr;
  if (need > 0) {
    hipError_t e = hipSuccess;
    ws = route_scratch_ptr(&e);
    if (!ws) return device_status(e, "route scratch address");
  }
  return device_status(launch_route(topk_ids, T, k, E, counts, offsets, perm, inv, active,
                                    n_active, bad_id_flag, ws, (hipStream_t)stream),
                       "route launch");
}

gnf4_status gnf4_route_logits(const float *logits, int32_t T, int32_t k, int32_t E,
                              int32_t *topk_ids, float *topk_w, int32_t *counts,
                              int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *active,
                              int32_t *n_active, int32_t *bad_id_flag, void *workspace,
                              size_t workspace_bytes, gnf4_stream_t stream) {
  if (E < 1 || E > GNF4_MAX_EXPERTS)
    return fail(GNF4_ERR_INVALID_ARG, "E = %d outside [1, %d]", E, GNF4_MAX_EXPERTS);
  if (k < 1 || k > 64 || k > E)
    return fail(GNF4_ERR_INVALID_ARG, "k = %d outside [1, min(64, E = %d)]", k, E);
  if (T < 0) return fail(GNF4_ERR_INVALID_ARG, "T = %d is negative", T);
  if ((int64_t)T * k >= ((int64_t)1 << 31) - 1024)
    return fail(GNF4_ERR_INVALID_ARG, "T*k too large");
  if (!counts || !offsets || !active || !n_active || !bad_id_flag)
    return fail(GNF4_ERR_INVALID_ARG, "an output pointer is NULL");
  if (T > 0 && (!logits || !topk_ids || !topk_w || !perm || !inv))
    return fail(GNF4_ERR_INVALID_ARG, "logits, topk_ids, topk_w, perm or inv is NULL");
  gnf4_status st = check_route_workspace(T, k, E, workspace, workspace_bytes);
  if (st != GNF4_OK) return st;
  hipError_t e = launch_topk(logits, T, E, k, topk_ids, topk_w, (hipStream_t)stream);
  if (e != hipSuccess) return device_status(e, "top-k launch");
  return device_status(launch_route(topk_ids, T, k, E, counts, offsets, perm, inv, active,
                                    n_active, bad_id_flag, workspace, (hipStream_t)stream),
                       "route launch");
}

gnf4_status gnf4_swiglu(const float *Y, int32_t rows, int32_t I, uint16_t *H,
                        gnf4_stream_t stream) {
  if (rows < 0) return fail(GNF4_ERR_INVALID_ARG, "rows = %d is negative", rows);
  if (I < 4 || I % 4 || I > GNF4_MAX_N / 2)
    return fail(GNF4_ERR_INVALID_ARG, "I = %d must be a positive multiple of 4 up to %d", I,
                GNF4_MAX_N / 2);
  if (rows == 0) return ok();
  if (!Y || !H) return fail(GNF4_ERR_INVALID_ARG, "Y or H is NULL");
  if (!aligned16(Y) || ((uintptr_t)H & 7u))
    return fail(GNF4_ERR_INVALID_ARG, "Y must be 16-byte and H 8-byte aligned");
  return device_status(launch_swiglu(Y, rows, I, H, (hipStream_t)stream), "swiglu launch");
}

}  // extern "C"

// Shared by both GEMM entry points: validation, then the path chosen from
// T*k (exactly one of Y / H is non-NULL).
// Routing to run before the GEMM (gnf4_route_grouped_gemm): the ids and the
// routing outputs; fused into the one-token GEMV when that path runs.
struct FusedRoute {
  const int32_t *ids;
  int32_t *counts, *offsets, *perm, *inv, *active, *n_active, *bad;
  const float *logits;        // instead of ids: the router's top-k first
  int32_t *topk_ids;
  float *topk_w;
  void *workspace;            // the route's (checked by the caller)
};

static gnf4_status grouped_gemm_any(const gnf4_weights *w, const uint16_t *X, int32_t gather,
                                    const int32_t *offsets, const int32_t *perm,
                                    const int32_t *active, const int32_t *n_active, int32_t T,
                                    int32_t k, float *Y, uint16_t *H, gnf4_stream_t stream,
                                    const FusedRoute *fr = nullptr) {
  gnf4_status st = check_weights(w);
  if (st != GNF4_OK) return st;
  if (gather != 0 && gather != 1) return fail(GNF4_ERR_INVALID_ARG, "gather must be 0 or 1");
  if (k < 1 || k > 64) return fail(GNF4_ERR_INVALID_ARG, "k = %d outside [1, 64]", k);
  if (T < 0) return fail(GNF4_ERR_INVALID_ARG, "T = %d is negative", T);
  if ((int64_t)T * k >= ((int64_t)1 << 31) - 1024)
    return fail(GNF4_ERR_INVALID_ARG, "T*k too large");
  if (H && w->N % 2)
    return fail(GNF4_ERR_INVALID_ARG, "the SwiGLU epilogue needs an even N (gate and up halves)");
  if (T == 0) return ok();
  if (!X || !offsets || !perm || !active || !n_active || !(Y || H))
    return fail(GNF4_ERR_INVALID_ARG, "a pointer argument is NULL");
  if (!aligned16(X) || (Y && !aligned16(Y)) || (H && ((uintptr_t)H & 1u)))
    return fail(GNF4_ERR_INVALID_ARG, "X and Y must be 16-byte aligned, H 2-byte aligned");
  GemmArgs a{};
  a.w = to_kernel(w);
  a.X = X;
  a.gather = gather;
  a.offsets = offsets;
  a.perm = perm;
  a.active = active;
  a.n_active = n_active;
  a.T = T;
  a.k = k;
  a.Y = Y;
  a.H = H;
  const int64_t rows = (int64_t)T * k;
  hipError_t e;
  if (fr) {
    if (T == 1 && gather == 1 && rows <= kGemvMaxRows && w->K <= kGemvMaxK) {
      a.ids = fr->ids;                            // one launch: routing inside the GEMV
      a.logits = fr->logits;
      a.r_topk_ids = fr->topk_ids;
      a.r_topk_w = fr->topk_w;
      a.r_counts = fr->counts;
      a.r_offsets = fr->offsets;
      a.r_perm = fr->perm;
      a.r_inv = fr->inv;
      a.r_active = fr->active;
      a.r_n_active = fr->n_active;
      a.r_bad = fr->bad;
      return device_status(launch_gemv(a, (hipStream_t)stream), "fused route + grouped GEMM launch");
    }
    if (fr->logits) {
      e = launch_topk(fr->logits, T, w->E, k, fr->topk_ids, fr->topk_w, (hipStream_t)stream);
      if (e != hipSuccess) return device_status(e, "top-k launch");
    }
    e = launch_route(fr->logits ? fr->topk_ids : fr->ids, T, k, w->E, fr->counts, fr->offsets,
                     fr->perm, fr->inv, fr->active, fr->n_active, fr->bad, fr->workspace,
                     (hipStream_t)stream);
    if (e != hipSuccess) return device_status(e, "route launch");
  }
  if (rows <= kGemvMaxRows && w->K <= kGemvMaxK)
    e = launch_gemv(a, (hipStream_t)stream);
  else if (w->K % 64 == 0)
    e = launch_mfma(a, (hipStream_t)stream);
  else if (w->K <= kGemvMaxK)
    e = launch_gemv(a, (hipStream_t)stream);
  else
    return fail(GNF4_ERR_UNSUPPORTED, "MXFP4 with K %% 64 != 0 needs K <= %d", kGemvMaxK);
  return device_status(e, "grouped GEMM launch");
}

extern "C" {

gnf4_status gnf4_grouped_gemm(const gnf4_weights *w, const uint16_t *X, int32_t gather,
                              const int32_t *offsets, const int32_t *perm, const int32_t *active,
                              const int32_t *n_active, int32_t T, int32_t k, float *Y,
                              gnf4_stream_t stream) {
  if (!Y && T > 0) return fail(GNF4_ERR_INVALID_ARG, "a pointer argument is NULL");
  return grouped_gemm_any(w, X, gather, offsets, perm, active, n_active, T, k, Y, nullptr, stream);
}

gnf4_status gnf4_route_grouped_gemm(const int32_t *topk_ids, int32_t T, int32_t k,
                                    int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv,
                                    int32_t *active, int32_t *n_active, int32_t *bad_id_flag,
                                    void *workspace, size_t workspace_bytes,
                                    const gnf4_weights *w, const uint16_t *X, float *Y, uint16_t *H,
                                    gnf4_stream_t stream) {
  gnf4_status st = check_weights(w);
  if (st != GNF4_OK) return st;
  if (k < 1 || k > 64) return fail(GNF4_ERR_INVALID_ARG, "k = %d outside [1, 64]", k);
  if (T < 0) return fail(GNF4_ERR_INVALID_ARG, "T = %d is negative", T);
  if ((int64_t)T * k >= ((int64_t)1 << 31) - 1024)
    return fail(GNF4_ERR_INVALID_ARG, "T*k too large");
  if (!counts || !offsets || !active || !n_active || !bad_id_flag)
    return fail(GNF4_ERR_INVALID_ARG, "an output pointer is NULL");
  if (T > 0 && (!topk_ids || !perm || !inv))
    return fail(GNF4_ERR_INVALID_ARG, "topk_ids, perm or inv is NULL");
  if (T > 0 && (Y == nullptr) == (H == nullptr))
    return fail(GNF4_ERR_INVALID_ARG, "exactly one of Y and H must be given");
  st = check_route_workspace(T, k, w->E, workspace, workspace_bytes);
  if (st != GNF4_OK) return st;
  if (T == 0)                                     // routing of nothing: counts, offsets, flags
    return gnf4_route(topk_ids, T, k, w->E, counts, offsets, perm, inv, active, n_active,
                      bad_id_flag, workspace, workspace_bytes, stream);
  const FusedRoute fr = {topk_ids, counts, offsets, perm, inv, active, n_active, bad_id_flag,
                         nullptr, nullptr, nullptr, workspace};
  return grouped_gemm_any(w, X, 1, offsets, perm, active, n_active, T, k, Y, H, stream, &fr);
}

gnf4_status gnf4_route_logits_grouped_gemm(const float *logits, int32_t T, int32_t k,
                                           int32_t *topk_ids, float *topk_w, int32_t *counts,
                                           int32_t *offsets, int32_t *perm, int32_t *inv,
                                           int32_t *active, int32_t *n_active,
                                           int32_t *bad_id_flag, void *workspace,
                                           size_t workspace_bytes, const gnf4_weights *w,
                                           const uint16_t *X, float *Y, uint16_t *H,
                                           gnf4_stream_t stream) {
  gnf4_status st = check_weights(w);
  if (st != GNF4_OK) return st;
  if (k < 1 || k > 64 || k > w->E)
    return fail(GNF4_ERR_INVALID_ARG, "k = %d outside [1, min(64, E = %d)]", k, w->E);
  if (T < 0) return fail(GNF4_ERR_INVALID_ARG, "T = %d is negative", T);
  if ((int64_t)T * k >= ((int64_t)1 << 31) - 1024)
    return fail(GNF4_ERR_INVALID_ARG, "T*k too large");
  if (!counts || !offsets || !active || !n_active || !bad_id_flag)
    return fail(GNF4_ERR_INVALID_ARG, "an output pointer is NULL");
  if (T > 0 && (!logits || !topk_ids || !topk_w || !perm || !inv))
    return fail(GNF4_ERR_INVALID_ARG, "logits, topk_ids, topk_w, perm or inv is NULL");
  if (T > 0 && (Y == nullptr) == (H == nullptr))
    return fail(GNF4_ERR_INVALID_ARG, "exactly one of Y and H must be given");
  st = check_route_workspace(T, k, w->E, workspace, workspace_bytes);
  if (st != GNF4_OK) return st;
  if (T == 0)
    return gnf4_route_logits(logits, T, k, w->E, topk_ids, topk_w, counts, offsets, perm, inv,
                             active, n_active, bad_id_flag, workspace, workspace_bytes, stream);
  const FusedRoute fr = {nullptr, counts, offsets, perm, inv, active, n_active, bad_id_flag,
                         logits, topk_ids, topk_w, workspace};
  return grouped_gemm_any(w, X, 1, offsets, perm, active, n_active, T, k, Y, H, stream, &fr);
}

gnf4_status gnf4_grouped_gemm_swiglu(const gnf4_weights *w, const uint16_t *X, int32_t gather,
                                     const int32_t *offsets, const int32_t *perm,
                                     const int32_t *active, const int32_t *n_active, int32_t T,
                                     int32_t k, uint16_t *H, gnf4_stream_t stream) {
  if (!H && T > 0) return fail(GNF4_ERR_INVALID_ARG, "a pointer argument is NULL");
  return grouped_gemm_any(w, X, gather, offsets, perm, active, n_active, T, k, nullptr, H, stream);
}

gnf4_status gnf4_grouped_gemm_dx(const gnf4_weights *w, const uint16_t *dY,
                                 const int32_t *offsets, int32_t T, int32_t k, float *dA,
                                 gnf4_stream_t stream) {
  gnf4_status st = check_weights(w);
  if (st != GNF4_OK) return st;
  if (k < 1 || k > 64) return fail(GNF4_ERR_INVALID_ARG, "k = %d outside [1, 64]", k);
  if (T < 0) return fail(GNF4_ERR_INVALID_ARG, "T = %d is negative", T);
  if ((int64_t)T * k >= ((int64_t)1 << 31) - 1024)
    return fail(GNF4_ERR_INVALID_ARG, "T*k too large");
  if (w->N % 8) return fail(GNF4_ERR_INVALID_ARG, "N = %d must be a multiple of 8", w->N);
  if ((int64_t)T * k * w->N * 2 >= ((int64_t)1 << 32))
    return fail(GNF4_ERR_UNSUPPORTED, "dY must be below 4 GiB (T*k*N*2 bytes)");
  if (T == 0) return ok();
  if (!dY || !offsets || !dA) return fail(GNF4_ERR_INVALID_ARG, "a pointer argument is NULL");
  if (!aligned16(dY) || !aligned16(dA))
    return fail(GNF4_ERR_INVALID_ARG, "dY and dA must be 16-byte aligned");
  DxArgs a;
  a.w = to_kernel(w);
  a.dY = dY;
  a.offsets = offsets;
  a.rows = T * k;
  a.dA = dA;
  return device_status(launch_gemm_dx(a, (hipStream_t)stream), "grouped GEMM dx launch");
}

gnf4_status gnf4_grouped_gemm_combine(const gnf4_weights *w, const uint16_t *X,
                                      const int32_t *offsets, const int32_t *perm,
                                      const int32_t *inv, const int32_t *active,
                                      const int32_t *n_active, const float *topk_w, int32_t T,
                                      int32_t k, float *Y, float *out, gnf4_stream_t stream) {
  gnf4_status st = check_weights(w);
  if (st != GNF4_OK) return st;
  if (k < 1 || k > 64) return fail(GNF4_ERR_INVALID_ARG, "k = %d outside [1, 64]", k);
  if (T < 0) return fail(GNF4_ERR_INVALID_ARG, "T = %d is negative", T);
  if ((int64_t)T * k >= ((int64_t)1 << 31) - 1024)
    return fail(GNF4_ERR_INVALID_ARG, "T*k too large");
  if (w->N % 4) return fail(GNF4_ERR_INVALID_ARG, "N = %d must be a multiple of 4", w->N);
  if (T == 0) return ok();
  if (!X || !offsets || !perm || !inv || !active || !n_active || !topk_w || !out)
    return fail(GNF4_ERR_INVALID_ARG, "a pointer argument is NULL");
  if (!aligned16(X) || !aligned16(out))
    return fail(GNF4_ERR_INVALID_ARG, "X and out must be 16-byte aligned");
  GemmArgs a{};
  a.w = to_kernel(w);
  a.X = X;
  a.gather = 0;
  a.offsets = offsets;
  a.perm = perm;
  a.active = active;
  a.n_active = n_active;
  a.T = T;
  a.k = k;
  if (gemv_combine_fits(a))
    return device_status(launch_gemv_combine(a, topk_w, inv, out, (hipStream_t)stream),
                         "grouped GEMM + combine launch");
  if (!Y) return fail(GNF4_ERR_INVALID_ARG, "Y (scratch for T*k rows) is NULL and T > 1");
  st = grouped_gemm_any(w, X, 0, offsets, perm, active, n_active, T, k, Y, nullptr, stream);
  if (st != GNF4_OK) return st;
  return device_status(launch_combine(Y, inv, topk_w, T, k, w->N, out, (hipStream_t)stream),
                       "combine launch");
}

gnf4_status gnf4_combine(const float *Y, const int32_t *inv, const float *topk_w, int32_t T,
                         int32_t k, int32_t N, float *out, gnf4_stream_t stream) {
  if (k < 1 || k > 64) return fail(GNF4_ERR_INVALID_ARG, "k = %d outside [1, 64]", k);
  if (T < 0) return fail(GNF4_ERR_INVALID_ARG, "T = %d is negative", T);
  if (N < 4 || N % 4 || N > GNF4_MAX_N)
    return fail(GNF4_ERR_INVALID_ARG, "N = %d must be a positive multiple of 4 up to %d", N,
                GNF4_MAX_N);
  if ((int64_t)T * k >= ((int64_t)1 << 31) - 1024)
    return fail(GNF4_ERR_INVALID_ARG, "T*k too large");
  if (T == 0) return ok();
  if (!Y || !inv || !topk_w || !out) return fail(GNF4_ERR_INVALID_ARG, "a pointer argument is NULL");
  if (!aligned16(Y) || !aligned16(out))
    return fail(GNF4_ERR_INVALID_ARG, "Y and out must be 16-byte aligned");
  return device_status(launch_combine(Y, inv, topk_w, T, k, N, out, (hipStream_t)stream),
                       "combine launch");
}

gnf4_status gnf4_dequant(const gnf4_weights *w, int32_t e, float *out, gnf4_stream_t stream) {
  gnf4_status st = check_weights(w);
  if (st != GNF4_OK) return st;
  if (e < 0 || e >= w->E) return fail(GNF4_ERR_INVALID_ARG, "expert %d outside [0, %d)", e, w->E);
  if (!out) return fail(GNF4_ERR_INVALID_ARG, "out is NULL");
  if ((int64_t)w->N * w->K / 32 > 0x7fffffffLL * 256)
    return fail(GNF4_ERR_UNSUPPORTED, "expert too large");
  Weights k = to_kernel(w);
  return device_status(launch_dequant(k, e, out, (hipStream_t)stream), "dequant launch");
}

gnf4_status gnf4_dequant_experts_bf16(const gnf4_weights *w, const int32_t *experts,
                                      const int32_t *count, int32_t max_experts, uint16_t *out,
                                      gnf4_stream_t stream) {
  gnf4_status st = check_weights(w);
  if (st != GNF4_OK) return st;
  if (max_experts < 0 || max_experts > w->E)
    return fail(GNF4_ERR_INVALID_ARG, "max_experts = %d outside [0, E = %d]", max_experts, w->E);
  if (max_experts == 0) return ok();
  if (!experts || !count || !out) return fail(GNF4_ERR_INVALID_ARG, "a pointer argument is NULL");
  if (!aligned16(out)) return fail(GNF4_ERR_INVALID_ARG, "out must be 16-byte aligned");
  if ((int64_t)max_experts * w->N * (w->K / 8) > 0x7fffffffLL * 256)
    return fail(GNF4_ERR_UNSUPPORTED, "too many weights for one call");
  Weights k = to_kernel(w);
  return device_status(launch_dequant_bf16(k, experts, count, max_experts, out, (hipStream_t)stream),
                       "bf16 dequant launch");
}

gnf4_status gnf4_quantize(int32_t format, const float *W, int32_t rows, int32_t K, uint8_t *codes,
                          void *scales, float *scales2, gnf4_stream_t stream) {
  if (format < GNF4_NF4 || format > GNF4_MXFP4)
    return fail(GNF4_ERR_INVALID_ARG, "unknown format %d", format);
  const int blk = format == GNF4_MXFP4 ? 32 : 64;
  if (K < blk || K % blk || K > GNF4_MAX_K)
    return fail(GNF4_ERR_INVALID_ARG, "K = %d must be a positive multiple of %d up to %d", K, blk,
                GNF4_MAX_K);
  if (rows < 0) return fail(GNF4_ERR_INVALID_ARG, "rows = %d is negative", rows);
  if (rows == 0) return ok();
  if (!W || !codes || !scales) return fail(GNF4_ERR_INVALID_ARG, "a pointer argument is NULL");
  if (format == GNF4_NF4_DQ && !scales2) return fail(GNF4_ERR_INVALID_ARG, "NF4_DQ needs scales2");
  if (!aligned16(codes) || ((uintptr_t)W & 3u))
    return fail(GNF4_ERR_INVALID_ARG, "codes must be 16-byte and W 4-byte aligned");
  if ((int64_t)rows * (K / 32) > 0x7fffffffLL * 200)
    return fail(GNF4_ERR_UNSUPPORTED, "weight tensor too large");
  return device_status(launch_quantize(format, W, rows, K, codes, scales, scales2,
                                       (hipStream_t)stream),
                       "quantize launch");
}

// ------------------------------------------------ expert streaming cache

static gnf4_status check_cache_shape(int32_t E, int32_t S) {
  if (E < 1 || E > GNF4_MAX_EXPERTS)
    return fail(GNF4_ERR_INVALID_ARG, "E = %d outside [1, %d]", E, GNF4_MAX_EXPERTS);
  if (S < 1 || S > E) return fail(GNF4_ERR_INVALID_ARG, "S = %d outside [1, E = %d]", S, E);
  return ok();
}

size_t gnf4_expert_cache_state_words(int32_t E, int32_t S) {
  if (E < 1 || E > GNF4_MAX_EXPERTS || S < 1 || S > E) return 0;
  return (size_t)1 + (size_t)E + 2 * (size_t)S;
}

size_t gnf4_expert_cache_copies_words(int32_t T, int32_t k, int32_t E, int32_t S) {
  if (T < 0 || k < 1 || E < 1 || S < 1) return 0;
  const int64_t m = std::min<int64_t>(std::min<int64_t>((int64_t)T * k, E), S);
  return (size_t)(1 + 2 * m);
}

gnf4_status gnf4_expert_cache_reset(int32_t *state, int32_t E, int32_t S, gnf4_stream_t stream) {
  gnf4_status st = check_cache_shape(E, S);
  if (st != GNF4_OK) return st;
  if (!state) return fail(GNF4_ERR_INVALID_ARG, "state is NULL");
  return device_status(launch_cache_reset(state, E, S, (hipStream_t)stream), "cache reset launch");
}

gnf4_status gnf4_expert_cache_stage(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E,
                                    int32_t S, int32_t *state, int32_t *slot_ids, int32_t *copies,
                                    gnf4_stream_t stream) {
  gnf4_status st = check_cache_shape(E, S);
  if (st != GNF4_OK) return st;
  if (k < 1 || k > 64) return fail(GNF4_ERR_INVALID_ARG, "k = %d outside [1, 64]", k);
  if (T < 0) return fail(GNF4_ERR_INVALID_ARG, "T = %d is negative", T);
  if ((int64_t)T * k >= ((int64_t)1 << 31) - 1024)
    return fail(GNF4_ERR_INVALID_ARG, "T*k too large");
  if (!state || !copies) return fail(GNF4_ERR_INVALID_ARG, "state or copies is NULL");
  if (T > 0 && (!topk_ids || !slot_ids))
    return fail(GNF4_ERR_INVALID_ARG, "topk_ids or slot_ids is NULL");
  if ((int64_t)S < std::min<int64_t>(E, (int64_t)T * k))
    return fail(GNF4_ERR_UNSUPPORTED,
                "S = %d slots cannot hold the up to %lld distinct experts of T*k = %lld ids", S,
                (long long)std::min<int64_t>(E, (int64_t)T * k), (long long)T * k);
  return device_status(launch_cache_stage(topk_ids, T * k, E, S, state, slot_ids, copies,
                                          (hipStream_t)stream),
                       "cache stage launch");
}

// Device address of a pinned host (or device) buffer, or NULL if the GPU
// cannot address it (pageable host memory).
static const void *device_view(const void *p) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return at.devicePointer;
}

gnf4_status gnf4_expert_cache_fill(const gnf4_weights *host_w, const gnf4_weights *cache_w,
                                   const int32_t *copies, int32_t max_copies,
                                   gnf4_stream_t stream) {
  gnf4_status st = check_weights(host_w);
  if (st != GNF4_OK) return st;
  st = check_weights(cache_w);
  if (st != GNF4_OK) return st;
  if (host_w->format != cache_w->format || host_w->N != cache_w->N || host_w->K != cache_w->K)
    return fail(GNF4_ERR_INVALID_ARG, "host and cache weights differ in format or shape");
  if (cache_w->E > host_w->E)
    return fail(GNF4_ERR_INVALID_ARG, "cache has %d slots for %d experts", cache_w->E, host_w->E);
  if (max_copies < 0 || max_copies > cache_w->E)
    return fail(GNF4_ERR_INVALID_ARG, "max_copies = %d outside [0, S = %d]", max_copies,
                cache_w->E);
  if (!copies) return fail(GNF4_ERR_INVALID_ARG, "copies is NULL");
  const int fmt = host_w->format;
  const int64_t N = host_w->N, K = host_w->K;
  const int64_t nblk = N * (K / 64);
  const int64_t seg[3] = {N * (K / 2),
                          fmt == GNF4_NF4 ? nblk * 4 : fmt == GNF4_NF4_DQ ? nblk : N * (K / 32),
                          fmt == GNF4_NF4_DQ ? nblk / 256 * 4 : 0};
  const int nseg = fmt == GNF4_NF4_DQ ? 3 : 2;
  if (fmt == GNF4_NF4_DQ && nblk % 256)
    return fail(GNF4_ERR_UNSUPPORTED,
                "NF4_DQ streaming needs N*K/64 = %lld to be a multiple of 256 (whole "
                "second-level groups per expert)", (long long)nblk);
  for (int g = 0; g < nseg; ++g)
    if (seg[g] % 16)
      return fail(GNF4_ERR_UNSUPPORTED, "an expert's packed segment of %lld bytes is not a "
                  "multiple of 16", (long long)seg[g]);
  const void *hs[3] = {host_w->codes, host_w->scales, host_w->scales2};
  void *cs[3] = {(void *)cache_w->codes, (void *)cache_w->scales, (void *)cache_w->scales2};
  for (int g = 0; g < nseg; ++g)
    if (!aligned16(hs[g]) || !aligned16(cs[g]))
      return fail(GNF4_ERR_INVALID_ARG, "host and cache arrays must be 16-byte aligned");
  if (max_copies == 0) return ok();
  CacheFillArgs f{};
  for (int g = 0; g < nseg; ++g) {
    f.src[g] = device_view(hs[g]);
    if (!f.src[g])
      return fail(GNF4_ERR_INVALID_ARG, "host weights must be pinned host memory (or device "
                  "memory) that the GPU can address");
    f.dst[g] = cs[g];
    f.seg_units[g] = seg[g] / 16;
    f.units += seg[g] / 16;
  }
  f.nseg = nseg;
  f.chunks = cache_fill_chunks(f.units);
  f.E = host_w->E;
  f.S = cache_w->E;
  f.copies = copies;
  return device_status(launch_cache_fill(f, max_copies, (hipStream_t)stream), "cache fill launch");
}

void gnf4_nf4_codebook(float out[16]) {
  if (!out) return;
  for (int i = 0; i < 16; ++i) {
    uint32_t b = kNF4Bits[i];
    std::memcpy(&out[i], &b, 4);
  }
}

gnf4_status gnf4_read_probe(const void *src, size_t nbytes, int32_t workgroups, uint32_t *sink,
                            gnf4_stream_t stream) {
  if (nbytes == 0) return ok();
  if (!src || !sink) return fail(GNF4_ERR_INVALID_ARG, "src or sink is NULL");
  if (!aligned16(src) || nbytes % 16)
    return fail(GNF4_ERR_INVALID_ARG, "src must be 16-byte aligned and nbytes a multiple of 16");
  if (workgroups < 0) return fail(GNF4_ERR_INVALID_ARG, "workgroups = %d is negative", workgroups);
  if (nbytes > ((size_t)1 << 46)) return fail(GNF4_ERR_UNSUPPORTED, "nbytes too large");
  return device_status(launch_read_probe(src, (int64_t)nbytes, workgroups, sink, (hipStream_t)stream),
                       "read probe launch");
}

void gnf4_nf4_codebook_bf16(uint16_t out[16], float *scale) {
  if (out)
    for (int i = 0; i < 16; ++i) out[i] = (uint16_t)nf4_bf16_bits((uint32_t)i);
  if (scale) *scale = kNF4Scale;
}

const char *gnf4_last_error(void) { return g_err; }

const char *gnf4_build_id(void) { return "gnf4 " GNF4_REVISION " gfx950"; }

}  // extern "C"
