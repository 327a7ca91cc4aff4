// C ABI (include/moe.h): host-side validation, workspace carving and stream-ordered launches.
// Nothing here synchronises the host or reads device memory.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/moe.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace moe;

namespace {

thread_local hipError_t g_last_hip = hipSuccess;

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool al256p(const void* p) { return ((uintptr_t)p & 255u) == 0; }

int check_dims(const moe_dims* d) {
  if (!d) return MOE_ERR_NULL;
  if (d->reserved != 0) return MOE_ERR_SHAPE;
  if (d->T < 0 || d->E < 1 || d->E > 1024 || d->k < 1 || d->k > d->E || d->k > 64) return MOE_ERR_SHAPE;
  if (d->d <= 0 || d->f <= 0 || d->d % 128 || d->f % 128 || d->d > 65536 || d->f > 65536) return MOE_ERR_SHAPE;
  if (d->T * d->k >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  if (d->dtype != MOE_BF16 && d->dtype != MOE_FP8_E4M3 && d->dtype != MOE_MXFP8) return MOE_ERR_DTYPE;
  // the fp8 and MXFP8 tiles are 256 columns wide along both d and f
  if (d->dtype != MOE_BF16 && (d->d % 256 || d->f % 256)) return MOE_ERR_SHAPE;
  // launch grids of the ragged GEMMs must fit in 32 bits
  const int64_t A = d->T * d->k;
  const int bm = d->dtype != MOE_BF16 ? kFp8BM : kGemmBM;
  const int64_t rows = (A + bm - 1) / bm + (A < d->E ? A : d->E);
  if (rows * (d->f / 64 > d->d / 128 ? d->f / 64 : d->d / 128) >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  // the MXFP8 weight gradients index the 128-padded expert segments with 32-bit rows
  if (d->dtype == MOE_MXFP8 && mx_padded_rows(A, (int)d->E) >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

bool is_fp8(const moe_dims* d) { return d->dtype == MOE_FP8_E4M3; }
bool is_mx(const moe_dims* d) { return d->dtype == MOE_MXFP8; }
int row_tile(const moe_dims* d) { return d->dtype != MOE_BF16 ? kFp8BM : kGemmBM; }
// d_topk_w partial sums per routed pair written by the activation-gradient GEMM
int dact_parts(const moe_dims* d) {
  return d->dtype != MOE_BF16 ? (int)d->f / 256 : dact_parts_bf16((int)d->f);
}

MoeShape shape_of(const moe_dims* d) {
  return MoeShape{(int)d->T, (int)d->d, (int)d->f, (int)d->E, (int)d->k};
}

// fp8: asq/ass (As in e4m3 + scales); dyq/dys, dHq/dHs; xbf (x dequantised to bf16 for the
// bf16 weight gradients).
// MXFP8 (codes + E8M0 exponents): asq/ass; xq/xe, w1q/w1e and w2q/w2e (forward quantisation of
// x, W1 and W2); dyq/dys, dHq/dHs, w1q/w1e and w2q/w2e (W1, W2 along the data gradients' K);
// for the weight gradients poff (padded expert offsets) and tqa/tea, tqb/teb (the two operands
// of one product quantised along the token axis, reused by dW2 and then dW1).
struct FwdLayout {
  size_t tiles, ntiles, op, asq, ass, xss, xq, xe, xes, w1q, w1e, w2q, w2e, total;
};
struct BwdLayout {
  size_t tiles, ntiles, tokrow, dH, dXp, dwp, wg_units, wg_meta, wg_pslot, wg_partial, dyq, dys, dyss, dyes, dHq, dHs, xbf,
      w1q, w1e, w2q, w2e, poff, tqa, tea, tqb, teb, total;
  int max_partials;
};
// MXFP8 adds W1 and W2 quantised along the data gradients' K (row blocks), produced by the
// forward's single pass over each weight matrix and read by the backward.
struct SavedLayout {
  size_t H, As, w1q, w1e, w2q, w2e, total;
};

FwdLayout fwd_layout(const moe_dims* d) {
  const int64_t A = d->T * d->k;
  FwdLayout L{};
  size_t off = 0;
  L.tiles = off;
  off += al256((size_t)max_row_tiles(A, (int)d->E, row_tile(d)) * sizeof(int2) + 16);
  L.ntiles = off;
  off += 256;
  L.op = off;
  off += al256((size_t)A * d->d * 2);
  if (is_fp8(d)) {
    L.asq = off;
    off += al256((size_t)A * d->f);
    L.ass = off;
    off += al256((size_t)A * (d->f / 128) * sizeof(float));
    L.xss = off;  // x's row scales in the sorted order, by k block
    off += al256((size_t)A * (d->d / 128) * sizeof(float));
  }
  if (is_mx(d)) {
    const size_t E = d->E, dd = d->d, ff = d->f, T = d->T;
    L.asq = off;
    off += al256((size_t)A * ff);
    L.ass = off;
    off += al256((size_t)A * (ff / 32));
    L.xq = off;
    off += al256(T * dd);
    L.xe = off;
    off += al256(T * (dd / 32));
    L.xes = off;  // x's exponents in the sorted order
    off += al256((size_t)A * (dd / 32));
    L.w1q = off;
    off += al256(E * dd * 2 * ff);
    L.w1e = off;
    off += al256(E * dd * 2 * ff / 32);
    L.w2q = off;
    off += al256(E * ff * dd);
    L.w2e = off;
    off += al256(E * ff * dd / 32);
  }
  L.total = off;
  return L;
}

BwdLayout bwd_layout(const moe_dims* d) {
  const int64_t A = d->T * d->k;
  BwdLayout L{};
  size_t off = 0;
  L.tiles = off;
  off += al256((size_t)max_row_tiles(A, (int)d->E, row_tile(d)) * sizeof(int2) + 16);
  L.ntiles = off;
  off += 256;
  L.tokrow = off;
  off += al256((size_t)(A + kTokrowPad) * sizeof(int32_t));
  L.dH = off;
  off += al256((size_t)A * 2 * d->f * 2);
  L.dXp = off;
  off += al256((size_t)A * d->d * 2);
  L.dwp = off;
  off += al256((size_t)A * dact_parts(d) * sizeof(float));
  L.max_partials = wg_max_partials(shape_of(d));
  L.wg_units = off;
  off += al256((size_t)(d->E + L.max_partials) * sizeof(int2));
  L.wg_meta = off;
  off += 256;
  L.wg_pslot = off;
  off += al256((size_t)d->E * sizeof(int32_t));
  L.wg_partial = off;
  off += al256((size_t)L.max_partials * d->d * 2 * d->f * sizeof(float));
  if (is_fp8(d)) {
    L.dyq = off;
    off += al256((size_t)d->T * d->d);
    L.dys = off;
    off += al256((size_t)d->T * (d->d / 128) * sizeof(float));
    L.dyss = off;  // dy's row scales in the sorted order, by k block
    off += al256((size_t)A * (d->d / 128) * sizeof(float));
    L.dHq = off;
    off += al256((size_t)A * 2 * d->f);
    L.dHs = off;
    off += al256((size_t)A * (2 * d->f / 128) * sizeof(float));
    L.xbf = off;
    off += al256((size_t)d->T * d->d * 2);
  }
  if (is_mx(d)) {
    const size_t dd = d->d, ff = d->f, T = d->T;
    L.dyq = off;
    off += al256(T * dd);
    L.dys = off;
    off += al256(T * (dd / 32));
    L.dyes = off;  // dy's exponents in the sorted order
    off += al256((size_t)A * (dd / 32));
    L.dHq = off;
    off += al256((size_t)A * 2 * ff);
    L.dHs = off;
    off += al256((size_t)A * (2 * ff / 32));
    const size_t E = d->E;
    const size_t P = (size_t)mx_padded_rows(A, (int)E);
    const size_t ca = ff > dd ? ff : dd, cb = dd > 2 * ff ? dd : 2 * ff;  // As or x; dy or dH
    L.poff = off;
    off += al256((E + 1) * sizeof(int32_t));
    L.tqa = off;
    off += al256(P * ca);
    L.tea = off;
    off += al256(P / 32 * ca);
    L.tqb = off;
    off += al256(P * cb);
    L.teb = off;
    off += al256(P / 32 * cb);
  }
  L.total = off;
  return L;
}

WgSplit wg_split_of(const BwdLayout& L, char* w, const int32_t* offsets) {
  WgSplit sp;
  sp.units = (int2*)(w + L.wg_units);
  sp.meta = (int32_t*)(w + L.wg_meta);
  sp.pslot = (int32_t*)(w + L.wg_pslot);
  sp.partial = (float*)(w + L.wg_partial);
  sp.offsets = offsets;
  sp.max_partials = L.max_partials;
  return sp;
}

SavedLayout saved_layout(const moe_dims* d) {
  const int64_t A = d->T * d->k;
  SavedLayout L{};
  L.H = 0;
  L.As = al256((size_t)A * 2 * d->f * 2);
  size_t off = L.As + al256((size_t)A * d->f * 2);
  if (d->dtype == MOE_MXFP8) {
    const size_t E = d->E, dd = d->d, ff = d->f;
    L.w1q = off;
    off += al256(E * dd * 2 * ff);
    L.w1e = off;
    off += al256(E * dd * 2 * ff / 32);
    L.w2q = off;
    off += al256(E * ff * dd);
    L.w2e = off;
    off += al256(E * ff * dd / 32);
  }
  L.total = off;
  return L;
}

int hip_status(hipError_t e) {
  if (e != hipSuccess) {
    g_last_hip = e;
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

moe_stage_hook g_hook = nullptr;
void* g_hook_user = nullptr;

// Enqueue one stage, bracketed by the profiling hook when one is set.
#define MOE_TRY(name, expr)                                   \
  do {                                                        \
    if (g_hook) g_hook(name, 1, (void*)st, g_hook_user);      \
    int _rc = hip_status(expr);                               \
    if (g_hook) g_hook(name, 0, (void*)st, g_hook_user);      \
    if (_rc != MOE_OK) return _rc;                            \
  } while (0)

}  // namespace

// Fixed scratch of moe_route_noalloc: the plan's per-(expert, segment) count and base tables,
// 2*E*S int32 with at most 512 segments and 1024 experts (4 MiB) for every shape check_dims
// accepts.  Each GPU the library runs on holds its own copy until the process ends.  In host code
// `scratch` names a host-side stand-in, not the device address: kernels get the address that
// hipGetSymbolAddress returns for the device (noalloc_scratch below), never the array's name.
constexpr size_t kRouteScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) uint8_t scratch[kRouteScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the device that owns `st`, looked up once per device with that
// device current (the caller's current device is restored).
hipError_t noalloc_scratch(hipStream_t st, void** out) {
  hipDevice_t dev = 0;
  hipError_t e = hipStreamGetDevice(st, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    int cur = 0;
    hipError_t r = hipGetDevice(&cur);
    if (r == hipSuccess && cur != dev) r = hipSetDevice(dev);
    void* p = nullptr;
    if (r == hipSuccess) r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (r == hipSuccess) r = back;
    }
    g_scratch_err[dev] = r;
    g_scratch_ptr[dev] = (r == hipSuccess) ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int moe_workspace_bytes(const moe_dims* dims, int which, size_t* out) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!out) return MOE_ERR_NULL;
  switch (which) {
    case MOE_WS_ROUTE: *out = al256(plan_ws_bytes(dims->T * dims->k, dims->E)); return MOE_OK;
    case MOE_WS_FORWARD: *out = fwd_layout(dims).total; return MOE_OK;
    case MOE_WS_BACKWARD: *out = bwd_layout(dims).total; return MOE_OK;
    case MOE_WS_ROUTER: *out = al256(router_ws_bytes(dims->T, (int)dims->d, (int)dims->E)); return MOE_OK;
    default: return MOE_ERR_SHAPE;
  }
}

int moe_saved_bytes(const moe_dims* dims, size_t* out) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!out) return MOE_ERR_NULL;
  *out = saved_layout(dims).total;
  return MOE_OK;
}

int moe_plan(const moe_dims* dims, const int32_t* topk_ids, int32_t* counts, int32_t* offsets, int32_t* perm,
             int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  const int64_t A = dims->T * dims->k;
  const size_t need = al256(plan_ws_bytes(A, dims->E));
  if (!counts || !offsets) return MOE_ERR_NULL;
  if (A > 0 && (!topk_ids || !perm || !inv_perm)) return MOE_ERR_NULL;
  if (need > 0 && !ws) return MOE_ERR_NULL;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (ws && !al256p(ws)) return MOE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  MOE_TRY("plan", launch_plan(topk_ids, A, (int)dims->E, counts, offsets, perm, inv_perm, ws, st));

  return MOE_OK;
}

int moe_route(const moe_dims* dims, const float* logits, int32_t* topk_ids, float* topk_w, int32_t* counts,
              int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  const int64_t A = dims->T * dims->k;
  if (!counts || !offsets) return MOE_ERR_NULL;
  if (A > 0 && (!logits || !topk_ids || !topk_w || !perm || !inv_perm)) return MOE_ERR_NULL;
  const size_t need = al256(plan_ws_bytes(A, dims->E));
  if (need > 0 && !ws) return MOE_ERR_NULL;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (ws && !al256p(ws)) return MOE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  MOE_TRY("router", launch_router(logits, (int)dims->T, (int)dims->E, (int)dims->k, topk_ids, topk_w, st));
  MOE_TRY("plan", launch_plan(topk_ids, A, (int)dims->E, counts, offsets, perm, inv_perm, ws, st));

  return MOE_OK;
}

int moe_route_noalloc(const moe_dims* dims, const float* logits, int32_t* topk_ids, float* topk_w, int32_t* counts,
                      int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  const int64_t A = dims->T * dims->k;
  if (!counts || !offsets) return MOE_ERR_NULL;
  if (A > 0 && (!logits || !topk_ids || !topk_w || !perm || !inv_perm)) return MOE_ERR_NULL;
  if (plan_ws_bytes(A, dims->E) > kRouteScratchBytes) return MOE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  void* ws = nullptr;
  rc = hip_status(noalloc_scratch(st, &ws));
  if (rc) return rc;
  // the plan writes every table entry it reads, so the scratch needs no clearing between calls
  MOE_TRY("router", launch_router(logits, (int)dims->T, (int)dims->E, (int)dims->k, topk_ids, topk_w, st));
  MOE_TRY("plan", launch_plan(topk_ids, A, (int)dims->E, counts, offsets, perm, inv_perm, ws, st));
  return MOE_OK;
}

int moe_forward(const moe_dims* dims, const void* x, const float* x_scale, const void* W1, const float* W1_scale,
                const void* W2, const float* W2_scale, const float* topk_w, const int32_t* offsets,
                const int32_t* perm, const int32_t* inv_perm, void* y, void* saved, void* ws, size_t ws_bytes,
                void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  const bool fp8 = is_fp8(dims);
  if (!fp8 && (x_scale || W1_scale || W2_scale)) return MOE_ERR_DTYPE;
  if (dims->T == 0) return MOE_OK;  // an empty layer has nothing to compute
  if (!x || !W1 || !W2 || !topk_w || !offsets || !perm || !inv_perm || !y || !saved || !ws) return MOE_ERR_NULL;
  if (fp8 && (!x_scale || !W1_scale || !W2_scale)) return MOE_ERR_NULL;
  const FwdLayout L = fwd_layout(dims);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!al16(x) || !al16(W1) || !al16(W2) || !al16(y) || !al256p(saved) || !al256p(ws)) return MOE_ERR_ALIGN;
  if (fp8 && (!al16(x_scale) || !al16(W1_scale) || !al16(W2_scale))) return MOE_ERR_ALIGN;
  const MoeShape s = shape_of(dims);
  const SavedLayout SL = saved_layout(dims);
  char* w = (char*)ws;
  char* sv = (char*)saved;
  int2* tiles = (int2*)(w + L.tiles);
  int32_t* ntiles = (int32_t*)(w + L.ntiles);
  uint16_t* Op = (uint16_t*)(w + L.op);
  uint16_t* H = (uint16_t*)(sv + SL.H);
  uint16_t* As = (uint16_t*)(sv + SL.As);
  hipStream_t st = (hipStream_t)stream;
  if (is_mx(dims)) {
    uint8_t *Asq = (uint8_t*)(w + L.asq), *Ase = (uint8_t*)(w + L.ass);
    uint8_t *xq = (uint8_t*)(w + L.xq), *xe = (uint8_t*)(w + L.xe), *xes = (uint8_t*)(w + L.xes);
    uint8_t *w1q = (uint8_t*)(w + L.w1q), *w1e = (uint8_t*)(w + L.w1e);
    uint8_t *w2q = (uint8_t*)(w + L.w2q), *w2e = (uint8_t*)(w + L.w2e);
    uint8_t *w1bq = (uint8_t*)(sv + SL.w1q), *w1be = (uint8_t*)(sv + SL.w1e);
    uint8_t *w2bq = (uint8_t*)(sv + SL.w2q), *w2be = (uint8_t*)(sv + SL.w2e);
    MOE_TRY("mx_quant_x", launch_mx_quant((const uint16_t*)x, 1, s.T, s.d, 0, xq, xe, st));
    // each weight matrix read once: blocks along the forward K (workspace) and along the data
    // gradients' K (saved, for the backward)
    MOE_TRY("mx_quant_w1", launch_mx_quant_dual((const uint16_t*)W1, s.E, s.d, 2 * s.f, w1q, w1e, w1bq, w1be, st));
    MOE_TRY("mx_quant_w2", launch_mx_quant_dual((const uint16_t*)W2, s.E, s.f, s.d, w2q, w2e, w2bq, w2be, st));
    MOE_TRY("tile_map", launch_tile_map(offsets, s.E, kFp8BM, tiles, ntiles, st));
    MOE_TRY("ksort_x", launch_kstep_sort(xe, s.d / 128, perm, s.k, offsets, s.E, (int64_t)s.T * s.k, xes, st));
    MOE_TRY("gemm_up", launch_mx_up(s, xq, xes, w1q, w1e, topk_w, offsets, perm, tiles, ntiles, H, As, Asq, Ase, st));
    MOE_TRY("gemm_down", launch_mx_down(s, Asq, Ase, w2q, w2e, offsets, perm, tiles, ntiles, Op, st));
    MOE_TRY("combine", launch_combine(Op, inv_perm, s.T, s.d, s.k, (uint16_t*)y, st));
    return MOE_OK;
  }
  if (fp8) {
    uint8_t* Asq = (uint8_t*)(w + L.asq);
    float* Ass = (float*)(w + L.ass);
    float* xss = (float*)(w + L.xss);
    const uint8_t *x8 = (const uint8_t*)x, *W18 = (const uint8_t*)W1, *W28 = (const uint8_t*)W2;
    MOE_TRY("tile_map", launch_tile_map(offsets, s.E, kFp8BM, tiles, ntiles, st));
    MOE_TRY("ksort_x", launch_kstep_sort(x_scale, s.d / 128, perm, s.k, offsets, s.E, (int64_t)s.T * s.k, xss, st));
    MOE_TRY("gemm_up", launch_fp8_up(s, x8, xss, W18, W1_scale, topk_w, offsets, perm, tiles, ntiles, H, As, Asq,
                                     Ass, st));
    MOE_TRY("gemm_down", launch_fp8_down(s, Asq, Ass, W28, W2_scale, offsets, perm, tiles, ntiles, Op, st));
    MOE_TRY("combine", launch_combine(Op, inv_perm, s.T, s.d, s.k, (uint16_t*)y, st));
    return MOE_OK;
  }
  MOE_TRY("tile_map", launch_tile_map(offsets, s.E, kGemmBM, tiles, ntiles, st));
  MOE_TRY("gemm_up", launch_gemm_up(s, (const uint16_t*)x, (const uint16_t*)W1, topk_w, offsets, perm, tiles, ntiles, H, As, st));
  MOE_TRY("gemm_down", launch_gemm_down(s, As, (const uint16_t*)W2, offsets, perm, tiles, ntiles, Op, st));
  MOE_TRY("combine", launch_combine(Op, inv_perm, s.T, s.d, s.k, (uint16_t*)y, st));

  return MOE_OK;
}

int moe_forward_fused(const moe_dims* dims, const void* x, const void* W1, const void* W2, const float* topk_w,
                      const int32_t* offsets, const int32_t* perm, const int32_t* inv_perm, void* y, void* saved,
                      void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (dims->dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (dims->T == 0) return MOE_OK;
  if (!x || !W1 || !W2 || !topk_w || !offsets || !perm || !inv_perm || !y || !saved || !ws) return MOE_ERR_NULL;
  const FwdLayout L = fwd_layout(dims);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!al16(x) || !al16(W1) || !al16(W2) || !al16(y) || !al256p(saved) || !al256p(ws)) return MOE_ERR_ALIGN;
  const MoeShape s = shape_of(dims);
  const SavedLayout SL = saved_layout(dims);
  char* w = (char*)ws;
  char* sv = (char*)saved;
  // the forward's tile table and count words hold the work queue and its counters
  int2* items = (int2*)(w + L.tiles);
  int32_t* qinfo = (int32_t*)(w + L.ntiles);
  uint16_t* Op = (uint16_t*)(w + L.op);
  uint16_t* H = (uint16_t*)(sv + SL.H);
  uint16_t* As = (uint16_t*)(sv + SL.As);
  hipStream_t st = (hipStream_t)stream;
  MOE_TRY("fwd_queue", launch_fwd_queue(s, offsets, items, qinfo, st));
  MOE_TRY("gemm_fused", launch_fused_forward(s, (const uint16_t*)x, (const uint16_t*)W1, (const uint16_t*)W2, topk_w,
                                             offsets, perm, items, qinfo, H, As, Op, st));
  MOE_TRY("combine", launch_combine(Op, inv_perm, s.T, s.d, s.k, (uint16_t*)y, st));
  return MOE_OK;
}

// MXFP8 weight gradients: dW2 = As^T dy and dW1 = x^T dH with every operand quantised along the
// token axis in 32-row blocks inside each expert's 128-padded segment.
static int mx_weight_grads(const MoeShape& s, const BwdLayout& L, char* w, const uint16_t* x, const uint16_t* dy,
                           const uint16_t* As, const uint16_t* dH, const int32_t* offsets, const int32_t* perm,
                           uint16_t* dW1, uint16_t* dW2, hipStream_t st) {
  int32_t* poff = (int32_t*)(w + L.poff);
  uint8_t *tqa = (uint8_t*)(w + L.tqa), *tea = (uint8_t*)(w + L.tea);
  uint8_t *tqb = (uint8_t*)(w + L.tqb), *teb = (uint8_t*)(w + L.teb);
  const WgSplit spm = wg_split_of(L, w, poff);
  MOE_TRY("mx_pad", launch_mx_pad_offsets(offsets, s.E, poff, st));
  MOE_TRY("wg_split", launch_wg_split(s, poff, spm, st));
  MOE_TRY("mx_quant_as_t", launch_mx_quant_tokens(As, s.f, 0, s, offsets, perm, poff, tqa, tea, st));
  MOE_TRY("mx_quant_dy_t", launch_mx_quant_tokens(dy, s.d, 1, s, offsets, perm, poff, tqb, teb, st));
  MOE_TRY("gemm_dw2", launch_mx_wg(0, s, tqa, tea, s.f, tqb, teb, s.d, poff, spm, dW2, st));
  MOE_TRY("wg_reduce", launch_wg_reduce(s, spm, (int64_t)s.f * s.d, dW2, st));
  MOE_TRY("mx_quant_x_t", launch_mx_quant_tokens(x, s.d, 1, s, offsets, perm, poff, tqa, tea, st));
  MOE_TRY("mx_quant_dh_t", launch_mx_quant_tokens(dH, 2 * s.f, 0, s, offsets, perm, poff, tqb, teb, st));
  MOE_TRY("gemm_dw1", launch_mx_wg(1, s, tqa, tea, s.d, tqb, teb, 2 * s.f, poff, spm, dW1, st));
  MOE_TRY("wg_reduce", launch_wg_reduce(s, spm, (int64_t)s.d * 2 * s.f, dW1, st));
  return MOE_OK;
}

int moe_backward(const moe_dims* dims, const void* dy, const void* x, const float* x_scale, const void* W1,
                 const float* W1_scale, const void* W2, const float* W2_scale, const int32_t* topk_ids,
                 const float* topk_w, const int32_t* offsets, const int32_t* perm, const int32_t* inv_perm,
                 const void* saved, void* dx, void* dW1, void* dW2, float* d_topk_w, float* d_logits, void* ws,
                 size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  const bool fp8 = is_fp8(dims);
  if (!fp8 && (x_scale || W1_scale || W2_scale)) return MOE_ERR_DTYPE;
  if (dims->T == 0) {
    // no routed pair: every expert's weight gradient is exactly zero, nothing else to write
    if (!offsets || !dW1 || !dW2 || !ws) return MOE_ERR_NULL;
    const BwdLayout L0 = bwd_layout(dims);
    if (ws_bytes < L0.total) return MOE_ERR_WORKSPACE;
    if (!al16(dW1) || !al16(dW2) || !al256p(ws)) return MOE_ERR_ALIGN;
    const MoeShape s = shape_of(dims);
    hipStream_t st = (hipStream_t)stream;
    const WgSplit sp = wg_split_of(L0, (char*)ws, offsets);
    MOE_TRY("wg_split", launch_wg_split(s, offsets, sp, st));
    MOE_TRY("gemm_dw2", launch_gemm_dw2(s, nullptr, nullptr, offsets, nullptr, nullptr, sp, (uint16_t*)dW2, st));
    MOE_TRY("gemm_dw1", launch_gemm_dw1(s, nullptr, nullptr, offsets, nullptr, nullptr, sp, (uint16_t*)dW1, st));
    return MOE_OK;
  }
  if (!dy || !x || !W1 || !W2 || !topk_w || !offsets || !perm || !inv_perm || !saved || !dx || !dW1 || !dW2 ||
      !d_topk_w || !ws)
    return MOE_ERR_NULL;
  if (d_logits && !topk_ids) return MOE_ERR_NULL;
  if (fp8 && (!x_scale || !W1_scale || !W2_scale)) return MOE_ERR_NULL;
  const BwdLayout L = bwd_layout(dims);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!al16(dy) || !al16(x) || !al16(W1) || !al16(W2) || !al16(dx) || !al16(dW1) || !al16(dW2) || !al256p(saved) ||
      !al256p(ws))
    return MOE_ERR_ALIGN;
  if (fp8 && (!al16(x_scale) || !al16(W1_scale) || !al16(W2_scale))) return MOE_ERR_ALIGN;
  const MoeShape s = shape_of(dims);
  const SavedLayout SL = saved_layout(dims);
  char* w = (char*)ws;
  const char* sv = (const char*)saved;
  int2* tiles = (int2*)(w + L.tiles);
  int32_t* ntiles = (int32_t*)(w + L.ntiles);
  uint16_t* dH = (uint16_t*)(w + L.dH);
  uint16_t* dXp = (uint16_t*)(w + L.dXp);
  float* dwp = (float*)(w + L.dwp);
  int32_t* tokrow = (int32_t*)(w + L.tokrow);
  const uint16_t* H = (const uint16_t*)(sv + SL.H);
  const uint16_t* As = (const uint16_t*)(sv + SL.As);
  hipStream_t st = (hipStream_t)stream;
  const WgSplit sp = wg_split_of(L, w, offsets);
  if (is_mx(dims)) {
    uint8_t *dyq = (uint8_t*)(w + L.dyq), *dye = (uint8_t*)(w + L.dys), *dyes = (uint8_t*)(w + L.dyes);
    uint8_t *dHq = (uint8_t*)(w + L.dHq), *dHe = (uint8_t*)(w + L.dHs);
    // W1, W2 in row blocks (K = 2f and d), quantised by the forward
    const uint8_t *w1q = (const uint8_t*)(sv + SL.w1q), *w1e = (const uint8_t*)(sv + SL.w1e);
    const uint8_t *w2q = (const uint8_t*)(sv + SL.w2q), *w2e = (const uint8_t*)(sv + SL.w2e);
    MOE_TRY("mx_quant_dy", launch_mx_quant((const uint16_t*)dy, 1, s.T, s.d, 0, dyq, dye, st));
    MOE_TRY("tile_map", launch_tile_map(offsets, s.E, kFp8BM, tiles, ntiles, st));
    MOE_TRY("ksort_dy", launch_kstep_sort(dye, s.d / 128, perm, s.k, offsets, s.E, (int64_t)s.T * s.k, dyes, st));
    MOE_TRY("gemm_dact", launch_mx_dact(s, dyq, dyes, w2q, w2e, H, topk_w, offsets, perm, tiles, ntiles, dH, dHq, dHe,
                                        dwp, st));
    MOE_TRY("gemm_dx", launch_mx_dx(s, dHq, dHe, w1q, w1e, offsets, perm, tiles, ntiles, dXp, st));
    MOE_TRY("combine_dx", launch_combine(dXp, inv_perm, s.T, s.d, s.k, (uint16_t*)dx, st));
    rc = mx_weight_grads(s, L, w, (const uint16_t*)x, (const uint16_t*)dy, As, dH, offsets, perm, (uint16_t*)dW1,
                         (uint16_t*)dW2, st);
    if (rc) return rc;
    MOE_TRY("dlogits", launch_dlogits(dwp, dact_parts(dims), inv_perm, topk_ids, topk_w, s.T, s.E, s.k, d_topk_w,
                                      d_logits, st));
    return MOE_OK;
  }
  if (fp8) {
    uint8_t* dyq = (uint8_t*)(w + L.dyq);
    float* dys = (float*)(w + L.dys);
    float* dyss = (float*)(w + L.dyss);
    uint8_t* dHq = (uint8_t*)(w + L.dHq);
    float* dHs = (float*)(w + L.dHs);
    const uint8_t *W18 = (const uint8_t*)W1, *W28 = (const uint8_t*)W2;
    MOE_TRY("quant_dy", launch_quant_rows((const uint16_t*)dy, s.T, s.d, dyq, dys, st));
    MOE_TRY("tile_map", launch_tile_map(offsets, s.E, kFp8BM, tiles, ntiles, st));
    MOE_TRY("ksort_dy", launch_kstep_sort(dys, s.d / 128, perm, s.k, offsets, s.E, (int64_t)s.T * s.k, dyss, st));
    MOE_TRY("gemm_dact", launch_fp8_dact(s, dyq, dyss, W28, W2_scale, H, topk_w, offsets, perm, tiles, ntiles, dH, dHq,
                                         dHs, dwp, st));
    MOE_TRY("gemm_dx", launch_fp8_dx(s, dHq, dHs, W18, W1_scale, offsets, perm, tiles, ntiles, dXp, st));
    MOE_TRY("combine_dx", launch_combine(dXp, inv_perm, s.T, s.d, s.k, (uint16_t*)dx, st));
    // weight gradients in bf16 MFMA: x dequantised to bf16 once, with dy, As and dH as they are
    uint16_t* xbf = (uint16_t*)(w + L.xbf);
    MOE_TRY("dequant_x", launch_dequant_rows((const uint8_t*)x, x_scale, s.T, s.d, xbf, st));
    MOE_TRY("tokrow", launch_tokrow(perm, offsets, s.E, (int64_t)s.T * s.k, s.k, tokrow, st));
    MOE_TRY("wg_split", launch_wg_split(s, offsets, sp, st));
    MOE_TRY("gemm_dw2", launch_gemm_dw2(s, As, (const uint16_t*)dy, offsets, perm, tokrow, sp, (uint16_t*)dW2, st));
    MOE_TRY("wg_reduce", launch_wg_reduce(s, sp, (int64_t)s.f * s.d, (uint16_t*)dW2, st));
    MOE_TRY("gemm_dw1", launch_gemm_dw1(s, xbf, dH, offsets, perm, tokrow, sp, (uint16_t*)dW1, st));
    MOE_TRY("wg_reduce", launch_wg_reduce(s, sp, (int64_t)s.d * 2 * s.f, (uint16_t*)dW1, st));
    MOE_TRY("dlogits", launch_dlogits(dwp, dact_parts(dims), inv_perm, topk_ids, topk_w, s.T, s.E, s.k, d_topk_w,
                                      d_logits, st));
    return MOE_OK;
  }
  MOE_TRY("tile_map", launch_tile_map(offsets, s.E, kGemmBM, tiles, ntiles, st));
  MOE_TRY("gemm_dact", launch_gemm_dact(s, (const uint16_t*)dy, (const uint16_t*)W2, H, topk_w, offsets, perm, tiles, ntiles, dH,
                           dwp, st));
  MOE_TRY("gemm_dx", launch_gemm_dx(s, dH, (const uint16_t*)W1, offsets, perm, tiles, ntiles, dXp, st));
  MOE_TRY("combine_dx", launch_combine(dXp, inv_perm, s.T, s.d, s.k, (uint16_t*)dx, st));
  MOE_TRY("tokrow", launch_tokrow(perm, offsets, s.E, (int64_t)s.T * s.k, s.k, tokrow, st));
  MOE_TRY("wg_split", launch_wg_split(s, offsets, sp, st));
  MOE_TRY("gemm_dw2", launch_gemm_dw2(s, As, (const uint16_t*)dy, offsets, perm, tokrow, sp, (uint16_t*)dW2, st));
  MOE_TRY("wg_reduce", launch_wg_reduce(s, sp, (int64_t)s.f * s.d, (uint16_t*)dW2, st));
  MOE_TRY("gemm_dw1", launch_gemm_dw1(s, (const uint16_t*)x, dH, offsets, perm, tokrow, sp, (uint16_t*)dW1, st));
  MOE_TRY("wg_reduce", launch_wg_reduce(s, sp, (int64_t)s.d * 2 * s.f, (uint16_t*)dW1, st));
  MOE_TRY("dlogits", launch_dlogits(dwp, dact_parts(dims), inv_perm, topk_ids, topk_w, s.T, s.E, s.k, d_topk_w, d_logits,
                                   st));

  return MOE_OK;
}

int moe_router_logits(const moe_dims* dims, const void* x, const void* Wg, float* logits, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (dims->dtype == MOE_FP8_E4M3) return MOE_ERR_DTYPE;  // the gate reads x in bf16
  if (dims->T == 0) return MOE_OK;
  if (!x || !Wg || !logits) return MOE_ERR_NULL;
  if (!al16(x) || !al16(Wg) || !al16(logits)) return MOE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  MOE_TRY("router_logits", launch_router_logits((const uint16_t*)x, (const uint16_t*)Wg, (int)dims->T,
                                                (int)dims->d, (int)dims->E, logits, st));
  return MOE_OK;
}

int moe_router_backward(const moe_dims* dims, const void* x, const void* Wg, const float* d_logits, void* dx,
                        void* dWg, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (dims->dtype == MOE_FP8_E4M3) return MOE_ERR_DTYPE;
  const int T = (int)dims->T, d = (int)dims->d, E = (int)dims->E;
  const size_t need = al256(router_ws_bytes(dims->T, d, E));
  if (dWg && need > 0 && !ws) return MOE_ERR_NULL;
  if (dWg && ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (T > 0 && (dx || dWg) && (!d_logits || (dWg && !x) || (dx && !Wg))) return MOE_ERR_NULL;
  if ((x && !al16(x)) || (Wg && !al16(Wg)) || (d_logits && !al16(d_logits)) || (dx && !al16(dx)) ||
      (dWg && !al16(dWg)) || (ws && !al256p(ws)))
    return MOE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  if (dx && T > 0)
    MOE_TRY("router_dx", launch_router_dx(d_logits, (const uint16_t*)Wg, T, d, E, (uint16_t*)dx, st));
  // an empty layer still writes dWg (zeros)
  if (dWg) MOE_TRY("router_dwg", launch_router_dwg((const uint16_t*)x, d_logits, T, d, E, (uint16_t*)dWg, (float*)ws, st));
  return MOE_OK;
}

int moe_permute(const moe_dims* dims, const void* x, const int32_t* inv_perm, void* xp, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (dims->dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (dims->T == 0) return MOE_OK;
  if (!x || !inv_perm || !xp) return MOE_ERR_NULL;
  if (!al16(x) || !al16(xp)) return MOE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  MOE_TRY("permute", launch_permute((const uint16_t*)x, inv_perm, (int)dims->T, (int)dims->d, (int)dims->k,
                                   (uint16_t*)xp, st));
  return MOE_OK;
}

int moe_combine(const moe_dims* dims, const void* op, const int32_t* inv_perm, void* y, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (dims->dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (dims->T == 0) return MOE_OK;  // an empty layer has nothing to combine
  if (!op || !inv_perm || !y) return MOE_ERR_NULL;
  if (!al16(op) || !al16(y)) return MOE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  MOE_TRY("combine", launch_combine((const uint16_t*)op, inv_perm, (int)dims->T, (int)dims->d, (int)dims->k,
                                   (uint16_t*)y, st));

  return MOE_OK;
}

// batch x rows x cols below 2^40 elements, each side within int range (checked without overflow)
static bool mx_size_ok(int64_t batch, int64_t rows, int64_t cols) {
  if (batch < 0 || rows < 0 || cols < 0 || rows > (1 << 30) || cols > (1 << 30)) return false;
  if (rows == 0 || cols == 0) return true;
  return batch <= (((int64_t)1 << 40) - 1) / (rows * cols);  // rows * cols <= 2^60: no overflow
}

int moe_mxfp8_quantize(const void* src, int64_t batch, int64_t rows, int64_t cols, int block_axis, void* codes,
                       void* exps, void* stream) {
  if (block_axis != 0 && block_axis != 1) return MOE_ERR_SHAPE;
  if (!mx_size_ok(batch, rows, cols)) return MOE_ERR_SHAPE;
  if (block_axis == 1 ? (cols % 32 != 0) : (rows % 32 != 0 || cols % 8 != 0)) return MOE_ERR_SHAPE;
  if (batch * rows * cols == 0) return MOE_OK;
  if (!src || !codes || !exps) return MOE_ERR_NULL;
  if (!al16(src) || !al16(codes) || ((uintptr_t)exps & 7u)) return MOE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  MOE_TRY("mx_quant", launch_mx_quant((const uint16_t*)src, batch, (int)rows, (int)cols, block_axis == 0 ? 1 : 0,
                                      (uint8_t*)codes, (uint8_t*)exps, st));
  return MOE_OK;
}

int moe_mxfp8_quantize_weights(const void* src, int64_t batch, int64_t rows, int64_t cols, void* col_codes,
                               void* col_exps, void* row_codes, void* row_words, void* stream) {
  if (!mx_size_ok(batch, rows, cols)) return MOE_ERR_SHAPE;
  if (rows % 32 != 0 || cols % 256 != 0) return MOE_ERR_SHAPE;
  if (batch * rows * cols == 0) return MOE_OK;
  if (!src || !col_codes || !col_exps || !row_codes || !row_words) return MOE_ERR_NULL;
  if (!al16(src) || !al16(col_codes) || !al16(row_codes) || ((uintptr_t)col_exps & 7u) || ((uintptr_t)row_words & 3u))
    return MOE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  MOE_TRY("mx_quant", launch_mx_quant_dual((const uint16_t*)src, batch, (int)rows, (int)cols, (uint8_t*)col_codes,
                                           (uint8_t*)col_exps, (uint8_t*)row_codes, (uint8_t*)row_words, st));
  return MOE_OK;
}

int moe_set_stage_hook(moe_stage_hook hook, void* user) {
  g_hook = hook;
  g_hook_user = user;
  return MOE_OK;
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "dims outside the supported range";
    case MOE_ERR_DTYPE: return "dtype not supported by this call";
    case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_bytes()";
    case MOE_ERR_ALIGN: return "buffer not aligned (tensors 16 bytes, ws/saved 256 bytes)";
    case MOE_ERR_HIP: return hipGetErrorString(g_last_hip);
    default: return "unknown status";
  }
}

}  // extern "C"
