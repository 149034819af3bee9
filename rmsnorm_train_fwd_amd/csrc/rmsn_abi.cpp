// rmsn_abi.cpp -- the C ABI of include/rmsnorm_train.h: validation, planning,
// launch. Every check runs on the host before anything is enqueued and never
// dereferences a device pointer, so the error paths run without a GPU.
#include "rmsnorm_train.h"

#include <math.h>
#include <string.h>

#include "rmsn_abi_internal.hpp"
#include "rmsn_launch.hpp"

namespace {

using namespace rmsn;

constexpr int64_t kWidths[] = {256, 512, 1536, 2048, 4096, 5120, 6144};
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;
constexpr int64_t kSmallTreeTiles = 8;   // tiles per chunk at most, for small row counts
constexpr int64_t kMaxStride = int64_t(1) << 40;
constexpr int32_t kMaxGrid = 1 << 24;

// Small row counts, per width: at or below these, the dw tree gives each
// chunk at most kSmallTreeTiles tiles, and the backward runs as one launch
// (row tasks + column tasks) unless a launch override says otherwise. The
// values are where the single launch stopped beating main kernel + fold
// (above them, on its tree of up to 256 chunks) on MI355X, kernel-active time
// with cold caches; the column tasks re-read x and dy, so the crossover falls
// as rows get wider. Both paths give the same bits for a given tree.
int64_t small_rows(int64_t width) {
  switch (width) {
    case 256: return 1280;
    case 512: return 960;
    case 1536: return 640;
    case 2048: return 640;
    case 4096: return 512;
    case 5120: return 512;
    default: return 384;  // 6144
  }
}

bool width_ok(int64_t w) {
  for (int64_t k : kWidths)
    if (k == w) return true;
  return false;
}

int rows_per_subchain_group(int64_t width) {  // R: row groups per workgroup
  return bwd_rows_per_rowtask((int)width);
}


struct Span {
  uintptr_t lo = 0, hi = 0;  // [lo, hi); empty if lo == hi
  bool empty() const { return lo == hi; }
};

bool overlap(const Span& a, const Span& b) {
  return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

Span dense_span(const void* p, int64_t bytes) {
  Span s;
  if (p && bytes > 0) {
    s.lo = (uintptr_t)p;
    s.hi = s.lo + (uintptr_t)bytes;
  }
  return s;
}

// Byte extent of a strided BF16 row input: base .. last element + 1.
Span row_span(const void* p, const rmsn_layout& L, int64_t st, int64_t sh) {
  if (!p || L.T == 0) return Span{};
  const int64_t last = (L.T - 1) * (L.T > 1 ? st : 0) + (L.heads - 1) * (L.heads > 1 ? sh : 0) + L.width;
  return dense_span(p, last * 2);
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

rmsn_status check_layout(const rmsn_layout* L) {
  if (!L) return RMSN_E_NULL;
  if (L->T < 0 || L->heads < 1 || !width_ok(L->width)) return RMSN_E_SHAPE;
  if (L->T > kMaxRows || L->heads > kMaxRows || L->T * L->heads > kMaxRows) return RMSN_E_SHAPE;
  const int64_t pairs[2][2] = {{L->x_stride_t, L->x_stride_h}, {L->g_stride_t, L->g_stride_h}};
  for (const auto& s : pairs) {
    const int64_t st = s[0], sh = s[1];
    if (L->heads > 1) {
      if (sh < L->width || sh > kMaxStride) return RMSN_E_STRIDE;
      if (sh % 8) return RMSN_E_ALIGN;
    }
    if (L->T > 1) {
      // wide: (heads - 1) * stride_h can exceed 64 bits within the bounds above
      const __int128 need = (__int128)(L->heads - 1) * (L->heads > 1 ? sh : 0) + L->width;
      if (st < need || st > kMaxStride) return RMSN_E_STRIDE;
      if (st % 8) return RMSN_E_ALIGN;
    }
    // The view's byte extent must fit the 48-bit address space (computed
    // wide: T * stride_t alone can exceed 64 bits within the per-field bounds).
    if (L->T > 0) {
      const __int128 last = (__int128)(L->T - 1) * (L->T > 1 ? st : 0) +
                            (__int128)(L->heads - 1) * (L->heads > 1 ? sh : 0) + L->width;
      if (last * 2 > ((__int128)1 << 48)) return RMSN_E_SHAPE;
    }
  }
  return RMSN_OK;
}

rmsn_status check_launch(const rmsn_launch* o) {
  if (!o) return RMSN_OK;
  if (o->grid < 0 || o->fold_grid < 0 || o->grid > kMaxGrid || o->fold_grid > kMaxGrid)
    return RMSN_E_LAUNCH;
  if (o->path != RMSN_PATH_AUTO && o->path != RMSN_PATH_SMALL && o->path != RMSN_PATH_LARGE)
    return RMSN_E_LAUNCH;
  return RMSN_OK;
}

bool eps_ok(float eps) { return isfinite(eps) && eps >= 0.0f; }

// Weight codes: BF16 or FP32 storage, plain or zero-centred (1 + w).
bool w_code_ok(int c) {
  return c == RMSN_BF16 || c == RMSN_F32 || c == RMSN_BF16_ZERO_CENTRED ||
         c == RMSN_F32_ZERO_CENTRED;
}
bool w_is_f32(int c) { return c == RMSN_F32 || c == RMSN_F32_ZERO_CENTRED; }
int w_zero_centred(int c) {
  return c == RMSN_BF16_ZERO_CENTRED || c == RMSN_F32_ZERO_CENTRED ? 1 : 0;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

void make_plan(const rmsn_layout& L, int /*det*/, const rmsn_launch* o, rmsn_bwd_plan* p) {
  memset(p, 0, sizeof *p);
  const int64_t rows = L.T * L.heads;
  p->rows = rows;
  // The dw tree: depends on the row count and the width only. Tiles of R
  // rows are dealt to the chunks in turn. Small row counts: at most 8 tiles
  // per chunk (one load round trip per sub-chain on the single-launch path,
  // and at most two 32-chunk fold groups);
  // otherwise kMaxChunks chunks (one per workgroup of the main kernel that a
  // 256-CU part holds at once, so all chunks run in one round with no tail),
  // or one per tile if there are fewer.
  const int64_t R = rows_per_subchain_group(L.width);
  const int64_t tiles = cdiv(rows, R);
  const bool small = rows <= small_rows(L.width);
  int64_t K = small ? cdiv(tiles, kSmallTreeTiles) : kMaxChunks;
  if (K > tiles) K = tiles;
  p->chunks = K;
  p->subchains = (int32_t)R;
  p->fold_group = kFoldGroup;
  int path = o ? o->path : RMSN_PATH_AUTO;
  if (rows == 0) path = RMSN_PATH_SMALL;  // only dw = 0 to write
  if (path == RMSN_PATH_AUTO)
    path = small ? RMSN_PATH_SMALL : RMSN_PATH_LARGE;
  p->path = path;
  const int32_t col_tiles = (int32_t)(L.width / small_col_tile((int)L.width));
  if (path == RMSN_PATH_SMALL) {
    const int64_t tiles = cdiv(rows, small_rows_per_rowtask((int)L.width));
    p->grid = (o && o->grid) ? o->grid : (int32_t)(tiles < kMaxGrid ? tiles : kMaxGrid);
    if (rows == 0) p->grid = 0;
    p->fold_grid = (o && o->fold_grid) ? o->fold_grid : col_tiles;
    p->workspace_bytes = 0;
  } else {
    p->grid = (o && o->grid) ? o->grid : (int32_t)p->chunks;
    p->fold_grid = (o && o->fold_grid) ? o->fold_grid : (int32_t)(L.width / kFoldTile);
    p->workspace_bytes = (size_t)p->chunks * (size_t)L.width * sizeof(double);
  }
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

RowIn row_in(const void* p, int64_t st, int64_t sh) {
  return RowIn{static_cast<const uint16_t*>(p), st, sh};
}

}  // namespace

namespace rmsn {

// ---------------------------------------------------------------- backward --
rmsn_status bwd_common(int form, const void* dy, const void* x, const void* e, const void* w,
                       int w_dtype, const float* rstd, int det, const rmsn_layout* L,
                       void* dx, void* dz, void* dw, int dw_dtype, void* ws,
                       size_t ws_bytes, WorkspaceSource ws_source, const rmsn_launch* o,
                       void* stream) {
  rmsn_status st = check_layout(L);
  if (st) return st;
  if (!w_code_ok(w_dtype)) return RMSN_E_DTYPE;
  if (dw_dtype != RMSN_BF16 && dw_dtype != RMSN_F32) return RMSN_E_DTYPE;
  if (det != 0 && det != 1) return RMSN_E_ARG;
  if ((st = check_launch(o))) return st;
  const int64_t rows = L->T * L->heads;
  if (!w || !dw) return RMSN_E_NULL;
  if (rows > 0 && (!dy || !x || !rstd || !dx)) return RMSN_E_NULL;
  if (form == kGate && rows > 0 && (!e || !dz)) return RMSN_E_NULL;
  if (!aligned(w, 16) || !aligned(dw, 16)) return RMSN_E_ALIGN;
  if (rows > 0) {
    if (!aligned(dy, 16) || !aligned(x, 16) || !aligned(dx, 16) || !aligned(rstd, 4))
      return RMSN_E_ALIGN;
    if (e && !aligned(e, 16)) return RMSN_E_ALIGN;
    if (dz && !aligned(dz, 16)) return RMSN_E_ALIGN;
  }
  rmsn_bwd_plan plan;
  make_plan(*L, det, o, &plan);
  if (ws_source && plan.workspace_bytes > 0) {
    if ((st = ws_source(stream, plan.workspace_bytes, &ws, &ws_bytes))) return st;
  }
  if (plan.workspace_bytes > 0) {
    if (!ws || ws_bytes < plan.workspace_bytes) return RMSN_E_WORKSPACE;
    if (!aligned(ws, 16)) return RMSN_E_ALIGN;
  }
  const int64_t W = L->width;
  const int64_t wbytes = W * (w_is_f32(w_dtype) ? 4 : 2);
  const int64_t rbytes = rows * W * 2;
  const bool e_uses_g = (form == kResidual);
  const Span ins[] = {
      row_span(dy, *L, L->g_stride_t, L->g_stride_h),
      row_span(x, *L, L->x_stride_t, L->x_stride_h),
      e_uses_g ? row_span(e, *L, L->g_stride_t, L->g_stride_h)
               : row_span(e, *L, L->x_stride_t, L->x_stride_h),
      dense_span(w, wbytes),
      dense_span(rstd, rows * 4),
  };
  const Span outs[] = {
      dense_span(dx, rbytes),
      form == kGate ? dense_span(dz, rbytes) : Span{},
      dense_span(dw, W * (dw_dtype == RMSN_F32 ? 4 : 2)),
      dense_span(ws, (int64_t)plan.workspace_bytes),
  };
  for (const Span& a : outs) {
    for (const Span& b : ins)
      if (overlap(a, b)) return RMSN_E_ALIAS;
    for (const Span& b : outs)
      if (&a != &b && overlap(a, b)) return RMSN_E_ALIAS;
  }

  BwdArgs a;
  a.dy = row_in(dy, L->g_stride_t, L->g_stride_h);
  a.x = row_in(x, L->x_stride_t, L->x_stride_h);
  a.e = e_uses_g ? row_in(e, L->g_stride_t, L->g_stride_h) : row_in(e, L->x_stride_t, L->x_stride_h);
  a.w = w;
  a.rstd = rstd;
  a.dx = static_cast<uint16_t*>(dx);
  a.dz = static_cast<uint16_t*>(dz);
  a.dw = dw;
  a.dw_bf16 = dw_dtype == RMSN_BF16;
  a.ws = static_cast<double*>(ws);
  a.rows = rows;
  a.chunks = plan.chunks;
  a.heads = (int32_t)L->heads;
  a.w_one = w_zero_centred(w_dtype);
  const bool wf32 = w_is_f32(w_dtype);
  const hipStream_t s = as_stream(stream);
  hipError_t err;
  if (plan.path == RMSN_PATH_SMALL) {
    err = launch_bwd_small((int)W, wf32, form, a, plan.grid, plan.fold_grid, s);
  } else {
    err = launch_bwd_large((int)W, wf32, form, det != 0, a, plan.grid, s);
    if (err == hipSuccess) err = launch_fold((int)W, a, plan.fold_grid, s);
  }
  return err == hipSuccess ? RMSN_OK : RMSN_E_HIP;
}

}  // namespace rmsn

using rmsn::bwd_common;

// ================================================================ C ABI ====

RMSN_API const char* rmsn_status_str(rmsn_status s) {
  switch (enum_code(s)) {
    case RMSN_OK: return "ok";
    case RMSN_E_NULL: return "a required pointer is NULL";
    case RMSN_E_DTYPE: return "unsupported dtype";
    case RMSN_E_SHAPE: return "unsupported shape (T, heads or width)";
    case RMSN_E_STRIDE: return "strides make rows overlap or run backwards";
    case RMSN_E_ALIGN: return "misaligned pointer or stride";
    case RMSN_E_ALIAS: return "an output overlaps an input or another output";
    case RMSN_E_WORKSPACE: return "workspace missing or too small";
    case RMSN_E_LAUNCH: return "bad launch override";
    case RMSN_E_ARG: return "bad argument (eps or flag)";
    case RMSN_E_HIP: return "HIP runtime error at launch";
  }
  return "unknown status";
}

RMSN_API rmsn_status rmsnorm_train_bwd_query(const rmsn_layout* L, int deterministic,
                                             const rmsn_launch* launch, rmsn_bwd_plan* plan) {
  rmsn_status st = check_layout(L);
  if (st) return st;
  if (deterministic != 0 && deterministic != 1) return RMSN_E_ARG;
  if ((st = check_launch(launch))) return st;
  if (!plan) return RMSN_E_NULL;
  make_plan(*L, deterministic, launch, plan);
  return RMSN_OK;
}

static rmsn_status fwd_common(int form, const void* x, const void* e, const void* w,
                              int w_dtype, float eps, const rmsn_layout* L, void* y,
                              void* h_out, float* rstd, void* stream) {
  rmsn_status st = check_layout(L);
  if (st) return st;
  if (!w_code_ok(w_dtype)) return RMSN_E_DTYPE;
  if (!eps_ok(eps)) return RMSN_E_ARG;
  const int64_t rows = L->T * L->heads;
  if (!w) return RMSN_E_NULL;
  if (form != kResidual && h_out) return RMSN_E_ARG;  // h_out only with a residual
  if (rows > 0 && (!x || !y || !rstd || (form != kPlain && !e))) return RMSN_E_NULL;
  if (rows > 0 && form == kResidual && !h_out) return RMSN_E_NULL;
  if (!aligned(w, 16)) return RMSN_E_ALIGN;
  if (rows > 0) {
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(rstd, 4)) return RMSN_E_ALIGN;
    if (e && !aligned(e, 16)) return RMSN_E_ALIGN;
    if (h_out && !aligned(h_out, 16)) return RMSN_E_ALIGN;
  }
  const int64_t W = L->width;
  const int64_t rbytes = rows * W * 2;
  const Span ins[] = {
      row_span(x, *L, L->x_stride_t, L->x_stride_h),
      row_span(e, *L, L->x_stride_t, L->x_stride_h),
      dense_span(w, W * (w_is_f32(w_dtype) ? 4 : 2)),
  };
  const Span outs[] = {dense_span(y, rbytes), dense_span(h_out, rbytes), dense_span(rstd, rows * 4)};
  for (const Span& a : outs) {
    for (const Span& b : ins)
      if (overlap(a, b)) return RMSN_E_ALIAS;
    for (const Span& b : outs)
      if (&a != &b && overlap(a, b)) return RMSN_E_ALIAS;
  }
  if (rows == 0) return RMSN_OK;

  FwdArgs a;
  a.x = row_in(x, L->x_stride_t, L->x_stride_h);
  a.e = row_in(e, L->x_stride_t, L->x_stride_h);
  a.w = w;
  a.y = static_cast<uint16_t*>(y);
  a.h = static_cast<uint16_t*>(h_out);
  a.rstd = rstd;
  a.rows = rows;
  a.heads = (int32_t)L->heads;
  a.w_one = w_zero_centred(w_dtype);
  a.eps = eps;
  const int64_t tiles = cdiv(rows, fwd_rows_per_tile((int)W, form));
  const int grid = (int)(tiles < kMaxGrid ? tiles : kMaxGrid);
  hipError_t err = launch_fwd((int)W, w_is_f32(w_dtype), form, a, grid, as_stream(stream));
  return err == hipSuccess ? RMSN_OK : RMSN_E_HIP;
}

RMSN_API rmsn_status rmsnorm_train_fwd(const void* x, const void* residual, const void* w,
                                       rmsn_dtype w_dtype, float eps, const rmsn_layout* L,
                                       void* y, void* h_out, float* rstd, void* stream) {
  return fwd_common(residual ? kResidual : kPlain, x, residual, w, enum_code(w_dtype), eps, L, y,
                    h_out, rstd, stream);
}

RMSN_API rmsn_status rmsnorm_silu_gate_train_fwd(const void* x, const void* z, const void* w,
                                                 rmsn_dtype w_dtype, float eps,
                                                 const rmsn_layout* L, void* y, float* rstd,
                                                 void* stream) {
  return fwd_common(kGate, x, z, w, enum_code(w_dtype), eps, L, y, nullptr, rstd, stream);
}

RMSN_API rmsn_status rmsnorm_train_bwd(const void* dy, const void* x, const void* dh,
                                       const void* w, rmsn_dtype w_dtype, const float* rstd,
                                       int deterministic, const rmsn_layout* L, void* dx,
                                       void* dw, rmsn_dtype dw_dtype, void* workspace,
                                       size_t workspace_bytes, const rmsn_launch* launch,
                                       void* stream) {
  return bwd_common(dh ? kResidual : kPlain, dy, x, dh, w, enum_code(w_dtype), rstd,
                    deterministic, L, dx, nullptr, dw, enum_code(dw_dtype), workspace,
                    workspace_bytes, nullptr, launch, stream);
}

RMSN_API rmsn_status rmsnorm_silu_gate_train_bwd(const void* dy, const void* x, const void* z,
                                                 const void* w, rmsn_dtype w_dtype,
                                                 const float* rstd, int deterministic,
                                                 const rmsn_layout* L, void* dx, void* dz,
                                                 void* dw, rmsn_dtype dw_dtype, void* workspace,
                                                 size_t workspace_bytes,
                                                 const rmsn_launch* launch, void* stream) {
  return bwd_common(kGate, dy, x, z, w, enum_code(w_dtype), rstd, deterministic, L, dx, dz, dw,
                    enum_code(dw_dtype), workspace, workspace_bytes, nullptr, launch, stream);
}
