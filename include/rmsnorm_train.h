/*
 * rmsnorm_train.h -- C ABI of the MI355X (gfx950) RMSNorm-for-training library.
 *
 * Sources for what the calls compute (the pages this project follows):
 *  [A] PR #8626 merge text (shown on the PR #8512 page), opening paragraph:
 *      the forward returns y (BF16) and rstd (FP32); the backward returns dx
 *      (BF16) and dw (FP32); deterministic=True/False share the forward and
 *      differ only in the backward; forms: [T, H] rows with BF16 or FP32
 *      weight, a fused residual add, per-head views [T,24,256] (strided) and
 *      [T,4,256] (contiguous) with a shared w[256].
 *  [B] Same text, "Key": [T,24,256] has strides (12288, 512, 1); the residual
 *      form adds the BF16 output h_new. PR #8848 page, "Key": h_new =
 *      BF16(h + u), combined gradient.
 *  [C] PR #8512 page, description: the deterministic backward sums each dw
 *      column in a fixed row order with exact products and compensated
 *      (TwoSum) summation, then a fixed-order FP64 fold and one rounding to
 *      FP32, so dw does not depend on the grid size or the number of compute
 *      units; small token counts run one launch instead of a main kernel plus
 *      a separate dw reduction. "Residual rows": the forward returns
 *      h = x + residual and y = RMSNorm(h); the backward takes the gradients
 *      of y and h and returns the gradient of h and dw.
 *  [D] PR #8848 page, description: the non-deterministic backward is one
 *      kernel with blocked FP32 dw sums.
 *  [E] PR #8656 page, description: SiLU-gated RMSNorm training, deterministic
 *      and non-deterministic, FP32 weight gradient.
 *  [F] Review on the PR #8512 page: a dw that shares storage with w must be
 *      rejected. Review on the PR #8848 page: launch bindings must reject
 *      multi-dimensional grids (this ABI only has a 1-D grid override).
 *
 * Math (the pages never print it; textbook RMSNorm, eps inside the root):
 *   rstd = 1/sqrt(mean_j x_j^2 + eps);  y_j = (x_j*rstd)*w_j
 *   dx_j = rstd*(g_j - xhat_j*mean_k(g_k*xhat_k)), g_j = dy_j*w_j, xhat = x*rstd
 *   dw_j = sum over rows of dy_j*xhat_j
 * Gate: y_j = xhat_j*w_j*silu(z_j); g_j = dy_j*w_j*silu(z_j);
 *   dz_j = dy_j*xhat_j*w_j*sigmoid(z_j)*(1 + z_j*(1 - sigmoid(z_j)));
 *   dw_j = sum over rows of dy_j*xhat_j*silu(z_j).
 * GPU arithmetic: FP32 statistics, FP32 products, one round-to-nearest-even
 * to BF16 per BF16 output; dw as described for each mode below.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless stated. The caller owns every buffer,
 *    including the workspace. The library never allocates, frees or
 *    synchronises and keeps no pointer after return; calls are asynchronous
 *    on `stream` (a hipStream_t; NULL = the default stream). Its only mutable
 *    global state is the per-device address of the device array behind
 *    rmsnorm_train_bwd_noalloc, looked up once per device under a lock; every
 *    other call is free of shared state and safe from several host threads.
 *  - Rows: a layout describes T tokens x `heads` rows per token; row
 *    r = t*heads + h of a row input starts at base + t*stride_t + h*stride_h
 *    (elements). Row outputs (y, h_out, dx / grad_h, dz) are dense
 *    [T, heads, width]; rstd is dense [T*heads]; dw is [width].
 *  - Supported widths: 256, 512, 1536, 2048, 4096, 5120, 6144 ([C]).
 *  - Sizes: T >= 0, heads >= 1, T*heads <= 2^31 - 1 rows, and each view's
 *    extent (last element + 1, in bytes) at most 2^48 (else RMSN_E_SHAPE).
 *  - Strides, for each pair (x_*, g_*): with heads > 1, width <= stride_h <=
 *    2^40; with T > 1, (heads - 1)*stride_h + width <= stride_t <= 2^40, i.e.
 *    rows never overlap (else RMSN_E_STRIDE). A stride whose dimension has
 *    size 1 is not used and not checked.
 *  - Alignment: every BF16 row pointer, w and dw 16-byte aligned; strides
 *    multiples of 8 elements; rstd 4-byte aligned; workspace 16-byte aligned.
 *  - Overlap: no output may share a byte with an input or another output
 *    (extents are [base, base + last element]); dw never overlaps w ([F]).
 *  - Errors: every check runs before anything is enqueued; on error nothing is
 *    launched and no output is touched. RMSN_E_HIP means that the HIP runtime
 *    refused one of this call's own launches after validation (outputs then
 *    undefined). The library never reads or clears the calling thread's HIP
 *    last-error state (hipGetLastError), so an earlier, unrelated error stays
 *    the caller's to see and does not turn a good call into RMSN_E_HIP.
 *  - T == 0 is valid: the forward enqueues nothing; the backward writes
 *    dw = 0. Row pointers may then be NULL.
 */
#ifndef RMSNORM_TRAIN_H
#define RMSNORM_TRAIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RMSN_OK = 0,
  RMSN_E_NULL = 1,        /* a required pointer is NULL */
  RMSN_E_DTYPE = 2,       /* unknown weight code, or a dw code other than RMSN_BF16 / RMSN_F32 */
  RMSN_E_SHAPE = 3,       /* T < 0, heads < 1, width unsupported, size overflow */
  RMSN_E_STRIDE = 4,      /* strides make rows overlap or run backwards */
  RMSN_E_ALIGN = 5,       /* misaligned pointer or stride */
  RMSN_E_ALIAS = 6,       /* an output overlaps an input or another output */
  RMSN_E_WORKSPACE = 7,   /* workspace NULL or smaller than the query result */
  RMSN_E_LAUNCH = 8,      /* bad launch override */
  RMSN_E_ARG = 9,         /* eps not finite or negative; bad flag value */
  RMSN_E_HIP = 10         /* the HIP runtime rejected a launch */
} rmsn_status;

/* Storage format of w (and of dw, which takes RMSN_BF16 or RMSN_F32 only).
 * The *_ZERO_CENTRED weight codes select the zero-centred-weight RMSNorm: the
 * stored w is centred on zero and every formula below uses 1 + w in its place
 * (rounded once to FP32 on the GPU); dw is then the gradient with respect to
 * the stored w, which is the same sum. The pages name this variant only in
 * the title of a related PR on the PR #8512 page ("zero-centred input
 * RMSNorm") and never define it; this is the plainest reading that keeps the
 * name RMSNorm (a mean-subtracted input would be LayerNorm). */
typedef enum {
  RMSN_BF16 = 0,
  RMSN_F32 = 1,
  RMSN_BF16_ZERO_CENTRED = 2,  /* w stored as BF16, used as 1 + w */
  RMSN_F32_ZERO_CENTRED = 3    /* w stored as FP32, used as 1 + w */
} rmsn_dtype;

/* Row geometry (all counts and strides in elements). */
typedef struct {
  int64_t T;           /* tokens, >= 0 */
  int64_t heads;       /* rows per token, >= 1 ([T, H] rows: heads = 1) */
  int64_t width;       /* elements per row (see supported widths) */
  int64_t x_stride_t;  /* token stride of x, residual, z (and h in the bwd) */
  int64_t x_stride_h;  /* head stride of the same tensors (unused if heads == 1) */
  int64_t g_stride_t;  /* token stride of dy and dh */
  int64_t g_stride_h;  /* head stride of dy and dh (unused if heads == 1) */
} rmsn_layout;

/* Backward paths. */
enum {
  RMSN_PATH_AUTO = 0,
  RMSN_PATH_SMALL = 1,  /* one launch: row tasks for dx + column tasks for dw */
  RMSN_PATH_LARGE = 2   /* main kernel (dx + FP64 chunk partials) + FP64 fold */
};

/* Launch override, for tests of grid independence. NULL = automatic.
 * grid / fold_grid: 1-D workgroup counts (0 = automatic; >= 1 otherwise) of
 * the main kernel and the fold on the large path, and of the row tasks (dx)
 * and the column tasks (dw) of the single launch on the small path. */
typedef struct {
  int32_t grid;
  int32_t fold_grid;
  int32_t path;        /* RMSN_PATH_* */
} rmsn_launch;

/* What a backward call will do (host-only query, no HIP call). */
typedef struct {
  int32_t path;          /* RMSN_PATH_SMALL or RMSN_PATH_LARGE */
  int64_t rows;          /* T * heads */
  int64_t chunks;        /* K: chunks of the dw tree (see rmsnorm_train_bwd) */
  int32_t subchains;     /* R: rows per tile = sub-chains per chunk (fixed per width) */
  int32_t fold_group;    /* chunks per first-level fold group */
  int32_t grid;          /* large path: main-kernel workgroups; small path: row tasks */
  int32_t fold_grid;     /* large path: fold workgroups; small path: column tasks */
  size_t workspace_bytes;
} rmsn_bwd_plan;

/* ---------------------------------------------------------------- forward --
 * y = RMSNorm(x) * w (BF16), rstd (FP32) for every row ([A]).
 * residual != NULL selects the fused residual form ([B], [C] "Residual rows"):
 * h_out = RNE_bf16(x + residual) (the exact sum rounded once), and y, rstd
 * are computed from that BF16 h. h_out must be NULL iff residual is NULL.
 * x, residual: BF16 rows in the x strides of L. w: [width] of w_dtype.
 * eps: finite, >= 0 (the pages use 1e-6).                                   */
rmsn_status rmsnorm_train_fwd(const void* x, const void* residual, const void* w,
                              rmsn_dtype w_dtype, float eps, const rmsn_layout* L, void* y,
                              void* h_out, float* rstd, void* stream);

/* ---------------------------------------------------------------- backward --
 * dx (BF16) and dw (FP32 or BF16) from dy (BF16, g strides), x (BF16, x strides; the
 * BF16 h of the forward in the residual form), the forward's rstd and w.
 * dh != NULL selects the residual form: the row output is grad_h = dh + dx
 * (one rounding), dh in the g strides ([C] "Residual rows").
 * deterministic != 0 ([C]): per column, the rows form tiles of R
 *   consecutive rows (R fixed per width) and the tiles are dealt in turn to K
 *   chunks: chunk k holds tiles k, k+K, k+2K, ... K depends only on T*heads
 *   and the width: ceil(tiles/8) when T*heads <= S, otherwise min(tiles,
 *   256), with S = 1280 at width 256, 960 at 512, 640 at 1536 and 2048,
 *   512 at 4096 and 5120, and 384 at 6144 (up to S rows the automatic
 *   path is the single launch). Row q of each of a chunk's tiles,
 *   in ascending tile order, forms sub-chain q, summed with exact products
 *   (dy*x is exact in FP32, times rstd by an FMA-based TwoProduct) and
 *   TwoSum-compensated FP32 accumulation; the R sub-chains merge in order in
 *   FP64; chunk partials fold in FP64 in a fixed two-level order (groups of
 *   32 consecutive chunks, then the groups); one rounding to dw_dtype. The result
 *   is bit-identical for every grid, every path and every device.
 * deterministic == 0 ([D]): same chunks and sub-chains, FP32 block sums of
 *   dy*xhat over 8 rows of a sub-chain flushed into a TwoSum-compensated
 *   pair, FP64 combine. No bitwise guarantee is made for this mode.
 * dw_dtype: RMSN_F32, or RMSN_BF16 for dw in the weight's 16-bit format ([E]
 *   times the gated step both ways; its stepg_f32 is the one with FP32 dw).
 *   In both modes the FP64 value is rounded once, straight to dw_dtype.
 * workspace: at least the bytes rmsnorm_train_bwd_query reports (0 on the
 *   small path; may then be NULL). Its contents on entry do not matter.     */
rmsn_status rmsnorm_train_bwd(const void* dy, const void* x, const void* dh, const void* w,
                              rmsn_dtype w_dtype, const float* rstd, int deterministic,
                              const rmsn_layout* L, void* dx, void* dw, rmsn_dtype dw_dtype,
                              void* workspace, size_t workspace_bytes, const rmsn_launch* launch,
                              void* stream);

/* ------------------------------------------------- backward, no allocation --
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the call
 * rmsnorm_train_bwd makes (same forms, modes, kernels and results, bit for
 * bit), without the workspace arguments. Its workspace is a device array
 * inside the library, 12 MiB per GPU (256 chunks x 6144 columns of FP64, the
 * largest any plan needs), held by each GPU the library runs on until the
 * process ends; a plan needing more would return RMSN_E_WORKSPACE. The call
 * uses the array of the calling thread's current HIP device, so `stream` must
 * belong to that device (a stream of another device: RMSN_E_ARG, nothing
 * enqueued); the first call on a device looks up the array's address there
 * (RMSN_E_HIP if that fails). It calls no allocator.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (nothing in it needs clearing). Calls that can overlap in time on
 * one GPU (unordered streams, several host threads) race on the array and
 * must not be made; calls ordered on one stream are safe.                   */
rmsn_status rmsnorm_train_bwd_noalloc(const void* dy, const void* x, const void* dh,
                                      const void* w, rmsn_dtype w_dtype, const float* rstd,
                                      int deterministic, const rmsn_layout* L, void* dx,
                                      void* dw, rmsn_dtype dw_dtype, const rmsn_launch* launch,
                                      void* stream);

/* Host-only: the plan (path, chunking, grids, workspace bytes) of a backward
 * call with this layout, mode and override. Validates L and the override.   */
rmsn_status rmsnorm_train_bwd_query(const rmsn_layout* L, int deterministic,
                                    const rmsn_launch* launch, rmsn_bwd_plan* plan);

/* ------------------------------------------------------------- SiLU gate --
 * Forward ([E]): y = RMSNorm(x) * w * silu(z) (BF16), rstd (FP32).
 * x and z: BF16 rows in the x strides of L.                                 */
rmsn_status rmsnorm_silu_gate_train_fwd(const void* x, const void* z, const void* w,
                                        rmsn_dtype w_dtype, float eps, const rmsn_layout* L,
                                        void* y, float* rstd, void* stream);

/* Backward ([E]): dx, dz (BF16) and dw (dw_dtype) from dy (g strides), x, z
 * (x strides), the forward's rstd and w. Modes, dw_dtype and workspace as in
 * rmsnorm_train_bwd (the query is shared). In the deterministic mode the
 * per-row term is TwoProduct(dy*x, RN(rstd*silu(z))): one rounding inside it.
 */
rmsn_status rmsnorm_silu_gate_train_bwd(const void* dy, const void* x, const void* z,
                                        const void* w, rmsn_dtype w_dtype, const float* rstd,
                                        int deterministic, const rmsn_layout* L, void* dx,
                                        void* dz, void* dw, rmsn_dtype dw_dtype, void* workspace,
                                        size_t workspace_bytes, const rmsn_launch* launch,
                                        void* stream);

/* Human-readable name of a status code (static string; never NULL). */
const char* rmsn_status_str(rmsn_status s);

#ifdef __cplusplus
}
#endif
#endif /* RMSNORM_TRAIN_H */
