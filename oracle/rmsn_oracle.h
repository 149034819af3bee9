/*
 * rmsn_oracle.h -- plain FP64 CPU oracle for RMSNorm training (test infrastructure).
 *
 * THIS IS TEST INFRASTRUCTURE. Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it. The HIP library never links,
 * includes or calls anything here, and nothing here includes the HIP library.
 *
 * What it computes (every passage cited is on the pages this project follows):
 *   - Forward: y (BF16 on the GPU) and rstd (FP32 on the GPU). Stated in the
 *     opening paragraph of the PR #8626 merge text (shown on the PR #8512 page)
 *     and in the opening paragraph of the PR #8848 page.
 *   - Backward: dx and the column-reduced weight gradient dw, same passages.
 *   - Fused residual add: forward returns h = x + residual and y = RMSNorm(h);
 *     backward takes the gradients of y and h and returns the gradient of h
 *     and dw (PR #8512 page, description, "Residual rows"). h is the BF16
 *     rounding of the sum ("h_new = BF16(h + u)", PR #8848 page, "Key").
 *   - Per-head views [T, heads, 256] sharing one w[256] (PR #8626 merge text,
 *     "Key"): each (token, head) pair is one row; dw sums over all of them.
 *   - SiLU-gated form y = RMSNorm(x) * w * silu(z) (PR #8656 page, description,
 *     which names the op; the formula itself is the plain reading of the op's
 *     name, with backward outputs dx, dz, dw).
 *
 * The method's own formula is never printed on the pages. The oracle takes the
 * textbook RMSNorm: rstd = 1 / sqrt(sum_j x_j^2 / width + eps), eps inside the
 * root, mean over width, no (1 + w) offset, y_j = x_j * rstd * w_j.
 *   - Zero-centred weight (PR #8512 page, the related-PR title "zero-centred
 *     input RMSNorm", never defined there; read as the RMSNorm whose stored
 *     weight is centred on zero and enters as 1 + w): every form above with
 *     the effective weight 1 + w (orc_zero_centred_weight). The gradient with
 *     respect to the stored w equals that with respect to 1 + w, so dw is the
 *     same sum.
 *
 * Everything is computed in IEEE double from inputs converted exactly to double.
 * No blocking, fusion or reordering: rows in ascending order, columns in
 * ascending order, dw summed over rows in ascending row order.
 *
 * Pins (tests that tie this oracle to facts other than itself): closed-form
 * special rows, complex-step and central finite-difference derivatives of the
 * forward, the scale-invariance identity sum_j dx_j x_j = eps rstd^3 sum_j g_j x_j,
 * exact (fsum) summation checks for dw, BF16 rounding against the IEEE
 * round-to-nearest-even definition and torch's CPU cast.
 */
#ifndef RMSN_ORACLE_H
#define RMSN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A strided BF16 view: element (t, h, j) sits at p[t*st + h*sh + j]. */
typedef struct {
  const uint16_t* p;
  int64_t T, heads, width, st, sh;
} orc_view;

/* ---- number formats ------------------------------------------------------ */
double orc_bf16_to_f64(uint16_t b);        /* exact */
uint16_t orc_f64_to_bf16(double d);        /* round to nearest, ties to even */
void orc_bf16_to_f64_array(const uint16_t* in, int64_t n, double* out);
void orc_f64_to_bf16_array(const double* in, int64_t n, uint16_t* out);

/* Effective weight of the zero-centred form: out[j] = 1 + w[j] (in double). */
void orc_zero_centred_weight(int64_t n, const double* w, double* out);

/* ---- dense FP64 rows: x is [rows, width] row-major ------------------------ */
void orc_rmsnorm_fwd_f64(int64_t rows, int64_t width, const double* x, const double* w,
                         double eps, double* y, double* rstd);
/* dx may be NULL; dw (length width) may be NULL. */
void orc_rmsnorm_bwd_f64(int64_t rows, int64_t width, const double* dy, const double* x,
                         const double* w, double eps, double* dx, double* dw);
void orc_gate_fwd_f64(int64_t rows, int64_t width, const double* x, const double* z,
                      const double* w, double eps, double* y, double* rstd);
void orc_gate_bwd_f64(int64_t rows, int64_t width, const double* dy, const double* x,
                      const double* z, const double* w, double eps, double* dx, double* dz,
                      double* dw);

/* ---- BF16 views (the layouts the library accepts) ------------------------ *
 * Rows are numbered r = t*heads + h. `sel` lists the rows whose row outputs
 * (y, rstd, dx, dz) are wanted, in the order given (nsel entries); sel == NULL
 * means all rows in order. Row outputs are dense [nsel, width] / [nsel].
 * dw, when non-NULL, is always the sum over ALL rows. w is given in double
 * (converted exactly from its BF16 or FP32 storage by the caller).
 * Return 0 on success, -1 on a bad argument (row index out of range, shape
 * mismatch between views).                                                   */
int orc_fwd_bf16(const orc_view* x, const double* w, double eps, const int64_t* sel,
                 int64_t nsel, double* y, double* rstd);
/* Fused residual forward: h = RNE_bf16(x + res) for every row (dense output,
 * [rows, width] BF16 bits), then the forward on h for the selected rows.     */
int orc_res_fwd_bf16(const orc_view* x, const orc_view* res, const double* w, double eps,
                     const int64_t* sel, int64_t nsel, uint16_t* h, double* y, double* rstd);
/* Backward. dh == NULL for the plain form; otherwise out = dh + dx (the
 * gradient of h in the fused residual form), and x is the BF16 h.            */
int orc_bwd_bf16(const orc_view* dy, const orc_view* x, const orc_view* dh, const double* w,
                 double eps, const int64_t* sel, int64_t nsel, double* out, double* dw);
int orc_gate_fwd_bf16(const orc_view* x, const orc_view* z, const double* w, double eps,
                      const int64_t* sel, int64_t nsel, double* y, double* rstd);
int orc_gate_bwd_bf16(const orc_view* dy, const orc_view* x, const orc_view* z,
                      const double* w, double eps, const int64_t* sel, int64_t nsel,
                      double* dx, double* dz, double* dw);

#ifdef __cplusplus
}
#endif
#endif
