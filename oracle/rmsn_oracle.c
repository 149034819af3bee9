/*
 * rmsn_oracle.c -- plain FP64 CPU oracle for RMSNorm training.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg. It shares no code with the HIP library.
 *
 * Definitions (the pages never print the formula; this is the textbook
 * RMSNorm that their problem statement names -- see rmsn_oracle.h):
 *   rstd   = 1 / sqrt( (1/n) sum_j x_j^2 + eps )          n = row width
 *   xhat_j = x_j * rstd
 *   y_j    = xhat_j * w_j
 *   g_j    = dy_j * w_j                       (gradient reaching xhat)
 *   c      = (1/n) sum_j g_j * xhat_j
 *   dx_j   = rstd * (g_j - xhat_j * c)
 *   dw_j   = sum over rows of dy_j * xhat_j
 * Fused residual (PR #8512 page, description, "Residual rows"; PR #8848 page,
 * "Key": h_new = BF16(h + u), combined grad): h = RNE_bf16(x + res); y and
 * rstd from h; grad_h = dh + dx(h); dw from h.
 * SiLU gate (PR #8656 page, description): s = 1/(1+exp(-z)), silu = z*s,
 *   y_j  = xhat_j * w_j * silu_j,  g_j = dy_j * w_j * silu_j,  dx as above,
 *   dz_j = dy_j * xhat_j * w_j * s_j * (1 + z_j (1 - s_j)),
 *   dw_j = sum over rows of dy_j * xhat_j * silu_j.
 * Every quantity is IEEE double; loops run in ascending index order.
 */
#include "rmsn_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- number formats ------------------------------------------------------ */

double orc_bf16_to_f64(uint16_t b) {
  /* A BF16 value is the upper half of an IEEE binary32 with the same bits. */
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

uint16_t orc_f64_to_bf16(double d) {
  /* BF16: 1 sign bit, 8 exponent bits (bias 127), 7 stored significand bits.
   * Normal values have 8 significant bits; below 2^-126 the spacing stays
   * 2^-133 (subnormals). Round |d| to the nearest multiple of the spacing of
   * its binade, ties to even (nearbyint in the default rounding mode). */
  uint16_t sign = signbit(d) ? 0x8000u : 0u;
  if (isnan(d)) return (uint16_t)(sign | 0x7FC0u);
  double a = fabs(d);
  if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
  if (a == 0.0) return sign;
  int e;
  (void)frexp(a, &e);              /* a = m * 2^e, 0.5 <= m < 1 */
  int lo = e - 1;                  /* 2^lo <= a < 2^(lo+1) */
  if (lo < -126) lo = -126;        /* subnormal range: fixed spacing */
  double n = ldexp(a, 7 - lo);     /* a / spacing, exact; n < 256 */
  double r = nearbyint(n);         /* round half to even */
  double v = ldexp(r, lo - 7);     /* exact */
  if (v >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u); /* overflow */
  float f = (float)v;              /* exact: v is a BF16 value */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7FFFu));
}

void orc_bf16_to_f64_array(const uint16_t* in, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_to_f64(in[i]);
}

void orc_f64_to_bf16_array(const double* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_bf16(in[i]);
}

/* ---- zero-centred weight ------------------------------------------------ */

void orc_zero_centred_weight(int64_t n, const double* w, double* out) {
  /* The stored weight is centred on zero; the norm multiplies by 1 + w. */
  for (int64_t j = 0; j < n; ++j) out[j] = 1.0 + w[j];
}

/* ---- one row ------------------------------------------------------------- */

static double row_rstd(int64_t n, const double* x, double eps) {
  double ss = 0.0;
  for (int64_t j = 0; j < n; ++j) ss += x[j] * x[j];
  return 1.0 / sqrt(ss / (double)n + eps);
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

static void row_fwd(int64_t n, const double* x, const double* w, double eps, double* y,
                    double* rstd) {
  double r = row_rstd(n, x, eps);
  if (y)
    for (int64_t j = 0; j < n; ++j) y[j] = (x[j] * r) * w[j];
  if (rstd) *rstd = r;
}

/* gate == NULL: plain form. dx, dz, dw may each be NULL. dw accumulates. */
static void row_bwd(int64_t n, const double* dy, const double* x, const double* gate,
                    const double* w, double eps, double* dx, double* dz, double* dw) {
  double r = row_rstd(n, x, eps);
  double c = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    double xh = x[j] * r;
    double g = dy[j] * w[j];
    if (gate) g *= gate[j] * sigmoid(gate[j]);
    c += g * xh;
  }
  c /= (double)n;
  for (int64_t j = 0; j < n; ++j) {
    double xh = x[j] * r;
    double g = dy[j] * w[j];
    double s = 1.0, silu = 1.0;
    if (gate) {
      s = sigmoid(gate[j]);
      silu = gate[j] * s;
      g *= silu;
    }
    if (dx) dx[j] = r * (g - xh * c);
    if (dz && gate) dz[j] = dy[j] * xh * w[j] * s * (1.0 + gate[j] * (1.0 - s));
    if (dw) dw[j] += dy[j] * xh * silu;
  }
}

/* ---- dense FP64 entry points -------------------------------------------- */

void orc_rmsnorm_fwd_f64(int64_t rows, int64_t width, const double* x, const double* w,
                         double eps, double* y, double* rstd) {
  for (int64_t i = 0; i < rows; ++i)
    row_fwd(width, x + i * width, w, eps, y ? y + i * width : NULL, rstd ? rstd + i : NULL);
}

void orc_rmsnorm_bwd_f64(int64_t rows, int64_t width, const double* dy, const double* x,
                         const double* w, double eps, double* dx, double* dw) {
  if (dw)
    for (int64_t j = 0; j < width; ++j) dw[j] = 0.0;
  for (int64_t i = 0; i < rows; ++i)
    row_bwd(width, dy + i * width, x + i * width, NULL, w, eps, dx ? dx + i * width : NULL,
            NULL, dw);
}

void orc_gate_fwd_f64(int64_t rows, int64_t width, const double* x, const double* z,
                      const double* w, double eps, double* y, double* rstd) {
  for (int64_t i = 0; i < rows; ++i) {
    const double* xi = x + i * width;
    const double* zi = z + i * width;
    double r = row_rstd(width, xi, eps);
    if (y)
      for (int64_t j = 0; j < width; ++j)
        y[i * width + j] = (xi[j] * r) * w[j] * (zi[j] * sigmoid(zi[j]));
    if (rstd) rstd[i] = r;
  }
}

void orc_gate_bwd_f64(int64_t rows, int64_t width, const double* dy, const double* x,
                      const double* z, const double* w, double eps, double* dx, double* dz,
                      double* dw) {
  if (dw)
    for (int64_t j = 0; j < width; ++j) dw[j] = 0.0;
  for (int64_t i = 0; i < rows; ++i)
    row_bwd(width, dy + i * width, x + i * width, z + i * width, w, eps,
            dx ? dx + i * width : NULL, dz ? dz + i * width : NULL, dw);
}

/* ---- BF16 views ----------------------------------------------------------- */

static int same_shape(const orc_view* a, const orc_view* b) {
  return a->T == b->T && a->heads == b->heads && a->width == b->width;
}

static int view_ok(const orc_view* v) {
  return v && v->p && v->T >= 0 && v->heads >= 1 && v->width >= 1;
}

static void load_row(const orc_view* v, int64_t r, double* out) {
  int64_t t = r / v->heads, h = r % v->heads;
  const uint16_t* p = v->p + t * v->st + h * v->sh;
  for (int64_t j = 0; j < v->width; ++j) out[j] = orc_bf16_to_f64(p[j]);
}

static int sel_ok(const int64_t* sel, int64_t nsel, int64_t rows) {
  if (!sel) return 1;
  for (int64_t i = 0; i < nsel; ++i)
    if (sel[i] < 0 || sel[i] >= rows) return 0;
  return 1;
}

int orc_fwd_bf16(const orc_view* x, const double* w, double eps, const int64_t* sel,
                 int64_t nsel, double* y, double* rstd) {
  if (!view_ok(x) || !w) return -1;
  int64_t rows = x->T * x->heads, n = x->width;
  if (!sel) nsel = rows;
  if (!sel_ok(sel, nsel, rows)) return -1;
  double* xr = malloc(sizeof(double) * (size_t)n);
  if (!xr) return -1;
  for (int64_t i = 0; i < nsel; ++i) {
    load_row(x, sel ? sel[i] : i, xr);
    row_fwd(n, xr, w, eps, y ? y + i * n : NULL, rstd ? rstd + i : NULL);
  }
  free(xr);
  return 0;
}

int orc_res_fwd_bf16(const orc_view* x, const orc_view* res, const double* w, double eps,
                     const int64_t* sel, int64_t nsel, uint16_t* h, double* y, double* rstd) {
  if (!view_ok(x) || !view_ok(res) || !same_shape(x, res) || !w || !h) return -1;
  int64_t rows = x->T * x->heads, n = x->width;
  if (!sel) nsel = rows;
  if (!sel_ok(sel, nsel, rows)) return -1;
  double* a = malloc(sizeof(double) * (size_t)n);
  double* b = malloc(sizeof(double) * (size_t)n);
  if (!a || !b) {
    free(a);
    free(b);
    return -1;
  }
  /* h = RNE_bf16(x + res). Both addends are BF16 values; their double sum is
   * exact unless the exponents differ by more than 44, in which case the
   * smaller addend is far below half a BF16 ulp of the larger and the double
   * sum rounds to the same BF16 value as the exact sum would. */
  for (int64_t r = 0; r < rows; ++r) {
    load_row(x, r, a);
    load_row(res, r, b);
    for (int64_t j = 0; j < n; ++j) h[r * n + j] = orc_f64_to_bf16(a[j] + b[j]);
  }
  for (int64_t i = 0; i < nsel; ++i) {
    int64_t r = sel ? sel[i] : i;
    orc_bf16_to_f64_array(h + r * n, n, a);
    row_fwd(n, a, w, eps, y ? y + i * n : NULL, rstd ? rstd + i : NULL);
  }
  free(a);
  free(b);
  return 0;
}

/* Shared driver for the plain / residual / gated backward over views. */
static int bwd_views(const orc_view* dy, const orc_view* x, const orc_view* dh,
                     const orc_view* z, const double* w, double eps, const int64_t* sel,
                     int64_t nsel, double* dx, double* dz, double* dw) {
  if (!view_ok(dy) || !view_ok(x) || !same_shape(dy, x) || !w) return -1;
  if (dh && (!view_ok(dh) || !same_shape(dh, x))) return -1;
  if (z && (!view_ok(z) || !same_shape(z, x))) return -1;
  int64_t rows = x->T * x->heads, n = x->width;
  if (!sel) nsel = rows;
  if (!sel_ok(sel, nsel, rows)) return -1;
  double* xr = malloc(sizeof(double) * (size_t)n);
  double* gr = malloc(sizeof(double) * (size_t)n);
  double* zr = malloc(sizeof(double) * (size_t)n);
  double* hr = malloc(sizeof(double) * (size_t)n);
  if (!xr || !gr || !zr || !hr) {
    free(xr), free(gr), free(zr), free(hr);
    return -1;
  }
  if (dw) {
    /* dw over every row, ascending row order. */
    for (int64_t j = 0; j < n; ++j) dw[j] = 0.0;
    for (int64_t r = 0; r < rows; ++r) {
      load_row(x, r, xr);
      load_row(dy, r, gr);
      if (z) load_row(z, r, zr);
      row_bwd(n, gr, xr, z ? zr : NULL, w, eps, NULL, NULL, dw);
    }
  }
  if (dx || dz) {
    for (int64_t i = 0; i < nsel; ++i) {
      int64_t r = sel ? sel[i] : i;
      load_row(x, r, xr);
      load_row(dy, r, gr);
      if (z) load_row(z, r, zr);
      double* dxi = dx ? dx + i * n : NULL;
      row_bwd(n, gr, xr, z ? zr : NULL, w, eps, dxi, dz ? dz + i * n : NULL, NULL);
      if (dh && dxi) {
        load_row(dh, r, hr);
        for (int64_t j = 0; j < n; ++j) dxi[j] = hr[j] + dxi[j];
      }
    }
  }
  free(xr), free(gr), free(zr), free(hr);
  return 0;
}

int orc_bwd_bf16(const orc_view* dy, const orc_view* x, const orc_view* dh, const double* w,
                 double eps, const int64_t* sel, int64_t nsel, double* out, double* dw) {
  return bwd_views(dy, x, dh, NULL, w, eps, sel, nsel, out, NULL, dw);
}

int orc_gate_fwd_bf16(const orc_view* x, const orc_view* z, const double* w, double eps,
                      const int64_t* sel, int64_t nsel, double* y, double* rstd) {
  if (!view_ok(x) || !view_ok(z) || !same_shape(x, z) || !w) return -1;
  int64_t rows = x->T * x->heads, n = x->width;
  if (!sel) nsel = rows;
  if (!sel_ok(sel, nsel, rows)) return -1;
  double* xr = malloc(sizeof(double) * (size_t)n);
  double* zr = malloc(sizeof(double) * (size_t)n);
  if (!xr || !zr) {
    free(xr), free(zr);
    return -1;
  }
  for (int64_t i = 0; i < nsel; ++i) {
    int64_t r = sel ? sel[i] : i;
    load_row(x, r, xr);
    load_row(z, r, zr);
    orc_gate_fwd_f64(1, n, xr, zr, w, eps, y ? y + i * n : NULL, rstd ? rstd + i : NULL);
  }
  free(xr), free(zr);
  return 0;
}

int orc_gate_bwd_bf16(const orc_view* dy, const orc_view* x, const orc_view* z,
                      const double* w, double eps, const int64_t* sel, int64_t nsel,
                      double* dx, double* dz, double* dw) {
  if (!z) return -1;
  return bwd_views(dy, x, NULL, z, w, eps, sel, nsel, dx, dz, dw);
}
