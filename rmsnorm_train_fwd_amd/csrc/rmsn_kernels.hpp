// rmsn_kernels.hpp -- the gfx950 kernels of RMSNorm training.
//
//   k_fwd        forward: y, rstd (+ h for the fused residual, silu gate)
//   k_bwd_large  backward main kernel: dx (+dz) and FP64 dw chunk partials
//   k_fold       fixed-order FP64 fold of the chunk partials -> dw (FP32 or BF16)
//   k_bwd_small  single-launch backward for small row counts: row tasks for
//                dx, column tasks for dw over all rows, no workspace
//
// What they compute is stated in include/rmsnorm_train.h. The rows are
// streamed once from HBM with 16-byte loads; every thread keeps the weight
// slice it needs in registers for its whole lifetime.
#pragma once

#include <tuple>

#include "rmsn_device.hpp"
#include "rmsn_launch.hpp"

namespace rmsn {

// Enqueues k<<<grid, block, 0, s>>>(a...) through hipLaunchKernel and returns
// that launch's own status. A triple-chevron launch reports only through the
// thread's last-error state, which can hold an earlier, unrelated error (and
// reading it with hipGetLastError would clear it for the caller), so the
// library never reads or clears that state. Each argument is converted to the
// kernel's parameter type before its address is passed.
template <class... P, class... A>
hipError_t launch_kernel(void (*k)(P...), int grid, int block, hipStream_t s, A... a) {
  static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
  std::tuple<P...> v(a...);
  return std::apply(
      [&](P&... p) {
        void* args[] = {static_cast<void*>(&p)...};
        return hipLaunchKernel(reinterpret_cast<const void*>(k), dim3(grid), dim3(block), args,
                               0, s);
      },
      v);
}

__device__ __forceinline__ int64_t row_off(const RowIn& in, int64_t row, int heads) {
  const uint32_t t = (uint32_t)row / (uint32_t)heads;
  const uint32_t h = (uint32_t)row - t * (uint32_t)heads;
  return (int64_t)t * in.stride_t + (int64_t)h * in.stride_h;
}

// Forward shape per width and form. The forward has no dw tree to follow, so
// its row groups per workgroup are chosen on their own: one at 4096 and two at
// 1536 and 2048 (the backward has two, four and four), which measured faster
// than the backward's shape (e.g. the gated forward at [3534, 4096] 16.3 ->
// 14.4 us, the plain one at [131072, 1536] 129 -> 124 us, cold caches); the
// plain form at 6144 takes two 384-thread row groups of 16 columns per thread
// ([131072, 6144] 558 -> 528 us; its residual and gated forms were slower
// that way and keep one 768-thread row group). Other widths take the
// backward's shape, except the gated form at 5120, which keeps one 640-thread
// row group (8 columns per thread) where the other forms use two 320-thread
// row groups.
template <int H, int FORM> struct FwdCfg : Cfg<H> {};
template <int FORM> struct FwdCfg<4096, FORM> {
  static constexpr int TPR = 512, V = 1, R = 1, D = 1;
  static constexpr bool PIPE = true;
};
template <int FORM> struct FwdCfg<2048, FORM> {
  static constexpr int TPR = 256, V = 1, R = 2, D = 1;
  static constexpr bool PIPE = true;
};
template <int FORM> struct FwdCfg<1536, FORM> {
  static constexpr int TPR = 192, V = 1, R = 2, D = 1;
  static constexpr bool PIPE = true;
};
template <> struct FwdCfg<6144, kPlain> {
  static constexpr int TPR = 384, V = 2, R = 2, D = 1;
  static constexpr bool PIPE = true;
};
template <> struct FwdCfg<5120, kGate> {
  static constexpr int TPR = 640, V = 1, R = 1, D = 1;
  static constexpr bool PIPE = true;
};
template <int H, int FORM> using FGeo = GeoOf<H, FwdCfg<H, FORM>>;

// ------------------------------------------------------------------ forward --
//
// Per row: ss = sum x^2 (FP32, per-thread FMA chain, then the row-group sum),
// rstd = 1/sqrt(ss/H + eps) with IEEE sqrt and division, y = bf16((x*rstd)*w)
// [* silu(z)]. Residual: h = bf16(x + res) (FP32 sum of two BF16 values,
// rounded once; the FP32 sum can only be inexact when the addends' exponents
// differ by more than 16, and then the smaller one is far below half a BF16
// ulp, so the result is the rounded exact sum), and the norm reads that h.
template <int H, bool WF32, int FORM, int RPG>
__global__ __launch_bounds__((FGeo<H, FORM>::BLOCK)) void k_fwd(FwdArgs a) {
  using G = FGeo<H, FORM>;
  constexpr int R = G::R, V = G::V, E = G::E;
  const int q = row_group<G>(), lane = threadIdx.x % G::TPR;
  __shared__ float slots[RowSum<G, RPG>::kSlots];
  int parity = 0;
  float wr[E];
  load_w<G, WF32>(a.w, lane, wr, a.w_one);

  const int64_t tiles = (a.rows + R * RPG - 1) / (R * RPG);
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    int64_t row[RPG];
    bool ok[RPG];
    uint4 xv[RPG][V], ev[RPG][V];
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      row[i] = tile * (R * RPG) + i * R + q;
      ok[i] = row[i] < a.rows;
      const int64_t xo = ok[i] ? row_off(a.x, row[i], a.heads) : 0;
      const int64_t eo = ok[i] && FORM != kPlain ? row_off(a.e, row[i], a.heads) : 0;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        xv[i][v] = ok[i] ? ld16_stream(a.x.p + xo + elem0<G>(v, lane)) : make_uint4(0, 0, 0, 0);
        if constexpr (FORM != kPlain)
          ev[i][v] = ok[i] ? ld16_stream(a.e.p + eo + elem0<G>(v, lane)) : make_uint4(0, 0, 0, 0);
      }
    }
    float xf[RPG][E];
    float ss[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float f[8];
        unpack8(xv[i][v], f);
        if constexpr (FORM == kResidual) {
          float r8[8];
          unpack8(ev[i][v], r8);
#pragma unroll
          for (int k = 0; k < 8; ++k) f[k] = f[k] + r8[k];
          const uint4 hb = pack8(f);
          if (ok[i]) st16_stream(a.h + row[i] * H + elem0<G>(v, lane), hb);
          unpack8(hb, f);  // the norm reads the rounded h
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) xf[i][v * 8 + k] = f[k];
      }
      float s = 0.0f;
#pragma unroll
      for (int k = 0; k < E; ++k) s = __builtin_fmaf(xf[i][k], xf[i][k], s);
      ss[i] = s;
    }
    RowSum<G, RPG>::run(ss, slots, parity, q, lane);
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const float r = 1.0f / __builtin_sqrtf(ss[i] / (float)H + a.eps);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float f[8];
        float zf[8];
        if constexpr (FORM == kGate) unpack8(ev[i][v], zf);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          float t = (xf[i][v * 8 + k] * r) * wr[v * 8 + k];
          if constexpr (FORM == kGate) t = t * (zf[k] * sigmoid_f(zf[k]));
          f[k] = t;
        }
        if (ok[i]) st16_stream(a.y + row[i] * H + elem0<G>(v, lane), pack8(f));
      }
      if (ok[i] && lane == 0) a.rstd[row[i]] = r;
    }
  }
}

// ----------------------------------------------------------------- backward --
//
// One batch of D rows of one row group: loads, the rows' dw terms into the
// caller's accumulators, the row sum c = sum g*xhat, dx = rstd*(g - xhat*c/H)
// (+dh), dz for the gate, stores. The arithmetic of a row does not depend on
// D or on the kernel calling it, so dx has the same bits on every path.
struct NoDw {};  // accumulator policy of row tasks that only write dx

template <int H, int FORM, int D>
struct RowBatch {
  using G = Geo<H>;
  static constexpr int V = G::V, E = G::E;
  uint4 xv[D][V], gv[D][V], ev[D][V];
  float r[D];

  __device__ __forceinline__ void load(const BwdArgs& a, const int64_t (&row)[D],
                                       const bool (&ok)[D], int lane) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      // Masked entries (ok[d] false) carry a valid row index chosen by the
      // caller: they load real data, which is then ignored (no branches
      // around the loads, so they issue back to back).
      (void)ok;
      const int64_t xo = row_off(a.x, row[d], a.heads);
      const int64_t go = row_off(a.dy, row[d], a.heads);
      const int64_t eo = FORM != kPlain ? row_off(a.e, row[d], a.heads) : 0;
      r[d] = a.rstd[row[d]];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int e0 = elem0<G>(v, lane);
        xv[d][v] = ld16_stream(a.x.p + xo + e0);
        gv[d][v] = ld16_stream(a.dy.p + go + e0);
        if constexpr (FORM != kPlain) ev[d][v] = ld16_stream(a.e.p + eo + e0);
      }
    }
  }

  // Make the loaded words look redefined to the compiler, so that values
  // unpacked from them before this point are not kept live across it
  // (re-unpacking is two VALU ops per element; keeping them live would cost
  // 2-4 VGPRs per element and halve the waves in flight).
  __device__ __forceinline__ void opaque() {
#pragma unroll
    for (int d = 0; d < D; ++d) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        asm volatile("" : "+v"(xv[d][v].x), "+v"(xv[d][v].y), "+v"(xv[d][v].z), "+v"(xv[d][v].w));
        if constexpr (FORM != kGate)  // the gate's pass 2 reads x only
          asm volatile("" : "+v"(gv[d][v].x), "+v"(gv[d][v].y), "+v"(gv[d][v].z), "+v"(gv[d][v].w));
        if constexpr (FORM == kResidual)
          asm volatile("" : "+v"(ev[d][v].x), "+v"(ev[d][v].y), "+v"(ev[d][v].z), "+v"(ev[d][v].w));
      }
    }
  }

  // Pass 1 (per row): the row sum c = sum g*xhat, and the row's dw terms into
  // acc (they do not depend on c, so they are taken while x and dy are
  // unpacked anyway); the gate's dz, which does not depend on c either, is
  // computed and stored here too. Row sum across the row group. Pass 2: dx,
  // stores.
  // Acc is Dot2 (deterministic: exact dy*x times rstd, or RN(rstd*silu) for
  // the gate), Block8 (dy times xhat [* silu]) or NoDw (dx only).
  template <bool WF32, class Acc>
  __device__ __forceinline__ void compute_store(const BwdArgs& a, const float (&wr)[E],
                                                const int64_t (&row)[D], const bool (&ok)[D],
                                                int q, int lane, float* slots, int& parity,
                                                Acc* acc, bool sync = false) {
    float dot[D];
    // Gate: g*silu(z) per element, kept from pass 1 for dx in pass 2, so that
    // pass 2 reads x only and the sigmoid is taken once per element (one FP32
    // register per element instead of re-unpacking dy and z and a second
    // exp2 and reciprocal: the gated backward is close to the VALU limit).
    float gsl[FORM == kGate ? D : 1][FORM == kGate ? E : 1];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      float xf[E], gf[E], sl[E], sg[E], zz[E];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float t[8];
        unpack8(xv[d][v], t);
#pragma unroll
        for (int k = 0; k < 8; ++k) xf[v * 8 + k] = t[k];
        unpack8(gv[d][v], t);
#pragma unroll
        for (int k = 0; k < 8; ++k) gf[v * 8 + k] = t[k];
        if constexpr (FORM == kGate) {
          unpack8(ev[d][v], t);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            zz[v * 8 + k] = t[k];
            sg[v * 8 + k] = sigmoid_f(t[k]);
            sl[v * 8 + k] = t[k] * sg[v * 8 + k];
          }
        }
      }
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float g = gf[e] * wr[e];
        if constexpr (FORM == kGate) {
          g = g * sl[e];
          gsl[d][e] = g;
        }
        s = __builtin_fmaf(g, xf[e] * r[d], s);
      }
      dot[d] = s;
      if constexpr (FORM == kGate) {
#pragma unroll
        for (int v = 0; v < V; ++v) {
          float dz[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int e = v * 8 + k;
            const float xh = xf[e] * r[d];
            dz[k] = ((gf[e] * xh) * wr[e]) * (sg[e] * (1.0f + zz[e] * (1.0f - sg[e])));
          }
          // unconditional, as the dx stores below
          st16_stream(a.dz + row[d] * H + elem0<G>(v, lane), pack8(dz));
        }
      }
      if constexpr (!__is_same(Acc, NoDw)) {
        if (ok[d]) {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            if constexpr (__is_same(Acc, Dot2)) {
              float b = r[d];
              if constexpr (FORM == kGate) b = r[d] * sl[e];
              acc[e].add(gf[e] * xf[e], b);
            } else {
              float b = xf[e] * r[d];
              if constexpr (FORM == kGate) b = b * sl[e];
              acc[e].add(gf[e], b);
            }
          }
        }
      }
    }
    RowSum<G, D>::run(dot, slots, parity, q, lane);
    // Width 256 (half-wave row groups) has no barrier in its row sum; a
    // workgroup barrier here keeps the workgroup's waves on the same tiles:
    // measured 4-8% faster in the non-deterministic mode at large row counts,
    // and in the deterministic mode on long chunks only (`sync`: 5-7% faster
    // from 128 batches per chunk, slower on short ones).
    if constexpr (__is_same(Acc, Block8) && G::LANES == 32) __syncthreads();
    if constexpr (__is_same(Acc, Dot2) && G::LANES == 32) {
      if (sync) __syncthreads();  // uniform: one value per workgroup
    }
    opaque();
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const float c = dot[d] / (float)H;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float xf[8], gf[8], zf[8], out[8];
        unpack8(xv[d][v], xf);
        if constexpr (FORM != kGate) unpack8(gv[d][v], gf);
        if constexpr (FORM == kResidual) unpack8(ev[d][v], zf);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float xh = xf[k] * r[d];
          float g;
          if constexpr (FORM == kGate) g = gsl[d][v * 8 + k];
          else g = gf[k] * wr[v * 8 + k];
          float dx = r[d] * __builtin_fmaf(-xh, c, g);
          if constexpr (FORM == kResidual) dx = zf[k] + dx;  // grad_h = dh + dx
          out[k] = dx;
        }
        // Unconditional: a masked entry holds a copy of a real row of the
        // same call (its index was clamped to that row), so it stores the very
        // bytes that row's own pass stores; no branch around the stores.
        st16_stream(a.dx + row[d] * H + elem0<G>(v, lane), pack8(out));
      }
    }
  }
};

// Batch shape of the backward main kernel for one form: the width's default
// (D rows per batch, pipelined), except that (a) with two vectors per thread
// (V = 2) the residual and gated forms, which also carry dh or z, take one row
// per batch without the second buffer, which would not fit in registers; and
// (b) the residual form at 6144 takes a 2-row burst, measured faster there
// than the plain form's pipelined single row (and than 1-, 4-row bursts or
// 2 rows pipelined).
template <int H, int FORM>
struct BwdShape {
  static constexpr bool kWide = FORM != kPlain && Geo<H>::V > 1;
  static constexpr int D = kWide ? 1 : Geo<H>::D;
  static constexpr bool PIPE = kWide ? false : Geo<H>::PIPE;
};
template <>
struct BwdShape<6144, kResidual> {
  static constexpr int D = 2;
  static constexpr bool PIPE = false;
};

// Backward main kernel. Workgroup-strided over the chunks of the dw tree. The
// rows form tiles of R consecutive rows and chunk k holds the tiles k, k + K,
// k + 2K, ... (K = a.chunks), so the workgroups in flight together stream one
// contiguous window of each tensor. Row group q takes row q of each of the
// chunk's tiles in ascending order, D tiles per batch, accumulating sub-chain
// q; the R sub-chains merge in order through LDS in FP64 and the chunk partial
// goes to ws[k][:].
template <int H, bool WF32, int FORM, bool DET, int D>
__global__ __launch_bounds__(Geo<H>::BLOCK) void k_bwd_large(BwdArgs a) {
  using G = Geo<H>;
  constexpr int R = G::R, V = G::V, E = G::E, TPR = G::TPR;
  static_assert(8 % D == 0, "a batch must not straddle a flush of the 8-row blocks");
  const int q = row_group<G>(), lane = threadIdx.x % TPR;
  __shared__ float slots[RowSum<G, D>::kSlots];
  // R >= 4: every sub-chain's values at once, [R][H]; R == 2: a running sum, [H].
  __shared__ double merge[R >= 4 ? R * H : (R > 1 ? H : 1)];
  int parity = 0;
  float wr[E];
  load_w<G, WF32>(a.w, lane, wr, a.w_one);
  const int64_t K = a.chunks, tiles = (a.rows + R - 1) / R;

  for (int64_t k = blockIdx.x; k < K; k += gridDim.x) {
    // The chunk's tiles k, k + K, ... below `tiles`, D per batch. The host
    // plans K <= tiles, so every chunk has at least one tile and r0 (row 0 of
    // its first tile) is a real row; a chunk without tiles would contribute
    // zeros, which is what it writes.
    const int nb = k < tiles ? (int)(((tiles - k + K - 1) / K + D - 1) / D) : 0;
    const int64_t r0 = k * R;
    Dot2 dacc[DET ? E : 1];
    Block8 bacc[DET ? 1 : E];
    // Rows of batch b for this row group: (k + (b*D + d)*K)*R + q, d < D.
    // Rows past the end are masked and clamped to r0.
    auto rows_of = [&](int b, int64_t (&row)[D], bool (&ok)[D]) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int64_t rr = (k + (int64_t)(b * D + d) * K) * R + q;
        ok[d] = rr < a.rows;
        row[d] = ok[d] ? rr : r0;
      }
    };
    auto process = [&](RowBatch<H, FORM, D>& rb, int b) {
      int64_t row[D];
      bool ok[D];
      rows_of(b, row, ok);
      if constexpr (DET)
        rb.template compute_store<WF32>(a, wr, row, ok, q, lane, slots, parity, dacc, nb >= 128);
      else rb.template compute_store<WF32>(a, wr, row, ok, q, lane, slots, parity, bacc);
      if constexpr (!DET) {
        if (((b + 1) * D) % 8 == 0) {
#pragma unroll
          for (int e = 0; e < E; ++e) bacc[e].flush();
        }
        // Width 512 (one-wave row groups, no barrier in the row sum): one
        // barrier per batch here, measured 5% faster in this mode.
        if constexpr (G::WPR == 1 && G::LANES == 64) __syncthreads();
      }
    };
    auto load = [&](RowBatch<H, FORM, D>& rb, int b) {
      int64_t row[D];
      bool ok[D];
      rows_of(b, row, ok);
      rb.load(a, row, ok, lane);
    };
    // Two batch buffers in turn: the loads of batch b+1 are in flight while
    // batch b is reduced, written and accumulated. The steady-state loop
    // issues its loads unconditionally (a load under a branch would make the
    // compiler drain every outstanding load at the join); the last one or
    // two batches are peeled.
    if (nb == 0) {
      // no tiles (not planned by the host): nothing to process
    } else if constexpr (BwdShape<H, FORM>::PIPE) {
      RowBatch<H, FORM, D> ba, bb;
      load(ba, 0);
      int b = 0;
      for (; b + 2 < nb; b += 2) {
        load(bb, b + 1);
        process(ba, b);
        load(ba, b + 2);
        process(bb, b + 1);
      }
      if (b + 1 < nb) {
        load(bb, b + 1);
        process(ba, b);
        process(bb, b + 1);
      } else {
        process(ba, b);
      }
    } else {
      // one buffer: a batch of D rows per row group loads as one burst
      for (int b = 0; b < nb; ++b) {
        RowBatch<H, FORM, D> ba;
        load(ba, b);
        process(ba, b);
      }
    }
    double dv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if constexpr (DET) {
        dv[e] = dacc[e].value();
      } else {
        bacc[e].flush();
        dv[e] = bacc[e].value();
      }
    }
    double* out = a.ws + k * H;
    if constexpr (R == 1) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        double2* o = reinterpret_cast<double2*>(out + elem0<G>(v, lane));
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = make_double2(0.0 + dv[v * 8 + 2 * i], 0.0 + dv[v * 8 + 2 * i + 1]);
      }
    } else if constexpr (R >= 4) {
      // p = 0.0 + d_0 + d_1 + ... + d_{R-1}, in row-group order, one thread
      // per column after a single barrier.
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int i = 0; i < 8; ++i) merge[q * H + elem0<G>(v, lane) + i] = dv[v * 8 + i];
      __syncthreads();
      for (int i = threadIdx.x; i < H; i += G::BLOCK) {
        double p = 0.0;
        for (int qq = 0; qq < R; ++qq) p = p + merge[qq * H + i];
        out[i] = p;
      }
      __syncthreads();
    } else {
      // p = 0.0 + d_0 + d_1 + ... + d_{R-1}, in row-group order.
      for (int qq = 0; qq < R; ++qq) {
        if (q == qq) {
#pragma unroll
          for (int v = 0; v < V; ++v)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              double& m = merge[elem0<G>(v, lane) + i];
              m = (qq == 0 ? 0.0 : m) + dv[v * 8 + i];
            }
        }
        __syncthreads();
      }
      for (int i = threadIdx.x; i < H; i += G::BLOCK) out[i] = merge[i];
      __syncthreads();
    }
  }
}

// dw[j] from its FP64 value, rounded once to the output dtype.
__device__ __forceinline__ void store_dw(void* dw, int bf16, int j, double v) {
  if (bf16) static_cast<u16*>(dw)[j] = f64_to_bf16(v);
  else static_cast<float*>(dw)[j] = (float)v;
}

// Fold: dw[j] = RN( sum_g ( sum_{k in group g} ws[k][j] ) ), both sums in
// ascending order from 0.0, groups of kFoldGroup consecutive chunks, one
// rounding to FP32 or BF16 (defined in rmsn_bwd_large.hip).
__global__ __launch_bounds__(kFoldThreads) void k_fold(const double* __restrict__ ws,
                                                       void* __restrict__ dw, int dw_bf16, int H,
                                                       int64_t chunks);

// 2 or 4 BF16 values loaded as one 4- or 8-byte word.
template <int N> struct VecOf;
template <> struct VecOf<2> {
  typedef uint32_t T;
  __device__ static void unpack(T u, float (&f)[2]) { f[0] = bf_lo(u); f[1] = bf_hi(u); }
};
template <> struct VecOf<4> {
  typedef uint2 T;
  __device__ static void unpack(T u, float (&f)[4]) {
    f[0] = bf_lo(u.x); f[1] = bf_hi(u.x); f[2] = bf_lo(u.y); f[3] = bf_hi(u.y);
  }
};

// Small-path shape. Workgroup size: the main kernel's, capped at 512 threads
// (a row task needs whole row groups; the dw tree only needs the sub-chain
// count R, which stays that of the main kernel). CPT: columns per column-task
// thread; the dw work of a call is (chunks x R x width / CPT) threads, so a
// narrower slice per thread spreads it over more workgroups (2 at widths up
// to 512, 4 above; 8 measured slower everywhere).
template <int H>
struct SmallGeo {
  static constexpr int CPT = H <= 512 ? 2 : 4;
  static constexpr int BLOCK = Geo<H>::BLOCK > 768 ? 512 : Geo<H>::BLOCK;
  static constexpr int RS = BLOCK / Geo<H>::TPR;  // rows per row-task tile
  static_assert(RS >= 1 && RS * Geo<H>::TPR == BLOCK, "row tasks hold whole row groups");
};

// Small-row backward in one launch. The first col_grid workgroups are column
// tasks (dw), strided over column tiles, and are dispatched first because
// they are the longer tasks; the last row_grid workgroups are row tasks (dx,
// strided over row tiles of RS rows). A column-task thread (cv, q, kl) owns
// CPT columns, sub-chain q of chunk kl of the current fold group: it loads
// row q of the chunk's tiles 8 tiles at a time (one memory round trip; the
// tree gives a chunk at most 8 tiles when the row count is small) and runs
// Dot2 over them in ascending order, exactly as k_bwd_large does. Through
// LDS, the chunk partial is then 0.0 + d_0 + ... + d_{R-1} in sub-chain
// order, and the fold follows k_fold's order. rstd is an input, so dw needs
// nothing from the row tasks and no workgroup ever waits for another.
template <int H, bool WF32, int FORM>
__global__ __launch_bounds__(SmallGeo<H>::BLOCK) void k_bwd_small(BwdArgs a, int row_grid) {
  using G = Geo<H>;
  constexpr int R = G::R, TPR = G::TPR, BLOCK = SmallGeo<H>::BLOCK, RS = SmallGeo<H>::RS;
  constexpr int KL = kFoldGroup;               // chunk lanes: one pass = one fold group
  constexpr int CV = BLOCK / (KL * R);         // column vectors per tile
  constexpr int CPT = SmallGeo<H>::CPT;        // columns per thread
  constexpr int kTile = CV * CPT;              // columns per tile
  static_assert(CV >= 1 && CV * KL * R == BLOCK, "column-task layout");
  static_assert(H % kTile == 0, "column tiles must cover the row exactly");
  __shared__ float slots[RowSum<G, 1>::kSlots];
  __shared__ double part[KL][R][kTile];
  const int col_grid = gridDim.x - row_grid;
  if ((int)blockIdx.x >= col_grid) {
    const int q = row_group<G>(), lane = threadIdx.x % TPR;
    int parity = 0;
    float wr[G::E];
    load_w<G, WF32>(a.w, lane, wr, a.w_one);
    const int64_t tiles = (a.rows + RS - 1) / RS;
    for (int64_t t = blockIdx.x - col_grid; t < tiles; t += row_grid) {
      bool ok[1] = {t * RS + q < a.rows};
      int64_t row[1] = {ok[0] ? t * RS + q : t * RS};
      RowBatch<H, FORM, 1> rb;
      rb.load(a, row, ok, lane);
      rb.template compute_store<WF32>(a, wr, row, ok, q, lane, slots, parity, (NoDw*)nullptr);
    }
    return;
  }
  const int cv = threadIdx.x % CV;
  const int q = (threadIdx.x / CV) % R;
  const int kl = threadIdx.x / (CV * R);
  const int64_t K = a.chunks;
  const int64_t groups = (K + KL - 1) / KL;
  for (int tile = blockIdx.x; tile < H / kTile; tile += col_grid) {
    const int c0 = tile * kTile + cv * CPT;
    double total = 0.0;  // column c0 + kl, on threads (cv, q = 0, kl < CPT)
    for (int64_t g = 0; g < groups; ++g) {
      const int64_t k = g * KL + kl;
      if (k < K) {
        // Row q of the chunk's tiles: rb + i*step; rb - q is row 0 of the
        // current tile, which exists while it is below the row count. Masked
        // rows load r0 (row 0 of the chunk's first tile, a real row whenever
        // the loop runs) and are skipped.
        const int64_t r0 = k * R;
        const int64_t step = K * R;
        Dot2 acc[CPT];
        constexpr int NB = 8;  // tiles per round trip
        for (int64_t rb = r0 + q; rb - q < a.rows; rb += NB * step) {
          using VT = typename VecOf<CPT>::T;
          VT xv[NB], gv[NB], zv[NB];
          float rr[NB];
          bool ok[NB];
#pragma unroll
          for (int i = 0; i < NB; ++i) {
            const int64_t row = rb + i * step;
            ok[i] = row < a.rows;
            const int64_t rc = ok[i] ? row : r0;
            rr[i] = a.rstd[rc];
            xv[i] = *reinterpret_cast<const VT*>(a.x.p + row_off(a.x, rc, a.heads) + c0);
            gv[i] = *reinterpret_cast<const VT*>(a.dy.p + row_off(a.dy, rc, a.heads) + c0);
            if constexpr (FORM == kGate)
              zv[i] = *reinterpret_cast<const VT*>(a.e.p + row_off(a.e, rc, a.heads) + c0);
          }
#pragma unroll
          for (int i = 0; i < NB; ++i) {
            if (!ok[i]) continue;
            float xf[CPT], gf[CPT], zf[CPT];
            VecOf<CPT>::unpack(xv[i], xf);
            VecOf<CPT>::unpack(gv[i], gf);
            if constexpr (FORM == kGate) VecOf<CPT>::unpack(zv[i], zf);
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
              float b = rr[i];
              if constexpr (FORM == kGate) b = rr[i] * (zf[e] * sigmoid_f(zf[e]));
              acc[e].add(gf[e] * xf[e], b);
            }
          }
        }
#pragma unroll
        for (int e = 0; e < CPT; ++e) part[kl][q][cv * CPT + e] = acc[e].value();
      }
      __syncthreads();
      if (q == 0 && k < K) {
        // chunk partial: 0.0 + d_0 + d_1 + ... in sub-chain order
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
          double p = 0.0;
          for (int qq = 0; qq < R; ++qq) p = p + part[kl][qq][cv * CPT + e];
          part[kl][0][cv * CPT + e] = p;
        }
      }
      __syncthreads();
      // Group fold, one thread per column (thread (cv, 0, kl) takes column
      // c0 + kl): the group's chunk partials in ascending order from 0.0,
      // read from LDS 8 at a time ahead of the adds.
      if (q == 0 && kl < CPT) {
        const int n = (int)(K - g * KL < KL ? K - g * KL : KL);
        double s = 0.0;
        for (int k0 = 0; k0 < n; k0 += 8) {
          double v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = k0 + i < n ? part[k0 + i][0][cv * CPT + kl] : 0.0;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (k0 + i < n) s = s + v[i];
        }
        total = total + s;
      }
      __syncthreads();
    }
    if (q == 0 && kl < CPT) store_dw(a.dw, a.dw_bf16, c0 + kl, total);
  }
}

}  // namespace rmsn
