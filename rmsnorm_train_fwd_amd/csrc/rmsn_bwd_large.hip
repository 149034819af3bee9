// rmsn_bwd_large.hip -- backward main kernel instances, the fold kernel and
// their launchers.
#include "rmsn_kernels.hpp"

namespace rmsn {

// One workgroup of kFoldThreads threads covers kFoldTile columns: thread
// (g, c) sums group g of column c -- its kFoldGroup chunk partials are all
// loaded first, then added in ascending order from 0.0 -- the group sums meet
// in LDS, and one thread per column adds them in ascending group order from
// 0.0. The host plans at most kMaxChunks chunks, i.e. kFoldGroups groups, so
// one pass holds every group; more would take further passes in order.
__global__ __launch_bounds__(kFoldThreads) void k_fold(const double* __restrict__ ws,
                                                       void* __restrict__ dw, int dw_bf16, int H,
                                                       int64_t chunks) {
  __shared__ double gsum[kFoldGroups][kFoldTile];
  const int c = threadIdx.x % kFoldTile, g = threadIdx.x / kFoldTile;
  const int64_t groups = (chunks + kFoldGroup - 1) / kFoldGroup;
  for (int tile = blockIdx.x; tile < H / kFoldTile; tile += gridDim.x) {
    const int col = tile * kFoldTile + c;
    double t = 0.0;
    for (int64_t g0 = 0; g0 < groups; g0 += kFoldGroups) {
      if (g0 + g < groups) {
        const int64_t k0 = (g0 + g) * kFoldGroup;
        const int n = (int)(chunks - k0 < kFoldGroup ? chunks - k0 : kFoldGroup);
        const double* p = ws + k0 * H + col;
        double v[kFoldGroup];
#pragma unroll
        for (int i = 0; i < kFoldGroup; ++i) v[i] = i < n ? p[(int64_t)i * H] : 0.0;
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < kFoldGroup; ++i)
          if (i < n) s = s + v[i];
        gsum[g][c] = s;
      }
      __syncthreads();
      if (g == 0) {
        for (int j = 0; j < kFoldGroups && g0 + j < groups; ++j) t = t + gsum[j][c];
      }
      __syncthreads();
    }
    if (g == 0) store_dw(dw, dw_bf16, col, t);
  }
}

namespace {
template <int H, bool WF32, int FORM>
hipError_t large_mode(bool det, const BwdArgs& a, int grid, hipStream_t s) {
  constexpr int D = BwdShape<H, FORM>::D;
  if (det) return launch_kernel(k_bwd_large<H, WF32, FORM, true, D>, grid, Geo<H>::BLOCK, s, a);
  return launch_kernel(k_bwd_large<H, WF32, FORM, false, D>, grid, Geo<H>::BLOCK, s, a);
}

template <int H, bool WF32>
hipError_t large_form(int form, bool det, const BwdArgs& a, int grid, hipStream_t s) {
  switch (form) {
    case kPlain: return large_mode<H, WF32, kPlain>(det, a, grid, s);
    case kResidual: return large_mode<H, WF32, kResidual>(det, a, grid, s);
    case kGate: return large_mode<H, WF32, kGate>(det, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int H>
hipError_t large_width(bool w_f32, int form, bool det, const BwdArgs& a, int grid, hipStream_t s) {
  return w_f32 ? large_form<H, true>(form, det, a, grid, s)
               : large_form<H, false>(form, det, a, grid, s);
}
}  // namespace

hipError_t launch_bwd_large(int H, bool w_f32, int form, bool det, const BwdArgs& a, int grid,
                            hipStream_t s) {
  switch (H) {
    case 256: return large_width<256>(w_f32, form, det, a, grid, s);
    case 512: return large_width<512>(w_f32, form, det, a, grid, s);
    case 1536: return large_width<1536>(w_f32, form, det, a, grid, s);
    case 2048: return large_width<2048>(w_f32, form, det, a, grid, s);
    case 4096: return large_width<4096>(w_f32, form, det, a, grid, s);
    case 5120: return large_width<5120>(w_f32, form, det, a, grid, s);
    case 6144: return large_width<6144>(w_f32, form, det, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fold(int H, const BwdArgs& a, int grid, hipStream_t s) {
  return launch_kernel(k_fold, grid, kFoldThreads, s, a.ws, a.dw, a.dw_bf16, H, a.chunks);
}

}  // namespace rmsn
