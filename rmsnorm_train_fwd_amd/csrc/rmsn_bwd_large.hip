// rmsn_bwd_large.hip -- backward main kernel instances, the fold kernel and
// their launchers.
#include "rmsn_kernels.hpp"

namespace rmsn {

__global__ __launch_bounds__(kBlock) void k_fold(const double* __restrict__ ws,
                                                 float* __restrict__ dw, int H, int64_t chunks) {
  __shared__ double gsum[1024 / kFoldGroup][kColTile];
  const int lane = threadIdx.x % kColTile, wave = threadIdx.x / kColTile;
  constexpr int kWaves = kBlock / kColTile;
  const int64_t groups = (chunks + kFoldGroup - 1) / kFoldGroup;  // <= 32 (chunks <= 1024)
  for (int tile = blockIdx.x; tile < H / kColTile; tile += gridDim.x) {
    const int col = tile * kColTile + lane;
    for (int64_t g = wave; g < groups; g += kWaves) {
      const int64_t k0 = g * kFoldGroup;
      const int64_t k1 = k0 + kFoldGroup < chunks ? k0 + kFoldGroup : chunks;
      double s = 0.0;
      for (int64_t k = k0; k < k1; ++k) s = s + ws[k * H + col];
      gsum[g][lane] = s;
    }
    __syncthreads();
    if (wave == 0) {
      double t = 0.0;
      for (int64_t g = 0; g < groups; ++g) t = t + gsum[g][lane];
      dw[col] = (float)t;
    }
    __syncthreads();
  }
}

namespace {
constexpr int kBwdD = 2;  // rows per row group per batch

template <int H, bool WF32, int FORM>
hipError_t large_mode(bool det, const BwdArgs& a, int grid, hipStream_t s) {
  if (det) k_bwd_large<H, WF32, FORM, true, kBwdD><<<grid, kBlock, 0, s>>>(a);
  else k_bwd_large<H, WF32, FORM, false, kBwdD><<<grid, kBlock, 0, s>>>(a);
  return hipGetLastError();
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
  k_fold<<<grid, kBlock, 0, s>>>(a.ws, a.dw, H, a.chunks);
  return hipGetLastError();
}

}  // namespace rmsn
