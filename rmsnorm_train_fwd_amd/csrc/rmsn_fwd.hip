// rmsn_fwd.hip -- forward kernel instances and their launcher.
#include "rmsn_kernels.hpp"

namespace rmsn {

namespace {
constexpr int kFwdRPG = 2;  // rows per row group per tile

template <int H, bool WF32>
hipError_t fwd_form(int form, const FwdArgs& a, int grid, hipStream_t s) {
  switch (form) {
    case kPlain:
      return launch_kernel(k_fwd<H, WF32, kPlain, kFwdRPG>, grid, FGeo<H, kPlain>::BLOCK, s, a);
    case kResidual:
      return launch_kernel(k_fwd<H, WF32, kResidual, kFwdRPG>, grid, FGeo<H, kResidual>::BLOCK, s,
                           a);
    case kGate:
      return launch_kernel(k_fwd<H, WF32, kGate, kFwdRPG>, grid, FGeo<H, kGate>::BLOCK, s, a);
    default: return hipErrorInvalidValue;
  }
}

template <int H>
hipError_t fwd_width(bool w_f32, int form, const FwdArgs& a, int grid, hipStream_t s) {
  return w_f32 ? fwd_form<H, true>(form, a, grid, s) : fwd_form<H, false>(form, a, grid, s);
}
}  // namespace

template <int H>
int fwd_rows_per_tile_w(int form) {
  switch (form) {
    case kPlain: return FGeo<H, kPlain>::R * kFwdRPG;
    case kResidual: return FGeo<H, kResidual>::R * kFwdRPG;
    case kGate: return FGeo<H, kGate>::R * kFwdRPG;
    default: return 0;
  }
}

int fwd_rows_per_tile(int H, int form) {
  switch (H) {
    case 256: return fwd_rows_per_tile_w<256>(form);
    case 512: return fwd_rows_per_tile_w<512>(form);
    case 1536: return fwd_rows_per_tile_w<1536>(form);
    case 2048: return fwd_rows_per_tile_w<2048>(form);
    case 4096: return fwd_rows_per_tile_w<4096>(form);
    case 5120: return fwd_rows_per_tile_w<5120>(form);
    case 6144: return fwd_rows_per_tile_w<6144>(form);
    default: return 0;
  }
}

hipError_t launch_fwd(int H, bool w_f32, int form, const FwdArgs& a, int grid, hipStream_t s) {
  switch (H) {
    case 256: return fwd_width<256>(w_f32, form, a, grid, s);
    case 512: return fwd_width<512>(w_f32, form, a, grid, s);
    case 1536: return fwd_width<1536>(w_f32, form, a, grid, s);
    case 2048: return fwd_width<2048>(w_f32, form, a, grid, s);
    case 4096: return fwd_width<4096>(w_f32, form, a, grid, s);
    case 5120: return fwd_width<5120>(w_f32, form, a, grid, s);
    case 6144: return fwd_width<6144>(w_f32, form, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rmsn
