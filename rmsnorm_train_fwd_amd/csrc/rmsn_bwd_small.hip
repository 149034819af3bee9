// rmsn_bwd_small.hip -- single-launch small-row backward instances and launcher.
#include "rmsn_kernels.hpp"

namespace rmsn {

namespace {
template <int H, bool WF32>
hipError_t small_form(int form, const BwdArgs& a, int row_grid, int col_grid, hipStream_t s) {
  const int grid = row_grid + col_grid;
  constexpr int B = SmallGeo<H>::BLOCK;
  switch (form) {
    case kPlain: return launch_kernel(k_bwd_small<H, WF32, kPlain>, grid, B, s, a, row_grid);
    case kResidual: return launch_kernel(k_bwd_small<H, WF32, kResidual>, grid, B, s, a, row_grid);
    case kGate: return launch_kernel(k_bwd_small<H, WF32, kGate>, grid, B, s, a, row_grid);
    default: return hipErrorInvalidValue;
  }
}

template <int H>
hipError_t small_width(bool w_f32, int form, const BwdArgs& a, int rg, int cg, hipStream_t s) {
  return w_f32 ? small_form<H, true>(form, a, rg, cg, s) : small_form<H, false>(form, a, rg, cg, s);
}
}  // namespace

int small_col_tile(int H) {
  switch (H) {
    case 256: return SmallGeo<256>::BLOCK / (kFoldGroup * Geo<256>::R) * SmallGeo<256>::CPT;
    case 512: return SmallGeo<512>::BLOCK / (kFoldGroup * Geo<512>::R) * SmallGeo<512>::CPT;
    case 1536: return SmallGeo<1536>::BLOCK / (kFoldGroup * Geo<1536>::R) * SmallGeo<1536>::CPT;
    case 2048: return SmallGeo<2048>::BLOCK / (kFoldGroup * Geo<2048>::R) * SmallGeo<2048>::CPT;
    case 4096: return SmallGeo<4096>::BLOCK / (kFoldGroup * Geo<4096>::R) * SmallGeo<4096>::CPT;
    case 5120: return SmallGeo<5120>::BLOCK / (kFoldGroup * Geo<5120>::R) * SmallGeo<5120>::CPT;
    case 6144: return SmallGeo<6144>::BLOCK / (kFoldGroup * Geo<6144>::R) * SmallGeo<6144>::CPT;
    default: return 0;
  }
}

int small_rows_per_rowtask(int H) {
  switch (H) {
    case 256: return SmallGeo<256>::RS;
    case 512: return SmallGeo<512>::RS;
    case 1536: return SmallGeo<1536>::RS;
    case 2048: return SmallGeo<2048>::RS;
    case 4096: return SmallGeo<4096>::RS;
    case 5120: return SmallGeo<5120>::RS;
    case 6144: return SmallGeo<6144>::RS;
    default: return 0;
  }
}

int bwd_rows_per_rowtask(int H) {
  switch (H) {
    case 256: return Geo<256>::R;
    case 512: return Geo<512>::R;
    case 1536: return Geo<1536>::R;
    case 2048: return Geo<2048>::R;
    case 4096: return Geo<4096>::R;
    case 5120: return Geo<5120>::R;
    case 6144: return Geo<6144>::R;
    default: return 0;
  }
}

hipError_t launch_bwd_small(int H, bool w_f32, int form, const BwdArgs& a, int row_grid,
                            int col_grid, hipStream_t s) {
  switch (H) {
    case 256: return small_width<256>(w_f32, form, a, row_grid, col_grid, s);
    case 512: return small_width<512>(w_f32, form, a, row_grid, col_grid, s);
    case 1536: return small_width<1536>(w_f32, form, a, row_grid, col_grid, s);
    case 2048: return small_width<2048>(w_f32, form, a, row_grid, col_grid, s);
    case 4096: return small_width<4096>(w_f32, form, a, row_grid, col_grid, s);
    case 5120: return small_width<5120>(w_f32, form, a, row_grid, col_grid, s);
    case 6144: return small_width<6144>(w_f32, form, a, row_grid, col_grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rmsn
