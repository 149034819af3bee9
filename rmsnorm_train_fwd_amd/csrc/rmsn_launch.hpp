// rmsn_launch.hpp -- internal interface between the C ABI (rmsn_abi.cpp) and
// the kernel translation units. Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rmsn {

enum Form : int { kPlain = 0, kResidual = 1, kGate = 2 };

// Row r of a row input starts at base + (r / heads) * stride_t + (r % heads) * stride_h.
struct RowIn {
  const uint16_t* p;
  int64_t stride_t, stride_h;
};

struct FwdArgs {
  RowIn x;            // x
  RowIn e;            // residual (kResidual) or z (kGate); unused otherwise
  const void* w;
  uint16_t* y;        // dense [rows, H]
  uint16_t* h;        // dense [rows, H] (kResidual)
  float* rstd;        // [rows]
  int64_t rows;
  int32_t heads;
  int32_t w_one;      // 1: zero-centred weight, the kernels use 1 + w
  float eps;
};

struct BwdArgs {
  RowIn dy;           // g strides
  RowIn x;            // x strides (the BF16 h in the residual form)
  RowIn e;            // dh (kResidual, g strides) or z (kGate, x strides)
  const void* w;
  const float* rstd;  // [rows]
  uint16_t* dx;       // dense [rows, H] (grad_h in the residual form)
  uint16_t* dz;       // dense [rows, H] (kGate)
  void* dw;           // [H], FP32 or (dw_bf16) BF16
  int32_t dw_bf16;
  double* ws;         // [chunks, H] FP64 chunk partials (large path)
  int64_t rows;
  int64_t chunks;     // K: chunks of the dw tree, 1 <= K <= ceil(rows / R) when rows > 0
  int32_t heads;
  int32_t w_one;      // 1: zero-centred weight, the kernels use 1 + w
};

// Each returns the status of its own launches (hipLaunchKernel's result;
// hipErrorInvalidValue for a width / form combination that has no kernel) and
// leaves the thread's last-error state alone.
hipError_t launch_fwd(int H, bool w_f32, int form, const FwdArgs& a, int grid, hipStream_t s);
hipError_t launch_bwd_large(int H, bool w_f32, int form, bool det, const BwdArgs& a, int grid,
                            hipStream_t s);
hipError_t launch_fold(int H, const BwdArgs& a, int grid, hipStream_t s);
hipError_t launch_bwd_small(int H, bool w_f32, int form, const BwdArgs& a, int row_grid,
                            int col_grid, hipStream_t s);

// Grid sizes the kernels are written for (host-side planning).
int fwd_rows_per_tile(int H, int form);  // rows one workgroup handles per tile
int bwd_rows_per_rowtask(int H);   // R: row groups of the main kernel = rows per tile = sub-chains per chunk
int small_rows_per_rowtask(int H); // rows one small-path row workgroup handles
int small_col_tile(int H);         // columns per small-path column-task workgroup
constexpr int kMaxChunks = 256;    // chunks of the dw tree at most (one per CU at large T)
constexpr int kFoldGroup = 32;     // chunks per first-level group of the dw fold
constexpr int kFoldGroups = kMaxChunks / kFoldGroup;  // first-level groups at most
constexpr int kFoldTile = 32;      // columns per fold workgroup
constexpr int kFoldThreads = kFoldTile * kFoldGroups; // one thread per column x group

}  // namespace rmsn
