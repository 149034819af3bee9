// rmsn_noalloc.hip -- rmsnorm_train_bwd_noalloc: the backward of
// rmsnorm_train_bwd for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation).
//
// The only device memory the backward needs beyond its inputs and outputs is
// the large path's FP64 chunk partials (at most 256 chunks x width doubles).
// Here they live in `scratch`, one file-scope device array per GPU, held until
// the process ends. In host code the name `scratch` only stands in for the
// device array: its device address is taken once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// ever handed to a kernel. The partials need no initial contents (every chunk
// writes its own row of them before the fold reads it), so nothing is cleared.
#include <mutex>

#include "rmsn_abi_internal.hpp"
#include "rmsn_launch.hpp"

namespace {

constexpr int kMaxWidth = 6144;
constexpr size_t kScratchDoubles = (size_t)rmsn::kMaxChunks * kMaxWidth;
constexpr size_t kScratchBytes = kScratchDoubles * sizeof(double);  // 12 MiB
constexpr int kMaxDevices = 64;

}  // namespace

// 256 chunks x 6144 columns of FP64 partials: the largest workspace any plan needs.
static __device__ __align__(256) double scratch[kScratchDoubles];

namespace {

std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, once looked up

// Workspace source of the no-allocation entry point: the current device's
// `scratch`, looked up on the first call on that device. A stream of another
// device is refused (its kernels would reach this device's array).
rmsn_status scratch_source(void* stream, size_t need, void** ws, size_t* ws_bytes) {
  if (need > kScratchBytes) return RMSN_E_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RMSN_E_HIP;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
      return RMSN_E_HIP;
    if (sdev != dev) return RMSN_E_ARG;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RMSN_E_HIP;
    g_scratch[dev] = p;
  }
  *ws = g_scratch[dev];
  *ws_bytes = kScratchBytes;
  return RMSN_OK;
}

}  // namespace

RMSN_API rmsn_status rmsnorm_train_bwd_noalloc(const void* dy, const void* x, const void* dh,
                                               const void* w, rmsn_dtype w_dtype,
                                               const float* rstd, int deterministic,
                                               const rmsn_layout* L, void* dx, void* dw,
                                               rmsn_dtype dw_dtype, const rmsn_launch* launch,
                                               void* stream) {
  return rmsn::bwd_common(dh ? rmsn::kResidual : rmsn::kPlain, dy, x, dh, w,
                          rmsn::enum_code(w_dtype), rstd, deterministic, L, dx, nullptr, dw,
                          rmsn::enum_code(dw_dtype), nullptr, 0, scratch_source, launch, stream);
}
