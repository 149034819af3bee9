// Bandwidth probe for the measurement script: the streaming access pattern of
// the normalisation kernels with no arithmetic, to show the practical HBM
// ceiling on this device beside the kernels' own rate. Not part of the
// normalisation library and not declared in its header; only the benchmark
// loads it.
//
// Buffers are arrays of whole 16 KiB tiles (1024 vectors of 16 bytes), moved
// with non-temporal 16-byte loads and stores in one of two patterns:
//   pattern 0 (dealt): `grid` workgroups of 1024 threads; tiles are dealt to
//     them in turn (workgroup g takes tiles g, g + grid, ...), so the
//     workgroups in flight together stream one contiguous window, as the
//     backward's chunks do; one vector per thread per tile, and the loads of a
//     workgroup's next tile are in flight while the current one is written.
//   pattern 1 (one-shot): one 256-thread workgroup per tile, four vectors per
//     thread, consecutive workgroups on consecutive tiles (`grid` is ignored).
//   pattern 2 (one-shot, one vector): one 256-thread workgroup per 4 KiB, one
//     vector per thread (the plainest streaming kernel, and the fastest of a
//     sweep of block sizes, vectors per thread and grid-strided forms on
//     MI355X; `grid` is ignored).
//   nin = 1: out = a           (one stream read, one written: the forward)
//   nin = 2: out = a ^ b       (two read, one written: the backward)
//   nin = 0: a is read and folded into one vector per thread (read only)
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kBlock = 1024;
constexpr int64_t kTileBytes = (int64_t)kBlock * 16;

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

template <int NIN>
__global__ __launch_bounds__(kBlock) void k_stream(const v4u* __restrict__ a,
                                                   const v4u* __restrict__ b,
                                                   v4u* __restrict__ out, int64_t tiles) {
  int64_t t = blockIdx.x;
  if (t >= tiles) return;
  const int64_t g = gridDim.x;
  v4u ca, cb = {0u, 0u, 0u, 0u}, na, nb = {0u, 0u, 0u, 0u}, acc = {0u, 0u, 0u, 0u};
  auto load = [&](int64_t tt, v4u& va, v4u& vb) {
    const int64_t i = tt * kBlock + threadIdx.x;
    va = __builtin_nontemporal_load(a + i);
    if constexpr (NIN == 2) vb = __builtin_nontemporal_load(b + i);
  };
  auto consume = [&](int64_t tt, const v4u& va, const v4u& vb) {
    if constexpr (NIN == 0) {
      acc ^= va;
    } else {
      v4u v = va;
      if constexpr (NIN == 2) v ^= vb;
      __builtin_nontemporal_store(v, out + tt * kBlock + threadIdx.x);
    }
  };
  load(t, ca, cb);
  for (; t + g < tiles; t += g) {
    load(t + g, na, nb);
    consume(t, ca, cb);
    ca = na;
    cb = nb;
  }
  consume(t, ca, cb);
  if constexpr (NIN == 0) out[(int64_t)blockIdx.x * kBlock + threadIdx.x] = acc;
}

template <int NIN>
__global__ __launch_bounds__(256) void k_stream_oneshot(const v4u* __restrict__ a,
                                                         const v4u* __restrict__ b,
                                                         v4u* __restrict__ out) {
  const int64_t base = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  v4u va[4], vb[4], acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    va[u] = __builtin_nontemporal_load(a + base + u * 256);
    if constexpr (NIN == 2) vb[u] = __builtin_nontemporal_load(b + base + u * 256);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if constexpr (NIN == 0) {
      acc ^= va[u];
    } else {
      v4u v = va[u];
      if constexpr (NIN == 2) v ^= vb[u];
      __builtin_nontemporal_store(v, out + base + u * 256);
    }
  }
  if constexpr (NIN == 0) out[base] = acc;
}

template <int NIN>
__global__ __launch_bounds__(256) void k_stream_vec1(const v4u* __restrict__ a,
                                                      const v4u* __restrict__ b,
                                                      v4u* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  v4u va = __builtin_nontemporal_load(a + i);
  if constexpr (NIN == 0) {
    // read only: a store the data practically never asks for keeps the load live
    if ((va.x ^ va.y ^ va.z ^ va.w) == 0x9e3779b9u) out[blockIdx.x] = va;
  } else {
    if constexpr (NIN == 2) va ^= __builtin_nontemporal_load(b + i);
    __builtin_nontemporal_store(va, out + i);
  }
}

// Enqueues k<<<grid, block, 0, s>>>(args) and returns that launch's own status.
template <class... P>
int launch(void (*k)(P...), unsigned grid, unsigned block, hipStream_t s, P... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(k), dim3(grid), dim3(block), argv, 0, s);
}

}  // namespace

// Runs one probe pass over `bytes` bytes per stream, a multiple of 16 KiB, in
// pattern 0, 1 or 2 as above. nin is 0, 1 or 2 as above; b is read only for
// nin = 2; with nin = 0, out receives at most `bytes`. Returns a hipError_t
// value: hipErrorInvalidValue for bad arguments, before any launch.
extern "C" __attribute__((visibility("default"))) int rmsn_stream_probe(
    int nin, int pattern, const void* a, const void* b, void* out, int64_t bytes, int grid,
    void* stream) {
  if (nin < 0 || nin > 2 || pattern < 0 || pattern > 2 || a == nullptr || out == nullptr ||
      (nin == 2 && b == nullptr) || bytes <= 0 || bytes % kTileBytes != 0 ||
      bytes / kTileBytes > 0x1fffffff || grid < 1 || grid > 65535 ||
      ((uintptr_t)a | (uintptr_t)b | (uintptr_t)out) % 16 != 0)
    return (int)hipErrorInvalidValue;
  const int64_t tiles = bytes / kTileBytes;
  const v4u* pa = static_cast<const v4u*>(a);
  const v4u* pb = static_cast<const v4u*>(b);
  v4u* po = static_cast<v4u*>(out);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pattern == 1) {
    const unsigned g = (unsigned)tiles;
    switch (nin) {
      case 0: return launch(k_stream_oneshot<0>, g, 256, s, pa, pb, po);
      case 1: return launch(k_stream_oneshot<1>, g, 256, s, pa, pb, po);
      default: return launch(k_stream_oneshot<2>, g, 256, s, pa, pb, po);
    }
  }
  if (pattern == 2) {
    const unsigned g = (unsigned)(tiles * 4);  // 4 KiB per workgroup
    switch (nin) {
      case 0: return launch(k_stream_vec1<0>, g, 256, s, pa, pb, po);
      case 1: return launch(k_stream_vec1<1>, g, 256, s, pa, pb, po);
      default: return launch(k_stream_vec1<2>, g, 256, s, pa, pb, po);
    }
  }
  switch (nin) {
    case 0: return launch(k_stream<0>, (unsigned)grid, (unsigned)kBlock, s, pa, pb, po, tiles);
    case 1: return launch(k_stream<1>, (unsigned)grid, (unsigned)kBlock, s, pa, pb, po, tiles);
    default: return launch(k_stream<2>, (unsigned)grid, (unsigned)kBlock, s, pa, pb, po, tiles);
  }
}
