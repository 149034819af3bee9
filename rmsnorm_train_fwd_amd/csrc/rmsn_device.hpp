// rmsn_device.hpp -- device building blocks of the gfx950 RMSNorm-training kernels.
//
// Compiled for gfx950 only (wave64). All translation units that include this
// header build with -ffp-contract=off and without fast-math: the error-free
// transforms below (TwoSum, TwoProduct) are exact only if the compiler keeps
// every rounding where it is written. FP32 denormals are preserved (HIP's
// default), since TwoProduct error terms can be subnormal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rmsn {

typedef uint16_t u16;
typedef uint32_t u32;

// ----------------------------------------------------------------- formats --

// BF16 element 2i of a packed pair sits in the low half of 32-bit word i.
__device__ __forceinline__ float bf_lo(u32 w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(u32 w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two FP32 values -> packed BF16 pair, round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ u32 pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(u32, __builtin_convertvector(v, bf16x2_t));
}

// 8 BF16 values (one 16-byte vector) <-> 8 floats.
__device__ __forceinline__ void unpack8(const uint4& u, float (&f)[8]) {
  f[0] = bf_lo(u.x); f[1] = bf_hi(u.x);
  f[2] = bf_lo(u.y); f[3] = bf_hi(u.y);
  f[4] = bf_lo(u.z); f[5] = bf_hi(u.z);
  f[6] = bf_lo(u.w); f[7] = bf_hi(u.w);
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  uint4 u;
  u.x = pack_bf16x2(f[0], f[1]);
  u.y = pack_bf16x2(f[2], f[3]);
  u.z = pack_bf16x2(f[4], f[5]);
  u.w = pack_bf16x2(f[6], f[7]);
  return u;
}

// FP64 -> BF16 rounded once to nearest even. The FP64 value is first rounded
// to odd at FP32 precision (toward zero, last bit set when inexact), then
// rounded to nearest even into BF16; rounding to odd at 24 bits followed by
// rounding to 8 bits equals rounding the FP64 value once (Boldo and
// Melquiond, "Emulation of FMA and correctly rounded sums: proved algorithms
// using rounding to odd", 2008). BF16 shares FP32's exponent range.
__device__ __forceinline__ u16 f64_to_bf16(double d) {
  const float f = (float)d;                            // nearest even
  u32 b = __float_as_uint(f);
  if (__builtin_fabs((double)f) > __builtin_fabs(d)) b -= 1;  // one step toward zero
  if ((double)__uint_as_float(b) != d) b |= 1u;        // inexact: odd
  return (u16)(pack_bf16x2(__uint_as_float(b), 0.0f) & 0xffffu);
}

__device__ __forceinline__ uint4 ld16(const u16* p) { return *reinterpret_cast<const uint4*>(p); }

// Streaming loads/stores: data touched exactly once per call.
typedef u32 u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const u16* p) {
  u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Row outputs: 16-byte non-temporal stores. Write-through stores (system
// scope, sc0 sc1) measured faster in single cold-cache calls, but only because
// the memory-side cache then held up to its 256 MB of the call's output dirty
// past the end of the call; back to back, where every byte reaches HBM, they
// were equal or up to 5% slower at [131072, 4096].
__device__ __forceinline__ void st16_stream(u16* p, const uint4& v) {
  u32x4_t t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t*>(p));
}

// --------------------------------------------------- error-free transforms --

// Knuth's TwoSum: s + e == a + b exactly (no magnitude precondition).
__device__ __forceinline__ void two_sum(float a, float b, float& s, float& e) {
  s = a + b;
  float bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

// TwoProduct by FMA: p + e == a * b exactly (barring underflow).
__device__ __forceinline__ void two_prod(float a, float b, float& p, float& e) {
  p = a * b;
  e = __builtin_fmaf(a, b, -p);
}

// ------------------------------------------------------- cross-lane sums --
//
// Butterfly sums inside a wave. Every lane ends with the same bits: each step
// adds a lane's value to its partner's, and IEEE addition is commutative.

template <int CTRL>
__device__ __forceinline__ float dpp_partner_add(float v) {
  int p = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false);
  return v + __int_as_float(p);
}

// Sum over the 16 lanes of each DPP row.
__device__ __forceinline__ float sum16(float v) {
  v = dpp_partner_add<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v = dpp_partner_add<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  v = dpp_partner_add<0x141>(v);  // row_half_mirror: quad 0 <-> quad 1 of each 8
  v = dpp_partner_add<0x140>(v);  // row_mirror: half-row 0 <-> half-row 1
  return v;
}

// Sum over each half-wave (lanes 0-31 and 32-63 separately).
__device__ __forceinline__ float sum32(float v) {
  v = sum16(v);
  // v_permlane16_swap with both operands = v: one result holds the even rows,
  // the other the odd rows, so their sum is row(2k) + row(2k+1) in every lane.
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the whole wave.
__device__ __forceinline__ float sum64(float v) {
  v = sum32(v);
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int LANES>
__device__ __forceinline__ float lane_sum(float v) {
  static_assert(LANES == 32 || LANES == 64, "row groups are half or whole waves");
  if constexpr (LANES == 32) return sum32(v);
  else return sum64(v);
}

// ------------------------------------------------------ per-width layout --
//
// A row of `H` BF16 elements is handled by a row group of TPR threads; each
// thread owns V 16-byte vectors (8 elements each): vector v of lane l covers
// elements (v*TPR + l)*8 .. +7, so one load instruction of the row group
// reads TPR*16 contiguous bytes. A workgroup of BLOCK = TPR*R threads holds R
// row groups, which work on R different rows at a time; in the backward main
// kernel each row group takes D rows per batch, with the next batch's loads in
// flight during the current one (PIPE) or not. Per-column state (weight, dw
// accumulators) lives in registers; fewer columns per thread means more waves
// in flight, more columns means fewer, larger row groups. Cfg is the
// backward's shape (its R is the sub-chain count of the dw tree); the
// forward's (FwdCfg, with the kernels) is the same except where measurement
// chose otherwise.
template <int H> struct Cfg;
template <> struct Cfg<256>  { static constexpr int TPR = 32,  V = 1, R = 16, D = 2; static constexpr bool PIPE = true; };
template <> struct Cfg<512>  { static constexpr int TPR = 64,  V = 1, R = 8,  D = 1; static constexpr bool PIPE = true; };
template <> struct Cfg<1536> { static constexpr int TPR = 192, V = 1, R = 4,  D = 2; static constexpr bool PIPE = true; };
template <> struct Cfg<2048> { static constexpr int TPR = 256, V = 1, R = 4,  D = 1; static constexpr bool PIPE = true; };
template <> struct Cfg<4096> { static constexpr int TPR = 512, V = 1, R = 2,  D = 1; static constexpr bool PIPE = true; };
template <> struct Cfg<5120> { static constexpr int TPR = 320, V = 2, R = 2,  D = 1; static constexpr bool PIPE = true; };
template <> struct Cfg<6144> { static constexpr int TPR = 768, V = 1, R = 1,  D = 1; static constexpr bool PIPE = true; };


template <int H_, class C>
struct GeoOf {
  static constexpr int H = H_;
  static constexpr int TPR = C::TPR;
  static constexpr int V = C::V;
  static constexpr int R = C::R;                   // row groups per workgroup
  static constexpr int BLOCK = TPR * R;            // workgroup size
  static constexpr int LANES = TPR < 64 ? TPR : 64;
  static constexpr int WPR = TPR / LANES;          // waves per row group
  static constexpr int E = 8 * V;                  // elements per thread
  static constexpr int D = C::D;                   // rows per row group per backward batch
  static constexpr bool PIPE = C::PIPE;            // backward: next batch loads during this one
  static_assert(TPR * V * 8 == H, "layout must tile the row exactly");
  static_assert(TPR % 64 == 0 || TPR == 32, "row groups are half waves or whole waves");
  static_assert(BLOCK <= 1024 && BLOCK % 32 == 0, "workgroup size");
};

template <int H> using Geo = GeoOf<H, Cfg<H>>;  // backward

// Row group of this thread. With whole-wave row groups it is the same for
// every lane of a wave; saying so (readfirstlane) lets the compiler keep row
// indices, row addresses and rstd in scalar registers.
template <class G>
__device__ __forceinline__ int row_group() {
  const int q = threadIdx.x / G::TPR;
  if constexpr (G::TPR >= 64) return __builtin_amdgcn_readfirstlane(q);
  else return q;
}

// First element of vector v of a lane.
template <class G>
__device__ __forceinline__ int elem0(int v, int lane) {
  return (v * G::TPR + lane) * 8;
}

// Weight in registers: the E elements a thread owns, as FP32. With `one`
// set (zero-centred weight) each becomes 1 + w, rounded once to FP32.
template <class G, bool WF32>
__device__ __forceinline__ void load_w(const void* w, int lane, float (&wr)[G::E], int one) {
  constexpr int TPR = G::TPR;
#pragma unroll
  for (int v = 0; v < G::V; ++v) {
    const int e0 = (v * TPR + lane) * 8;
    if constexpr (WF32) {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(w) + e0);
      float4 a = p[0], b = p[1];
      wr[v * 8 + 0] = a.x; wr[v * 8 + 1] = a.y; wr[v * 8 + 2] = a.z; wr[v * 8 + 3] = a.w;
      wr[v * 8 + 4] = b.x; wr[v * 8 + 5] = b.y; wr[v * 8 + 6] = b.z; wr[v * 8 + 7] = b.w;
    } else {
      float f[8];
      unpack8(ld16(static_cast<const u16*>(w) + e0), f);
#pragma unroll
      for (int i = 0; i < 8; ++i) wr[v * 8 + i] = f[i];
    }
  }
  if (one) {
#pragma unroll
    for (int i = 0; i < G::E; ++i) wr[i] = 1.0f + wr[i];
  }
}

// Sum of D per-thread partials over each row group; every thread of the row
// group receives the totals. Row groups of one or half a wave use lane sums
// only. Wider row groups add the per-wave sums through LDS in wave order
// ((w0 + w1) + w2) + ..., with two alternating slot sets so that one barrier
// per call suffices. All threads of the workgroup must call it together.
template <class G, int D>
struct RowSum {
  static constexpr int R = G::R, WPR = G::WPR;
  static constexpr int kSlots = (WPR > 1) ? 2 * R * WPR * D : 1;

  __device__ static void run(float (&v)[D], float* slots, int& parity, int q, int lane) {
#pragma unroll
    for (int d = 0; d < D; ++d) v[d] = lane_sum<G::LANES>(v[d]);
    if constexpr (WPR > 1) {
      float* s = slots + (parity * R + q) * WPR * D;
      const int wv = lane / 64;
      if ((lane & 63) == 0) {
#pragma unroll
        for (int d = 0; d < D; ++d) s[wv * D + d] = v[d];
      }
      __syncthreads();
#pragma unroll
      for (int d = 0; d < D; ++d) {
        float t = s[d];
#pragma unroll
        for (int k = 1; k < WPR; ++k) t += s[k * D + d];
        v[d] = t;
      }
      parity ^= 1;
    }
  }
};

// ------------------------------------------------------------ dw tree --
//
// Deterministic dw: the rows of a call form tiles of R consecutive rows (R
// fixed per width), and the tiles are dealt to K chunks in turn: chunk k holds
// tiles k, k + K, k + 2K, ... (K from the row count and the width alone, see
// the host plan). Row q of each of chunk k's tiles, in ascending tile order,
// forms sub-chain q, summed by Dot2 (TwoProduct + TwoSum, compensation in
// FP32); the chunk partial is 0.0 + d_0 + d_1 + ... + d_{R-1} in FP64 with
// d_q = (double)s_q + (double)c_q;
// partials fold in FP64: consecutive groups of kFoldGroup chunks are summed in
// ascending order from 0.0, then the group sums in ascending order from 0.0,
// then one rounding to FP32. Every kernel below that produces dw follows this
// tree operation for operation, so dw has the same bits on every path.
struct Dot2 {
  float s = 0.0f, c = 0.0f;
  // Adds the exact product a*b (a itself exact, e.g. dy*x of two BF16 values).
  __device__ __forceinline__ void add(float a, float b) {
    float p, pe, t;
    two_prod(a, b, p, pe);
    two_sum(s, p, s, t);
    c = c + (t + pe);
  }
  __device__ __forceinline__ double value() const { return (double)s + (double)c; }
};

// Non-deterministic dw: FP32 sums over blocks of 8 rows of a sub-chain, each
// block flushed into a TwoSum-compensated pair.
struct Block8 {
  float b = 0.0f, s = 0.0f, c = 0.0f;
  __device__ __forceinline__ void add(float dy, float xh) { b = __builtin_fmaf(dy, xh, b); }
  __device__ __forceinline__ void flush() {
    float t;
    two_sum(s, b, s, t);
    c = c + t;
    b = 0.0f;
  }
  __device__ __forceinline__ double value() const { return (double)s + (double)c; }
};

// SiLU pieces in FP32: sigmoid by the hardware exp2 and reciprocal
// (v_exp_f32, v_rcp_f32; about 1 ulp each). Large negative z gives
// exp2 -> +inf and sigmoid -> 0; large positive z gives sigmoid -> 1.
__device__ __forceinline__ float sigmoid_f(float z) {
  float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
  return __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace rmsn
