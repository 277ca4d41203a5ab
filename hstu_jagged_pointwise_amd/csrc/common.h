// Device-side helpers shared by the libhstu kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// Load of data that no kernel in flight writes, through the scalar data cache
// when the address is wavefront-uniform (the constant address space lets the
// compiler select s_load).
template <typename T>
__device__ __forceinline__ T sload(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// ---------------------------------------------------------------------------
// Bias buckets. These compute the relative attention bias rab^{p,t} of
// eq. 2 ("What an HSTU layer changes", HSTU chapter). The bias encodes
// relative position and elapsed time (Yonas Stephen's course, "Problem 2").
// position: bp = min(i - j, P - 1) for a visible pair (i >= j)
// time:     bt = min(floor(log2(max(t_i - t_j, 0) + 1)), T - 1), exact integers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int pos_bucket(int dpos, int P) {
  dpos = dpos < 0 ? 0 : dpos;
  return dpos < P - 1 ? dpos : P - 1;
}

// General form. Timestamps of one sequence (history plus candidates) must
// span less than 2^62 seconds, so that the difference and the +1 cannot overflow.
__device__ __forceinline__ int time_bucket64(int64_t tq, int64_t tk) {
  int64_t d = tq - tk;
  d = d < 0 ? 0 : d;
  return 63 - __builtin_clzll((uint64_t)d + 1ull);
}

// Fast form, valid when the true dt = tq - tk satisfies -2^31-1 <= dt <= 2^31-2.
// Then dt + 1 fits in int32, and it equals the wrapped 32-bit difference of the
// low words, tq1 - tk_lo, where tq1 = low32(tq) + 1. The result is the count of
// leading zeros of max(dt + 1, 1), in [1, 31]. The bucket is 31 - clz, which
// callers usually fold into a table indexed by clz.
__device__ __forceinline__ int time_clz_fast(uint32_t tq1, uint32_t tk_lo) {
  int d = (int)(tq1 - tk_lo);
  d = d < 1 ? 1 : d;
  return __builtin_clz((uint32_t)d);
}

// True when every dt in [qmin - kmax, qmax - kmin] stays in the fast range.
__device__ __forceinline__ bool time_fast_ok(int64_t qmin, int64_t qmax, int64_t kmin,
                                             int64_t kmax) {
  return (qmax - kmin <= (int64_t)2147483646) && (qmin - kmax >= -(int64_t)2147483649LL);
}

// ---------------------------------------------------------------------------
// numerics
// ---------------------------------------------------------------------------
// SiLU(x) = x * sigmoid(x) = x / (1 + e^{-x}), phi1 and phi2 of the HSTU layer.
// Uses the hardware exp2 and reciprocal (about 1 ulp each). That is ample when
// the result is rounded to bf16.
__device__ __forceinline__ float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}
// SiLU of x given x' = -log2(e) x, times -log2(e): x' * sigmoid(x), one multiply fewer.
__device__ __forceinline__ float silu_prescaled(float xp) {
  return xp * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(xp));
}
// Accurate SiLU for fp32 outputs (correctly rounded expf and a true divide).
__device__ __forceinline__ float silu_precise(float x) { return x / (1.0f + expf(-x)); }

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
__device__ __forceinline__ bf16 f2bf(float x) { return (bf16)x; }  // round to nearest even

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16>(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// 64-bit min/max across a wavefront (64 lanes).
__device__ __forceinline__ int64_t wave_min64(int64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    int64_t w = __shfl_xor(v, o, 64);
    v = w < v ? w : v;
  }
  return v;
}
__device__ __forceinline__ int64_t wave_max64(int64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    int64_t w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace hstu
