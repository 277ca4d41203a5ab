// Small kernels around the hot path: the candidate logit (one linear head on
// the final M-FALCON embedding) and the bucket export used by the tests.
#include "common.h"
#include "kernels.h"

namespace hstu {

template <typename T>
__global__ __launch_bounds__(256) void rowdot_kernel(const T* __restrict__ y, int64_t ld_y,
                                                     const float* __restrict__ w,
                                                     float* __restrict__ logit, int64_t rows, int d) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  float s = 0.f;
  for (int c = lane; c < d; c += 64) s = fmaf(to_f32<T>(y[row * ld_y + c]), w[c], s);
  s = wave_sum(s);
  if (lane == 0) logit[row] = s;
}

// bf16 rows in 16-byte pieces: each lane loads 8 values of y and 8 of w at once (one pass
// for a row of 512), instead of a strided loop of 2-byte loads.
__global__ __launch_bounds__(256) void rowdot_bf16x8_kernel(const bf16* __restrict__ y,
                                                            int64_t ld_y,
                                                            const float* __restrict__ w,
                                                            float* __restrict__ logit,
                                                            int64_t rows, int d) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  float s = 0.f;
  for (int c = 8 * lane; c < d; c += 512) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(y + row * ld_y + c);
    const f32x4 w0 = *reinterpret_cast<const f32x4*>(w + c);
    const f32x4 w1 = *reinterpret_cast<const f32x4*>(w + c + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) s = fmaf((float)v[e], w0[e], s);
#pragma unroll
    for (int e = 0; e < 4; ++e) s = fmaf((float)v[4 + e], w1[e], s);
  }
  s = wave_sum(s);
  if (lane == 0) logit[row] = s;
}

hipError_t launch_rowdot(const void* y, int64_t ld_y, const float* w, float* logit, int64_t rows,
                         int d, int bf16flag, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (bf16flag && d % 8 == 0 && ld_y % 8 == 0 && (uintptr_t)y % 16 == 0 && (uintptr_t)w % 16 == 0) {
    hipLaunchKernelGGL(rowdot_bf16x8_kernel, grid, dim3(256), 0, s, (const bf16*)y, ld_y, w, logit,
                       rows, d);
    return hipGetLastError();
  }
  if (bf16flag)
    hipLaunchKernelGGL((rowdot_kernel<bf16>), grid, dim3(256), 0, s, (const bf16*)y, ld_y, w, logit,
                       rows, d);
  else
    hipLaunchKernelGGL((rowdot_kernel<float>), grid, dim3(256), 0, s, (const float*)y, ld_y, w,
                       logit, rows, d);
  return hipGetLastError();
}

// Bucket indices for every (query i, key j) pair of one sequence. Hidden pairs
// (j > i) are written as -1. The time bucket comes from the general 64-bit
// function. Where the 32-bit fast form applies to the pair, both forms are
// evaluated, and a disagreement is written as -2 so that the tests catch it.
__global__ void debug_buckets_kernel(const int64_t* __restrict__ off, const int64_t* __restrict__ ts,
                                     int seq, int n, int P, int T, int32_t* __restrict__ pb,
                                     int32_t* __restrict__ tb) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n * n) return;
  const int i = (int)(idx / n), j = (int)(idx % n);
  if (j > i) {
    pb[idx] = -1;
    tb[idx] = -1;
    return;
  }
  pb[idx] = pos_bucket(i - j, P);
  if (!ts) {
    tb[idx] = 0;
    return;
  }
  const int64_t s0 = off[seq];
  const int64_t ti = ts[s0 + i], tj = ts[s0 + j];
  int bt = time_bucket64(ti, tj);
  bt = bt < T - 1 ? bt : T - 1;
  if (time_fast_ok(ti, ti, tj, tj)) {
    int bf = 31 - time_clz_fast((uint32_t)ti + 1u, (uint32_t)tj);
    bf = bf < T - 1 ? bf : T - 1;
    if (bf != bt) bt = -2;
  }
  tb[idx] = bt;
}

hipError_t launch_debug_buckets(const int64_t* offsets, const int64_t* ts, int seq, int n, int P,
                                int T, int32_t* pos_bucket_out, int32_t* time_bucket_out,
                                hipStream_t s) {
  const int64_t total = (int64_t)n * n;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(debug_buckets_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     offsets, ts, seq, n, P, T, pos_bucket_out, time_bucket_out);
  return hipGetLastError();
}

}  // namespace hstu
