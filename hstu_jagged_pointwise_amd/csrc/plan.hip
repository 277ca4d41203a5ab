// Jagged tile planner. The HSTU chapter ("Three more scaling components",
// ragged kernels) says padding every user to the maximum length wastes most
// of the compute. This planner emits one work item per (sequence, query tile)
// that actually exists, with no padding to the longest sequence. Under the
// causal mask a query tile t needs key tiles 0..t only, so its cost grows with
// t. Items are ordered by decreasing t (longest first), which makes the
// dispatch order approximate longest-processing-time scheduling across the
// compute units. The order never changes results: every item writes its own
// output rows and no reduction crosses items.
#include "common.h"
#include "kernels.h"

namespace hstu {

constexpr int kPlanThreads = 1024;
constexpr int kPlanBins = 2048;

__global__ __launch_bounds__(kPlanThreads) void plan_causal_kernel(const int64_t* __restrict__ off,
                                                                   int B, int tile_rows, int nbins,
                                                                   int2* __restrict__ items,
                                                                   int n_items) {
  __shared__ int cnt[kPlanBins];
  __shared__ int start[kPlanBins];
  const int tid = threadIdx.x;
  for (int i = tid; i < nbins; i += kPlanThreads) cnt[i] = 0;
  __syncthreads();
  // histogram of items by query-tile index (clamped into the last bin)
  for (int b = tid; b < B; b += kPlanThreads) {
    const int64_t n = off[b + 1] - off[b];
    const int nq = (int)((n + tile_rows - 1) / tile_rows);
    for (int t = 0; t < nq; ++t) atomicAdd(&cnt[t < nbins ? t : nbins - 1], 1);
  }
  __syncthreads();
  // start[t] = number of items with a larger bin (descending order), by a
  // Hillis-Steele suffix scan in shared memory
  for (int i = tid; i < nbins; i += kPlanThreads) start[i] = cnt[i];
  __syncthreads();
  for (int o = 1; o < nbins; o <<= 1) {
    int v[kPlanBins / kPlanThreads];
#pragma unroll
    for (int r = 0; r < kPlanBins / kPlanThreads; ++r) {
      const int i = tid + r * kPlanThreads;
      v[r] = (i < nbins && i + o < nbins) ? start[i + o] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kPlanBins / kPlanThreads; ++r) {
      const int i = tid + r * kPlanThreads;
      if (i < nbins) start[i] += v[r];
    }
    __syncthreads();
  }
  // inclusive suffix sum -> exclusive, then reuse cnt as the fill cursor
  for (int i = tid; i < nbins; i += kPlanThreads) {
    start[i] -= cnt[i];
    cnt[i] = 0;
  }
  __syncthreads();
  for (int b = tid; b < B; b += kPlanThreads) {
    const int64_t n = off[b + 1] - off[b];
    const int nq = (int)((n + tile_rows - 1) / tile_rows);
    for (int t = 0; t < nq; ++t) {
      const int bin = t < nbins ? t : nbins - 1;
      const int pos = start[bin] + atomicAdd(&cnt[bin], 1);
      if (pos < n_items) items[pos] = make_int2(b, t);
    }
  }
}

hipError_t launch_plan_causal(const int64_t* offsets, int B, int tile_rows, int max_tiles,
                              int2* items, int n_items, hipStream_t s) {
  int nbins = max_tiles < 1 ? 1 : (max_tiles > kPlanBins ? kPlanBins : max_tiles);
  hipLaunchKernelGGL(plan_causal_kernel, dim3(1), dim3(kPlanThreads), 0, s, offsets, B, tile_rows,
                     nbins, items, n_items);
  return hipGetLastError();
}

}  // namespace hstu
