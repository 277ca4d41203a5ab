// Jagged tile planner. The HSTU chapter ("Three more scaling components",
// ragged kernels) says padding every user to the maximum length wastes most
// of the compute. This planner emits one work item per (sequence, query tile)
// that actually exists, with no padding to the longest sequence. Under the
// causal mask a query tile t needs key tiles 0..t only, so its cost grows with
// t. Items are ordered by decreasing t (longest first), which makes the
// dispatch order approximate longest-processing-time scheduling across the
// compute units. Within one t the order follows LDS atomics, so it can change
// from run to run. The forward outputs and dq, dk, dv never depend on it: every
// item writes its own rows. The bias-table gradients do, in their last bits:
// their per-item partial sums are added in item order.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace hstu {

constexpr int kPlanThreads = 1024;
constexpr int kPlanGroup = 32;  // threads per sequence in the planner's passes
constexpr int kPlanBins = 2048;
constexpr int kPlanMaxRangeGroups = 8192;  // key-range workgroups along x at most

// one workgroup of kPlanThreads threads
__device__ void plan_block(const int64_t* __restrict__ off, int B, int tile_rows, int nbins,
                           int2* __restrict__ items, int n_items) {
  __shared__ int cnt[kPlanBins];
  __shared__ int start[kPlanBins];
  const int tid = threadIdx.x;
  for (int i = tid; i < nbins; i += kPlanThreads) cnt[i] = 0;
  __syncthreads();
  // histogram of items by query-tile index (clamped into the last bin)
  // kPlanGroup threads per sequence, striding over its query tiles, so that a few long
  // sequences do not leave one thread to count all of their tiles
  const int grp = tid / kPlanGroup, gl = tid % kPlanGroup;
  for (int b = grp; b < B; b += kPlanThreads / kPlanGroup) {
    const int64_t n = off[b + 1] - off[b];
    const int nq = (int)((n + tile_rows - 1) / tile_rows);
    for (int t = gl; t < nq; t += kPlanGroup) atomicAdd(&cnt[t < nbins ? t : nbins - 1], 1);
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
  for (int b = grp; b < B; b += kPlanThreads / kPlanGroup) {
    const int64_t n = off[b + 1] - off[b];
    const int nq = (int)((n + tile_rows - 1) / tile_rows);
    for (int t = gl; t < nq; t += kPlanGroup) {
      const int bin = t < nbins ? t : nbins - 1;
      const int pos = start[bin] + atomicAdd(&cnt[bin], 1);
      if (pos < n_items) items[pos] = make_int2(b, t);
    }
  }
}

// Timestamp range of every 32-key block (the keys one attention wavefront
// classifies at a time). Each half-wavefront reduces one block; the attention
// kernel then decides a block's bias class from two scalar loads instead of
// reducing timestamps itself on every key tile.
__device__ void key_range_block(const int64_t* __restrict__ off, const int64_t* __restrict__ ts,
                                KeyRange* __restrict__ out, int b) {
  const int64_t s0 = off[b], n = off[b + 1] - s0;
  const int64_t nblk = (n + 31) / 32;
  const int64_t base = key_range_slot(s0, b);
  constexpr int kHalves = kPlanThreads / 32;
  const int l32 = threadIdx.x & 31, half = threadIdx.x >> 5;
  for (int64_t j = (int64_t)blockIdx.y * kHalves + half; j < nblk;
       j += (int64_t)gridDim.y * kHalves) {
    const int64_t key = 32 * j + l32;
    const bool ok = key < n;
    int64_t mn = ok ? ts[s0 + key] : INT64_MAX;
    int64_t mx = ok ? ts[s0 + key] : INT64_MIN;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) {  // stays inside the half-wavefront
      const int64_t a1 = __shfl_xor(mn, o, 64), a2 = __shfl_xor(mx, o, 64);
      mn = a1 < mn ? a1 : mn;
      mx = a2 > mx ? a2 : mx;
    }
    if (l32 == 0) out[base + j] = KeyRange{mn, mx};
  }
}

// The planner (workgroup (0, 0)) and, given timestamps, the key ranges (workgroups
// (1 + i, y), which take sequences i, i + gridDim.x - 1, ...) in one launch: they are
// independent and both small.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int64_t* __restrict__ off, int B,
                                                            int tile_rows, int nbins,
                                                            int2* __restrict__ items, int n_items,
                                                            const int64_t* __restrict__ ts,
                                                            KeyRange* __restrict__ kr) {
  if (blockIdx.x == 0) {
    if (blockIdx.y == 0) plan_block(off, B, tile_rows, nbins, items, n_items);
    return;
  }
  for (int b = (int)blockIdx.x - 1; b < B; b += (int)gridDim.x - 1) key_range_block(off, ts, kr, b);
}

hipError_t launch_plan(const int64_t* offsets, int B, int tile_rows, int max_tiles, int2* items,
                       int n_items, const int64_t* ts, int64_t max_len, KeyRange* kr,
                       hipStream_t s) {
  if (B <= 0) return hipSuccess;
  const int nbins = max_tiles < 1 ? 1 : (max_tiles > kPlanBins ? kPlanBins : max_tiles);
  const bool ranges = ts && kr && max_len > 0;
  const int64_t blocks = (max_len + 31) / 32;
  const unsigned gy =
      ranges ? (unsigned)std::min<int64_t>((blocks + kPlanThreads / 32 - 1) / (kPlanThreads / 32), 64)
             : 1u;
  // key-range workgroups stride over the sequences, so any batch size fits the grid
  const unsigned gx = ranges ? (unsigned)std::min<int64_t>(B, kPlanMaxRangeGroups) : 0u;
  const dim3 grid(1u + gx, gy);
  hipLaunchKernelGGL(plan_kernel, grid, dim3(kPlanThreads), 0, s, offsets, B, tile_rows, nbins,
                     items, n_items, ranges ? ts : nullptr, ranges ? kr : nullptr);
  return hipGetLastError();
}

}  // namespace hstu
