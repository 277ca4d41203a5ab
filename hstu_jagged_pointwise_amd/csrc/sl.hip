// Stochastic Length sampling of jagged training sequences (HSTU chapter, "Three
// more scaling components", Stochastic Length: long histories are usually cut to
// a shorter subsequence, occasionally kept whole; alpha = 1.6 turns 4,096 into 776).
//
// The host decides each sequence's new length (n, or L = floor(N^(alpha/2)));
// these kernels pick which actions a cut sequence keeps and gather them. A cut
// sequence keeps the m positions whose (key, position) pairs are the m smallest,
// in their original order; with uniform random keys that is a uniformly random
// order-preserving subsequence.
#include "common.h"
#include "kernels.h"

namespace hstu {

namespace {
constexpr int kSlThreads = 256;   // also the number of histogram bins
constexpr int kSlWaves = kSlThreads / 64;
constexpr int kSlLdsKeys = 8192;  // sequences up to this length keep their keys in LDS (32 KB)

// Lane l's mask of the lanes below it.
__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}
}  // namespace

// Workgroup-shared state of the selection.
struct SlShared {
  uint32_t keys[kSlLdsKeys];
  int hist[kSlThreads];
  uint32_t prefix;
  int rank;
  int wave_lt[kSlWaves], wave_eq[kSlWaves];
};

// Radix select and ordered compaction of one cut sequence of n keys, read from LDS
// (kLds, n <= kSlLdsKeys) or from global memory. kSlBatch independent loads are
// issued before they are used, so their latencies overlap.
constexpr int kSlBatch = 8;

template <bool kLds>
__device__ __forceinline__ void sl_select_seq(SlShared& sh, const uint32_t* __restrict__ gk, int n,
                                              int m, int64_t s, int64_t* __restrict__ out_src) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  auto key_at = [&](int j) -> uint32_t {
    if constexpr (kLds) return sh.keys[j];
    else return gk[j];
  };
  if (tid == 0) {
    sh.prefix = 0;
    sh.rank = m;  // 1-based rank still to find among the keys that match the prefix
  }
  uint32_t mask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    sh.hist[tid] = 0;
    __syncthreads();
    const uint32_t prefix = sh.prefix;
    for (int j0 = tid; j0 < n; j0 += kSlThreads * kSlBatch) {
      uint32_t v[kSlBatch];
#pragma unroll
      for (int u = 0; u < kSlBatch; ++u) {
        const int j = j0 + u * kSlThreads;
        v[u] = j < n ? key_at(j) : 0u;
      }
#pragma unroll
      for (int u = 0; u < kSlBatch; ++u) {
        const int j = j0 + u * kSlThreads;
        if (j < n && (v[u] & mask) == prefix) atomicAdd(&sh.hist[(v[u] >> shift) & 255u], 1);
      }
    }
    __syncthreads();
    if (w == 0) {  // wave 0 finds the bin holding the rank: lane l owns bins 4l .. 4l+3
      const int h0 = sh.hist[4 * lane], h1 = sh.hist[4 * lane + 1], h2 = sh.hist[4 * lane + 2],
                h3 = sh.hist[4 * lane + 3];
      const int own = h0 + h1 + h2 + h3;
      int incl = own;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(incl, d);
        if (lane >= d) incl += t;
      }
      const int k = sh.rank;
      const uint64_t hit = __ballot(incl >= k);
      if (lane == __ffsll((unsigned long long)hit) - 1) {
        int c = incl - own, d = 4 * lane;
        if (c + h0 < k) {
          c += h0, ++d;
          if (c + h1 < k) {
            c += h1, ++d;
            if (c + h2 < k) c += h2, ++d;
          }
        }
        sh.rank = k - c;
        sh.prefix = prefix | ((uint32_t)d << shift);
      }
    }
    mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t K = sh.prefix;  // key of the m-th smallest pair
  const int r = sh.rank;         // pairs with key K that are kept (1..count of K)
  // ordered compaction: wave w owns positions [w*C, min((w+1)*C, n)), C a multiple of 64
  const int C = ((n + kSlWaves - 1) / kSlWaves + 63) & ~63;
  const int lo = min(w * C, n), hi = min(lo + C, n);
  int lt = 0, eq = 0;
  for (int j0 = lo + lane; j0 < hi; j0 += 64 * kSlBatch) {
    uint32_t v[kSlBatch];
#pragma unroll
    for (int u = 0; u < kSlBatch; ++u) {
      const int j = j0 + 64 * u;
      v[u] = j < hi ? key_at(j) : 0xffffffffu;
    }
#pragma unroll
    for (int u = 0; u < kSlBatch; ++u) {
      const bool in = j0 + 64 * u < hi;
      lt += in && v[u] < K;
      eq += in && v[u] == K;
    }
  }
  // wave totals
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    lt += __shfl_xor(lt, d);
    eq += __shfl_xor(eq, d);
  }
  if (lane == 0) {
    sh.wave_lt[w] = lt;
    sh.wave_eq[w] = eq;
  }
  __syncthreads();
  int out = 0, eq_seen = 0;  // kept pairs and key-K pairs before this wave's chunk
  for (int q = 0; q < w; ++q) {
    out += sh.wave_lt[q] + min(max(r - eq_seen, 0), sh.wave_eq[q]);
    eq_seen += sh.wave_eq[q];
  }
  const uint64_t below = lanes_below(lane);
  for (int j0 = lo + lane; j0 < hi + lane; j0 += 64 * kSlBatch) {
    uint32_t v[kSlBatch];
#pragma unroll
    for (int u = 0; u < kSlBatch; ++u) {
      const int j = j0 + 64 * u;
      v[u] = j < hi ? key_at(j) : 0xffffffffu;
    }
#pragma unroll
    for (int u = 0; u < kSlBatch; ++u) {
      const int j = j0 + 64 * u;
      const bool is_eq = j < hi && v[u] == K;
      const uint64_t eq_bal = __ballot(is_eq);
      const bool keep = (j < hi && v[u] < K) || (is_eq && eq_seen + __popcll(eq_bal & below) < r);
      const uint64_t keep_bal = __ballot(keep);
      if (keep) out_src[out + __popcll(keep_bal & below)] = s + j;
      out += __popcll(keep_bal);
      eq_seen += __popcll(eq_bal);
    }
  }
}

// One workgroup per sequence: src[new_off[b] + i] = global source row of the i-th kept action.
//
// A cut sequence keeps the m smallest (key, position) pairs. A radix select over
// the 32-bit keys, most significant byte first, finds the key K of the m-th
// smallest pair and how many of the pairs with key K are kept (r, the ones with
// the smallest positions). Then every position with key < K is kept, and so are
// the first r positions with key == K.
__global__ __launch_bounds__(kSlThreads) void sl_select_kernel(const int64_t* __restrict__ off,
                                                               const int64_t* __restrict__ new_off,
                                                               const uint32_t* __restrict__ keys,
                                                               int64_t* __restrict__ src) {
  __shared__ SlShared sh;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int64_t s = off[b], n = off[b + 1] - s;
  const int64_t o = new_off[b], m = new_off[b + 1] - o;
  if (m == n) {  // kept whole
    for (int64_t j = tid; j < n; j += kSlThreads) src[o + j] = s + j;
    return;
  }
  if (m <= 0) return;
  const uint32_t* gk = keys + s;
  if (n <= kSlLdsKeys) {
    // stage the keys: 16-byte loads for the aligned middle, single keys for the ends
    const int nn = (int)n;
    const int mis = (int)((reinterpret_cast<uintptr_t>(gk) >> 2) & 3);
    const int head = min(nn, (4 - mis) & 3);
    const int nv = (nn - head) >> 2;
    const u32x4* gv = reinterpret_cast<const u32x4*>(gk + head);
#pragma unroll 4
    for (int i = tid; i < nv; i += kSlThreads) {
      const u32x4 v = gv[i];
      uint32_t* d = &sh.keys[head + 4 * i];
      d[0] = v.x, d[1] = v.y, d[2] = v.z, d[3] = v.w;
    }
    if (tid < head) sh.keys[tid] = gk[tid];
    const int tail = head + 4 * nv;
    if (tail + tid < nn) sh.keys[tail + tid] = gk[tail + tid];  // at most 3 keys
    sl_select_seq<true>(sh, gk, (int)n, (int)m, s, src + o);
  } else {
    sl_select_seq<false>(sh, gk, (int)n, (int)m, s, src + o);  // fewer than 2^31 rows
  }
}

// out_x[r] = x[src[r]] (row_bytes a multiple of 16), out_ts[r] = ts[src[r]].
__global__ __launch_bounds__(256) void sl_gather_kernel(const int64_t* __restrict__ src,
                                                        int64_t rows, const char* __restrict__ x,
                                                        int64_t row_bytes, const int64_t* __restrict__ ts,
                                                        char* __restrict__ out_x,
                                                        int64_t* __restrict__ out_ts) {
  const int64_t chunks = x ? row_bytes / 16 : 0;
  const int64_t per_row = chunks + (ts ? 1 : 0);
  const int64_t total = rows * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / per_row, c = i % per_row;
    const int64_t from = src[r];
    if (c < chunks) {
      *reinterpret_cast<u32x4*>(out_x + r * row_bytes + 16 * c) =
          *reinterpret_cast<const u32x4*>(x + from * row_bytes + 16 * c);
    } else {
      out_ts[r] = ts[from];
    }
  }
}

hipError_t launch_sl_select(const int64_t* off, const int64_t* new_off, int B,
                            const uint32_t* keys, int64_t* src, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(sl_select_kernel, dim3((unsigned)B), dim3(kSlThreads), 0, s, off, new_off,
                     keys, src);
  return hipGetLastError();
}

hipError_t launch_sl_gather(const int64_t* src, int64_t rows, const void* x, int64_t row_bytes,
                            const int64_t* ts, void* out_x, int64_t* out_ts, hipStream_t s) {
  if (rows <= 0 || (!x && !ts)) return hipSuccess;
  const int64_t per_row = (x ? row_bytes / 16 : 0) + (ts ? 1 : 0);
  const int64_t total = rows * per_row;
  const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(sl_gather_kernel, dim3(grid), dim3(256), 0, s, src, rows,
                     (const char*)x, row_bytes, ts, (char*)out_x, out_ts);
  return hipGetLastError();
}

}  // namespace hstu
