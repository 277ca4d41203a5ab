// Backward pass of the HSTU pointwise attention (eq. 2, "What an HSTU layer
// changes", HSTU chapter) on the vector ALUs, any supported widths: fp32
// accumulation, with the scores and the activation in fp64.
//
// Forward, per head and visible pair j <= i:
//   z_ij = q_i.k_j + rab(i, j),  a_ij = SiLU(z_ij) / N,  o_i = sum_j a_ij v_j.
// With g_i = dL/do_i:
//   dv_j = sum_i a_ij g_i,  dz_ij = (g_i.v_j) SiLU'(z_ij) / N,
//   dq_i = sum_j dz_ij k_j,  dk_j = sum_i dz_ij q_i,
//   d rab_pos[h][bp_ij] and d rab_time[h][bt_ij] collect dz_ij.
// There is no softmax, so unlike softmax attention no row statistic of the
// forward pass is needed: every pair's gradient depends on that pair alone.
//
// Two kernels, so that no output is summed by atomics across workgroups:
// * the key-side kernel: one workgroup per (64-key tile, head) walks the queries
//   that see the tile and accumulates dk and dv in registers. It also sums dz by
//   bucket into per-wave LDS bins and writes one partial row per workgroup;
// * the query-side kernel: one workgroup per (64-query tile, head) walks the
//   visible keys and accumulates dq.
// A last kernel adds the bucket partials of all work items in a fixed order.
#include "attn_common.h"

namespace hstu {

namespace {
constexpr int BR = kSimpleRows;  // rows (keys or queries) owned by a workgroup
constexpr int BS = 16;           // rows of the other side per LDS step
constexpr int kBwdWaves = 4;

// SiLU(z) / N and SiLU'(z) / N from one sigmoid, in fp64. Where z is very negative,
// a = SiLU(z) / N is tiny and its relative error equals the absolute error of z,
// so z (the q.k and g.v dot products) is accumulated in fp64 too: a key near the
// end of a sequence has few queries, and its dv and dk rows are made of such terms.
__device__ __forceinline__ void silu_and_grad(double z, float inv_n, float* a, float* da) {
  const double sg = 1.0 / (1.0 + exp(-z));
  *a = (float)(z * sg * (double)inv_n);
  *da = (float)(sg * (1.0 + z * (1.0 - sg)) * (double)inv_n);
}

__device__ __forceinline__ int time_bucket_clamped(int64_t tq, int64_t tk, int T) {
  const int bt = time_bucket64(tq, tk);
  return bt < T - 1 ? bt : T - 1;
}
}  // namespace

// Sequence, first row and row count of the key tile of a work item. The planner
// lists (sequence, tile t) longest first for the query side, where tile t costs
// t + 1 steps; key tile ntiles - 1 - t costs as many on the key side.
struct BwdTile {
  int seq;
  int64_t base;  // global row of the sequence's first action
  int64_t n;     // sequence length
  int64_t r0;    // first row of the tile within the sequence
  int rows;
  bool valid;
};

__device__ __forceinline__ BwdTile bwd_decode(const AttnBwdArgs& a, int item, bool key_side) {
  BwdTile t;
  t.valid = false;
  if (item >= a.n_items) return t;
  const uint64_t raw = sload(reinterpret_cast<const uint64_t*>(a.items + item));
  const int seq = (int)(uint32_t)raw, tile = (int)(uint32_t)(raw >> 32);
  if (seq < 0 || seq >= a.batch || tile < 0) return t;
  t.seq = seq;
  t.base = sload(a.offsets + seq);
  t.n = sload(a.offsets + seq + 1) - t.base;
  const int64_t ntiles = (t.n + BR - 1) / BR;
  if (tile >= ntiles) return t;
  const int64_t kt = key_side ? ntiles - 1 - tile : tile;
  t.r0 = kt * BR;
  t.rows = (int)(t.n - t.r0 < BR ? t.n - t.r0 : BR);
  t.valid = true;
  return t;
}

template <typename T, int DQK, int DV>
__global__ __launch_bounds__(256) void attn_bwd_kv_simple(AttnBwdArgs a) {
  __shared__ float Ks[BR][DQK + 1];
  __shared__ float Vs[BR][DV + 1];
  __shared__ float Qs[BS][DQK + 1];
  __shared__ float Gs[BS][DV + 1];
  __shared__ float Ps[BR][BS + 1];
  __shared__ float Zs[BR][BS + 1];
  __shared__ int64_t tqs[BS];
  extern __shared__ float bins[];  // [kBwdWaves][P + T] when bias_partial is set

  const int item = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const BwdTile t = bwd_decode(a, item, true);
  const int tid = threadIdx.x, row = tid >> 2, sub = tid & 3, w = tid >> 6;
  const int nb = a.P + a.T;
  float* my_bins = bins + w * nb;
  if (a.bias_partial) {
    for (int i = tid; i < kBwdWaves * nb; i += 256) bins[i] = 0.f;
  }
  if (t.valid) {
    const T* q = (const T*)a.q;
    const T* k = (const T*)a.k;
    const T* v = (const T*)a.v;
    const T* g = (const T*)a.dout;
    const bool has_time = a.ts != nullptr;
    const float* rp = a.rab_pos ? a.rab_pos + (int64_t)h * a.P : nullptr;
    const float* rt = (a.rab_time && has_time) ? a.rab_time + (int64_t)h * a.T : nullptr;
    for (int i = tid; i < BR * DQK; i += 256) {
      const int r = i / DQK, c = i % DQK;
      Ks[r][c] = r < t.rows ? to_f32<T>(k[(t.base + t.r0 + r) * a.ld_k + (int64_t)h * DQK + c]) : 0.f;
    }
    for (int i = tid; i < BR * DV; i += 256) {
      const int r = i / DV, c = i % DV;
      Vs[r][c] = r < t.rows ? to_f32<T>(v[(t.base + t.r0 + r) * a.ld_v + (int64_t)h * DV + c]) : 0.f;
    }
    const bool row_ok = row < t.rows;
    const int64_t j = t.r0 + row;  // this thread's key position
    const int64_t tk = (has_time && row_ok) ? a.ts[t.base + j] : 0;
    constexpr int NK = DQK / 4, NV = DV / 4;
    float dk[NK], dv[NV];
#pragma unroll
    for (int c = 0; c < NK; ++c) dk[c] = 0.f;
#pragma unroll
    for (int c = 0; c < NV; ++c) dv[c] = 0.f;

    for (int64_t q0 = t.r0; q0 < t.n; q0 += BS) {
      __syncthreads();
      for (int i = tid; i < BS * DQK; i += 256) {
        const int r = i / DQK, c = i % DQK;
        Qs[r][c] = q0 + r < t.n ? to_f32<T>(q[(t.base + q0 + r) * a.ld_q + (int64_t)h * DQK + c]) : 0.f;
      }
      for (int i = tid; i < BS * DV; i += 256) {
        const int r = i / DV, c = i % DV;
        Gs[r][c] = q0 + r < t.n ? to_f32<T>(g[(t.base + q0 + r) * a.ld_do + (int64_t)h * DV + c]) : 0.f;
      }
      if (tid < BS) tqs[tid] = (has_time && q0 + tid < t.n) ? a.ts[t.base + q0 + tid] : 0;
      __syncthreads();
#pragma unroll
      for (int m = 0; m < BS / 4; ++m) {
        const int qi = sub + 4 * m;
        const int64_t i = q0 + qi;
        float p = 0.f, dz = 0.f;
        if (row_ok && i < t.n && j <= i) {
          double s = 0.0, dp = 0.0;
#pragma unroll 8
          for (int c = 0; c < DQK; ++c) s = fma((double)Qs[qi][c], (double)Ks[row][c], s);
#pragma unroll 8
          for (int c = 0; c < DV; ++c) dp = fma((double)Gs[qi][c], (double)Vs[row][c], dp);
          const int bp = pos_bucket((int)(i - j), a.P);
          const int bt = has_time ? time_bucket_clamped(tqs[qi], tk, a.T) : 0;
          double z = s;
          if (rp) z += rp[bp];
          if (rt) z += rt[bt];
          float dsl;
          silu_and_grad(z, a.inv_n, &p, &dsl);
          dz = (float)(dp * (double)dsl);
          if (a.bias_partial) {
            atomicAdd(&my_bins[bp], dz);
            if (has_time) atomicAdd(&my_bins[a.P + bt], dz);
          }
        }
        Ps[row][qi] = p;
        Zs[row][qi] = dz;
      }
      __syncthreads();
#pragma unroll 4
      for (int qi = 0; qi < BS; ++qi) {
        const float p = Ps[row][qi], dz = Zs[row][qi];
#pragma unroll
        for (int c = 0; c < NV; ++c) dv[c] = fmaf(p, Gs[qi][c * 4 + sub], dv[c]);
#pragma unroll
        for (int c = 0; c < NK; ++c) dk[c] = fmaf(dz, Qs[qi][c * 4 + sub], dk[c]);
      }
    }
    if (row_ok) {
      T* dko = (T*)a.dk;
      T* dvo = (T*)a.dv;
      const int64_t r = t.base + j;
#pragma unroll
      for (int c = 0; c < NK; ++c) dko[r * a.ld_dk + (int64_t)h * DQK + c * 4 + sub] = from_f32<T>(dk[c]);
#pragma unroll
      for (int c = 0; c < NV; ++c) dvo[r * a.ld_dv + (int64_t)h * DV + c * 4 + sub] = from_f32<T>(dv[c]);
    }
  }
  if (a.bias_partial) {  // this work item's bucket sums, waves added in a fixed order
    __syncthreads();
    float* out = a.bias_partial + ((int64_t)item * a.H + h) * nb;
    for (int i = tid; i < nb; i += 256) {
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < kBwdWaves; ++q) s += bins[q * nb + i];
      out[i] = s;
    }
  }
}

template <typename T, int DQK, int DV>
__global__ __launch_bounds__(256) void attn_bwd_q_simple(AttnBwdArgs a) {
  __shared__ float Qs[BR][DQK + 1];
  __shared__ float Gs[BR][DV + 1];
  __shared__ float Ks[BS][DQK + 1];
  __shared__ float Vs[BS][DV + 1];
  __shared__ float Zs[BR][BS + 1];
  __shared__ int64_t tks[BS];

  const int item = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const BwdTile t = bwd_decode(a, item, false);
  if (!t.valid) return;  // uniform across the workgroup
  const int tid = threadIdx.x, row = tid >> 2, sub = tid & 3;
  const T* q = (const T*)a.q;
  const T* k = (const T*)a.k;
  const T* v = (const T*)a.v;
  const T* g = (const T*)a.dout;
  const bool has_time = a.ts != nullptr;
  const float* rp = a.rab_pos ? a.rab_pos + (int64_t)h * a.P : nullptr;
  const float* rt = (a.rab_time && has_time) ? a.rab_time + (int64_t)h * a.T : nullptr;
  for (int i = tid; i < BR * DQK; i += 256) {
    const int r = i / DQK, c = i % DQK;
    Qs[r][c] = r < t.rows ? to_f32<T>(q[(t.base + t.r0 + r) * a.ld_q + (int64_t)h * DQK + c]) : 0.f;
  }
  for (int i = tid; i < BR * DV; i += 256) {
    const int r = i / DV, c = i % DV;
    Gs[r][c] = r < t.rows ? to_f32<T>(g[(t.base + t.r0 + r) * a.ld_do + (int64_t)h * DV + c]) : 0.f;
  }
  const bool row_ok = row < t.rows;
  const int64_t i = t.r0 + row;  // this thread's query position
  const int64_t tq = (rt && row_ok) ? a.ts[t.base + i] : 0;
  const int64_t kend = t.r0 + t.rows;
  constexpr int NK = DQK / 4;
  float dq[NK];
#pragma unroll
  for (int c = 0; c < NK; ++c) dq[c] = 0.f;
  for (int64_t k0 = 0; k0 < kend; k0 += BS) {
    __syncthreads();
    for (int x = tid; x < BS * DQK; x += 256) {
      const int r = x / DQK, c = x % DQK;
      Ks[r][c] = k0 + r < kend ? to_f32<T>(k[(t.base + k0 + r) * a.ld_k + (int64_t)h * DQK + c]) : 0.f;
    }
    for (int x = tid; x < BS * DV; x += 256) {
      const int r = x / DV, c = x % DV;
      Vs[r][c] = k0 + r < kend ? to_f32<T>(v[(t.base + k0 + r) * a.ld_v + (int64_t)h * DV + c]) : 0.f;
    }
    if (tid < BS) tks[tid] = (rt && k0 + tid < kend) ? a.ts[t.base + k0 + tid] : 0;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < BS / 4; ++m) {
      const int key = sub + 4 * m;
      const int64_t j = k0 + key;
      float dz = 0.f;
      if (row_ok && j <= i) {
        double s = 0.0, dp = 0.0;
#pragma unroll 8
        for (int c = 0; c < DQK; ++c) s = fma((double)Qs[row][c], (double)Ks[key][c], s);
#pragma unroll 8
        for (int c = 0; c < DV; ++c) dp = fma((double)Gs[row][c], (double)Vs[key][c], dp);
        double z = s;
        if (rp) z += rp[pos_bucket((int)(i - j), a.P)];
        if (rt) z += rt[time_bucket_clamped(tq, tks[key], a.T)];
        float p, dsl;
        silu_and_grad(z, a.inv_n, &p, &dsl);
        dz = (float)(dp * (double)dsl);
      }
      Zs[row][key] = dz;
    }
    __syncthreads();
#pragma unroll 4
    for (int key = 0; key < BS; ++key) {
      const float dz = Zs[row][key];
#pragma unroll
      for (int c = 0; c < NK; ++c) dq[c] = fmaf(dz, Ks[key][c * 4 + sub], dq[c]);
    }
  }
  if (!row_ok) return;
  T* dqo = (T*)a.dq;
#pragma unroll
  for (int c = 0; c < NK; ++c)
    dqo[(t.base + i) * a.ld_dq + (int64_t)h * DQK + c * 4 + sub] = from_f32<T>(dq[c]);
}

// d_rab_pos[h][p] = sum over items of partial[item][h][p] (d_rab_time: bins P..P+T-1),
// one wavefront per output, lanes strided over items, then a fixed butterfly.
__global__ __launch_bounds__(256) void bias_grad_reduce_kernel(const float* __restrict__ partial,
                                                               int n_items, int H, int P, int T,
                                                               float* __restrict__ d_pos,
                                                               float* __restrict__ d_time) {
  const int lane = threadIdx.x & 63;
  const int64_t o = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nb = P + T;
  if (o >= (int64_t)H * nb) return;
  const int h = (int)(o / nb), bin = (int)(o % nb);
  float s = 0.f;
  if (partial)
    for (int it = lane; it < n_items; it += 64) s += partial[((int64_t)it * H + h) * nb + bin];
  s = wave_sum(s);
  if (lane) return;
  if (bin < P) {
    if (d_pos) d_pos[(int64_t)h * P + bin] = s;
  } else if (d_time) {
    d_time[(int64_t)h * T + (bin - P)] = s;
  }
}

template <typename T>
static hipError_t dispatch_bwd_simple(const AttnBwdArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.n_items * (unsigned)a.H);
  const size_t bins = a.bias_partial ? (size_t)kBwdWaves * (a.P + a.T) * sizeof(float) : 0;
#define HSTU_BWD_CASE(DQ, DVV)                                                                   \
  if (a.d_qk == DQ && a.d_v == DVV) {                                                            \
    hipLaunchKernelGGL((attn_bwd_kv_simple<T, DQ, DVV>), grid, dim3(256), bins, s, a);          \
    hipLaunchKernelGGL((attn_bwd_q_simple<T, DQ, DVV>), grid, dim3(256), 0, s, a);              \
    return hipGetLastError();                                                                    \
  }
  HSTU_BWD_CASE(32, 32) HSTU_BWD_CASE(32, 64) HSTU_BWD_CASE(32, 128)
  HSTU_BWD_CASE(64, 32) HSTU_BWD_CASE(64, 64) HSTU_BWD_CASE(64, 128)
  HSTU_BWD_CASE(128, 32) HSTU_BWD_CASE(128, 64) HSTU_BWD_CASE(128, 128)
#undef HSTU_BWD_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_attn_bwd_simple(const AttnBwdArgs& a, int use_bf16, hipStream_t s) {
  if (a.n_items <= 0 || a.H <= 0) return hipSuccess;
  return use_bf16 ? dispatch_bwd_simple<bf16>(a, s) : dispatch_bwd_simple<float>(a, s);
}

hipError_t launch_bias_grad_reduce(const float* partial, int n_items, int H, int P, int T,
                                   float* d_rab_pos, float* d_rab_time, hipStream_t s) {
  if (!d_rab_pos && !d_rab_time) return hipSuccess;
  const int64_t outs = (int64_t)H * (P + T);
  hipLaunchKernelGGL(bias_grad_reduce_kernel, dim3((unsigned)((outs + 3) / 4)), dim3(256), 0, s,
                     partial, n_items, H, P, T, d_rab_pos, d_rab_time);
  return hipGetLastError();
}

}  // namespace hstu
