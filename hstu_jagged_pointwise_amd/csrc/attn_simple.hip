// Generic HSTU attention kernel on the vector ALUs (fp32 math throughout).
//
// Computes eq. 2 of the HSTU layer ("What an HSTU layer changes", HSTU
// chapter): O_i = sum_j SiLU(q_i.k_j + rab(i,j)) / N * v_j. There is no
// softmax, so no running max and no rescaling: one pass over the keys,
// accumulating pointwise-activated scores times values.
// This kernel serves fp32 inputs, mixed head widths and bias tables too large
// for the MFMA kernel's LDS. A workgroup of 256 threads owns 64 query rows of
// one head. It walks the visible keys in tiles of 16 held in LDS. Each thread
// owns one query row and a quarter of its output columns.
#include "attn_common.h"

namespace hstu {

namespace {
constexpr int SBM = kSimpleRows;  // query rows per workgroup
constexpr int SBN = 16;           // keys per LDS tile
}  // namespace

template <typename T, int DQK, int DV, bool CAND>
__global__ __launch_bounds__(256) void attn_simple_kernel(AttnArgs a) {
  __shared__ float Qs[SBM][DQK + 1];
  __shared__ float Ks[SBN][DQK + 1];
  __shared__ float Vs[SBN][DV];
  __shared__ float Ps[SBM][SBN + 1];
  __shared__ int64_t tks[SBN];

  const TileDecode t = decode<CAND>(a, SBM);
  if (!t.valid) return;  // uniform across the workgroup
  const int tid = threadIdx.x;
  const int row = tid >> 2, sub = tid & 3;
  const int h = t.h;
  const T* q = (const T*)a.q;
  const T* k = (const T*)a.k;
  const T* v = (const T*)a.v;
  const bool has_pos = a.rab_pos != nullptr;
  const bool has_time = a.rab_time != nullptr && a.ts_q != nullptr && a.ts_k != nullptr;
  const float* rp = has_pos ? a.rab_pos + (int64_t)h * a.P : nullptr;
  const float* rt = has_time ? a.rab_time + (int64_t)h * a.T : nullptr;

  for (int i = tid; i < SBM * DQK; i += 256) {
    const int r = i / DQK, c = i % DQK;
    Qs[r][c] = r < t.rows ? to_f32<T>(q[(t.q_local + r) * a.ld_q + (int64_t)h * DQK + c]) : 0.f;
  }
  const bool row_ok = row < t.rows;
  const int64_t tq = (has_time && row_ok) ? a.ts_q[t.q_base + row] : 0;
  const int64_t qpos = CAND ? t.qpos0 : t.qpos0 + row;

  constexpr int NC = DV / 4;
  float acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = 0.f;

  for (int64_t k0 = 0; k0 < t.kend; k0 += SBN) {
    __syncthreads();
    for (int i = tid; i < SBN * DQK; i += 256) {
      const int r = i / DQK, c = i % DQK;
      Ks[r][c] = (k0 + r < t.nk) ? to_f32<T>(k[(t.k_base + k0 + r) * a.ld_k + (int64_t)h * DQK + c])
                                 : 0.f;
    }
    for (int i = tid; i < SBN * DV; i += 256) {
      const int r = i / DV, c = i % DV;
      Vs[r][c] = (k0 + r < t.nk) ? to_f32<T>(v[(t.k_base + k0 + r) * a.ld_v + (int64_t)h * DV + c])
                                 : 0.f;
    }
    if (tid < SBN) tks[tid] = (has_time && k0 + tid < t.nk) ? a.ts_k[t.k_base + k0 + tid] : 0;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < SBN / 4; ++m) {
      const int key = sub + 4 * m;
      const int64_t j = k0 + key;
      float s = 0.f;
#pragma unroll 8
      for (int c = 0; c < DQK; ++c) s = fmaf(Qs[row][c], Ks[key][c], s);
      const bool vis = row_ok && j < t.kend && (CAND || j <= qpos);
      float p = 0.f;
      if (vis) {
        float x = s;
        if (has_pos) x += rp[pos_bucket((int)(qpos - j), a.P)];
        if (has_time) {
          const int bt = time_bucket64(tq, tks[key]);
          x += rt[bt < a.T - 1 ? bt : a.T - 1];
        }
        p = silu_precise(x);
      }
      Ps[row][key] = p;
    }
    __syncthreads();
#pragma unroll 4
    for (int key = 0; key < SBN; ++key) {
      const float p = Ps[row][key];
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] = fmaf(p, Vs[key][c * 4 + sub], acc[c]);
    }
  }
  if (!row_ok) return;
  if (CAND) {
    // the candidate's own key: relative position 0, elapsed time 0
    const T* kc = (const T*)a.kc;
    const T* vc = (const T*)a.vc;
    float s = 0.f;
    for (int c = 0; c < DQK; ++c)
      s = fmaf(Qs[row][c], to_f32<T>(kc[(t.q_local + row) * a.ld_kc + (int64_t)h * DQK + c]), s);
    if (has_pos) s += rp[0];
    if (has_time) s += rt[0];
    const float p = silu_precise(s);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      acc[c] = fmaf(p, to_f32<T>(vc[(t.q_local + row) * a.ld_vc + (int64_t)h * DV + c * 4 + sub]),
                    acc[c]);
  }
  const int64_t obase = (t.q_local + row) * a.ld_o + (int64_t)h * DV;
  if (a.out_f32) {
    float* o = (float*)a.out;
#pragma unroll
    for (int c = 0; c < NC; ++c) o[obase + c * 4 + sub] = acc[c] * a.inv_n;
  } else {
    T* o = (T*)a.out;
#pragma unroll
    for (int c = 0; c < NC; ++c) o[obase + c * 4 + sub] = from_f32<T>(acc[c] * a.inv_n);
  }
}

template <typename T, bool CAND>
static hipError_t dispatch_simple(const AttnArgs& a, dim3 grid, hipStream_t s) {
#define HSTU_SIMPLE_CASE(DQ, DVV)                                                               \
  if (a.d_qk == DQ && a.d_v == DVV) {                                                           \
    hipLaunchKernelGGL((attn_simple_kernel<T, DQ, DVV, CAND>), grid, dim3(256), 0, s, a);       \
    return hipGetLastError();                                                                   \
  }
  HSTU_SIMPLE_CASE(32, 32) HSTU_SIMPLE_CASE(32, 64) HSTU_SIMPLE_CASE(32, 128)
  HSTU_SIMPLE_CASE(64, 32) HSTU_SIMPLE_CASE(64, 64) HSTU_SIMPLE_CASE(64, 128)
  HSTU_SIMPLE_CASE(128, 32) HSTU_SIMPLE_CASE(128, 64) HSTU_SIMPLE_CASE(128, 128)
#undef HSTU_SIMPLE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_attn_simple(const AttnArgs& a, int use_bf16, bool cand, hipStream_t s) {
  dim3 grid;
  if (!cand) {
    grid = dim3((unsigned)a.n_items * (unsigned)a.H);
  } else {
    grid = dim3((unsigned)((a.max_user_rows + SBM - 1) / SBM) * (unsigned)a.H, (unsigned)a.n_users);
  }
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  if (use_bf16) return cand ? dispatch_simple<bf16, true>(a, grid, s) : dispatch_simple<bf16, false>(a, grid, s);
  return cand ? dispatch_simple<float, true>(a, grid, s) : dispatch_simple<float, false>(a, grid, s);
}

}  // namespace hstu
