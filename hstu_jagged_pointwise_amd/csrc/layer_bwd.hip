// Kernels of the HSTU layer's backward pass other than attention and the GEMMs
// ("What an HSTU layer changes", HSTU chapter, eqs. 1 and 3):
//   * SiLU of the stored f1 pre-activation z1, and dz1 = d[U|V|Q|K] (.) SiLU'(z1);
//   * the backward of Norm(AV) (.) U (LayerNorm over the H*d_v row, biased variance):
//       y = xhat gamma + beta, out = y (.) u, with g = dL/dout:
//       du = g y,  dy = g u,  dxhat = dy gamma,
//       do = rstd (dxhat - mean(dxhat) - xhat mean(dxhat xhat)),
//       dgamma = sum over rows of dy xhat,  dbeta = sum over rows of dy;
//   * column sums (bias gradients) and split-K sums, each in a fixed order, so
//     results repeat bit for bit;
//   * a tiled transpose that feeds the weight-gradient GEMMs, whose reduction
//     runs over tokens.
// All of these are bound by HBM bandwidth; rows are read with coalesced accesses.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace hstu {

// ------------------------------------------------------------------ transpose
// out[c * ld_out + r] = in[r * ld_in + c] for r < R, c < C; out[c * ld_out + r] = 0
// for R <= r < Rpad. 64 x 64 tiles through LDS (padded row, no bank conflicts).
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ in, int64_t ld_in,
                                                        T* __restrict__ out, int64_t ld_out,
                                                        int64_t R, int64_t Rpad, int C) {
  __shared__ T tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.y * 64;
  const int c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i;
    const int c = c0 + tx;
    tile[i][tx] = (r < R && c < C) ? in[r * ld_in + c] : (T)0.f;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i;
    const int64_t r = r0 + tx;
    if (c < C && r < Rpad) out[(int64_t)c * ld_out + r] = tile[tx][i];
  }
}

hipError_t launch_transpose(const void* in, int64_t ld_in, void* out, int64_t ld_out, int64_t R,
                            int64_t Rpad, int C, int use_bf16, hipStream_t s) {
  if (Rpad <= 0 || C <= 0) return hipSuccess;
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)((Rpad + 63) / 64));
  if (use_bf16)
    hipLaunchKernelGGL(transpose_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)in, ld_in,
                       (bf16*)out, ld_out, R, Rpad, C);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, s, (const float*)in, ld_in,
                       (float*)out, ld_out, R, Rpad, C);
  return hipGetLastError();
}

// ------------------------------------------------------------------ column sums
// Sums over rows in a fixed order. A workgroup covers 16 columns; its 16 row groups
// (one per 16-lane slice) each add every 16th row (or chunk) in order, 8 loads in
// flight, and the 16 group sums are then added in group order through LDS. The
// result depends only on the data, never on timing.
constexpr int kSumGroups = 16;

template <typename T>
__device__ __forceinline__ float grouped_column_sum(const T* __restrict__ x, int64_t stride,
                                                    int64_t n, int64_t c, int g) {
  float s = 0.f;
  int64_t r = g;
  for (; r + 7 * kSumGroups < n; r += 8 * kSumGroups) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = to_f32<T>(x[(r + u * kSumGroups) * stride + c]);
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; r < n; r += kSumGroups) s += to_f32<T>(x[r * stride + c]);
  return s;
}

// out[c] = sum over r < n of x[r * stride + c] (zeros when n == 0).
template <typename T>
__global__ __launch_bounds__(256) void column_sum_kernel(const T* __restrict__ x, int64_t stride,
                                                         int64_t n, int64_t C,
                                                         float* __restrict__ out) {
  __shared__ float part[kSumGroups][16];
  const int cl = threadIdx.x & 15, g = threadIdx.x >> 4;
  const int64_t c = (int64_t)blockIdx.x * 16 + cl;
  part[g][cl] = c < C ? grouped_column_sum<T>(x, stride, n, c, g) : 0.f;
  __syncthreads();
  if (g == 0 && c < C) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < kSumGroups; ++q) s += part[q][cl];
    out[c] = s;
  }
}

// out[c] = sum over k < n of partial[k * stride + c] for wide outputs (split-K sums):
// one thread per column, the few partials in order.
__global__ __launch_bounds__(256) void sum_rows_wide_kernel(const float* __restrict__ partial,
                                                            int64_t stride, int n, int64_t C,
                                                            float* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  float s = 0.f;
  for (int k = 0; k < n; ++k) s += partial[(int64_t)k * stride + c];
  out[c] = s;
}

hipError_t launch_sum_rows(const float* partial, int64_t stride, int n, int64_t C, float* out,
                           hipStream_t s) {
  if (C <= 0 || !out) return hipSuccess;
  if (n <= 8 && C >= 4096)
    hipLaunchKernelGGL(sum_rows_wide_kernel, dim3((unsigned)((C + 255) / 256)), dim3(256), 0, s,
                       partial, stride, n, C, out);
  else
    hipLaunchKernelGGL(column_sum_kernel<float>, dim3((unsigned)((C + 15) / 16)), dim3(256), 0, s,
                       partial, stride, (int64_t)n, C, out);
  return hipGetLastError();
}

// partial[ch][c] = sum of x[r][c] over the rows of chunk ch, in order, 8 loads in flight.
template <typename T>
__global__ __launch_bounds__(256) void colsum_partial_kernel(const T* __restrict__ x, int64_t ld,
                                                             int64_t R, int C, int64_t rows_per,
                                                             float* __restrict__ partial) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int ch = blockIdx.y;
  if (c >= C) return;
  const int64_t r0 = (int64_t)ch * rows_per;
  const int64_t r1 = r0 + rows_per < R ? r0 + rows_per : R;
  float s = 0.f;
  int64_t r = r0;
  for (; r + 7 < r1; r += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = to_f32<T>(x[(r + u) * ld + c]);
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; r < r1; ++r) s += to_f32<T>(x[r * ld + c]);
  partial[(int64_t)ch * C + c] = s;
}

int colsum_chunks(int64_t R) {
  const int64_t c = (R + 63) / 64;
  return (int)(c < 1 ? 1 : (c > 256 ? 256 : c));
}

hipError_t launch_colsum(const void* x, int64_t ld, int64_t R, int C, int use_bf16, float* partial,
                         float* out, hipStream_t s) {
  if (!out || C <= 0) return hipSuccess;
  const int nch = colsum_chunks(R);
  const int64_t rows_per = (R + nch - 1) / nch;
  const dim3 grid((unsigned)((C + 255) / 256), (unsigned)nch);
  if (use_bf16)
    hipLaunchKernelGGL(colsum_partial_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)x, ld, R, C,
                       rows_per, partial);
  else
    hipLaunchKernelGGL(colsum_partial_kernel<float>, grid, dim3(256), 0, s, (const float*)x, ld, R,
                       C, rows_per, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_sum_rows(partial, C, nch, C, out, s);
}

// ------------------------------------------------------------------ SiLU pieces
// act[r][c] = SiLU(z1[r][c]) in the activation type, the same rounding as the f1
// GEMM epilogue (fast exp2/rcp for bf16, expf for fp32).
template <typename T>
__global__ __launch_bounds__(256) void silu_act_kernel(const float* __restrict__ z, int64_t ld_z,
                                                       T* __restrict__ act, int64_t ld_a, int64_t R,
                                                       int C) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= R * C) return;
  const int64_t r = idx / C;
  const int c = (int)(idx % C);
  const float x = z[r * ld_z + c];
  act[r * ld_a + c] = from_f32<T>(std::is_same<T, bf16>::value ? silu_fast(x) : silu_precise(x));
}

// d[r][c] *= SiLU'(z1[r][c]) (in place, activation type).
template <typename T>
__global__ __launch_bounds__(256) void silu_grad_kernel(const float* __restrict__ z, int64_t ld_z,
                                                        T* __restrict__ d, int64_t ld_d, int64_t R,
                                                        int C) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= R * C) return;
  const int64_t r = idx / C;
  const int c = (int)(idx % C);
  const float x = z[r * ld_z + c];
  const float sg = 1.0f / (1.0f + expf(-x));
  const float dsl = sg * (1.0f + x * (1.0f - sg));
  d[r * ld_d + c] = from_f32<T>(to_f32<T>(d[r * ld_d + c]) * dsl);
}

// The same for bf16 rows of 8-column groups (C and both leading dimensions multiples
// of 8, 16-byte aligned rows): one thread per group, 16-byte loads and stores.
__global__ __launch_bounds__(256) void silu_grad_vec_kernel(const float* __restrict__ z,
                                                            int64_t ld_z, bf16* __restrict__ d,
                                                            int64_t ld_d, int64_t R, int C) {
  const int G = C / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= R * G) return;
  const int64_t r = idx / G;
  const int c = 8 * (int)(idx % G);
  const f32x4 z0 = *reinterpret_cast<const f32x4*>(z + r * ld_z + c);
  const f32x4 z1 = *reinterpret_cast<const f32x4*>(z + r * ld_z + c + 4);
  bf16x8 v = *reinterpret_cast<const bf16x8*>(d + r * ld_d + c);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = e < 4 ? z0[e] : z1[e - 4];
    const float sg = 1.0f / (1.0f + expf(-x));
    const float dsl = sg * (1.0f + x * (1.0f - sg));
    v[e] = (bf16)((float)v[e] * dsl);
  }
  *reinterpret_cast<bf16x8*>(d + r * ld_d + c) = v;
}

hipError_t launch_silu_act(const float* z, int64_t ld_z, void* act, int64_t ld_a, int64_t R, int C,
                           int use_bf16, hipStream_t s) {
  const int64_t n = R * C;
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (use_bf16)
    hipLaunchKernelGGL(silu_act_kernel<bf16>, grid, dim3(256), 0, s, z, ld_z, (bf16*)act, ld_a, R, C);
  else
    hipLaunchKernelGGL(silu_act_kernel<float>, grid, dim3(256), 0, s, z, ld_z, (float*)act, ld_a, R,
                       C);
  return hipGetLastError();
}

hipError_t launch_silu_grad(const float* z, int64_t ld_z, void* d, int64_t ld_d, int64_t R, int C,
                            int use_bf16, hipStream_t s) {
  const int64_t n = R * C;
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  const bool vec = use_bf16 && C % 8 == 0 && ld_z % 8 == 0 && ld_d % 8 == 0 &&
                   ((uintptr_t)z & 15) == 0 && ((uintptr_t)d & 15) == 0;
  if (vec)
    hipLaunchKernelGGL(silu_grad_vec_kernel, dim3((unsigned)((n / 8 + 255) / 256)), dim3(256), 0, s,
                       z, ld_z, (bf16*)d, ld_d, R, C);
  else if (use_bf16)
    hipLaunchKernelGGL(silu_grad_kernel<bf16>, grid, dim3(256), 0, s, z, ld_z, (bf16*)d, ld_d, R, C);
  else
    hipLaunchKernelGGL(silu_grad_kernel<float>, grid, dim3(256), 0, s, z, ld_z, (float*)d, ld_d, R,
                       C);
  return hipGetLastError();
}

// ------------------------------------------------------------------ gate backward
// One wavefront per row (values in registers, NPL per lane, width w <= 64 * NPL).
// A workgroup walks rows blockIdx.x, blockIdx.x + gridDim.x, ... (4 at a time) and
// writes one partial row of dgamma and of dbeta, its 4 wavefronts added in order.
template <typename T, int NPL>
__global__ __launch_bounds__(256) void ln_gate_bwd_kernel(
    const float* __restrict__ o, int64_t ld_o, const T* __restrict__ u, int64_t ld_u,
    const float* __restrict__ gamma, const float* __restrict__ beta, float eps,
    const T* __restrict__ g, int64_t ld_g, T* __restrict__ d_o, int64_t ld_do, T* __restrict__ du,
    int64_t ld_du, float* __restrict__ part_gamma, float* __restrict__ part_beta, int64_t rows,
    int w) {
  __shared__ float red[2][4][64 * NPL];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  float gam[NPL], bet[NPL], pg[NPL], pb[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int c = lane + 64 * i;
    gam[i] = (c < w && gamma) ? gamma[c] : 1.f;
    bet[i] = (c < w && beta) ? beta[c] : 0.f;
    pg[i] = pb[i] = 0.f;
  }
  const float inv_w = 1.0f / (float)w;
  for (int64_t row = (int64_t)blockIdx.x * 4 + wv; row < rows; row += (int64_t)gridDim.x * 4) {
    float x[NPL], uu[NPL], gg[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int c = lane + 64 * i;
      const bool ok = c < w;
      x[i] = ok ? o[row * ld_o + c] : 0.f;
      uu[i] = ok ? to_f32<T>(u[row * ld_u + c]) : 0.f;
      gg[i] = ok ? to_f32<T>(g[row * ld_g + c]) : 0.f;
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) sum += x[i];
    const float mean = wave_sum(sum) * inv_w;
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int c = lane + 64 * i;
      const float d = c < w ? x[i] - mean : 0.f;
      sq = fmaf(d, d, sq);
    }
    const float rstd = 1.0f / sqrtf(wave_sum(sq) * inv_w + eps);
    float s1 = 0.f, s2 = 0.f;
    float xh[NPL], dxh[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int c = lane + 64 * i;
      const bool ok = c < w;
      xh[i] = ok ? (x[i] - mean) * rstd : 0.f;
      const float y = xh[i] * gam[i] + bet[i];
      const float dy = gg[i] * uu[i];
      if (ok) du[row * ld_du + c] = from_f32<T>(gg[i] * y);
      pg[i] = fmaf(dy, xh[i], pg[i]);
      pb[i] += dy;
      dxh[i] = dy * gam[i];
      s1 += dxh[i];
      s2 = fmaf(dxh[i], xh[i], s2);
    }
    const float m1 = wave_sum(s1) * inv_w, m2 = wave_sum(s2) * inv_w;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int c = lane + 64 * i;
      if (c < w) d_o[row * ld_do + c] = from_f32<T>(rstd * (dxh[i] - m1 - xh[i] * m2));
    }
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    red[0][wv][lane + 64 * i] = pg[i];
    red[1][wv][lane + 64 * i] = pb[i];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < w; c += 256) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a += red[0][q][c];
      b += red[1][q][c];
    }
    part_gamma[(int64_t)blockIdx.x * w + c] = a;
    part_beta[(int64_t)blockIdx.x * w + c] = b;
  }
}

int ln_gate_bwd_blocks(int64_t rows) {
  const int64_t b = (rows + 63) / 64;  // about 64 rows per workgroup
  return (int)(b < 1 ? 1 : (b > 1024 ? 1024 : b));
}

hipError_t launch_ln_gate_bwd(const float* o, int64_t ld_o, const void* u, int64_t ld_u,
                              const float* gamma, const float* beta, float eps, const void* g,
                              int64_t ld_g, void* d_o, int64_t ld_do, void* du, int64_t ld_du,
                              float* part_gamma, float* part_beta, int64_t rows, int w,
                              int use_bf16, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int nb = ln_gate_bwd_blocks(rows);
#define HSTU_LNB(NPL)                                                                          \
  if (w <= 64 * NPL) {                                                                         \
    if (use_bf16)                                                                              \
      hipLaunchKernelGGL((ln_gate_bwd_kernel<bf16, NPL>), dim3(nb), dim3(256), 0, s, o, ld_o,  \
                         (const bf16*)u, ld_u, gamma, beta, eps, (const bf16*)g, ld_g,         \
                         (bf16*)d_o, ld_do, (bf16*)du, ld_du, part_gamma, part_beta, rows, w); \
    else                                                                                       \
      hipLaunchKernelGGL((ln_gate_bwd_kernel<float, NPL>), dim3(nb), dim3(256), 0, s, o, ld_o, \
                         (const float*)u, ld_u, gamma, beta, eps, (const float*)g, ld_g,       \
                         (float*)d_o, ld_do, (float*)du, ld_du, part_gamma, part_beta, rows,   \
                         w);                                                                   \
    return hipGetLastError();                                                                  \
  }
  HSTU_LNB(1) HSTU_LNB(2) HSTU_LNB(4) HSTU_LNB(8) HSTU_LNB(16)
#undef HSTU_LNB
  return hipErrorInvalidValue;
}

}  // namespace hstu
