// The two outer linear projections of the HSTU layer ("What an HSTU layer
// changes", HSTU chapter, eqs. 1 and 3; Figure 3 notes the block has only these
// two). The GEMMs run over all jagged tokens of the batch at once. A row is a
// token, so the ragged batch needs no padding at all.
//
//   f1: [U|V|Q|K] = SiLU(X W1^T + b1)   (epilogue: bias, SiLU)
//   f2: Y = G W2^T + b2 (+ X)           (epilogue: bias, optional residual)
//
// W is stored [out, in], so both operands are contiguous along the reduction
// dimension and feed v_mfma_f32_32x32x16_bf16 directly from LDS rows. A 128x128
// workgroup tile has 4 wavefronts, each owning 64x64 (2x2 MFMA blocks), with
// K staged through LDS 32 at a time. fp32 inputs take a plain vector-ALU tiled
// kernel.
#include "common.h"
#include "kernels.h"

namespace hstu {

namespace {
constexpr int GBM = 128, GBN = 128, GBK = 32, GLD = GBK + 8;
}

template <typename OutT>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(const bf16* __restrict__ A, int64_t lda,
                                                           const bf16* __restrict__ W, int64_t ldw,
                                                           const float* __restrict__ bias,
                                                           const bf16* __restrict__ R, int64_t ldr,
                                                           OutT* __restrict__ C, int64_t ldc,
                                                           int64_t M, int N, int K, int silu) {
  __shared__ __attribute__((aligned(16))) bf16 As[GBM * GLD];
  __shared__ __attribute__((aligned(16))) bf16 Ws[GBN * GLD];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int wm = w >> 1, wn = w & 1;
  const int64_t m0 = (int64_t)blockIdx.y * GBM;
  const int n0 = blockIdx.x * GBN;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  for (int k0 = 0; k0 < K; k0 += GBK) {
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int c = tid + 256 * it;
      const int row = c >> 2, kc = (c & 3) * 8;
      bf16x8 av, wv;
      const bool kok = k0 + kc < K;
      if (kok && m0 + row < M) {
        av = *reinterpret_cast<const bf16x8*>(A + (m0 + row) * lda + k0 + kc);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) av[i] = (bf16)0.f;
      }
      if (kok && n0 + row < N) {
        wv = *reinterpret_cast<const bf16x8*>(W + (int64_t)(n0 + row) * ldw + k0 + kc);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) wv[i] = (bf16)0.f;
      }
      *reinterpret_cast<bf16x8*>(&As[row * GLD + kc]) = av;
      *reinterpret_cast<bf16x8*>(&Ws[row * GLD + kc]) = wv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < GBK / 16; ++kk) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&As[(wm * 64 + 32 * i + l32) * GLD + 16 * kk + 8 * hl]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(&Ws[(wn * 64 + 32 * j + l32) * GLD + 16 * kk + 8 * hl]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  // acc[i][j][r] = C[m0 + wm*64 + 32i + 8(r/4) + 4hl + r%4][n0 + wn*64 + 32j + l32]
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + 32 * j + l32;
    if (n >= N) continue;
    const float bn = bias ? bias[n] : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * hl + (r & 3);
        if (m >= M) continue;
        float y = acc[i][j][r] + bn;
        if (silu) y = silu_fast(y);
        if (R) y += (float)R[m * ldr + n];
        C[m * ldc + n] = from_f32<OutT>(y);
      }
  }
}

// fp32: 64x64 tile, 256 threads with 4x4 outputs each, K staged 16 at a time
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int64_t lda,
                                                       const float* __restrict__ W, int64_t ldw,
                                                       const float* __restrict__ bias,
                                                       const float* __restrict__ R, int64_t ldr,
                                                       float* __restrict__ C, int64_t ldc, int64_t M,
                                                       int N, int K, int silu) {
  __shared__ float As[16][64 + 4];
  __shared__ float Ws[16][64 + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * 64;
  const int n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    __syncthreads();
    for (int i = tid; i < 64 * 16; i += 256) {
      const int r = i >> 4, kk = i & 15;
      As[kk][r] = (m0 + r < M && k0 + kk < K) ? A[(m0 + r) * lda + k0 + kk] : 0.f;
      Ws[kk][r] = (n0 + r < N && k0 + kk < K) ? W[(int64_t)(n0 + r) * ldw + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a4[4], w4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a4[i] = As[kk][ty * 4 + i]; w4[i] = Ws[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a4[i], w4[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      float y = acc[i][j] + (bias ? bias[n] : 0.f);
      if (silu) y = silu_precise(y);
      if (R) y += R[m * ldr + n];
      C[m * ldc + n] = y;
    }
  }
}

hipError_t launch_gemm(const void* A, int64_t lda, const void* W, int64_t ldw, const float* bias,
                       const void* R, int64_t ldr, void* C, int64_t ldc, int64_t M, int N, int K,
                       int silu, int bf16flag, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (bf16flag) {
    const dim3 grid((unsigned)((N + GBN - 1) / GBN), (unsigned)((M + GBM - 1) / GBM));
    hipLaunchKernelGGL((gemm_bf16_kernel<bf16>), grid, dim3(256), 0, s, (const bf16*)A, lda,
                       (const bf16*)W, ldw, bias, (const bf16*)R, ldr, (bf16*)C, ldc, M, N, K, silu);
  } else {
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, (const float*)A, lda,
                       (const float*)W, ldw, bias, (const float*)R, ldr, (float*)C, ldc, M, N, K,
                       silu);
  }
  return hipGetLastError();
}

}  // namespace hstu
