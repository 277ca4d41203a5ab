// The two outer linear projections of the HSTU layer ("What an HSTU layer
// changes", HSTU chapter, eqs. 1 and 3; Figure 3 notes the block has only these
// two). The GEMMs run over all jagged tokens of the batch at once. A row is a
// token, so the ragged batch needs no padding at all.
//
//   f1: [U|V|Q|K] = SiLU(X W1^T + b1)   (epilogue: bias, SiLU)
//   f2: Y = G W2^T + b2 (+ X)           (epilogue: bias, optional residual)
//
// W is stored [out, in], so both operands are contiguous along the reduction
// dimension and feed v_mfma_f32_32x32x16_bf16 directly from LDS rows. Workgroup
// tiles are 128x128, or 64x64 when the grid would otherwise leave compute units
// idle; K is staged through double-buffered LDS 64 at a time. fp32 inputs take a
// plain vector-ALU tiled kernel.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace hstu {

namespace {
constexpr int GBK = 64;          // K per pipeline stage
constexpr int GLD = GBK + 8;     // padded LDS row (elements): conflict-free ds_read_b128
constexpr int GSPR = GLD / 8;    // 16-byte slots per LDS row (8 data + 1 pad)

__device__ __forceinline__ void dma16(const bf16* g, bf16* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
}  // namespace

// BM x BN workgroup tile, 4 wavefronts as 2 x 2, each wavefront (BM/2) x (BN/2) of
// 32x32 MFMA blocks. K streams through two LDS stages filled by global_load_lds
// (the next stage loads while the current one is multiplied; one barrier per stage).
// Rows past M or N repeat the last valid row; K must be a multiple of 8, and the
// K tail of the last stage is zero-filled by a plain store.
template <int BM, int BN, typename OutT>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(const bf16* __restrict__ A, int64_t lda,
                                                           const bf16* __restrict__ W, int64_t ldw,
                                                           const float* __restrict__ bias,
                                                           const bf16* __restrict__ R, int64_t ldr,
                                                           OutT* __restrict__ C, int64_t ldc,
                                                           int64_t M, int N, int K, int silu) {
  constexpr int WM = BM / 2, WN = BN / 2;      // per-wavefront tile
  constexpr int FM = WM / 32, FN = WN / 32;    // 32x32 blocks per wavefront
  constexpr int A_SLOTS = BM * GSPR, W_SLOTS = BN * GSPR;
  constexpr int A_INSTR = (A_SLOTS + 63) / 64, W_INSTR = (W_SLOTS + 63) / 64;
  __shared__ __attribute__((aligned(16))) bf16 As0[A_INSTR * 512];
  __shared__ __attribute__((aligned(16))) bf16 As1[A_INSTR * 512];
  __shared__ __attribute__((aligned(16))) bf16 Ws0[W_INSTR * 512];
  __shared__ __attribute__((aligned(16))) bf16 Ws1[W_INSTR * 512];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int wm = w >> 1, wn = w & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nks = (K + GBK - 1) / GBK;
  auto issue = [&](auto bufc, int k0) {
    constexpr int buf = decltype(bufc)::value;
    bf16* Ad = buf ? As1 : As0;
    bf16* Wd = buf ? Ws1 : Ws0;
    const bool ktail = k0 + GBK > K;
#pragma unroll
    for (int i = w; i < A_INSTR; i += 4) {
      const int slot = 64 * i + lane;
      if (slot < A_SLOTS) {
        const int row = slot / GSPR, pc = slot % GSPR;
        int c = pc < 8 ? pc : 0;
        if (ktail && k0 + 8 * c >= K) c = 0;  // out-of-range K chunk: fetch any valid chunk
        const int64_t gr = min(m0 + row, M - 1);
        dma16(A + gr * lda + k0 + 8 * c, &Ad[512 * i]);
      }
    }
#pragma unroll
    for (int i = w; i < W_INSTR; i += 4) {
      const int slot = 64 * i + lane;
      if (slot < W_SLOTS) {
        const int row = slot / GSPR, pc = slot % GSPR;
        int c = pc < 8 ? pc : 0;
        if (ktail && k0 + 8 * c >= K) c = 0;
        const int64_t gr = min(n0 + row, N - 1);
        dma16(W + gr * ldw + k0 + 8 * c, &Wd[512 * i]);
      }
    }
  };
  auto finish = [&](auto bufc, int k0) {
    constexpr int buf = decltype(bufc)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (k0 + GBK > K) {
      // zero the K tail so that it adds nothing (the DMA filled it with valid data)
      __syncthreads();
      bf16* Ad = buf ? As1 : As0;
      bf16* Wd = buf ? Ws1 : Ws0;
      const int kv = K - k0;  // valid K in this stage, a multiple of 8
      for (int e = tid; e < BM * 8; e += 256) {
        const int row = e >> 3, c = e & 7;
        if (8 * c >= kv) {
#pragma unroll
          for (int q = 0; q < 8; ++q) Ad[row * GLD + 8 * c + q] = (bf16)0.f;
        }
      }
      for (int e = tid; e < BN * 8; e += 256) {
        const int row = e >> 3, c = e & 7;
        if (8 * c >= kv) {
#pragma unroll
          for (int q = 0; q < 8; ++q) Wd[row * GLD + 8 * c + q] = (bf16)0.f;
        }
      }
    }
  };
  auto compute = [&](auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const bf16* Ad = buf ? As1 : As0;
    const bf16* Wd = buf ? Ws1 : Ws0;
#pragma unroll
    for (int kk = 0; kk < GBK / 16; ++kk) {
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&Ad[(wm * WM + 32 * i + l32) * GLD + 16 * kk + 8 * hl]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(&Wd[(wn * WN + 32 * j + l32) * GLD + 16 * kk + 8 * hl]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  issue(B0{}, 0);
  finish(B0{}, 0);
  __syncthreads();
  for (int ks = 0; ks < nks; ks += 2) {
    if (ks + 1 < nks) issue(B1{}, (ks + 1) * GBK);
    compute(B0{});
    if (ks + 1 < nks) finish(B1{}, (ks + 1) * GBK);
    __syncthreads();
    if (ks + 1 >= nks) break;
    if (ks + 2 < nks) issue(B0{}, (ks + 2) * GBK);
    compute(B1{});
    if (ks + 2 < nks) finish(B0{}, (ks + 2) * GBK);
    __syncthreads();
  }
  // acc[i][j][r] = C[m0 + wm*WM + 32i + 8(r/4) + 4hl + r%4][n0 + wn*WN + 32j + l32]
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + wn * WN + 32 * j + l32;
    if (n >= N) continue;
    const float bn = bias ? bias[n] : 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * WM + 32 * i + 8 * (r >> 2) + 4 * hl + (r & 3);
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
    // 128x128 tiles when they give at least ~one workgroup per compute unit, else 64x64
    const int64_t big = ((N + 127) / 128) * ((M + 127) / 128);
    if (big >= 256) {
      const dim3 grid((unsigned)((N + 127) / 128), (unsigned)((M + 127) / 128));
      hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, bf16>), grid, dim3(256), 0, s, (const bf16*)A,
                         lda, (const bf16*)W, ldw, bias, (const bf16*)R, ldr, (bf16*)C, ldc, M, N,
                         K, silu);
    } else {
      const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
      hipLaunchKernelGGL((gemm_bf16_kernel<64, 64, bf16>), grid, dim3(256), 0, s, (const bf16*)A,
                         lda, (const bf16*)W, ldw, bias, (const bf16*)R, ldr, (bf16*)C, ldc, M, N,
                         K, silu);
    }
  } else {
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, (const float*)A, lda,
                       (const float*)W, ldw, bias, (const float*)R, ldr, (float*)C, ldc, M, N, K,
                       silu);
  }
  return hipGetLastError();
}

}  // namespace hstu
