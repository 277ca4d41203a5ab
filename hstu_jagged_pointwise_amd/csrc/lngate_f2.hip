// Norm(AV) (.) U fused into the output projection f2 (eqs. 2-3 of the HSTU layer,
// "What an HSTU layer changes" and "Gating instead of a separate FFN", HSTU chapter):
//
//   Y = ((LN(O) * gamma + beta) (.) U) W2^T + b2 (+ X)
//
// for layers whose pooled width K = H*d_v and model width N are small (K <= 128, N <= 256):
// there one workgroup holds a block of 64 whole rows of the gated value and all of W2 in
// LDS, so the gated value never goes to HBM and the layer needs one launch fewer. A
// workgroup
//   1. requests W2 (N x K bf16), the 64 rows of O (fp32, the sum of nsplit partial rows
//      plus, for M-FALCON candidates, the candidate's own weighted value), the 64 rows of
//      the gate U, gamma and beta, all at once;
//   2. layer-normalises each row exactly as the stand-alone LN gate does (fp32 statistics,
//      mean then squared deviations, biased variance), applies gamma, beta and U, and
//      writes the bf16 result into LDS in the layout the matrix cores read;
//   3. multiplies it by W2^T with v_mfma_f32_32x32x16_bf16 (4 wavefronts as 2 x 2, each
//      32 rows x N/2 columns);
//   4. stages each wavefront's fp32 tile in LDS and writes whole 16-byte row segments of
//      Y with b2 and the residual added.
// The gated value is rounded to bf16 before the product, as the two-kernel form stores it.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace hstu {

namespace {
constexpr int kRows = 64;  // rows per workgroup

template <int K, int N>
struct LnF2Shape {
  static constexpr int LD = K + 8;             // padded bf16 row (ds_read_b128 phases hit distinct banks)
  static constexpr int LPR = K / 4;            // lanes per row in the normalisation (4 columns each)
  static constexpr int RPP = 64 / LPR;         // rows per wavefront pass
  static constexpr int PASSES = (kRows / 4) / RPP;  // passes per wavefront (16 rows each)
  static constexpr int WCH = N * K / 8 / 256;  // 16-byte W2 chunks per thread
  static constexpr int WN = N / 2, FN = WN / 32;
  static constexpr int EP = WN + 4;            // padded fp32 row of the epilogue tile
  static constexpr int OPER = (kRows + N) * LD;           // bf16 elements of A and W2
  static constexpr int EPI = 4 * 32 * EP * 2;             // the 4 epilogue tiles, in bf16 units
  static constexpr int LDS = OPER > EPI ? OPER : EPI;
  static_assert(K == 64 || K == 128, "K: 64 or 128 (4 columns per lane, at most 64 lanes)");
  static_assert(N % 64 == 0 && (N * K / 8) % 256 == 0, "N: a multiple of 64");
};

template <int K, int N>
__global__ __launch_bounds__(256) void ln_gate_f2_kernel(
    const float* __restrict__ o, int64_t ld_o, int nsplit, int64_t split_stride,
    const bf16* __restrict__ u, int64_t ld_u, const float* __restrict__ gamma,
    const float* __restrict__ beta, float eps, const bf16* __restrict__ w2, int64_t ldw,
    const float* __restrict__ b2, const bf16* __restrict__ R, int64_t ldr, bf16* __restrict__ y,
    int64_t ldy, int64_t rows, const float* __restrict__ self_w, const bf16* __restrict__ vself,
    int64_t ld_vself, int dv, int H) {
  using S = LnF2Shape<K, N>;
  constexpr int LD = S::LD, LPR = S::LPR, RPP = S::RPP, PASSES = S::PASSES;
  __shared__ __attribute__((aligned(16))) bf16 lds[S::LDS];
  bf16* As = lds;                // kRows x LD: the gated rows
  bf16* Ws = lds + kRows * LD;   // N x LD: W2
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * kRows;

  // ---- 1. requests: W2 first (shared by every workgroup, so mostly from L2), then the rows
  bf16x8 wch[S::WCH];
#pragma unroll
  for (int i = 0; i < S::WCH; ++i) {
    const int ch = tid + 256 * i, n = ch / (K / 8), c = ch % (K / 8);
    wch[i] = *reinterpret_cast<const bf16x8*>(w2 + (int64_t)n * ldw + 8 * c);
  }
  const int sl = lane % LPR;       // this lane's 4 columns: 4 sl .. 4 sl + 3
  const int c = 4 * sl;
  const f32x4 gv = gamma ? *reinterpret_cast<const f32x4*>(gamma + c) : f32x4{1.f, 1.f, 1.f, 1.f};
  const f32x4 bv = beta ? *reinterpret_cast<const f32x4*>(beta + c) : f32x4{};
  f32x4 x[PASSES];
  bf16x4 ub[PASSES];
  bool live[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int rl = 16 * w + RPP * p + lane / LPR;  // row within the block
    const int64_t row = m0 + rl;
    live[p] = row < rows;
    ub[p] = live[p] ? *reinterpret_cast<const bf16x4*>(u + row * ld_u + c) : bf16x4{};
    x[p] = f32x4{};
    if (self_w && live[p]) {  // the candidate's own value, weighted (4 columns lie in one head)
      const float sw = self_w[row * H + c / dv];
      const bf16x4 vv = *reinterpret_cast<const bf16x4*>(vself + row * ld_vself + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[p][e] = sw * (float)vv[e];
    }
  }
  for (int sp = 0; sp < nsplit; ++sp) {  // partial rows, summed in split order
    f32x4 part[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int64_t row = m0 + 16 * w + RPP * p + lane / LPR;
      part[p] = live[p] ? *reinterpret_cast<const f32x4*>(o + (int64_t)sp * split_stride + row * ld_o + c)
                        : f32x4{};
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[p][e] += part[p][e];
  }
#pragma unroll
  for (int i = 0; i < S::WCH; ++i) {
    const int ch = tid + 256 * i, n = ch / (K / 8), cc = ch % (K / 8);
    *reinterpret_cast<bf16x8*>(&Ws[n * LD + 8 * cc]) = wch[i];
  }

  // ---- 2. normalise, scale, shift, gate; bf16 rows into LDS
  auto seg_sum = [](float v) {  // over the LPR lanes of one row (xor stays inside them)
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
  };
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const float mean = seg_sum(x[p][0] + x[p][1] + x[p][2] + x[p][3]) / (float)K;
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float d = x[p][e] - mean;
      sq = fmaf(d, d, sq);
    }
    const float rstd = rsqrtf(seg_sum(sq) / (float)K + eps);
    bf16x4 g;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      g[e] = (bf16)(((x[p][e] - mean) * rstd * gv[e] + bv[e]) * (float)ub[p][e]);
    const int rl = 16 * w + RPP * p + lane / LPR;
    *reinterpret_cast<bf16x4*>(&As[rl * LD + c]) = g;  // rows past the data hold zeros
  }
  __syncthreads();

  // ---- 3. Y tile = A W2^T: wavefront (wm, wn) owns rows 32 wm.. and columns WN wn..
  const int wm = w >> 1, wn = w & 1;
  f32x16 acc[S::FN];
#pragma unroll
  for (int j = 0; j < S::FN; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
#pragma unroll
  for (int kk = 0; kk < K / 16; ++kk) {
    const bf16x8 af = *reinterpret_cast<const bf16x8*>(&As[(32 * wm + l32) * LD + 16 * kk + 8 * hl]);
    bf16x8 bfr[S::FN];
#pragma unroll
    for (int j = 0; j < S::FN; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8*>(&Ws[(S::WN * wn + 32 * j + l32) * LD + 16 * kk + 8 * hl]);
#pragma unroll
    for (int j = 0; j < S::FN; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr[j], acc[j], 0, 0, 0);
  }
  __syncthreads();  // every wavefront is done with A and W2; the space takes the epilogue

  // ---- 4. epilogue: b2 at staging, residual at the 16-byte row-segment writes
  constexpr int EP = S::EP;
  float* E = reinterpret_cast<float*>(lds) + w * 32 * EP;
#pragma unroll
  for (int j = 0; j < S::FN; ++j) {
    const int nl = 32 * j + l32;
    const float bn = b2 ? b2[S::WN * wn + nl] : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) E[(8 * (r >> 2) + 4 * hl + (r & 3)) * EP + nl] = acc[j][r] + bn;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): own LDS writes done (same wavefront reads)
  constexpr int SEGS = 32 * (S::WN / 8);
#pragma unroll
  for (int s = lane; s < SEGS; s += 64) {
    const int ml = s / (S::WN / 8), cs = s % (S::WN / 8);
    const int64_t m = m0 + 32 * wm + ml;
    if (m >= rows) continue;
    const int n = S::WN * wn + 8 * cs;
    const f32x4 lo = *reinterpret_cast<const f32x4*>(&E[ml * EP + 8 * cs]);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(&E[ml * EP + 8 * cs + 4]);
    float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    if (R) {
      const bf16x8 rv = *reinterpret_cast<const bf16x8*>(&R[m * ldr + n]);
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] += (float)rv[q];
    }
    bf16x8 ob;
#pragma unroll
    for (int q = 0; q < 8; ++q) ob[q] = (bf16)v[q];
    *reinterpret_cast<bf16x8*>(&y[m * ldy + n]) = ob;
  }
}
}  // namespace

bool ln_gate_f2_supported(int K, int N, int bf16flag, const void* w2, const float* gamma,
                          const float* beta) {
  auto al16 = [](const void* q) { return q == nullptr || ((uintptr_t)q % 16) == 0; };
  return bf16flag && (K == 64 || K == 128) && (N == 64 || N == 128 || N == 256) && al16(w2) &&
         al16(gamma) && al16(beta);
}

hipError_t launch_ln_gate_f2(const float* o, int64_t ld_o, int nsplit, int64_t split_stride,
                             const void* u, int64_t ld_u, const float* gamma, const float* beta,
                             float eps, const void* w2, int64_t ldw, const float* b2, const void* R,
                             int64_t ldr, void* y, int64_t ldy, int64_t rows, int K, int N,
                             hipStream_t s, const float* self_w, const void* vself,
                             int64_t ld_vself, int dv) {
  if (rows <= 0) return hipSuccess;
  if (!ln_gate_f2_supported(K, N, 1, w2, gamma, beta) || !w2) return hipErrorInvalidValue;
  // 16-byte rows of O, W2, R and Y; 8-byte rows of U and the candidates' values
  if (ld_o % 4 != 0 || (nsplit > 1 && split_stride % 4 != 0) || ld_u % 4 != 0 || ldw % 8 != 0 ||
      ldy % 8 != 0 || (R && ldr % 8 != 0))
    return hipErrorInvalidValue;
  if (self_w && (dv <= 0 || dv % 4 != 0 || K % dv != 0 || !vself || ld_vself % 4 != 0))
    return hipErrorInvalidValue;
  auto al = [](const void* q, uintptr_t a) { return ((uintptr_t)q % a) == 0; };
  if (!al(o, 16) || !al(u, 8) || !al(w2, 16) || !al(y, 16) || (R && !al(R, 16)) ||
      (gamma && !al(gamma, 16)) || (beta && !al(beta, 16)) || (self_w && !al(vself, 8)))
    return hipErrorInvalidValue;
  nsplit = nsplit < 1 ? 1 : nsplit;
  const int H = self_w ? K / dv : 1;
  const dim3 grid((unsigned)((rows + kRows - 1) / kRows));
  auto go = [&](auto kc, auto nc) {
    constexpr int KK = decltype(kc)::value, NN = decltype(nc)::value;
    hipLaunchKernelGGL((ln_gate_f2_kernel<KK, NN>), grid, dim3(256), 0, s, o, ld_o, nsplit,
                       split_stride, (const bf16*)u, ld_u, gamma, beta, eps, (const bf16*)w2, ldw,
                       b2, (const bf16*)R, ldr, (bf16*)y, ldy, rows, self_w, (const bf16*)vself,
                       ld_vself, dv, H);
  };
  using K64 = std::integral_constant<int, 64>;
  using K128 = std::integral_constant<int, 128>;
  using N256 = std::integral_constant<int, 256>;
  if (K == 64) {
    if (N == 64) go(K64{}, K64{});
    else if (N == 128) go(K64{}, K128{});
    else go(K64{}, N256{});
  } else {
    if (N == 64) go(K128{}, K64{});
    else if (N == 128) go(K128{}, K128{});
    else go(K128{}, N256{});
  }
  return hipGetLastError();
}

}  // namespace hstu
