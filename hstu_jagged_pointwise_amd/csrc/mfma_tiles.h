// Building blocks shared by the MFMA attention kernels that stream one side through
// LDS and keep the other in registers (v_mfma_f32_32x32x16_bf16 on gfx950): operand
// fragments, the accumulator's row order, exact time buckets and register-staged
// tile copies.
#pragma once
#include "common.h"
#include "kernels.h"

namespace hstu {
namespace mt {
constexpr int TR = 64;         // rows of the streamed side per LDS tile
constexpr int kMaxPosB = 1024; // position-table entries kept in LDS
constexpr int kTimeB = 64;     // reachable time buckets (<= 63)

__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x4 tr4(const bf16* lds_ptr) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(lds_ptr));
  return __builtin_bit_cast(bf16x4, r);
}
__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS tiles: rows padded to D + 8 elements (conflict-free 16-byte row reads).
template <int D>
__device__ __forceinline__ int toff(int row, int col) {
  return row * (D + 8) + col;
}

// Operand fragment of a row-major LDS tile M whose rows are the contraction index,
// in the accumulator's row order: k-slot (hl, i) of the 16-row step at row r0 is row
// r0 + 8*(i/4) + 4*hl + i%4, at column 32*c + lane%32.
template <int D>
__device__ __forceinline__ bf16x8 trfrag(const bf16* M, int r0, int c, int lane) {
  const int hl = lane >> 5, g16 = lane >> 4, rho = lane & 15;
  const int row = r0 + 4 * hl + (rho >> 2);
  const int col = c * 32 + 16 * (g16 & 1) + 4 * (rho & 3);
  const bf16x4 v1 = tr4(&M[toff<D>(row, col)]);
  const bf16x4 v2 = tr4(&M[toff<D>(row + 8, col)]);
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = v1[i];
    r[4 + i] = v2[i];
  }
  return r;
}

// Row (within the 32-row block) of accumulator slot r for this lane.
__device__ __forceinline__ int acc_row(int r, int hl) { return 8 * (r >> 2) + 4 * hl + (r & 3); }

__device__ __forceinline__ int tbucket(int64_t dt, int T) {
  dt = dt < 0 ? 0 : dt;
  const int b = 63 - __builtin_clzll((uint64_t)dt + 1ull);
  return b < T - 1 ? b : T - 1;
}

__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Timestamps of the streamed side's 64 rows and the ranges of its two 32-row blocks,
// fetched into registers together with the next tile's data and stored to LDS after
// the current tile's compute, so that their load latency is hidden by that compute.
struct SideTs {
  int64_t tv;
  KeyRange r;
};

// Register-staged copy of 64 rows x D of two row-major tensors into LDS tiles
// (rows past `rows` become zeros).
template <int D>
struct TileStage {
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int PER = TR * CPR / 256;     // chunks per thread per tensor
  u32x4 x[PER], y[PER];
  __device__ void load(const bf16* X, int64_t ldx, const bf16* Y, int64_t ldy, int64_t row0,
                       int rows, int col0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + 256 * i, r = c / CPR, cc = c % CPR;
      const bool ok = r < rows;
      x[i] = ok ? *reinterpret_cast<const u32x4*>(X + (row0 + r) * ldx + col0 + 8 * cc) : u32x4{};
      y[i] = ok ? *reinterpret_cast<const u32x4*>(Y + (row0 + r) * ldy + col0 + 8 * cc) : u32x4{};
    }
  }
  __device__ void store(bf16* XS, bf16* YS) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + 256 * i, r = c / CPR, cc = c % CPR;
      *reinterpret_cast<u32x4*>(&XS[toff<D>(r, 8 * cc)]) = x[i];
      *reinterpret_cast<u32x4*>(&YS[toff<D>(r, 8 * cc)]) = y[i];
    }
  }
};
}  // namespace mt
}  // namespace hstu
