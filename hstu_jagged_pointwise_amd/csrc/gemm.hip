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
// idle. K streams through a 4-stage LDS ring, with three stages in flight, filled by
// global_load_lds: 32 of K per stage for 128x128 tiles, 64 for 64x64 tiles (whose
// workgroups do 4x less MFMA work per stage, so they need more of K in flight to
// cover the load latency). Tiles are ordered so that the tiles of one
// row block of A run on one XCD (sharing its L2). The epilogue stages each
// wavefront's tile in LDS and writes whole 16-byte row segments. fp32 inputs
// take a plain vector-ALU tiled kernel.
#include "common.h"
#include "kernels.h"
#include "mfma_tiles.h"

#include <type_traits>

namespace hstu {

namespace {
constexpr int NST = 4;  // LDS ring stages: NST-1 stages load while one is multiplied
// K per pipeline stage of a BM-row tile
constexpr int stage_k(int bm) { return bm >= 128 ? 32 : 64; }

// s_waitcnt vmcnt(N) through the builtin (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt and lgkmcnt at their maxima), so that the compiler sees it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// One 16-byte-per-lane load into LDS (buffer_load_dwordx4 ... lds): lane L's 16 bytes at
// base + voff land in slot L of the 1 KiB span at lds. The descriptor has no range limit:
// the callers keep every address inside the data. Written as assembly, so that the
// compiler does not track these loads: the next stage's loads are issued between the
// current stage's MFMAs, and with the loads visible the compiler would make the LDS
// reads after each such branch wait for every load in flight. The ring's own waits
// (wait_vmcnt before each barrier) order the loads with the reads. The instruction has
// no register result; its operands (offset, descriptor, M0) are read when it issues.
__device__ __forceinline__ void stage_fetch(const char* base, bf16* lds, uint32_t voff) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, -1, 0x00020000);
  const uint32_t m0v = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(r), "s"(m0v)
      : "memory", "m0");
}
// Workgroup barrier that leaves in-flight global->LDS loads alone (__syncthreads
// also waits for every outstanding vector memory operation, which would drain the
// ring). This wavefront's LDS operations complete first.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
}  // namespace

// LDS ring geometry of a BM x BN tile: each stage holds BM rows of A then BN rows
// of W, GBK elements each, padded by 8 (the 16 rows of one ds_read_b128 phase fall
// in distinct banks). A stage is filled by whole 64-lane DMA instructions, dealt
// to the 4 wavefronts round robin and padded to an equal count per wavefront (the
// per-wavefront waits count instructions).
template <int BM, int BN>
struct GemmShape {
  static constexpr int GBK = stage_k(BM);
  static constexpr int GLD = GBK + 8, GSPR = GLD / 8, CPR = GBK / 8;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int SLOTS = (BM + BN) * GSPR;
  static constexpr int INSTR = (SLOTS + 63) / 64;
  static constexpr int PERW = (INSTR + 3) / 4;           // instructions per wavefront (padded)
  static constexpr int A_INSTR = BM * GSPR / 64;          // instructions that read A
  static constexpr int STAGE = (4 * PERW) * 512;          // bf16 elements per stage (incl. junk)
  static_assert(BM * GSPR % 64 == 0, "A rows fill whole instructions");
};

// C[M,N] = epi(A[M,K] W[N,K]^T + bias): 4 wavefronts as 2 x 2, each (BM/2) x (BN/2)
// of 32x32 MFMA blocks. Rows past M or N repeat the last valid row; K must be a
// multiple of 8, and the K tail of the last stage is zeroed in LDS.
template <int BM, int BN, typename OutT>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(const bf16* __restrict__ A, int64_t lda,
                                                         const bf16* __restrict__ W, int64_t ldw,
                                                         const float* __restrict__ bias,
                                                         const bf16* __restrict__ R, int64_t ldr,
                                                         OutT* __restrict__ C, int64_t ldc, int64_t M,
                                                         int N, int K, int silu, int tiles_n,
                                                         int tiles_total, int64_t ksplit,
                                                         int64_t c_split, bf16* __restrict__ act,
                                                         bf16* __restrict__ rem, int rem_c0,
                                                         int sc_c0, int sc_c1, float sc,
                                                         int cw_len0, int cw_off0, int cw_off1) {
  using G = GemmShape<BM, BN>;
  constexpr int GBK = G::GBK;
  constexpr int FM = G::FM, FN = G::FN, PERW = G::PERW, STAGE = G::STAGE;
  constexpr int GLD = G::GLD, GSPR = G::GSPR, CPR = G::CPR;
  __shared__ __attribute__((aligned(16))) bf16 S0[STAGE];
  __shared__ __attribute__((aligned(16))) bf16 S1[STAGE];
  __shared__ __attribute__((aligned(16))) bf16 S2[STAGE];
  __shared__ __attribute__((aligned(16))) bf16 S3[STAGE];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int l32 = lane & 31, hl = lane >> 5;
  const int wm = w >> 1, wn = w & 1;
  // XCD-aware order: workgroups are dealt to the 8 XCDs round robin; consecutive
  // logical tiles (same row block of A) go to one XCD and share its L2
  int tile;
  {
    const int b = blockIdx.x, x = b & 7, j = b >> 3;
    const int per = tiles_total >> 3, rem = tiles_total & 7;
    tile = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + j;
  }
  const int64_t m0 = (int64_t)(tile / tiles_n) * BM;
  const int n0 = (tile % tiles_n) * BN;
  // computed column n is column n + cw_off0 of W and C below cw_len0, else n - cw_len0 +
  // cw_off1 (two windows of whole tiles; the identity when cw_len0 = N and both offsets 0)
  const int n0a = n0 < cw_len0 ? n0 + cw_off0 : n0 - cw_len0 + cw_off1;
  {  // split-K: blockIdx.y takes K range [y * ksplit, (y + 1) * ksplit) into its own C slice
    const int64_t kofs = (int64_t)blockIdx.y * ksplit;
    A += kofs;
    W += kofs;
    C += (int64_t)blockIdx.y * c_split;
    K = (int)(K - kofs < ksplit ? K - kofs : ksplit);
  }

  // per-lane DMA sources of this wavefront's PERW instructions: the byte offset of the
  // row from the row-block base of A or W (rows past M or N repeat the last row) and the
  // byte offset of the 16-byte chunk within a stage (pad slots fetch chunk 0)
  uint32_t soff[PERW], coff[PERW];
  bool isA[PERW];
#pragma unroll
  for (int j = 0; j < PERW; ++j) {
    const int i = wu + 4 * j;
    const int slot = 64 * i + lane;
    const int row = slot / GSPR, pc = slot % GSPR;
    coff[j] = 16u * (uint32_t)(pc < CPR ? pc : 0);
    isA[j] = i < G::A_INSTR;
    if (i >= G::INSTR) {  // junk instruction: any valid A chunk
      soff[j] = 0;
      isA[j] = true;
    } else if (isA[j]) {
      const int64_t r = min(m0 + row, M - 1) - m0;
      soff[j] = (uint32_t)(r * lda * 2);
    } else {
      const int r = min(n0 + (row - BM), N - 1) - n0;
      soff[j] = (uint32_t)((int64_t)r * ldw * 2);
    }
  }
  const char* abase = (const char*)(A + m0 * lda);
  const char* wbase = (const char*)(W + (int64_t)n0a * ldw);
  const int nks = (K + GBK - 1) / GBK;
  // byte offset of the last 16-byte chunk of a row inside K: chunks of the last stage
  // that lie past K fetch that one instead (they are zeroed in LDS before use), so no
  // load leaves the row
  const uint32_t klast = (uint32_t)(K - 8) * 2u;
  // this wavefront's instruction j of stage ks
  auto issue_one = [&](auto bufc, int ks, int j) {
    constexpr int buf = decltype(bufc)::value;
    bf16* D = buf == 0 ? S0 : buf == 1 ? S1 : buf == 2 ? S2 : S3;
    const uint32_t kb = (uint32_t)ks * GBK * 2;
    stage_fetch(isA[j] ? abase : wbase, &D[512 * (wu + 4 * j)], soff[j] + min(kb + coff[j], klast));
  };
  auto issue = [&](auto bufc, int ks) {
#pragma unroll
    for (int j = 0; j < PERW; ++j) issue_one(bufc, ks, j);
  };
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // the MFMAs of stage ks, with this wavefront's loads of stage ks+NST-1 (into buffer
  // nbufc) issued one after each MFMA when `more`: a load can wait for room in the memory
  // pipeline, and the MFMAs issued before it run meanwhile
  auto compute = [&](auto bufc, int ks, auto nbufc, bool more) {
    constexpr int buf = decltype(bufc)::value;
    bf16* D = buf == 0 ? S0 : buf == 1 ? S1 : buf == 2 ? S2 : S3;
    if ((ks + 1) * GBK > K) {  // K tail: zero the chunks past K (uniform branch, last stage only)
      lds_barrier();
      const int kv = K - ks * GBK;  // a multiple of 8
      for (int e = tid; e < (BM + BN) * CPR; e += 256) {
        const int row = e / CPR, c = e % CPR;
        if (8 * c >= kv) {
          u32x4 z = {0u, 0u, 0u, 0u};
          *reinterpret_cast<u32x4*>(&D[row * GLD + 8 * c]) = z;
        }
      }
      lds_barrier();
    }
    // every k-step's fragments are read first, so that the reads of later k-steps
    // complete under the MFMAs of earlier ones
    constexpr int NKS = GBK / 16;
    bf16x8 af[NKS][FM], bfr[NKS][FN];
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[kk][i] = *reinterpret_cast<const bf16x8*>(&D[(wm * G::WM + 32 * i + l32) * GLD + 16 * kk + 8 * hl]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[kk][j] = *reinterpret_cast<const bf16x8*>(&D[(BM + wn * G::WN + 32 * j + l32) * GLD + 16 * kk + 8 * hl]);
    }
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk][i], bfr[kk][j], acc[i][j], 0, 0, 0);
          const int n = (kk * FM + i) * FN + j;  // this stage's MFMA count so far
          if (n < PERW && more) issue_one(nbufc, ks + NST - 1, n);
        }
    }
    constexpr int NMF = (GBK / 16) * FM * FN;
#pragma unroll
    for (int n = NMF; n < PERW; ++n)
      if (more) issue_one(nbufc, ks + NST - 1, n);
  };
  // prologue: NST-1 stages in flight
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  using B3 = std::integral_constant<int, 3>;
  if (0 < nks) issue(B0{}, 0);
  if (1 < nks) issue(B1{}, 1);
  if (2 < nks) issue(B2{}, 2);
  auto step = [&](auto bufc, int ks) {
    constexpr int buf = decltype(bufc)::value;
    using BI = std::integral_constant<int, (buf + NST - 1) % NST>;
    // stage ks landed once at most the later stages' instructions are outstanding
    if (ks + 2 < nks) wait_vmcnt<2 * PERW>();
    else if (ks + 1 < nks) wait_vmcnt<PERW>();
    else wait_vmcnt<0>();
    lds_barrier();
    // the buffer of stage ks-1 is free (every wavefront passed this barrier after using it);
    // stage ks+NST-1 goes into it during this stage's MFMAs
    compute(bufc, ks, BI{}, ks + NST - 1 < nks);
  };
  for (int ks = 0; ks < nks; ks += NST) {
    step(B0{}, ks);
    if (ks + 1 < nks) step(B1{}, ks + 1);
    if (ks + 2 < nks) step(B2{}, ks + 2);
    if (ks + 3 < nks) step(B3{}, ks + 3);
  }
  __syncthreads();  // every wavefront is done with the ring; reuse it for the epilogue

  // epilogue: each wavefront stages its WM x WN fp32 tile (bias and SiLU applied) in its
  // own ring buffer, then writes 16-byte row segments (residual added there)
  constexpr int EP = G::WN + 4;  // padded fp32 row
  static_assert(G::WM * EP * 4 <= STAGE * 2, "epilogue tile fits one ring buffer");
  float* E = (float*)(w == 0 ? S0 : w == 1 ? S1 : w == 2 ? S2 : S3);
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int nl = 32 * j + l32;
    const int n = n0 + wn * G::WN + nl;
    const float bn = (bias && n < N) ? bias[n0a + wn * G::WN + nl] : 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ml = 32 * i + 8 * (r >> 2) + 4 * hl + (r & 3);
        float y = acc[i][j][r] + bn;
        if (silu) y = silu_fast(y);
        E[ml * EP + nl] = y;
      }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): own LDS writes done (same wavefront reads)
  constexpr int SEGS = G::WM * (G::WN / 8);  // 8-column segments
#pragma unroll
  for (int s = lane; s < SEGS; s += 64) {
    const int ml = s / (G::WN / 8), cs = s % (G::WN / 8);
    const int64_t m = m0 + wm * G::WM + ml;
    if (m >= M || n0 + wn * G::WN + 8 * cs >= N) continue;
    const int n = n0a + wn * G::WN + 8 * cs;  // the column of C (and R, act, rem) written
    const f32x4 lo = *reinterpret_cast<const f32x4*>(&E[ml * EP + 8 * cs]);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(&E[ml * EP + 8 * cs + 4]);
    float y[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    if (R) {
      const bf16x8 rv = *reinterpret_cast<const bf16x8*>(&R[m * ldr + n]);
#pragma unroll
      for (int q = 0; q < 8; ++q) y[q] += (float)rv[q];
    }
    if constexpr (std::is_same<OutT, float>::value) {
      *reinterpret_cast<f32x4*>(&C[m * ldc + n]) = f32x4{y[0], y[1], y[2], y[3]};
      *reinterpret_cast<f32x4*>(&C[m * ldc + n + 4]) = f32x4{y[4], y[5], y[6], y[7]};
      if (act) {  // SiLU of the fp32 result too, in bf16 (the f1 activation of a recompute)
        bf16x8 o;
        float a8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          a8[q] = silu_fast(y[q]);
          o[q] = (bf16)a8[q];
        }
        *reinterpret_cast<bf16x8*>(&act[m * ldc + n]) = o;
        if (rem && n >= rem_c0) {  // and the rounding remainder of that activation
          bf16x8 r;
#pragma unroll
          for (int q = 0; q < 8; ++q) r[q] = (bf16)(a8[q] - (float)o[q]);
          *reinterpret_cast<bf16x8*>(&rem[m * ldc + n]) = r;
        }
      }
    } else {
      if (n >= sc_c0 && n < sc_c1)  // a column block stored scaled (8-column segments never straddle)
#pragma unroll
        for (int q = 0; q < 8; ++q) y[q] *= sc;
      bf16x8 o;
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = (bf16)y[q];
      *reinterpret_cast<bf16x8*>(&C[m * ldc + n]) = o;
      if (rem && n >= rem_c0) {  // the rounding remainder, so that C + rem carries ~16 bits
        bf16x8 r;
#pragma unroll
        for (int q = 0; q < 8; ++q) r[q] = (bf16)(y[q] - (float)o[q]);
        *reinterpret_cast<bf16x8*>(&rem[m * ldc + n]) = r;
      }
    }
  }
}

// TN form for weight gradients: C[M,N] = sum_k A[k,m] B[k,n] with A [K, lda] and
// B [K, ldb] row-major (the contraction runs over rows, e.g. tokens), fp32 out. A stage
// holds GBK rows of A (BM wide) then GBK rows of B (BN wide), each as stored, rows
// padded by 8; the MFMA fragments are read transposed (ds_read_b64_tr_b16), so no
// transposed copy of either operand is made. Both operands take the same contraction
// order within a 16-row step, so their products pair up. Columns past M or N repeat
// the last 8-column chunk; rows past K are zeroed in LDS.
template <int BM, int BN>
struct GemmTnShape {
  static constexpr int GBK = stage_k(BM);
  static constexpr int SPA = BM / 8 + 1, SPB = BN / 8 + 1;  // 16-byte slots per padded row
  static constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 32, FN = WN / 32;
  static constexpr int A_SLOTS = GBK * SPA, SLOTS = GBK * (SPA + SPB);
  static constexpr int INSTR = (SLOTS + 63) / 64;
  static constexpr int PERW = (INSTR + 3) / 4;
  static constexpr int STAGE = 4 * PERW * 512;  // bf16 elements per stage (incl. junk)
  static constexpr int BOFF = GBK * (BM + 8);    // B rows start here within a stage
};

template <int BM, int BN>
__global__ __launch_bounds__(256, 2) void gemm_tn_kernel(const bf16* __restrict__ A, int64_t lda,
                                                       const bf16* __restrict__ B, int64_t ldb,
                                                       float* __restrict__ C, int64_t ldc, int M,
                                                       int N, int64_t K, int tiles_n,
                                                       int tiles_total, int64_t ksplit,
                                                       int64_t c_split) {
  using G = GemmTnShape<BM, BN>;
  constexpr int GBK = G::GBK, FM = G::FM, FN = G::FN, PERW = G::PERW, STAGE = G::STAGE;
  __shared__ __attribute__((aligned(16))) bf16 S0[STAGE];
  __shared__ __attribute__((aligned(16))) bf16 S1[STAGE];
  __shared__ __attribute__((aligned(16))) bf16 S2[STAGE];
  __shared__ __attribute__((aligned(16))) bf16 S3[STAGE];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int l32 = lane & 31, hl = lane >> 5;
  const int wm = w >> 1, wn = w & 1;
  int tile;  // XCD-aware order, as in the NT kernel
  {
    const int b = blockIdx.x, x = b & 7, j = b >> 3;
    const int per = tiles_total >> 3, rem = tiles_total & 7;
    tile = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + j;
  }
  const int m0 = (tile / tiles_n) * BM;
  const int n0 = (tile % tiles_n) * BN;
  {  // split-K: blockIdx.y takes rows [y * ksplit, (y + 1) * ksplit) into its own C slice
    const int64_t kofs = (int64_t)blockIdx.y * ksplit;
    A += kofs * lda;
    B += kofs * ldb;
    C += (int64_t)blockIdx.y * c_split;
    K = K - kofs < ksplit ? K - kofs : ksplit;
  }
  // per-lane DMA source of each of this wavefront's instructions: matrix, row within the
  // stage, byte column (junk slots of the padded last instruction fetch A row 0, chunk 0)
  int srow[PERW];
  uint32_t scol[PERW];
  bool isA[PERW];
#pragma unroll
  for (int j = 0; j < PERW; ++j) {
    const int i = wu + 4 * j;
    const int slot = 64 * i + lane;
    if (i >= G::INSTR || slot >= G::SLOTS) {
      isA[j] = true;
      srow[j] = 0;
      scol[j] = 0;
    } else if (slot < G::A_SLOTS) {
      isA[j] = true;
      srow[j] = slot / G::SPA;
      const int pc = slot % G::SPA, c = pc < G::SPA - 1 ? pc : 0;
      scol[j] = (uint32_t)(2 * (min(m0 + 8 * c, M - 8) - m0));
    } else {
      const int sb = slot - G::A_SLOTS;
      isA[j] = false;
      srow[j] = sb / G::SPB;
      const int pc = sb % G::SPB, c = pc < G::SPB - 1 ? pc : 0;
      scol[j] = (uint32_t)(2 * (min(n0 + 8 * c, N - 8) - n0));
    }
  }
  const char* abase = (const char*)(A + m0);
  const char* bbase = (const char*)(B + n0);
  const int nks = (int)((K + GBK - 1) / GBK);
  auto issue = [&](auto bufc, int ks) {
    constexpr int buf = decltype(bufc)::value;
    bf16* D = buf == 0 ? S0 : buf == 1 ? S1 : buf == 2 ? S2 : S3;
#pragma unroll
    for (int j = 0; j < PERW; ++j) {
      const int i = wu + 4 * j;
      const int64_t r = min((int64_t)ks * GBK + srow[j], K - 1);  // rows past K: zeroed later
      const char* src = isA[j] ? abase + r * lda * 2 + scol[j] : bbase + r * ldb * 2 + scol[j];
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(&D[512 * i]), 16,
                                       0, 0);
    }
  };
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  auto compute = [&](auto bufc, int ks) {
    constexpr int buf = decltype(bufc)::value;
    bf16* D = buf == 0 ? S0 : buf == 1 ? S1 : buf == 2 ? S2 : S3;
    if ((int64_t)(ks + 1) * GBK > K) {  // rows past K (uniform branch, last stage only)
      lds_barrier();
      const int kv = (int)(K - (int64_t)ks * GBK);
      for (int e = tid; e < (GBK - kv) * (G::SPA + G::SPB - 2); e += 256) {
        const int row = kv + e / (G::SPA + G::SPB - 2), c = e % (G::SPA + G::SPB - 2);
        const int off = c < G::SPA - 1 ? row * (BM + 8) + 8 * c
                                       : G::BOFF + row * (BN + 8) + 8 * (c - (G::SPA - 1));
        *reinterpret_cast<u32x4*>(&D[off]) = u32x4{0u, 0u, 0u, 0u};
      }
      lds_barrier();
    }
#pragma unroll
    for (int kk = 0; kk < GBK / 16; ++kk) {
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = mt::trfrag<BM>(D, 16 * kk, wm * FM + i, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = mt::trfrag<BN>(D + G::BOFF, 16 * kk, wn * FN + j, lane);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  using B3 = std::integral_constant<int, 3>;
  if (0 < nks) issue(B0{}, 0);
  if (1 < nks) issue(B1{}, 1);
  if (2 < nks) issue(B2{}, 2);
  auto step = [&](auto bufc, int ks) {
    constexpr int buf = decltype(bufc)::value;
    using BI = std::integral_constant<int, (buf + NST - 1) % NST>;
    if (ks + 2 < nks) wait_vmcnt<2 * PERW>();
    else if (ks + 1 < nks) wait_vmcnt<PERW>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (ks + NST - 1 < nks) issue(BI{}, ks + NST - 1);
    compute(bufc, ks);
  };
  for (int ks = 0; ks < nks; ks += NST) {
    step(B0{}, ks);
    if (ks + 1 < nks) step(B1{}, ks + 1);
    if (ks + 2 < nks) step(B2{}, ks + 2);
    if (ks + 3 < nks) step(B3{}, ks + 3);
  }
  __syncthreads();  // every wavefront is done with the ring; reuse it for the epilogue

  constexpr int EP = G::WN + 4;  // padded fp32 row
  static_assert(G::WM * EP * 4 <= STAGE * 2, "epilogue tile fits one ring buffer");
  float* E = (float*)(w == 0 ? S0 : w == 1 ? S1 : w == 2 ? S2 : S3);
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        E[(32 * i + 8 * (r >> 2) + 4 * hl + (r & 3)) * EP + 32 * j + l32] = acc[i][j][r];
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): own LDS writes done (same wavefront reads)
  constexpr int SEGS = G::WM * (G::WN / 8);
#pragma unroll
  for (int sg = lane; sg < SEGS; sg += 64) {
    const int ml = sg / (G::WN / 8), cs = sg % (G::WN / 8);
    const int m = m0 + wm * G::WM + ml;
    const int n = n0 + wn * G::WN + 8 * cs;
    if (m >= M || n >= N) continue;
    const f32x4 lo = *reinterpret_cast<const f32x4*>(&E[ml * EP + 8 * cs]);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(&E[ml * EP + 8 * cs + 4]);
    *reinterpret_cast<f32x4*>(&C[(int64_t)m * ldc + n]) = lo;
    *reinterpret_cast<f32x4*>(&C[(int64_t)m * ldc + n + 4]) = hi;
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

hipError_t launch_gemm_ex(const void* A, int64_t lda, const void* W, int64_t ldw, const float* bias,
                          const void* R, int64_t ldr, void* C, int64_t ldc, int64_t M, int N, int K,
                          int silu, int bf16flag, int out_f32, int splits, int64_t ksplit,
                          int64_t c_split, void* act, hipStream_t s, void* lo, int lo_c0,
                          int sc_c0, int sc_c1, float sc) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (act && (!bf16flag || !out_f32 || splits > 1 || silu)) return hipErrorInvalidValue;
  if (lo && (!bf16flag || (out_f32 && !act) || splits > 1 || lo_c0 % 8 != 0))
    return hipErrorInvalidValue;
  if (sc_c1 > sc_c0 && (!bf16flag || out_f32 || sc_c0 % 8 != 0 || sc_c1 % 8 != 0))
    return hipErrorInvalidValue;
  if (bf16flag) {
    // the DMA and the epilogue move 16-byte rows segments
    if (N % 8 != 0 || K % 8 != 0 || lda % 8 != 0 || ldw % 8 != 0 || ldc % 8 != 0 ||
        (R && ldr % 8 != 0))
      return hipErrorInvalidValue;
    if (splits < 1) splits = 1;
    if (splits == 1) ksplit = K;
    // 128x128 tiles when they give at least ~one workgroup per compute unit, else 64x64
    const int64_t big = ((N + 127) / 128) * ((M + 127) / 128) * splits;
    // split K ranges are whole pipeline stages; a split tail carries no bias or residual
    const int gbk = stage_k(big >= 256 ? 128 : 64);
    if (splits > 1 && (ksplit % gbk != 0 || (int64_t)(splits - 1) * ksplit >= K || bias || R || silu))
      return hipErrorInvalidValue;
    auto go = [&](auto bm, auto outc) {
      constexpr int T = decltype(bm)::value;
      using O = typename decltype(outc)::type;
      const int tn = (N + T - 1) / T, tm = (int)((M + T - 1) / T);
      hipLaunchKernelGGL((gemm_bf16_kernel<T, T, O>), dim3(tn * tm, splits), dim3(256), 0, s,
                         (const bf16*)A, lda, (const bf16*)W, ldw, bias, (const bf16*)R, ldr, (O*)C,
                         ldc, M, N, K, silu, tn, tn * tm, ksplit, c_split, (bf16*)act,
                         (bf16*)lo, lo_c0, sc_c0, sc_c1, sc, N, 0, 0);
    };
    using I128 = std::integral_constant<int, 128>;
    using I64 = std::integral_constant<int, 64>;
    struct F { using type = float; };
    struct H { using type = bf16; };
    if (big >= 256) {
      if (out_f32) go(I128{}, F{}); else go(I128{}, H{});
    } else {
      if (out_f32) go(I64{}, F{}); else go(I64{}, H{});
    }
  } else {
    if (splits > 1) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, (const float*)A, lda,
                       (const float*)W, ldw, bias, (const float*)R, ldr, (float*)C, ldc, M, N, K,
                       silu);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_tn(const void* A, int64_t lda, const void* B, int64_t ldb, float* C,
                          int64_t ldc, int M, int N, int64_t K, int splits, int64_t ksplit,
                          int64_t c_split, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (M % 8 != 0 || N % 8 != 0 || lda % 8 != 0 || ldb % 8 != 0 || ldc % 4 != 0 || K <= 0)
    return hipErrorInvalidValue;
  if (splits < 1) splits = 1;
  if (splits == 1) ksplit = K;
  const int64_t big = (int64_t)((N + 127) / 128) * ((M + 127) / 128) * splits;
  const int gbk = stage_k(big >= 256 ? 128 : 64);
  if (splits > 1 && (ksplit % gbk != 0 || (int64_t)(splits - 1) * ksplit >= K))
    return hipErrorInvalidValue;
  auto go = [&](auto bm) {
    constexpr int T = decltype(bm)::value;
    const int tn = (N + T - 1) / T, tm = (M + T - 1) / T;
    hipLaunchKernelGGL((gemm_tn_kernel<T, T>), dim3(tn * tm, splits), dim3(256), 0, s,
                       (const bf16*)A, lda, (const bf16*)B, ldb, C, ldc, M, N, K, tn, tn * tm,
                       ksplit, c_split);
  };
  if (big >= 256)
    go(std::integral_constant<int, 128>{});
  else
    go(std::integral_constant<int, 64>{});
  return hipGetLastError();
}

hipError_t launch_gemm_2cols(const void* A, int64_t lda, const void* W, int64_t ldw,
                             const float* bias, void* C, int64_t ldc, int64_t M, int K, int silu,
                             int c0, int len0, int c1, int len1, hipStream_t s) {
  if (M <= 0 || len0 + len1 <= 0) return hipSuccess;
  const int N = len0 + len1;
  if (len0 < 0 || len1 < 0 || c0 < 0 || c1 < 0 || N % 8 != 0 || K % 8 != 0 || lda % 8 != 0 ||
      ldw % 8 != 0 || ldc % 8 != 0)
    return hipErrorInvalidValue;
  const int64_t big = ((N + 127) / 128) * ((M + 127) / 128);
  auto go = [&](auto bm) {
    constexpr int T = decltype(bm)::value;
    // each window is whole tiles, so that no tile straddles the two
    if (len0 % T != 0 || c0 % 8 != 0 || c1 % 8 != 0) return hipErrorInvalidValue;
    const int tn = (N + T - 1) / T, tm = (int)((M + T - 1) / T);
    hipLaunchKernelGGL((gemm_bf16_kernel<T, T, bf16>), dim3(tn * tm, 1), dim3(256), 0, s,
                       (const bf16*)A, lda, (const bf16*)W, ldw, bias, (const bf16*)nullptr,
                       (int64_t)0, (bf16*)C, ldc, M, N, K, silu, tn, tn * tm, (int64_t)K,
                       (int64_t)0, (bf16*)nullptr, (bf16*)nullptr, 0, 0, 0, 1.f, len0, c0,
                       c1);
    return hipGetLastError();
  };
  return big >= 256 ? go(std::integral_constant<int, 128>{})
                    : go(std::integral_constant<int, 64>{});
}

hipError_t launch_gemm(const void* A, int64_t lda, const void* W, int64_t ldw, const float* bias,
                       const void* R, int64_t ldr, void* C, int64_t ldc, int64_t M, int N, int K,
                       int silu, int bf16flag, hipStream_t s, void* lo, int lo_c0, int sc_c0,
                       int sc_c1, float sc) {
  return launch_gemm_ex(A, lda, W, ldw, bias, R, ldr, C, ldc, M, N, K, silu, bf16flag, 0, 1, K, 0,
                        nullptr, s, lo, lo_c0, sc_c0, sc_c1, sc);
}

}  // namespace hstu
