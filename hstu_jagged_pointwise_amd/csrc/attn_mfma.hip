// Fused HSTU pointwise attention on gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// Eq. 2 of the HSTU layer ("What an HSTU layer changes", HSTU chapter):
//   O_i = (1/N) sum_{j visible} SiLU(q_i.k_j + rab_pos[bp(i,j)] + rab_time[bt(i,j)]) v_j
// There is no softmax ("No sequence-wise softmax"), so the pass is single and
// needs no running maximum, no row sum and no rescaling of the accumulator.
// Each score is activated on its own and fed straight into the second
// contraction.
//
// Work decomposition. A workgroup (4 wavefronts) owns 128 query rows of one
// head. Each wavefront owns 32 rows. Keys stream through a double-buffered LDS
// tile of 64: the next tile's global loads are in flight while the current
// tile is computed, with one barrier per tile. Per 32-key block a wavefront runs:
//   S^T = K Q^T  with v_mfma_f32_32x32x16_bf16. Q stays in registers as the B
//                operand. The accumulator holds one query row per lane
//                (lane % 32) and 16 keys per lane.
//   P = SiLU(S + bias), on the vector ALU.
//   O += P V     again with the 32x32x16 MFMA. P goes in as the A operand
//                straight from registers; the key order of the accumulator
//                defines the contraction order, and V is read in that order
//                with ds_read_b64_tr_b16, which transposes row-major V on the
//                way out of LDS.
// Both 32-key blocks of a tile issue their S MFMAs first, so the matrix core
// works on block 1 while the vector ALU activates block 0.
//
// Bias classes, decided per (wavefront, 32-key block) from exact integer
// ranges. The lanes decide them in bulk, lane i for key block i of a group of
// 64 (32 tiles), and each tile reads its two blocks' classes from their lanes
// (v_readlane), so the per-tile cost is a few instructions:
//   * The position bucket min(i-j, P-1) is one constant when every i-j >= P-1.
//   * The time bucket is monotone in the elapsed time, so over the block's
//     elapsed-time range [min t_i - max t_j, max t_i - min t_j] (the key side
//     comes precomputed per 32-key block, see KeyRange) its values run from the
//     bucket of the lower end to the bucket of the upper end:
//       - one bucket: a constant;
//       - two adjacent buckets b, b+1: an element is in b+1 exactly when
//         t_i + 1 - t_j >= 2^(b+1), one 32-bit compare and select per element;
//       - more: the bucket of each element from the count of leading zeros of
//         the 32-bit t_i + 1 - t_j (a 64-bit path covers spans past 2^31 s).
//   * A constant bias is the starting value of the S^T accumulator (exact fp32,
//     16 moves per block; candidate mode adds it as an extra MFMA k-step, see
//     bias_step). A block whose position bucket varies gathers it per element
//     from an LDS-resident table.
// Masking is a select after SiLU (SiLU(-inf) would be NaN). It runs only on
// blocks that cross the causal diagonal (or the history tail for candidates).
// Blocks entirely above the diagonal are skipped.
//
// Candidate mode (M-FALCON): the queries are one user's candidates, all at
// position n_h. The keys are that user's history, all visible. The first key
// range also scores each candidate against its own key and stores the weight
// SiLU(score) / N per row and head; the layer norm that reads the summed rows
// adds weight * v_c there, so no split rereads V of the candidates. When a wavefront's
// candidates share one timestamp, a pair's whole bias depends on its key only;
// an extra MFMA k-step then multiplies a per-key bias by ones, and every unmasked block
// takes the fast path whatever its buckets.
#include "attn_common.h"

#include <type_traits>

namespace hstu {

namespace {
constexpr int MBM = kMfmaRows;  // 128 query rows per workgroup
constexpr int MBN = 64;         // keys per LDS tile
constexpr int kMaxP = 1024;     // position-table entries kept in LDS
// The position table in LDS is padded on both sides with its clamped values: entry
// kPadLo + d holds rab_pos[min(max(d, 0), P - 1)] for d = -kPadLo .. P - 1 + kPadHi. A
// 32 x 32 block whose bucket varies has every i - j in that range (see general_block), so
// its elements read the table at one base plus constant offsets, with no clamping.
constexpr int kPadLo = 64, kPadHi = 64;
constexpr int kTimeTab = 64;    // time-table entries ever reachable (buckets <= 63)
constexpr int kBufferWord3 = 0x00020000;  // buffer descriptor dword 3: 32-bit data format, raw

// One 16-byte-per-lane buffer load into LDS: lane L's chunk at base + voff lands in
// slot L of the 1 KiB span at lds. The descriptor's record count is limoff + 16, the
// end of the last valid chunk: a lane past it reads zeros. (The flat-encoded global
// form would make the compiler count every fetch against the LDS counter as well, so
// that a wait for an LDS read would also wait for the fetches in flight.)
__device__ __forceinline__ void fetch16(const char* base, uint32_t limoff, bf16* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)(limoff + 16u), kBufferWord3),
      (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ bf16x4 tr_read(const bf16* lds_ptr) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(lds_ptr));
  return __builtin_bit_cast(bf16x4, r);
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Element offset of (row, col) in a 64-row K or V tile: rows padded by 8 elements.
// With a row stride of D+8 elements the 16 rows of one row-fragment load
// (ds_read_b128) fall in distinct banks, and every read address is one base
// register plus an immediate, which keeps register pressure down.
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * (D + 8) + col;
}
template <int D>
constexpr int tile_elems() {
  return MBN * (D + 8);
}
// V tiles: unpadded rows whose 16-byte chunks are permuted by an XOR of the row. A
// transposing read (ds_read_b64_tr_b16) of 16 lanes covers 4 consecutive rows and 2
// adjacent chunks, and the lanes of the next 16 the next 2 chunks of the same rows;
// the XOR moves each of the 4 rows' chunks to a different quarter of the row, so the
// 32 lanes touch 32 distinct bank pairs.
template <int D>
__device__ __forceinline__ int vswz(int row) {
  return (row & 3) * (D / 32);
}
template <int D>
__device__ __forceinline__ int vtile_off(int row, int col) {
  return row * D + ((((col >> 3) ^ vswz<D>(row))) << 3) + (col & 7);
}

// exact time bucket of an elapsed time (negative counts as 0), clamped to the table
__device__ __forceinline__ int bucket_of(int64_t dt, int T) {
  dt = dt < 0 ? 0 : dt;
  const int b = 63 - __builtin_clzll((uint64_t)dt + 1ull);
  return b < T - 1 ? b : T - 1;
}

// Bias classes of one tile's two 32-key blocks for one wavefront (uniform
// values), packed so that two tiles' worth stays in few scalar registers.
// Byte kb of f describes block kb:
//   bit 0 act      some key of the block is visible to some row of the wavefront
//   bit 1 mask     the block needs the per-element visibility mask
//   bit 2 pos_c    one position bucket over the block (or no position bias)
//   bits 3-4 tmode time bias: 0 one bucket (or none), 1 two adjacent buckets, 2 general
//   bit 5 tfast    every elapsed time fits the 32-bit forms
// and bits 16 + 8*kb .. 21 + 8*kb hold the block's highest time bucket bhi
// (tmode 1: an element is in it when the 32-bit t_i + 1 - t_j >= 2^bhi).
struct TileClass {
  uint32_t f;
  float tlo[2], thi[2];  // time-table values of each block's lowest and highest bucket
};
struct BlockClass {  // one block's view of a TileClass
  uint32_t bits, bhi;
  float tlo, thi;
  __device__ bool act() const { return bits & 1u; }
  __device__ bool mask() const { return bits & 2u; }
  __device__ bool pos_c() const { return bits & 4u; }
  __device__ uint32_t tmode() const { return (bits >> 3) & 3u; }
  __device__ bool tfast() const { return bits & 32u; }
  __device__ int thr() const { return (int)(1u << bhi); }
};
__device__ __forceinline__ BlockClass block_class(const TileClass& c, int kb) {
  return BlockClass{(c.f >> (8 * kb)) & 0xffu, (c.f >> (16 + 8 * kb)) & 63u, c.tlo[kb], c.thi[kb]};
}
}  // namespace

bool attn_mfma_supported(int dtype_bf16, int d_qk, int d_v, int P, int T) {
  (void)T;
  return dtype_bf16 && d_qk == d_v && (d_qk == 32 || d_qk == 64 || d_qk == 128) && P <= kMaxP;
}

bool attn_mfma_strides_ok(const AttnArgs& a) {
  // the key-tile DMA shares one per-lane byte offset between K and V; offsets are 32-bit
  return a.ld_k == a.ld_v && a.ld_k > 0 && (int64_t)(MBN + 1) * a.ld_k * 2 < (int64_t(1) << 32);
}

// SPLIT (causal mode only): queries and keys come as bf16 pairs hi + lo (a.q / a.q_lo,
// a.k / a.k_lo, same strides) carrying about 16 significant bits, and each score is
// hi.hi + lo.hi + hi.lo: three MFMAs per k-step, the lo.lo term (about 2^-16 relative)
// left out. The layer path uses it for the Q and K it computes itself.
//
// Pre-scaled queries (candidate mode and SPLIT, i.e. the queries the library computes
// itself in its f1 projection): q arrives multiplied by -log2(e) (the projection stores
// it so, rounded to bf16 from fp32 like any stored query), and the bias tables are
// scaled the same way when they are copied to LDS. A score then comes out of the MFMA
// as x' = -log2(e) x, so that SiLU needs no multiply before the exponential:
// SiLU(x) = x' * rcp(1 + exp2(x')) / -log2(e), and the 1/-log2(e) joins the 1/N of the
// output scale.
template <int D, bool CAND, bool SPLIT>
__global__ __launch_bounds__(256, SPLIT ? (D <= 64 ? 2 : 1) : (D <= 64 ? 3 : 2)) void
attn_mfma_kernel(AttnArgs a) {
  static_assert(!(CAND && SPLIT), "split scores are for causal mode");
  constexpr bool PRE = CAND || SPLIT;
  constexpr float kPre = -kLog2e;     // the scale of pre-scaled queries and tables
  const float tscale = PRE ? kPre : 1.f;
  constexpr int NKK = D / 16;  // k-steps of the S^T contraction
  constexpr int NC = D / 32;   // 32-wide output column blocks
  constexpr int CPR = D / 8;   // 16-byte chunks per row
  constexpr int TE = tile_elems<D>();
  // two LDS buffers per matrix as separate objects, so that alias analysis can tell
  // the in-flight DMA target from the buffer being read (no conservative waits)
  __shared__ __attribute__((aligned(16))) bf16 Ks0[TE];
  __shared__ __attribute__((aligned(16))) bf16 Ks1[TE];
  __shared__ __attribute__((aligned(16))) bf16 Kl0[SPLIT ? TE : 8];  // K lo parts (SPLIT)
  __shared__ __attribute__((aligned(16))) bf16 Kl1[SPLIT ? TE : 8];
  __shared__ __attribute__((aligned(16))) bf16 Vs0[MBN * D];
  __shared__ __attribute__((aligned(16))) bf16 Vs1[MBN * D];
  __shared__ __attribute__((aligned(16))) uint32_t tk_lo[2][MBN];
  __shared__ int64_t tk64[2][MBN];
  __shared__ float rpx[kPadLo + kMaxP + kPadHi];
  __shared__ float rt[kTimeTab];
  __shared__ float rtc[32];

  const TileDecode t = decode<CAND>(a, MBM);
  if (!t.valid) return;  // uniform across the workgroup
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int wu = uniform(w);
  const int l32 = lane & 31, hl = lane >> 5;
  const int h = t.h;
  const bf16* q = (const bf16*)a.q;
  const bool has_pos = a.rab_pos != nullptr;
  const bool has_time = a.rab_time != nullptr && a.ts_q != nullptr && a.ts_k != nullptr &&
                        a.key_ranges != nullptr;
  const int P = a.P, T = a.T;

  // this lane's query row (the S^T column it holds)
  const int wrow = 32 * w + l32;
  const bool row_ok = wrow < t.rows;
  const bool wave_live = 32 * wu < t.rows;
  // positions inside one sequence fit in 32 bits (lengths are bounded by an int N)
  const int nk = (int)t.nk, kend = (int)t.kend, kbeg = (int)t.kbeg, qpos0 = (int)t.qpos0;

  // ---- key tiles go global -> LDS directly (buffer_load_dwordx4 ... lds): lane L of
  // one instruction fills 16-byte slot L of a contiguous 1 KiB span, so the LDS layout
  // comes from which source chunk each lane fetches. K rows are padded by one slot
  // (row-fragment reads, see tile_off); V rows are unpadded with their 16-byte chunks
  // permuted by an XOR of the row (see vtile_off). Rows past the data read zeros (see
  // fetch16): their scores are masked, and they multiply P = 0.
  constexpr int SPR = CPR + 1;        // 16-byte slots per K row
  constexpr int NSLOT = MBN * SPR;    // slots per K tile
  constexpr int NINSTR = NSLOT / 64;  // wave-instructions per K tile
  constexpr int NIW = (NINSTR + 3) / 4;
  static_assert(NSLOT % 64 == 0, "every DMA instruction fills 64 slots");
  static_assert(MBN * CPR == 4 * 64 * (NIW - 1), "each wavefront issues NIW - 1 V instructions");
  // Wavefront w issues instructions w, w+4, w+8, ... of each matrix tile. The byte
  // offset of each of its slots' source chunk from the tile's first row is computed
  // once (K and V share the row stride). The address is the tile's base (a buffer
  // descriptor) plus that 32-bit offset. Offsets grow with the row (a row's chunks span
  // less than the row stride), so a record count that ends at the last valid row's last
  // chunk keeps every fetch inside the data.
  const uint32_t ldb = (uint32_t)(a.ld_k * 2);
  uint32_t offk[NIW], offv[NIW - 1];
#pragma unroll
  for (int j = 0; j < NIW; ++j) {
    const int slot = 64 * (w + 4 * j) + lane;
    const int row = slot / SPR, pc = slot % SPR;
    offk[j] = (uint32_t)row * ldb + 16u * (uint32_t)(pc < CPR ? pc : 0);
  }
#pragma unroll
  for (int j = 0; j < NIW - 1; ++j) {
    const int slot = 64 * (w + 4 * j) + lane;
    const int row = slot / CPR;
    offv[j] = (uint32_t)row * ldb + 16u * (uint32_t)((slot % CPR) ^ vswz<D>(row));
  }
  const char* kg = (const char*)a.k + (int64_t)h * D * 2;
  const char* vg = (const char*)a.v + (int64_t)h * D * 2;
  struct DmaSrc {
    const char* kb;
    const char* vb;
    const char* klb;  // K lo parts (SPLIT), same row stride as K
    uint32_t lim;     // last key row of the data, counted from the tile's first row
    uint32_t limoff;  // offset of that row's last chunk (rows past the tile: its last row's);
                      // the descriptor's record count is limoff + 16
  };
  auto lim_off = [&](uint32_t lim) {
    return (lim < (uint32_t)MBN - 1 ? lim : (uint32_t)MBN - 1) * ldb + 16u * (CPR - 1);
  };
  // the source of the tile being fetched: set for the first tile, then advanced by one
  // tile of rows per step (K and V share the row stride)
  DmaSrc nsrc{kg + (t.k_base + kbeg) * a.ld_k * 2, vg + (t.k_base + kbeg) * a.ld_v * 2,
              SPLIT ? (const char*)a.k_lo + (int64_t)h * D * 2 + (t.k_base + kbeg) * a.ld_k * 2
                    : nullptr,
              (uint32_t)(nk - 1 - kbeg), 0u};
  nsrc.limoff = lim_off(nsrc.lim);
  const int64_t tile_bytes = (int64_t)MBN * a.ld_k * 2;
  // this wavefront's instruction pair j (K and V; the last K instruction has no V
  // partner) for one tile
  auto dma_pair = [&](auto bufc, const DmaSrc& src, int j) {
    constexpr int buf = decltype(bufc)::value;
    bf16* Kd = buf ? Ks1 : Ks0;
    bf16* Vd = buf ? Vs1 : Vs0;
    const int i = wu + 4 * j;
    fetch16(src.kb, src.limoff, &Kd[512 * i], offk[j]);
    if constexpr (SPLIT) fetch16(src.klb, src.limoff, &(buf ? Kl1 : Kl0)[512 * i], offk[j]);
    if (j < NIW - 1) fetch16(src.vb, src.limoff, &Vd[512 * i], offv[j]);
  };
  static_assert(NINSTR == 4 * (NIW - 1) + 1, "only wavefront 0 issues a last K instruction");
  auto dma_tile = [&](auto bufc, const DmaSrc& src) {
#pragma unroll
    for (int j = 0; j < NIW - 1; ++j) dma_pair(bufc, src, j);
    if (wu == 0) dma_pair(bufc, src, NIW - 1);
  };
  int64_t ptk = 0;
  // each wavefront fetches the timestamps of 16 of the tile's keys
  auto ts_fetch = [&](int k0) {
    if (has_time && lane < 16) {
      const int key = k0 + 16 * w + lane;
      ptk = key < nk ? a.ts_k[t.k_base + key] : 0;
    }
  };
  auto finish_tile = [&](auto bufc, bool store_ts) {
    constexpr int buf = decltype(bufc)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (store_ts && has_time && lane < 16) {
      tk_lo[buf][16 * w + lane] = (uint32_t)ptk;
      tk64[buf][16 * w + lane] = ptk;
    }
  };

  // ---- bias classes, from the key blocks' precomputed timestamp ranges. Lane i of
  // the wavefront classifies key block 64 g + i of the range (32 keys each) for a
  // group g of 64 blocks, 32 tiles; each tile then reads its two blocks' classes
  // from their lanes. The ranges of the next group are fetched a group ahead.
  const KeyRange* krs = has_time ? a.key_ranges + key_range_slot(t.k_base, t.seq) : nullptr;
  struct LaneClass {
    uint32_t bits;  // a TileClass byte in bits 0-5, the highest time bucket in bits 8-13
    float tlo, thi;
  };
  auto lane_range = [&](int g) {
    KeyRange r{0, 0};
    const int kb0 = kbeg + 32 * (64 * g + lane);
    if (has_time && wave_live && kb0 < kend) r = krs[kb0 >> 5];
    return r;
  };

  const int nkt = (kend - kbeg + MBN - 1) / MBN;
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  // The first tile's keys, values, key timestamps and timestamp ranges are requested
  // before the bias tables, the queries and the query timestamps, so that both sets of
  // loads are in flight together: one memory round trip before the first tile, not two.
  KeyRange lrn{0, 0};  // this lane's timestamp range in the next group
  if (nkt > 0) {
    dma_tile(B0{}, nsrc);
    ts_fetch(kbeg);
    lrn = lane_range(0);
  }

  // bias-table entries: loaded into registers here (indices clamped into the tables, no
  // divergent branches) and written to LDS once the queries' loads are issued too
  float vp = 0.f, vt = 0.f, vtc = 0.f;
  if (has_pos) vp = a.rab_pos[(int64_t)h * P + min(max(tid - kPadLo, 0), P - 1)];
  if (has_time) {
    vt = a.rab_time[(int64_t)h * T + min(tid, T - 1)];     // rt[tid], tid < kTimeTab
    vtc = a.rab_time[(int64_t)h * T + min(max(31 - tid, 0), T - 1)];  // rtc[tid], tid < 32
  }
  const float pb = has_pos ? tscale * sload(a.rab_pos + (int64_t)h * P + P - 1) : 0.f;  // P-1

  // this lane's Q fragment; lanes past the tile's rows load its last row (no divergent
  // branch between the loads) and zero it once the loads have landed
  bf16x8 qf[NKK];
  bf16x8 qlf[SPLIT ? NKK : 1];  // lo parts of the queries (SPLIT)
  const int qrow = row_ok ? wrow : t.rows - 1;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int64_t qo = (t.q_local + qrow) * a.ld_q + (int64_t)h * D + 16 * kk + 8 * hl;
    qf[kk] = load_bf16x8(q + qo);
    if constexpr (SPLIT) qlf[kk] = load_bf16x8((const bf16*)a.q_lo + qo);
  }
  // candidate mode, first key range: the candidate's own key (relative position 0,
  // elapsed time 0) is loaded with Q and its weight SiLU(score) / N stored per row and
  // head, for the layer norm that follows to add weight * v_c (it reads the row anyway)
  if (CAND && blockIdx.z == 0) {
    const bf16* kc = (const bf16*)a.kc;
    float part = 0.f;
    if (row_ok) {
      bf16x8 kf[NKK];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        kf[kk] = load_bf16x8(kc + (t.q_local + wrow) * a.ld_kc + (int64_t)h * D + 16 * kk + 8 * hl);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int i = 0; i < 8; ++i) part = fmaf((float)qf[kk][i], (float)kf[kk][i], part);
    }
    part += __shfl_xor(part, 32, 64);
    float xs = part;  // pre-scaled like the queries
    if (has_pos) xs += kPre * sload(a.rab_pos + (int64_t)h * P);
    if (has_time) xs += kPre * sload(a.rab_time + (int64_t)h * T);
    if (hl == 0 && row_ok)
      a.self_w[(t.q_local + wrow) * a.H + h] = silu_prescaled(xs) * (a.inv_n / kPre);
  }
  const int64_t tq = (has_time && row_ok) ? a.ts_q[t.q_base + wrow] : 0;
  const uint32_t tq1 = (uint32_t)tq + 1u;
  const int64_t qmin = uniform64(wave_min64(row_ok ? tq : INT64_MAX));
  const int64_t qmax = uniform64(wave_max64(row_ok ? tq : INT64_MIN));
  // (the pin keeps the scaling here: folded into the loads' branches it would wait there)
  asm volatile("" : "+v"(vp), "+v"(vt), "+v"(vtc));
  if (has_pos) {
    const int np = kPadLo + P + kPadHi;
    if (tid < np) rpx[tid] = tscale * vp;
    for (int i = tid + 256; i < np; i += 256)
      rpx[i] = tscale * a.rab_pos[(int64_t)h * P + min(max(i - kPadLo, 0), P - 1)];
  }
  if (has_time) {
    if (tid < kTimeTab) rt[tid] = tscale * vt;
    if (tid < 32) rtc[tid] = tscale * vtc;
  }
  if (!row_ok) {
    const bf16x8 z = {};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qf[kk] = z;
      if constexpr (SPLIT) qlf[kk] = z;
    }
  }
  const int qpos = CAND ? qpos0 : qpos0 + wrow;
  const int wrow0 = qpos0 + 32 * wu;                        // the wavefront's first row
  const int wlast = qpos0 + min(32 * wu + 31, t.rows - 1);  // its last live row
  // candidate mode: the wavefront's candidates share one timestamp (or there is no time
  // bias), so a pair's bias depends on the key alone
  const bool keyb_ok = CAND && (!has_time || qmin == qmax);

  // constant fragment of the bias k-step (candidate mode), [0] = [1] = 1 in the first
  // half-wavefront, rebuilt at each use rather than held in registers
  const uint32_t ones_w = hl == 0 ? 0x3f803f80u : 0u;  // two bf16 ones in one word
  auto ones = [&]() {
    u32x4 f = {ones_w, 0u, 0u, 0u};
    return __builtin_bit_cast(bf16x8, f);
  };

  f32x16 o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[c][r] = 0.f;

  auto lane_classify = [&](int g, const KeyRange& r) {
    const int kb0 = kbeg + 32 * (64 * g + lane);
    const bool act = wave_live && kb0 < kend && (CAND || kb0 <= wlast);
    const bool mask = CAND ? (kb0 + 32 > kend) : (kb0 + 31 > wrow0);
    const int min_dpos = (CAND ? qpos0 : wrow0) - (kb0 + 31);
    const bool pos_c = !has_pos || min_dpos >= P - 1;
    LaneClass c{(act ? 1u : 0u) | (mask ? 2u : 0u) | (pos_c ? 4u : 0u) | 32u, 0.f, 0.f};
    if (has_time && act) {
      const int64_t lo = qmin - r.hi, hi = qmax - r.lo;  // elapsed-time range
      const int blo = bucket_of(lo, T), bhi = bucket_of(hi, T);
      const bool tfast = time_fast_ok(qmin, qmax, r.lo, r.hi);
      const uint32_t tmode = blo == bhi ? 0u : ((bhi == blo + 1 && tfast) ? 1u : 2u);
      c.bits = (c.bits & 7u) | (tmode << 3) | (tfast ? 32u : 0u) |
               ((uint32_t)bhi << 8);
      c.tlo = rt[blo];
      c.thi = rt[bhi];
    }
    return c;
  };
  auto tile_class = [&](const LaneClass& lc, int kt) {
    const int l0 = (2 * kt) & 63;  // the tile's first block's lane
    const uint32_t b0 = __builtin_amdgcn_readlane(lc.bits, l0);
    const uint32_t b1 = __builtin_amdgcn_readlane(lc.bits, l0 + 1);
    auto rdf = [&](float v, int l) {
      return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
    };
    TileClass c;
    c.f = (b0 & 0xffu) | ((b1 & 0xffu) << 8) | ((b0 >> 8) << 16) | ((b1 >> 8) << 24);
    c.tlo[0] = rdf(lc.tlo, l0);
    c.tlo[1] = rdf(lc.tlo, l0 + 1);
    c.thi[0] = rdf(lc.thi, l0);
    c.thi[1] = rdf(lc.thi, l0 + 1);
    return c;
  };

  // Pipeline: tile t computes while tile t+1's keys and values stream into the
  // idle buffer. Every 32 tiles the lanes classify the next 64 key blocks from
  // timestamp ranges fetched 32 tiles earlier.
  LaneClass lcl{0u, 0.f, 0.f};
  if (nkt > 0) finish_tile(B0{}, true);
  __syncthreads();  // also publishes the bias tables in LDS
  if (nkt > 0) {
    lcl = lane_classify(0, lrn);
    if (nkt > 32) lrn = lane_range(1);
  }

  auto kfrag = [&](const bf16* Kt, int kb, int kk) {
    return load_bf16x8(&Kt[tile_off<D>(32 * kb + l32, 16 * kk + 8 * hl)]);
  };
  // fragment of the bias k-step: k-slots 0 and 1 hold bias_hi and bias_lo (a bf16
  // split, exact to ~2^-16 relative) of this lane's query or, for a per-key bias, key
  auto bias_frag = [&](float bias) {
    bf16x8 bfrag;
#pragma unroll
    for (int i = 0; i < 8; ++i) bfrag[i] = (bf16)0.f;
    const bf16 bhi = (bf16)bias;
    if (hl == 0) {
      bfrag[0] = bhi;
      bfrag[1] = (bf16)(bias - (float)bhi);
    }
    return bfrag;
  };
  const int g16 = lane >> 4, rho = lane & 15;
  // V fragment m = s2 * NC + c of 32-key block kb: the k-slot (hl, i) of step s2
  // is key 16*s2 + 8*(i/4) + 4*hl + i%4, the accumulator's key order
  auto vfrag = [&](const bf16* Vt, int kb, int m) {
    const int s2 = m / NC, c = m % NC;
    const int krow = 32 * kb + 16 * s2 + 4 * hl + (rho >> 2);
    const int col = c * 32 + 16 * (g16 & 1) + 4 * (rho & 3);
    const bf16x4 v1 = tr_read(&Vt[vtile_off<D>(krow, col)]);
    const bf16x4 v2 = tr_read(&Vt[vtile_off<D>(krow + 8, col)]);
    bf16x8 bv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bv[i] = v1[i];
      bv[4 + i] = v2[i];
    }
    return bv;
  };

  auto tile_step = [&](auto bufc, int kt) {
    constexpr int buf = decltype(bufc)::value;
    using BN_ = std::integral_constant<int, 1 - buf>;
    const int k0 = kbeg + kt * MBN;
    const bool more = kt + 1 < nkt;
    const int kn = k0 + MBN;  // the next tile's first key
    // the last tile refills the idle buffer with its own keys (harmless), so
    // that the DMA inside the fenced fast path needs no branch
    if (more) {
      nsrc.kb += tile_bytes;
      nsrc.vb += tile_bytes;
      if constexpr (SPLIT) nsrc.klb += tile_bytes;
      nsrc.lim -= MBN;
      nsrc.limoff = lim_off(nsrc.lim);
    }
    auto dma = [&](int j) { dma_pair(BN_{}, nsrc, j); };
    if (wu == 0) dma(NIW - 1);
    if (more) ts_fetch(kn);
    if (kt > 0 && (kt & 31) == 0) {  // a new group of 64 key blocks
      lcl = lane_classify(kt >> 5, lrn);
      if (kt + 32 < nkt) lrn = lane_range((kt >> 5) + 1);
    }
    const TileClass cls = tile_class(lcl, kt);
    const BlockClass c0 = block_class(cls, 0);
    const BlockClass c1 = block_class(cls, 1);
    const bf16* Kt = buf ? Ks1 : Ks0;
    const bf16* Klt = buf ? Kl1 : Kl0;
    const bf16* Vt = buf ? Vs1 : Vs0;
    // both blocks active, unmasked, one position bucket, one time bucket
    const bool fast = (cls.f & 0x1f1fu) == 0x0505u;
    // candidate mode with one timestamp per wavefront: both blocks live and unmasked suffice
    const bool keyb_tile = CAND && keyb_ok && (cls.f & 0x0303u) == 0x0101u;
    // causal mode: both blocks live, unmasked, one position bucket, one or two time
    // buckets each (the fast path's schedule plus a per-element two-bucket select)
    const bool fast2 = !CAND && (cls.f & 0x1717u) == 0x0505u;
    constexpr int E = 16 / NKK;  // scores activated per interleaved step
    // SiLU of accumulator slots st*E .. st*E+E-1 into bf16 A fragments, as c SiLU(x)
    // with c = -log2(e) (the output scale divides c out again). Pre-scaled scores
    // arrive as c x with their bias inside; otherwise a block on the fast paths starts
    // its S^T chain from 0 and its constant bias, scaled, is cb, which joins the score
    // in the same fma that scales it (cb = 0 when the accumulator holds the bias).
    auto act_step = [&](const f32x16& x, float cb, bf16x8* pa, int st) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int r = st * E + e;
        const float xp = PRE ? x[r] : fmaf(x[r], kPre, cb);
        pa[r >> 3][r & 7] = (bf16)silu_prescaled(xp);
      }
    };
    // the start of a block's S^T accumulator: the block's constant bias, or, given keyA,
    // a bias per key through one MFMA k-step (keyA on the key side, ones on the query
    // side). Candidate mode takes its constant bias through the same k-step (ones times
    // a bf16 hi/lo split), so that a candidate's scores round the same way whichever of
    // the two its wavefront takes.
    auto bias_step = [&](float bias, const bf16x8* keyA) -> f32x16 {
      if (keyA) return __builtin_amdgcn_mfma_f32_32x32x16_bf16(*keyA, ones(), f32x16{}, 0, 0, 0);
      if constexpr (CAND)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones(), bias_frag(bias), f32x16{}, 0, 0, 0);
      f32x16 xb;
#pragma unroll
      for (int r = 0; r < 16; ++r) xb[r] = bias;
      return xb;
    };
    // S^T of one block, starting from the constant part of its bias
    // one k-step of a block's S^T: hi.hi, then (SPLIT) lo.hi and hi.lo
    auto s_step = [&](f32x16 x, const bf16x8& kh, const bf16x8& kl, int kk) {
      x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qf[kk], x, 0, 0, 0);
      if constexpr (SPLIT) {
        x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kl, qf[kk], x, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qlf[kk], x, 0, 0, 0);
      }
      return x;
    };
    auto s_chain = [&](int kb, float bias, const bf16x8* keyA, bool with_dma) {
      bf16x8 kq[NKK], kql[SPLIT ? NKK : 1];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        kq[kk] = kfrag(Kt, kb, kk);
        if constexpr (SPLIT) kql[kk] = kfrag(Klt, kb, kk);
      }
      f32x16 x = bias_step(bias, keyA);
      if (with_dma) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        x = s_step(x, kq[kk], kql[SPLIT ? kk : 0], kk);
        if (with_dma) {  // the dependent chain has room for the next tile's DMA
          if (kk < NIW - 1) dma(kk);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      return x;
    };
    // Each tile ends in one shared tail, the only code that touches the output
    // accumulators: block 0's P V, carrying the SiLU of block 1's scores x1,
    // then block 1's P V. The paths before it hand over block 0's P fragments
    // pa0 and x1. A masked or inactive score is handed over as 0, whose SiLU is
    // exactly 0.
    bf16x8 pa0[2];
    f32x16 x1;
    // the fast paths' constant biases (plain causal mode: the chains start from 0 and
    // each block's constant joins its SiLU), else 0
    const float cb0 = PRE ? 0.f : kPre * (pb + c0.tlo);
    const float cb1 = PRE ? 0.f : kPre * (pb + c1.tlo);
    float cba = 0.f, cbb = 0.f;  // the constants of block 0 and block 1 as activated
    const float sb0 = PRE ? pb + c0.tlo : 0.f;  // the fast paths' accumulator starts
    const float sb1 = PRE ? pb + c1.tlo : 0.f;
    // Common case: both blocks live, no mask, one position bucket and one time
    // bucket per block, so the bias is a constant that starts the accumulator. The
    // path is one basic block (no branch, so nothing moves across the fences);
    // its instruction order is written out and fenced (sched_barrier) so that
    // the in-order wavefront issues one MFMA, then the independent vector work
    // that fits under it: block 0's S^T chain; block 1's S^T chain, each step
    // carrying the SiLU of 16/NKK of block 0's scores.
    //
    // Candidate mode, when the wavefront's candidates share one timestamp: every
    // candidate sits at position n_h, so the whole bias of a pair depends on its key
    // alone. The bias step then carries a per-key bias (key-side fragment) times ones
    // (query side), and any unmasked block takes this path, whatever its buckets.
    auto fast_path = [&](bool keyb) {
      bf16x8 kA[2];
      if constexpr (CAND) {
        // the whole bias of a key (position n_h - j, elapsed time t_c - t_j), one key per
        // lane: lane L takes key k0 + L (block 0 in the low half-wavefront, block 1 in the
        // high one), split into bf16 high and low parts packed in one word; the k-step
        // fragments carry the word in the low half-wavefront only
        const int j = k0 + lane;
        float b = has_pos ? rpx[kPadLo + min(qpos0 - j, P - 1)] : 0.f;
        if (has_time) {
          // both blocks' elapsed times fit the 32-bit form: the same bucket from the low
          // words (the count-of-leading-zeros table holds the same values as rt)
          if ((cls.f & 0x2020u) == 0x2020u)
            b += rtc[time_clz_fast((uint32_t)qmin + 1u, tk_lo[buf][lane])];
          else
            b += rt[bucket_of(qmin - tk64[buf][lane], T)];
        }
        const bf16 bh = (bf16)b;
        const bf16 bl = (bf16)(b - (float)bh);
        const uint32_t word = (uint32_t)__builtin_bit_cast(uint16_t, bh) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, bl) << 16);
        const uint32_t word1 = (uint32_t)__shfl_xor((int)word, 32, 64);  // block 1's key
        const u32x4 f0 = {hl == 0 ? word : 0u, 0u, 0u, 0u};
        const u32x4 f1 = {hl == 0 ? word1 : 0u, 0u, 0u, 0u};
        kA[0] = __builtin_bit_cast(bf16x8, f0);
        kA[1] = __builtin_bit_cast(bf16x8, f1);
      }
      cba = cb0;
      cbb = cb1;
      const f32x16 s0 = s_chain(0, sb0, CAND && keyb ? &kA[0] : nullptr, true);
      bf16x8 k1[NKK], k1l[SPLIT ? NKK : 1];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        k1[kk] = kfrag(Kt, 1, kk);
        if constexpr (SPLIT) k1l[kk] = kfrag(Klt, 1, kk);
      }
      f32x16 s1 = bias_step(sb1, CAND && keyb ? &kA[1] : nullptr);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        s1 = s_step(s1, k1[kk], k1l[SPLIT ? kk : 0], kk);
        act_step(s0, cba, pa0, kk);
        __builtin_amdgcn_sched_barrier(0);
      }
      x1 = s1;
    };

    // General path, one 32-key block at a time: any mix of masks, per-element
    // position buckets and per-element time buckets; the constant part of the
    // bias (the lower time bucket when two) starts the accumulator.
    // The upper bucket's excess over the constant, for the elements whose elapsed time
    // reaches it (two-bucket blocks); the general path uses the same code.
    auto two_bucket = [&](f32x16& x, int kb, const BlockClass& bc) {
      const uint32_t* tkl = tk_lo[buf] + 32 * kb + 4 * hl;
      const float dl = bc.thi - bc.tlo;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const u32x4 tk4 = *reinterpret_cast<const u32x4*>(tkl + 8 * g4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = (int)(tq1 - tk4[e]);
          x[4 * g4 + e] += d >= bc.thr() ? dl : 0.f;
        }
      }
    };
    // Fast path with two-bucket blocks (causal mode): the fast path's order, each
    // block's scores corrected right after its S^T chain.
    auto fast2_path = [&]() {
      cba = cb0;
      cbb = cb1;
      f32x16 s0 = s_chain(0, sb0, nullptr, true);
      if (c0.tmode() == 1) two_bucket(s0, 0, c0);
      bf16x8 k1[NKK], k1l[SPLIT ? NKK : 1];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        k1[kk] = kfrag(Kt, 1, kk);
        if constexpr (SPLIT) k1l[kk] = kfrag(Klt, 1, kk);
      }
      f32x16 s1 = bias_step(sb1, nullptr);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        s1 = s_step(s1, k1[kk], k1l[SPLIT ? kk : 0], kk);
        act_step(s0, cba, pa0, kk);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (c1.tmode() == 1) two_bucket(s1, 1, c1);
      x1 = s1;
    };

    auto general_block = [&](int kb, const BlockClass& bc) {
      if (!bc.act()) return f32x16{};
      const int kb0 = k0 + 32 * kb;
      if constexpr (CAND) {
        // Candidate mode: each pair's whole bias, formed as the per-key path forms it
        // (position term plus time term in fp32, split into a bf16 high and low part,
        // whose sum is exact in fp32), starts the accumulator. A candidate's scores then
        // round the same way whichever path its wavefront takes, so its output does not
        // depend on which candidates share its wavefront.
        f32x16 x;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = kb0 + 8 * (r >> 2) + 4 * hl + (r & 3);
          float b = has_pos ? rpx[kPadLo + max(0, min(qpos0 - j, P - 1))] : 0.f;
          if (has_time) b += rt[bucket_of(tq - tk64[buf][j - k0], T)];
          const bf16 bh = (bf16)b;
          x[r] = (float)bh + (float)(bf16)(b - (float)bh);
        }
        bf16x8 kq[NKK];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) kq[kk] = kfrag(Kt, kb, kk);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[kk], qf[kk], x, 0, 0, 0);
        if (bc.mask()) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int keyoff = 8 * (r >> 2) + 4 * hl + (r & 3);
            x[r] = kb0 + keyoff < kend ? x[r] : 0.f;
          }
        }
        return x;
      }
      f32x16 x = s_chain(kb, (bc.pos_c() ? pb : 0.f) + (bc.tmode() < 2 ? bc.tlo : 0.f), nullptr, false);
      // i - j = dbase - (8*(r/4) + r%4) for accumulator slot r
      const int dbase = qpos - kb0 - 4 * hl;
      if (!bc.pos_c()) {
        // Over the wavefront's rows (dead rows included) and the block's keys, i - j lies
        // in [wrow0 - kb0 - 31, wrow0 - kb0 + 31]. The block is active (kb0 <= wlast <=
        // wrow0 + 31) and its bucket varies (wrow0 - kb0 - 31 < P - 1), so that range is
        // inside [-62, P + 60], which the padded table covers. Slot r reads i - j =
        // dbase - off(r), off(r) = 8 (r / 4) + r % 4 <= 27: one base, constant offsets.
        const float* rq = rpx + (kPadLo - 27) + dbase;
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] += rq[27 - (8 * (r >> 2) + (r & 3))];
      }
      const uint32_t* tkl = tk_lo[buf] + 32 * kb + 4 * hl;
      if (bc.tmode() == 1) {
        two_bucket(x, kb, bc);  // two adjacent buckets
      } else if (bc.tmode() == 2) {
        if (bc.tfast()) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const u32x4 tk4 = *reinterpret_cast<const u32x4*>(tkl + 8 * g4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              x[4 * g4 + e] += rtc[time_clz_fast(tq1, tk4[e])];
          }
        } else {
          const int64_t* tk = tk64[buf] + 32 * kb + 4 * hl;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int bt = time_bucket64(tq, tk[8 * (r >> 2) + (r & 3)]);
            x[r] += rt[bt < 63 ? bt : 63];
          }
        }
      }
      if (bc.mask()) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int keyoff = 8 * (r >> 2) + 4 * hl + (r & 3);
          const bool vis = CAND ? (kb0 + keyoff < kend) : (dbase - (8 * (r >> 2) + (r & 3)) >= 0);
          x[r] = vis ? x[r] : 0.f;
        }
      }
      return x;
    };
    auto general_path = [&]() {
#pragma unroll
      for (int j = 0; j < NIW - 1; ++j) dma(j);
      const f32x16 x0 = general_block(0, c0);
#pragma unroll
      for (int st = 0; st < NKK; ++st) act_step(x0, 0.f, pa0, st);
      x1 = general_block(1, c1);
    };

    if (wave_live) {
      if (fast || keyb_tile)
        fast_path(keyb_tile);
      else if (fast2)
        fast2_path();
      else
        general_path();
    } else {
#pragma unroll
      for (int j = 0; j < NIW - 1; ++j) dma(j);
      // no live rows: P = 0 for both blocks (V holds finite data)
#pragma unroll
      for (int i = 0; i < 8; ++i) pa0[0][i] = pa0[1][i] = (bf16)0.f;
      x1 = f32x16{};
    }
    // shared tail: block 0's P V carrying block 1's SiLU, then block 1's P V
    {
      bf16x8 pa1[2];
      constexpr int NPV = 2 * NC;  // P V steps per block, one per activation step
      static_assert(NPV == NKK, "one P V step per activation step");
      bf16x8 vb = vfrag(Vt, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < NPV; ++m) {
        const bf16x8 vnext = vfrag(Vt, m + 1 < NPV ? 0 : 1, (m + 1) % NPV);
        o[m % NC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa0[m / NC], vb, o[m % NC], 0, 0, 0);
        act_step(x1, cbb, pa1, m);
        vb = vnext;
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int m = 0; m < NPV; ++m) {
        const bf16x8 vnext = vfrag(Vt, 1, (m + 1) % NPV);
        o[m % NC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa1[m / NC], vb, o[m % NC], 0, 0, 0);
        vb = vnext;
      }
    }
    finish_tile(BN_{}, more);
    __syncthreads();
  };
  for (int kt = 0; kt < nkt; kt += 2) {
    tile_step(B0{}, kt);
    if (kt + 1 < nkt) tile_step(B1{}, kt + 1);
  }

  __syncthreads();
  if (!wave_live) return;

  const float oscale = a.inv_n / kPre;  // P carries c = -log2(e)
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rw = 8 * (r >> 2) + 4 * hl + (r & 3);  // row within the wavefront
    const int rowl = 32 * w + rw;
    if (rowl >= t.rows) continue;
    const int64_t orow = (CAND ? (int64_t)blockIdx.z * a.part_stride : 0) +
                         (t.q_local + rowl) * a.ld_o + (int64_t)h * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int col = c * 32 + l32;
      const float val = o[c][r] * oscale;
      if (a.out_f32)
        ((float*)a.out)[orow + col] = val;
      else
        ((bf16*)a.out)[orow + col] = (bf16)val;
    }
  }
}

hipError_t launch_attn_mfma(const AttnArgs& a, bool cand, hipStream_t s) {
  dim3 grid;
  if (!cand)
    grid = dim3((unsigned)a.n_items * (unsigned)a.H);
  else
    grid = dim3((unsigned)((a.max_user_rows + MBM - 1) / MBM) * (unsigned)a.H, (unsigned)a.n_users,
                (unsigned)(a.kv_splits > 1 ? a.kv_splits : 1));
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  const bool split = a.q_lo != nullptr;
  if (split && (cand || !a.k_lo)) return hipErrorInvalidValue;
#define HSTU_MFMA_CASE(DD)                                                                  \
  if (a.d_qk == DD) {                                                                       \
    if (cand)                                                                               \
      hipLaunchKernelGGL((attn_mfma_kernel<DD, true, false>), grid, dim3(256), 0, s, a);    \
    else if (split)                                                                         \
      hipLaunchKernelGGL((attn_mfma_kernel<DD, false, true>), grid, dim3(256), 0, s, a);    \
    else                                                                                    \
      hipLaunchKernelGGL((attn_mfma_kernel<DD, false, false>), grid, dim3(256), 0, s, a);   \
    return hipGetLastError();                                                               \
  }
  HSTU_MFMA_CASE(32) HSTU_MFMA_CASE(64) HSTU_MFMA_CASE(128)
#undef HSTU_MFMA_CASE
  return hipErrorInvalidValue;
}

}  // namespace hstu
