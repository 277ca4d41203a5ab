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
// ranges:
//   * The position bucket min(i-j, P-1) is one constant when every i-j >= P-1.
//   * The time bucket is one constant when its value agrees at both ends of the
//     block's elapsed-time range [min t_i - max t_j, max t_i - min t_j]. The
//     bucket is monotone in the elapsed time, so agreement at both ends means
//     it holds everywhere.
//   * A constant bias becomes the accumulator's initial value, at no cost per
//     element. Otherwise each element gathers from LDS-resident tables. The
//     time bucket is then the count of leading zeros of the 32-bit elapsed time
//     + 1 (a 64-bit path covers spans past 2^31 s).
// Masking is a select after SiLU (SiLU(-inf) would be NaN). It runs only on
// blocks that cross the causal diagonal (or the history tail for candidates).
// Blocks entirely above the diagonal are skipped.
//
// Candidate mode (M-FALCON): the queries are one user's candidates, all at
// position n_h. The keys are that user's history, all visible. Each
// candidate's own key and value are added in the epilogue.
#include "attn_common.h"

#include <type_traits>

namespace hstu {

namespace {
constexpr int MBM = kMfmaRows;  // 128 query rows per workgroup
constexpr int MBN = 64;         // keys per LDS tile
constexpr int kMaxP = 1024;     // position-table entries kept in LDS
constexpr int kTimeTab = 64;    // time-table entries ever reachable (buckets <= 63)

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
  return MBN * (D + 8) + 64 * 8;  // + slack for the last DMA span
}

// exact time bucket of a non-negative elapsed time, clamped to the table
__device__ __forceinline__ int bucket_of(int64_t dt, int T) {
  dt = dt < 0 ? 0 : dt;
  const int b = 63 - __builtin_clzll((uint64_t)dt + 1ull);
  return b < T - 1 ? b : T - 1;
}
}  // namespace

bool attn_mfma_supported(int dtype_bf16, int d_qk, int d_v, int P, int T) {
  (void)T;
  return dtype_bf16 && d_qk == d_v && (d_qk == 32 || d_qk == 64 || d_qk == 128) && P <= kMaxP;
}

bool attn_mfma_strides_ok(const AttnArgs& a) {
  // the key-tile DMA shares one per-lane offset between K and V; offsets are 32-bit
  return a.ld_k == a.ld_v && a.ld_k > 0 && (int64_t)(MBN + 1) * a.ld_k < (int64_t(1) << 31);
}

template <int D, bool CAND>
__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(AttnArgs a) {
  constexpr int NKK = D / 16;       // k-steps of the S^T contraction
  constexpr int NC = D / 32;        // 32-wide output column blocks
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int TE = tile_elems<D>();
  // two LDS buffers per matrix as separate objects, so that alias analysis can tell
  // the in-flight DMA target from the buffer being read (no conservative waits)
  __shared__ __attribute__((aligned(16))) bf16 Ks0[TE];
  __shared__ __attribute__((aligned(16))) bf16 Ks1[TE];
  __shared__ __attribute__((aligned(16))) bf16 Vs0[TE];
  __shared__ __attribute__((aligned(16))) bf16 Vs1[TE];
  __shared__ __attribute__((aligned(16))) uint32_t tk_lo[2][MBN];
  __shared__ int64_t tk64[2][MBN];
  __shared__ int64_t kstat[2][2][2];  // [buffer][32-key block][min, max]
  __shared__ float rp[kMaxP];
  __shared__ float rt[kTimeTab];
  __shared__ float rtc[32];
  __shared__ float pself[4][32];

  const TileDecode t = decode<CAND>(a, MBM);
  if (!t.valid) return;  // uniform across the workgroup
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int h = t.h;
  const bf16* q = (const bf16*)a.q;
  const bf16* k = (const bf16*)a.k;
  const bf16* v = (const bf16*)a.v;
  const bool has_pos = a.rab_pos != nullptr;
  const bool has_time = a.rab_time != nullptr && a.ts_q != nullptr && a.ts_k != nullptr;
  const int P = a.P, T = a.T;

  if (has_pos)
    for (int i = tid; i < P; i += 256) rp[i] = a.rab_pos[(int64_t)h * P + i];
  if (has_time) {
    if (tid < kTimeTab) rt[tid] = a.rab_time[(int64_t)h * T + (tid < T - 1 ? tid : T - 1)];
    if (tid < 32) {
      const int bt = 31 - tid;
      rtc[tid] = a.rab_time[(int64_t)h * T + (bt < T - 1 ? bt : T - 1)];
    }
  }

  // this lane's query row (the S^T column it holds) and its Q fragment
  const int wrow = 32 * w + l32;
  const bool row_ok = wrow < t.rows;
  const bool wave_live = 32 * w < t.rows;
  bf16x8 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    if (row_ok) {
      qf[kk] = load_bf16x8(q + (t.q_local + wrow) * a.ld_q + (int64_t)h * D + 16 * kk + 8 * hl);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[kk][i] = (bf16)0.f;
    }
  }
  const int64_t tq = (has_time && row_ok) ? a.ts_q[t.q_base + wrow] : 0;
  const uint32_t tq1 = (uint32_t)tq + 1u;
  const int64_t qmin = uniform64(wave_min64(row_ok ? tq : INT64_MAX));
  const int64_t qmax = uniform64(wave_max64(row_ok ? tq : INT64_MIN));
  const int64_t qpos = CAND ? t.qpos0 : t.qpos0 + wrow;
  const int64_t wrow0 = t.qpos0 + 32 * w;  // causal position of the wavefront's first row
  const int64_t wlast = t.qpos0 + (int64_t)min(32 * w + 31, t.rows - 1);  // its last live row

  // constant A fragment for the bias k-step: A[key][0] = A[key][1] = 1
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (bf16)((hl == 0 && i < 2) ? 1.f : 0.f);

  f32x16 o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[c][r] = 0.f;

  // ---- key tiles go global -> LDS directly (global_load_lds_dwordx4): lane L of one
  // instruction fills 16-byte slot L of a contiguous 1 KiB span, so the padded
  // layout comes from which source chunk each lane fetches. Rows past the data
  // repeat the last valid row: their scores are masked and multiply finite values.
  constexpr int SPR = CPR + 1;                         // 16-byte slots per LDS row
  constexpr int NSLOT = MBN * SPR;                     // slots per matrix tile
  constexpr int NINSTR = (NSLOT + 63) / 64;            // wave-instructions per matrix tile
  int64_t ptk = 0;
  // Per-lane source offsets (elements from the tile's first row) of this wavefront's
  // DMA instructions, computed once. K and V share the row stride. A full tile
  // then needs only the uniform base pointer advanced; the tail tile clamps rows
  // past the data to the last valid row.
  constexpr int NIW = (NINSTR + 3) / 4;
  uint32_t soff[NIW];
#pragma unroll
  for (int j = 0; j < NIW; ++j) {
    const int slot = 64 * (w + 4 * j) + lane;
    const int row = slot / SPR, pc = slot % SPR;
    soff[j] = (uint32_t)(row * a.ld_k + 8 * (pc < CPR ? pc : 0));
  }
  auto issue_tile = [&](auto bufc, int64_t k0) {
    constexpr int buf = decltype(bufc)::value;
    bf16* Kd = buf ? Ks1 : Ks0;
    bf16* Vd = buf ? Vs1 : Vs0;
    const int64_t last = t.nk - 1;
    const bf16* kb = k + (t.k_base + k0) * a.ld_k + (int64_t)h * D;
    const bf16* vb = v + (t.k_base + k0) * a.ld_v + (int64_t)h * D;
    const bool full = k0 + MBN - 1 <= last;
#pragma unroll
    for (int j = 0; j < NIW; ++j) {
      const int i = w + 4 * j;
      if (i >= NINSTR) break;
      const int slot = 64 * i + lane;
      if (slot < NSLOT) {
        uint32_t off = soff[j];
        if (!full) {
          const int row = slot / SPR, pc = slot % SPR;
          const int64_t r = min(k0 + row, last) - k0;
          off = (uint32_t)(r * a.ld_k + 8 * (pc < CPR ? pc : 0));
        }
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(kb + off),
                                         (__attribute__((address_space(3))) void*)(&Kd[512 * i]),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(vb + off),
                                         (__attribute__((address_space(3))) void*)(&Vd[512 * i]),
                                         16, 0, 0);
      }
    }
    if (has_time && tid < MBN) ptk = (k0 + tid < t.nk) ? a.ts_k[t.k_base + k0 + tid] : 0;
  };
  auto finish_tile = [&](auto bufc, int64_t k0) {
    constexpr int buf = decltype(bufc)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (has_time && tid < MBN) {
      const bool ok = k0 + tid < t.nk;
      tk_lo[buf][tid] = (uint32_t)ptk;
      tk64[buf][tid] = ptk;
      // min and max over each half-wavefront (one 32-key block each)
      int64_t mn = ok ? ptk : INT64_MAX, mx = ok ? ptk : INT64_MIN;
#pragma unroll
      for (int o2 = 16; o2 >= 1; o2 >>= 1) {
        const int64_t a1 = __shfl_xor(mn, o2, 64), a2 = __shfl_xor(mx, o2, 64);
        mn = a1 < mn ? a1 : mn;
        mx = a2 > mx ? a2 : mx;
      }
      if ((tid & 31) == 0) {
        kstat[buf][tid >> 5][0] = mn;
        kstat[buf][tid >> 5][1] = mx;
      }
    }
  };

  const int64_t nkt = (t.kend - t.kbeg + MBN - 1) / MBN;
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  if (nkt > 0) {
    issue_tile(B0{}, t.kbeg);
    finish_tile(B0{}, t.kbeg);
  }
  __syncthreads();

  // per-lane key offset inside a 32-key block for accumulator slot r
  // keyoff(r) = 8*(r/4) + 4*hl + (r%4)
  auto tile_step = [&](auto bufc, int64_t kt) {
    constexpr int buf = decltype(bufc)::value;
    using BN_ = std::integral_constant<int, 1 - buf>;
    const int64_t k0 = t.kbeg + kt * MBN;
    if (kt + 1 < nkt) issue_tile(BN_{}, k0 + MBN);

    if (wave_live) {
      const bf16* Kt = buf ? Ks1 : Ks0;
      const bf16* Vt = buf ? Vs1 : Vs0;
      // ---- classify both 32-key blocks (wave-uniform scalars)
      bool act[2], need_mask[2], uni[2], pos_c[2], time_c[2], time_fast[2], time_sorted[2];
      float ubias[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int64_t kb0 = k0 + 32 * kb;
        act[kb] = kb0 < t.kend && (CAND || kb0 <= wlast);
        need_mask[kb] = CAND ? (kb0 + 32 > t.kend) : (kb0 + 31 > wrow0);
        const int64_t min_dpos = (CAND ? t.qpos0 : wrow0) - (kb0 + 31);
        pos_c[kb] = !has_pos || min_dpos >= P - 1;
        float b = has_pos && pos_c[kb] ? rp[P - 1] : 0.f;
        time_c[kb] = true;
        time_fast[kb] = true;
        time_sorted[kb] = true;
        if (has_time && act[kb]) {
          const int64_t kmin = uniform64(kstat[buf][kb][0]);
          const int64_t kmax = uniform64(kstat[buf][kb][1]);
          const int64_t lo = qmin - kmax, hi = qmax - kmin;  // elapsed-time range
          const int blo = bucket_of(lo, T), bhi = bucket_of(hi, T);
          time_c[kb] = blo == bhi;
          if (time_c[kb]) b += rt[blo < 63 ? blo : 63];
          time_fast[kb] = time_fast_ok(qmin, qmax, kmin, kmax);
          time_sorted[kb] = lo >= 0;
        }
        uni[kb] = pos_c[kb] && time_c[kb];
        ubias[kb] = b;
      }

      // ---- S^T. A uniform bias enters as one extra MFMA k-step: a constant all-ones
      // A fragment (keys x {0,1}) times a B fragment holding bias_hi, bias_lo
      // (bf16 split, exact to ~2^-16 relative) for every row. The accumulator then
      // starts from the inline zero, and no vector instruction touches the bias.
      auto qk = [&](int kb, bool with_bias, float bias) {
        f32x16 acc;
        const bf16x8 kf0 = load_bf16x8(&Kt[tile_off<D>(32 * kb + l32, 8 * hl)]);
        if (with_bias) {
          bf16x8 bfrag;
#pragma unroll
          for (int i = 0; i < 8; ++i) bfrag[i] = (bf16)0.f;
          const bf16 bhi = (bf16)bias;
          if (hl == 0) {
            bfrag[0] = bhi;
            bfrag[1] = (bf16)(bias - (float)bhi);
          }
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, bfrag, f32x16{}, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf0, qf[0], acc, 0, 0, 0);
        } else {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf0, qf[0], f32x16{}, 0, 0, 0);
        }
#pragma unroll
        for (int kk = 1; kk < NKK; ++kk) {
          const bf16x8 kf = load_bf16x8(&Kt[tile_off<D>(32 * kb + l32, 16 * kk + 8 * hl)]);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], acc, 0, 0, 0);
        }
        return acc;
      };
      // SiLU to bf16 A fragments, with the mask applied when asked
      auto activate = [&](const f32x16& x, int kb, bool mask, bf16x8* pa) {
        const int64_t kb0 = k0 + 32 * kb;
        const int dbase = (int)(qpos - kb0) - 4 * hl;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = silu_fast(x[r]);
          if (mask) {
            const int keyoff = 8 * (r >> 2) + 4 * hl + (r & 3);
            const bool vis = CAND ? (kb0 + keyoff < t.kend) : (dbase - (8 * (r >> 2) + (r & 3)) >= 0);
            p = vis ? p : 0.f;
          }
          pa[r >> 3][r & 7] = (bf16)p;
        }
      };
      // O += P V; the k-slot (hl, i) of step s2 is key 16*s2 + 8*(i/4) + 4*hl + i%4
      auto pv = [&](int kb, const bf16x8* pa) {
        const int g = lane >> 4, rho = lane & 15;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int krow = 32 * kb + 16 * s2 + 4 * hl + (rho >> 2);
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const int col = c * 32 + 16 * (g & 1) + 4 * (rho & 3);
            const bf16x4 v1 = tr_read(&Vt[tile_off<D>(krow, col)]);
            const bf16x4 v2 = tr_read(&Vt[tile_off<D>(krow + 8, col)]);
            bf16x8 bv;
#pragma unroll
            for (int i = 0; i < 4; ++i) { bv[i] = v1[i]; bv[4 + i] = v2[i]; }
            o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[s2], bv, o[c], 0, 0, 0);
          }
        }
      };

      const bool fast = act[0] && act[1] && uni[0] && uni[1] && !need_mask[0] && !need_mask[1];
      if (fast) {
        // Common case: both blocks live, uniform bias, no mask. The instruction order
        // is written out and fenced (sched_barrier) so that the in-order wavefront
        // issues one MFMA (~40 cycles in the matrix core), then the independent
        // vector work that fits under it:
        //   block 0: S^T chain;
        //   block 1: S^T chain, each step carrying the SiLU of ~2 of block 0's scores;
        //   block 0: P V, each step carrying the SiLU of 2 of block 1's scores;
        //   block 1: P V.
        constexpr int NS = NKK + 1;  // S steps per block (bias step + NKK)
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
        auto kfrag = [&](int kb, int kk) {
          return load_bf16x8(&Kt[tile_off<D>(32 * kb + l32, 16 * kk + 8 * hl)]);
        };
        const int g = lane >> 4, rho = lane & 15;
        auto vfrag = [&](int kb, int m) {  // m = s2 * NC + c
          const int s2 = m / NC, c = m % NC;
          const int krow = 32 * kb + 16 * s2 + 4 * hl + (rho >> 2);
          const int col = c * 32 + 16 * (g & 1) + 4 * (rho & 3);
          const bf16x4 v1 = tr_read(&Vt[tile_off<D>(krow, col)]);
          const bf16x4 v2 = tr_read(&Vt[tile_off<D>(krow + 8, col)]);
          bf16x8 bv;
#pragma unroll
          for (int i = 0; i < 4; ++i) { bv[i] = v1[i]; bv[4 + i] = v2[i]; }
          return bv;
        };
        auto act_range = [&](const f32x16& x, bf16x8* pa, int r0, int r1) {
#pragma unroll
          for (int r = r0; r < r1; ++r) pa[r >> 3][r & 7] = (bf16)silu_fast(x[r]);
        };
        const bf16x8 bf0 = bias_frag(ubias[0]), bf1 = bias_frag(ubias[1]);
        // block 0: S^T
        bf16x8 kq[NKK];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) kq[kk] = kfrag(0, kk);
        f32x16 s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, bf0, f32x16{}, 0, 0, 0);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[kk], qf[kk], s0, 0, 0, 0);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) kq[kk] = kfrag(1, kk);
        __builtin_amdgcn_sched_barrier(0);
        // block 1: S^T, carrying block 0's SiLU
        bf16x8 pa0[2], pa1[2];
        f32x16 s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, bf1, f32x16{}, 0, 0, 0);
        act_range(s0, pa0, 0, 16 / NS);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[kk], qf[kk], s1, 0, 0, 0);
          act_range(s0, pa0, (kk + 1) * 16 / NS, (kk + 2) * 16 / NS);
          __builtin_amdgcn_sched_barrier(0);
        }
        // block 0: P V, carrying block 1's SiLU
        constexpr int NPV = 2 * NC;
        bf16x8 vb = vfrag(0, 0);
#pragma unroll
        for (int m = 0; m < NPV; ++m) {
          const bf16x8 vnext = vfrag(m + 1 < NPV ? 0 : 1, (m + 1) % NPV);
          o[m % NC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa0[m / NC], vb, o[m % NC], 0, 0, 0);
          act_range(s1, pa1, m * 16 / NPV, (m + 1) * 16 / NPV);
          vb = vnext;
          __builtin_amdgcn_sched_barrier(0);
        }
        // block 1: P V
#pragma unroll
        for (int m = 0; m < NPV; ++m) {
          const bf16x8 vnext = vfrag(1, (m + 1) % NPV);
          o[m % NC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa1[m / NC], vb, o[m % NC], 0, 0, 0);
          vb = vnext;
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (!act[kb]) continue;
          const int64_t kb0 = k0 + 32 * kb;
          f32x16 x = qk(kb, uni[kb] && ubias[kb] != 0.f, ubias[kb]);
          if (!uni[kb]) {
            // per-element bias for this block
            const int dbase = (int)(qpos - kb0) - 4 * hl;  // i - j = dbase - (8*(r/4) + r%4)
            if (!pos_c[kb]) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                int d = dbase - (8 * (r >> 2) + (r & 3));
                d = d < 0 ? 0 : (d < P - 1 ? d : P - 1);
                x[r] += rp[d];
              }
            }
            // the constant part of the bias (position or time, whichever is constant)
            if (pos_c[kb] != time_c[kb] && ubias[kb] != 0.f) {
#pragma unroll
              for (int r = 0; r < 16; ++r) x[r] += ubias[kb];
            }
            if (has_time && !time_c[kb]) {
              const uint32_t* tkl = tk_lo[buf] + 32 * kb + 4 * hl;
              if (time_fast[kb] && time_sorted[kb]) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                  const u32x4 tk4 = *reinterpret_cast<const u32x4*>(tkl + 8 * g);
#pragma unroll
                  for (int e = 0; e < 4; ++e)
                    x[4 * g + e] += rtc[__builtin_clz((tq1 - tk4[e]) | 1u)];
                }
              } else if (time_fast[kb]) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                  const u32x4 tk4 = *reinterpret_cast<const u32x4*>(tkl + 8 * g);
#pragma unroll
                  for (int e = 0; e < 4; ++e) x[4 * g + e] += rtc[time_clz_fast(tq1, tk4[e])];
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
          }
          bf16x8 pa[2];
          activate(x, kb, need_mask[kb], pa);
          pv(kb, pa);
        }
      }
    }
    if (kt + 1 < nkt) finish_tile(BN_{}, k0 + MBN);
    __syncthreads();
  };
  for (int64_t kt = 0; kt < nkt; kt += 2) {
    tile_step(B0{}, kt);
    if (kt + 1 < nkt) tile_step(B1{}, kt + 1);
  }

  const bool add_self = CAND && blockIdx.z == 0;
  if (add_self) {
    // the candidate's own key and value: relative position 0, elapsed time 0
    const bf16* kc = (const bf16*)a.kc;
    float part = 0.f;
    if (row_ok) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 kf =
            load_bf16x8(kc + (t.q_local + wrow) * a.ld_kc + (int64_t)h * D + 16 * kk + 8 * hl);
#pragma unroll
        for (int i = 0; i < 8; ++i) part = fmaf((float)qf[kk][i], (float)kf[i], part);
      }
    }
    part += __shfl_xor(part, 32, 64);
    float x = part;
    if (has_pos) x += rp[0];
    if (has_time) x += rt[0];
    if (hl == 0) pself[w][l32] = row_ok ? silu_fast(x) : 0.f;
  }
  __syncthreads();
  if (!wave_live) return;

  const bf16* vc = (const bf16*)a.vc;
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
      float val = o[c][r];
      if (add_self)
        val = fmaf(pself[w][rw], (float)vc[(t.q_local + rowl) * a.ld_vc + (int64_t)h * D + col], val);
      val *= a.inv_n;
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
#define HSTU_MFMA_CASE(DD)                                                                  \
  if (a.d_qk == DD) {                                                                       \
    if (cand)                                                                               \
      hipLaunchKernelGGL((attn_mfma_kernel<DD, true>), grid, dim3(256), 0, s, a);           \
    else                                                                                    \
      hipLaunchKernelGGL((attn_mfma_kernel<DD, false>), grid, dim3(256), 0, s, a);          \
    return hipGetLastError();                                                               \
  }
  HSTU_MFMA_CASE(32) HSTU_MFMA_CASE(64) HSTU_MFMA_CASE(128)
#undef HSTU_MFMA_CASE
  return hipErrorInvalidValue;
}

}  // namespace hstu
