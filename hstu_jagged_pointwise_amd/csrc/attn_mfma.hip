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
// head. Each wavefront owns 32 rows. Keys stream through LDS in tiles of 64.
// Per 32-key block a wavefront runs:
//   S^T = K Q^T  with v_mfma_f32_32x32x16_bf16. Q stays in registers as the B
//                operand. The accumulator then holds one query row per lane
//                (lane % 32) and 16 keys per lane.
//   P = SiLU(S + bias), masked, on the vector ALU. The bias comes from
//                LDS-resident tables. The time bucket is a count of leading
//                zeros on the 32-bit elapsed time, with a 64-bit path for
//                tiles whose span is too wide.
//   O += P V     again with the 32x32x16 MFMA. P goes in as the A operand
//                straight from registers, with no LDS round trip: the key order
//                held in the accumulator defines the contraction order, and V
//                is read in that same order with ds_read_b64_tr_b16, which
//                transposes row-major V on the way out of LDS.
// Under the causal mask a wavefront skips key blocks that lie entirely above
// its rows, and applies the mask select only on blocks that cross the
// diagonal. The mask is a select after SiLU (SiLU(-inf) would be NaN).
// Candidate mode (M-FALCON): the queries are one user's candidates, all at
// position n_h. The keys are that user's history, all visible. Each
// candidate's own key and value are added in the epilogue.
#include "attn_common.h"

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
}  // namespace

bool attn_mfma_supported(int dtype_bf16, int d_qk, int d_v, int P, int T) {
  (void)T;
  return dtype_bf16 && d_qk == d_v && (d_qk == 32 || d_qk == 64 || d_qk == 128) && P <= kMaxP;
}

template <int D, bool CAND>
__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(AttnArgs a) {
  constexpr int LDK = D + 8;  // padded LDS row, in elements (keeps 16-byte alignment)
  constexpr int NKK = D / 16; // k-steps of the S^T contraction
  constexpr int NC = D / 32;  // 32-wide output column blocks
  __shared__ __attribute__((aligned(16))) bf16 Ks[MBN * LDK];
  __shared__ __attribute__((aligned(16))) bf16 Vs[MBN * LDK];
  __shared__ uint32_t tk_lo[MBN];
  __shared__ int64_t tk64[MBN];
  __shared__ float rp[kMaxP];
  __shared__ float rt[kTimeTab];
  __shared__ float rtc[32];
  __shared__ int64_t kstat[2];
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
  const int64_t qmin = wave_min64(row_ok ? tq : INT64_MAX);
  const int64_t qmax = wave_max64(row_ok ? tq : INT64_MIN);
  const int64_t qpos = CAND ? t.qpos0 : t.qpos0 + wrow;
  const int64_t wrow0 = t.qpos0 + 32 * w;  // causal position of the wavefront's first row

  f32x16 o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[c][r] = 0.f;

  const int64_t nkt = (t.kend + MBN - 1) / MBN;
  for (int64_t kt = 0; kt < nkt; ++kt) {
    const int64_t k0 = kt * MBN;
    __syncthreads();
    // stage K and V (64 keys x D) into LDS, zero past the data so that hidden
    // lanes multiply finite values
#pragma unroll
    for (int c = tid; c < MBN * D / 8; c += 256) {
      const int key = c / (D / 8), col = (c % (D / 8)) * 8;
      const bool ok = k0 + key < t.nk;
      bf16x8 kv, vv;
      if (ok) {
        const int64_t grow = t.k_base + k0 + key;
        kv = load_bf16x8(k + grow * a.ld_k + (int64_t)h * D + col);
        vv = load_bf16x8(v + grow * a.ld_v + (int64_t)h * D + col);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) { kv[i] = (bf16)0.f; vv[i] = (bf16)0.f; }
      }
      *reinterpret_cast<bf16x8*>(&Ks[key * LDK + col]) = kv;
      *reinterpret_cast<bf16x8*>(&Vs[key * LDK + col]) = vv;
    }
    if (has_time && tid < MBN) {
      const bool ok = k0 + tid < t.nk;
      const int64_t tk = ok ? a.ts_k[t.k_base + k0 + tid] : 0;
      tk_lo[tid] = (uint32_t)tk;
      tk64[tid] = tk;
      const int64_t mn = wave_min64(ok ? tk : INT64_MAX);
      const int64_t mx = wave_max64(ok ? tk : INT64_MIN);
      if (tid == 0) { kstat[0] = mn; kstat[1] = mx; }
    }
    __syncthreads();
    if (!wave_live) continue;
    const bool fast = !has_time || time_fast_ok(qmin, qmax, kstat[0], kstat[1]);

#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int64_t kb0 = k0 + 32 * kb;
      if (kb0 >= t.kend) continue;
      if (!CAND && kb0 > wrow0 + 31) continue;  // every key above every row of this wavefront
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 kf = load_bf16x8(&Ks[(32 * kb + l32) * LDK + 16 * kk + 8 * hl]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s, 0, 0, 0);
      }
      // s[r] = S[query wrow][key 32kb + 8(r/4) + 4hl + r%4]
      const bool need_mask = CAND ? (kb0 + 32 > t.nk) : (kb0 + 31 > wrow0);
      bf16x8 pa[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int keyl = 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
        const int64_t j = k0 + keyl;
        const int dpos = (int)(qpos - j);
        float x = s[r];
        if (has_pos) x += rp[pos_bucket(dpos, P)];
        if (has_time) {
          if (fast) {
            x += rtc[time_clz_fast(tq1, tk_lo[keyl])];
          } else {
            const int bt = time_bucket64(tq, tk64[keyl]);
            x += rt[bt < 63 ? bt : 63];
          }
        }
        float p = silu_fast(x);
        if (need_mask) {
          const bool vis = CAND ? (j < t.nk) : (dpos >= 0);
          p = vis ? p : 0.f;
        }
        pa[r >> 3][r & 7] = (bf16)p;
      }
      // O += P V; the k-slot (hl, i) of step s2 is key 16*s2 + 8*(i/4) + 4*hl + i%4
      const int g = lane >> 4, rho = lane & 15;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int kbase = 32 * kb + 16 * s2 + 4 * hl + (rho >> 2);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int col = c * 32 + 16 * (g & 1) + 4 * (rho & 3);
          const bf16x4 v1 = tr_read(&Vs[kbase * LDK + col]);
          const bf16x4 v2 = tr_read(&Vs[(kbase + 8) * LDK + col]);
          bf16x8 bv;
#pragma unroll
          for (int i = 0; i < 4; ++i) { bv[i] = v1[i]; bv[4 + i] = v2[i]; }
          o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[s2], bv, o[c], 0, 0, 0);
        }
      }
    }
  }

  if (CAND) {
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
    const int64_t orow = (t.q_local + rowl) * a.ld_o + (int64_t)h * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int col = c * 32 + l32;
      float val = o[c][r];
      if (CAND)
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
    grid = dim3((unsigned)((a.max_user_rows + MBM - 1) / MBM) * (unsigned)a.H, (unsigned)a.n_users);
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
