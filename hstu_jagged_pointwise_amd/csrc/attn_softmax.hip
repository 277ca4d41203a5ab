// Causal softmax attention over jagged sequences on gfx950 matrix cores (bf16 in,
// fp32 accumulate). This is the ablation the HSTU chapter describes ("No
// sequence-wise softmax"): the pointwise SiLU(z)/N is replaced by a softmax of each
// query row over its visible keys. Scores are the HSTU scores,
// z_ij = q_i.k_j + rab(i, j), with the same buckets and no extra scale:
//   O_i = sum_{j <= i} exp(z_ij) v_j / sum_{j <= i} exp(z_ij).
// It serves as the in-house softmax baseline against which the pointwise kernel is
// timed.
//
// A workgroup owns 128 query rows of one head (32 per wavefront). 64-key tiles of K
// and V stream through double-buffered LDS. Per 32-key block:
//   S^T = K Q^T (Q in registers): lanes l and l + 32 share query l % 32 and hold 16
//   keys each, so a row maximum is 16 local operations and one exchange with lane ^ 32.
//   Online softmax in base 2: the running maximum m, the running sum and the output
//   are rescaled by 2^(m_old - m_new) when m moves; p = 2^(z log2 e - m).
//   O^T += V^T P^T: P^T is the B operand straight from registers and V^T the A operand,
//   read transposed from LDS. The output accumulator then also holds one query per lane,
//   so the rescale is a per-lane scalar.
// Bias per block as in the other attention kernels: one scalar where the position
// and time buckets are constant over the block, a select between two scalars for two
// adjacent time buckets, and per-element buckets and mask otherwise.
#include "attn_common.h"
#include "mfma_tiles.h"

namespace hstu {

namespace {
using namespace mt;
constexpr int SR = kMfmaRows;  // query rows per workgroup
}  // namespace

bool attn_softmax_supported(int dtype_bf16, int d_qk, int d_v, int P) {
  return dtype_bf16 && d_qk == d_v && (d_qk == 32 || d_qk == 64 || d_qk == 128) && P <= kMaxPosB;
}

template <int D>
__global__ __launch_bounds__(256, D <= 64 ? 2 : 1) void attn_softmax_kernel(AttnArgs a) {
  constexpr int NKK = D / 16, NC = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][TR * (D + 8)];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][TR * (D + 8)];
  __shared__ int64_t tks[2][TR];
  __shared__ uint32_t tks32[2][TR];
  __shared__ KeyRange krs[2][2];
  __shared__ float rps[kMaxPosB];
  __shared__ float rts[kTimeB];

  const int item = blockIdx.x / a.H, h = blockIdx.x % a.H;
  if (item >= a.n_items) return;
  const uint64_t raw = sload(reinterpret_cast<const uint64_t*>(a.items + item));
  const int seq = (int)(uint32_t)raw, tile = (int)(uint32_t)(raw >> 32);
  if (seq < 0 || seq >= a.batch || tile < 0) return;
  const int64_t base = sload(a.q_offsets + seq);
  const int64_t n = sload(a.q_offsets + seq + 1) - base;
  const int64_t r0 = (int64_t)tile * SR;
  if (r0 >= n) return;  // uniform across the workgroup

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hl = lane >> 5;
  const bf16* q = (const bf16*)a.q;
  const bf16* k = (const bf16*)a.k;
  const bf16* v = (const bf16*)a.v;
  const int64_t* ts = a.ts_q;
  const bool has_ts = ts != nullptr;
  const int TT = a.T < kTimeB ? a.T : kTimeB;
  for (int i = tid; i < a.P; i += 256) rps[i] = a.rab_pos ? a.rab_pos[(int64_t)h * a.P + i] : 0.f;
  for (int i = tid; i < TT; i += 256)
    rts[i] = (a.rab_time && has_ts) ? a.rab_time[(int64_t)h * a.T + i] : 0.f;

  const int64_t q0w = r0 + 32 * w;
  const bool wave_live = q0w < n;
  const int64_t i = q0w + l32;  // this lane's query
  const bool row_ok = i < n;
  bf16x8 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    qf[kk] = row_ok ? ld8(q + (base + i) * a.ld_q + (int64_t)h * D + 16 * kk + 8 * hl) : bf16x8{};
  const int64_t tq = (has_ts && row_ok) ? ts[base + i] : 0;
  KeyRange qr{0, 0};
  if (has_ts && wave_live) {
    const KeyRange* p = a.key_ranges + key_range_slot(base, seq) + q0w / 32;
    qr.lo = sload(&p->lo);
    qr.hi = sload(&p->hi);
  }
  f32x16 o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) o[c] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;  // base-2 running maximum; this lane's half of the sum

  const int64_t kend = r0 + SR < n ? r0 + SR : n;
  const int nkt = (int)((kend + TR - 1) / TR);
  TileStage<D> st;
  auto load_tile = [&](int kt) {
    const int64_t k0 = (int64_t)kt * TR;
    const int rows = (int)(kend - k0 < TR ? kend - k0 : TR);
    st.load(k, a.ld_k, v, a.ld_v, base + k0, rows, h * D);
  };
  auto fetch_ts = [&](int kt) {
    const int64_t k0 = (int64_t)kt * TR;
    SideTs f{0, {0, 0}};
    if (has_ts && tid < TR && k0 + tid < kend) f.tv = ts[base + k0 + tid];
    if (has_ts && tid < 2 && k0 + 32 * tid < kend)
      f.r = a.key_ranges[key_range_slot(base, seq) + k0 / 32 + tid];
    return f;
  };
  auto store_ts = [&](const SideTs& f, int buf) {
    if (tid < TR) {
      tks[buf][tid] = f.tv;
      tks32[buf][tid] = (uint32_t)f.tv;
    }
    if (tid < 2) krs[buf][tid] = f.r;
  };
  load_tile(0);
  st.store(Ks[0], Vs[0]);
  store_ts(fetch_ts(0), 0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nkt;
    SideTs nf{0, {0, 0}};
    if (more) {
      load_tile(kt + 1);
      nf = fetch_ts(kt + 1);
    }
    const bf16* Kt = Ks[buf];
    const bf16* Vt = Vs[buf];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int64_t k0b = (int64_t)kt * TR + 32 * kb;
      if (!wave_live || k0b > q0w + 31 || k0b >= kend) continue;  // uniform
      f32x16 s = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        s = mfma(ld8(&Kt[toff<D>(32 * kb + l32, 16 * kk + 8 * hl)]), qf[kk], s);
      const bool full = q0w >= k0b + 31 && q0w + 31 < n;
      const bool posc = q0w - (k0b + 31) >= a.P - 1;
      int blo = 0, bhi = 0;
      bool fits32 = true;
      if (has_ts) {
        const KeyRange kr = krs[buf][kb];
        blo = tbucket(qr.lo - kr.hi, a.T);
        bhi = tbucket(qr.hi - kr.lo, a.T);
        fits32 = time_fast_ok(qr.lo, qr.hi, kr.lo, kr.hi);
      }
      // base-2 scores x = z log2(e); hidden pairs -inf (finite 0 on rows past the end,
      // whose output is never written, so that no row's maximum stays -inf)
      f32x16 x;
      if (full && posc && blo == bhi) {
        const float b2 = (rps[a.P - 1] + rts[blo]) * kLog2e;
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = fmaf(s[r], kLog2e, b2);
      } else if (full && posc && bhi == blo + 1 && fits32) {
        const float b_lo = (rps[a.P - 1] + rts[blo]) * kLog2e;
        const float b_hi = (rps[a.P - 1] + rts[bhi]) * kLog2e;
        const int thr = 1 << bhi;
        const uint32_t tq1 = (uint32_t)tq + 1u;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int d = (int)(tq1 - tks32[buf][32 * kb + acc_row(r, hl)]);
          x[r] = fmaf(s[r], kLog2e, d >= thr ? b_hi : b_lo);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jr = 32 * kb + acc_row(r, hl);
          const int64_t j = (int64_t)kt * TR + jr;
          float z = s[r] + rps[pos_bucket((int)(i - j), a.P)];
          if (has_ts) z += rts[tbucket(tq - tks[buf][jr], a.T)];
          x[r] = !row_ok ? 0.f : (j <= i && j < kend) ? z * kLog2e : -INFINITY;
        }
      }
      float bm = x[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) bm = fmaxf(bm, x[r]);
      bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
      const float m_new = fmaxf(m_run, bm);
      if (__ballot(m_new != m_run)) {  // some row's maximum moved: rescale
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[c][r] *= alpha;
        m_run = m_new;
      }
      bf16x8 pp[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(x[r] - m_run);
        l_run += p;
        pp[r >> 3][r & 7] = (bf16)p;
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int c = 0; c < NC; ++c) o[c] = mfma(trfrag<D>(Vt, 32 * kb + 16 * s2, c, lane), pp[s2], o[c]);
    }
    if (more) {
      st.store(Ks[buf ^ 1], Vs[buf ^ 1]);
      store_ts(nf, buf ^ 1);
    }
    __syncthreads();
  }
  if (!wave_live) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!row_ok) return;
  const float inv = 1.0f / l_tot;
  bf16* out = (bf16*)a.out;
  bf16* orow = out + (base + i) * a.ld_o + (int64_t)h * D;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {  // 4 consecutive columns per slot group
      bf16x4 w4;
#pragma unroll
      for (int e = 0; e < 4; ++e) w4[e] = (bf16)(o[c][4 * r4 + e] * inv);
      *reinterpret_cast<bf16x4*>(&orow[32 * c + 8 * r4 + 4 * hl]) = w4;
    }
}

hipError_t launch_attn_softmax(const AttnArgs& a, hipStream_t s) {
  if (a.n_items <= 0 || a.H <= 0) return hipSuccess;
  if (a.ts_q && !a.key_ranges) return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.n_items * (unsigned)a.H);
  switch (a.d_qk) {
    case 32: hipLaunchKernelGGL(attn_softmax_kernel<32>, grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL(attn_softmax_kernel<64>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(attn_softmax_kernel<128>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hstu
