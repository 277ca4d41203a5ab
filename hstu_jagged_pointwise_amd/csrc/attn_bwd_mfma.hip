// Backward pass of the HSTU pointwise attention on gfx950 matrix cores (bf16 in,
// fp32 accumulate), for d_qk == d_v in {32, 64, 128}.
//
// Gradients of eq. 2 ("What an HSTU layer changes", HSTU chapter), per head and
// visible pair j <= i, with z_ij = q_i.k_j + rab(i, j) and g_i = dL/do_i:
//   a_ij  = SiLU(z_ij) / N            dv_j = sum_i a_ij g_i
//   dz_ij = (g_i.v_j) SiLU'(z_ij) / N dq_i = sum_j dz_ij k_j,  dk_j = sum_i dz_ij q_i
// With no softmax every pair is independent, so no statistic of the forward pass
// is stored or needed; both kernels recompute z from Q and K.
//
// Query-side kernel: a workgroup owns 128 query rows of one head (32 per wavefront)
// and streams 64-key tiles of K and V through double-buffered LDS.
//   S^T = K Q^T and dP^T = V G^T (v_mfma_f32_32x32x16_bf16; Q and G stay in registers
//   as B operands): one query per lane, 16 keys per lane.
//   dZ = dP SiLU'(S + bias) / N on the vector ALU, packed to bf16.
//   dQ += dZ K: dZ is the A operand straight from registers, and K is read in the
//   accumulator's key order with ds_read_b64_tr_b16 (a transposing LDS read).
// Key-side kernel: the mirror image. A workgroup owns 128 keys (32 per wavefront),
// K and V stay in registers, and 64-query tiles of Q and G stream through LDS.
//   S = Q K^T and dP = G V^T: one key per lane, 16 queries per lane.
//   P = SiLU(S + bias) / N and dZ as above.
//   dV += P^T G and dK += dZ^T Q, with G and Q read transposed from LDS.
// The key-side kernel also sums dz per bias bucket into per-wavefront LDS bins,
// which are written as one partial row per work item and reduced in a fixed order.
// Most pairs of a block share a time bucket, so a per-element atomic would make the
// 64 lanes collide on one address. Blocks with one or two time buckets add their
// sums to per-lane running sums of the current bucket and the next, reduced across
// the wavefront only when the bucket moves on; other blocks reduce once per bucket
// of their range. The clamped position bucket is summed in a register. Only
// position buckets below the clamp, which differ across the lanes of an
// instruction, use LDS atomics.
//
// Bias per 32x32 block (wavefront-uniform): the position bucket min(i-j, P-1) is
// the constant P-1 when every i - j >= P - 1. The time bucket is monotone in the
// elapsed time, so it is one constant when the buckets of the block's smallest and
// largest elapsed times agree (from the per-32-row timestamp ranges). A block that
// is fully visible with both constant takes the bias as one scalar and adds the
// block's dz sum to two bins. One whose time range covers two adjacent buckets
// b, b+1 selects between two scalars per element (a pair is in b+1 exactly when
// dt + 1 >= 2^(b+1), a 32-bit compare when the block's elapsed times fit) and
// keeps two sums. Any other block computes buckets, mask and bins per element.
#include "attn_common.h"
#include "mfma_tiles.h"

namespace hstu {

namespace {
using namespace mt;
constexpr int WR = kMfmaRows;  // rows owned by a workgroup (4 wavefronts x 32)

// SiLU(z)/N and SiLU'(z)/N from one sigmoid (hardware exp2 and reciprocal).
__device__ __forceinline__ void silu2(float z, float inv_n, float& a, float& da) {
  const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
  a = z * sg * inv_n;
  da = sg * (1.0f + z * (1.0f - sg)) * inv_n;
}

struct WTile {
  int seq;
  int64_t base, n, r0;
  bool valid;
};

__device__ __forceinline__ WTile wdecode(const AttnBwdArgs& a, int item, bool key_side) {
  WTile t;
  t.valid = false;
  const uint64_t raw = sload(reinterpret_cast<const uint64_t*>(a.items + item));
  const int seq = (int)(uint32_t)raw, tile = (int)(uint32_t)(raw >> 32);
  if (seq < 0 || seq >= a.batch || tile < 0) return t;
  t.seq = seq;
  t.base = sload(a.offsets + seq);
  t.n = sload(a.offsets + seq + 1) - t.base;
  const int64_t ntiles = (t.n + WR - 1) / WR;
  if (tile >= ntiles) return t;
  t.r0 = (key_side ? ntiles - 1 - tile : tile) * WR;
  t.valid = true;
  return t;
}

// Timestamp range of the 32-row block starting at row `row` (a multiple of 32) of a sequence.
__device__ __forceinline__ KeyRange block_range(const AttnBwdArgs& a, const WTile& t, int64_t row) {
  const KeyRange* p = a.key_ranges + key_range_slot(t.base, t.seq) + row / 32;
  KeyRange r;
  r.lo = sload(&p->lo);
  r.hi = sload(&p->hi);
  return r;
}

}  // namespace

bool attn_bwd_mfma_supported(int dtype_bf16, int d_qk, int d_v, int P) {
  return dtype_bf16 && d_qk == d_v && (d_qk == 32 || d_qk == 64 || d_qk == 128) && P <= kMaxPosB;
}

// ------------------------------------------------------------------ query side
template <int D>
__global__ __launch_bounds__(256, 2) void attn_bwd_q_mfma(AttnBwdArgs a) {
  constexpr int NKK = D / 16, NC = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][TR * (D + 8)];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][TR * (D + 8)];
  __shared__ int64_t tks[2][TR];
  __shared__ uint32_t tks32[2][TR];  // low words, for the two-bucket test
  __shared__ KeyRange krs[2][2];     // timestamp ranges of the tile's two key blocks
  __shared__ float rps[kMaxPosB];
  __shared__ float rts[kTimeB];

  const int item = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const WTile t = wdecode(a, item, false);
  if (!t.valid) return;  // uniform across the workgroup
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hl = lane >> 5;
  const bf16* q = (const bf16*)a.q;
  const bf16* k = (const bf16*)a.k;
  const bf16* v = (const bf16*)a.v;
  const bf16* g = (const bf16*)a.dout;
  const bool has_ts = a.ts != nullptr;
  const int TT = a.T < kTimeB ? a.T : kTimeB;
  for (int i = tid; i < a.P; i += 256) rps[i] = a.rab_pos ? a.rab_pos[(int64_t)h * a.P + i] : 0.f;
  for (int i = tid; i < TT; i += 256)
    rts[i] = (a.rab_time && has_ts) ? a.rab_time[(int64_t)h * a.T + i] : 0.f;

  const int64_t q0w = t.r0 + 32 * w;  // this wavefront's first query
  const bool wave_live = q0w < t.n;
  const int64_t i = q0w + l32;        // this lane's query
  const bool row_ok = i < t.n;
  bf16x8 qf[NKK], gf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int64_t off = (t.base + i) * a.ld_q + (int64_t)h * D + 16 * kk + 8 * hl;
    const int64_t offg = (t.base + i) * a.ld_do + (int64_t)h * D + 16 * kk + 8 * hl;
    qf[kk] = row_ok ? ld8(q + off) : bf16x8{};
    gf[kk] = row_ok ? ld8(g + offg) : bf16x8{};
  }
  const int64_t tq = (has_ts && row_ok) ? a.ts[t.base + i] : 0;
  KeyRange qr{0, 0};
  if (has_ts && wave_live) qr = block_range(a, t, q0w);
  f32x16 dq[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) dq[c] = f32x16{};

  const int64_t kend = t.r0 + WR < t.n ? t.r0 + WR : t.n;  // keys any query of the tile sees
  const int nkt = (int)((kend + TR - 1) / TR);
  TileStage<D> st;
  auto load_tile = [&](int kt) {
    const int64_t k0 = (int64_t)kt * TR;
    const int rows = (int)(kend - k0 < TR ? kend - k0 : TR);
    st.load(k, a.ld_k, v, a.ld_v, t.base + k0, rows, h * D);
    return rows;
  };
  auto fetch_ts = [&](int kt) {
    const int64_t k0 = (int64_t)kt * TR;
    SideTs f{0, {0, 0}};
    if (has_ts && tid < TR && k0 + tid < kend) f.tv = a.ts[t.base + k0 + tid];
    if (has_ts && tid < 2 && k0 + 32 * tid < kend)
      f.r = a.key_ranges[key_range_slot(t.base, t.seq) + k0 / 32 + tid];
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
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        s = mfma(ld8(&Kt[toff<D>(32 * kb + l32, 16 * kk + 8 * hl)]), qf[kk], s);
        dp = mfma(ld8(&Vt[toff<D>(32 * kb + l32, 16 * kk + 8 * hl)]), gf[kk], dp);
      }
      // class of the block
      const bool full = q0w >= k0b + 31 && q0w + 31 < t.n;
      const bool posc = q0w - (k0b + 31) >= a.P - 1;
      int blo = 0, bhi = 0;
      bool fits32 = true;
      if (has_ts) {
        const KeyRange kr = krs[buf][kb];
        blo = tbucket(qr.lo - kr.hi, a.T);
        bhi = tbucket(qr.hi - kr.lo, a.T);
        fits32 = time_fast_ok(qr.lo, qr.hi, kr.lo, kr.hi);
      }
      bf16x8 pz[2];
      if (full && posc && blo == bhi) {
        const float bias = rps[a.P - 1] + rts[blo];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p, dsl;
          silu2(s[r] + bias, a.inv_n, p, dsl);
          pz[r >> 3][r & 7] = (bf16)(dp[r] * dsl);
        }
      } else if (full && posc && bhi == blo + 1 && fits32) {
        // two adjacent time buckets: a pair is in bhi exactly when dt + 1 >= 2^bhi,
        // and dt + 1 is the wrapped 32-bit difference of the low words
        const float b_lo = rps[a.P - 1] + rts[blo], b_hi = rps[a.P - 1] + rts[bhi];
        const int thr = 1 << bhi;
        const uint32_t tq1 = (uint32_t)tq + 1u;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int d = (int)(tq1 - tks32[buf][32 * kb + acc_row(r, hl)]);
          float p, dsl;
          silu2(s[r] + (d >= thr ? b_hi : b_lo), a.inv_n, p, dsl);
          pz[r >> 3][r & 7] = (bf16)(dp[r] * dsl);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jr = 32 * kb + acc_row(r, hl);  // key row within the tile
          const int64_t j = (int64_t)kt * TR + jr;
          const bool vis = row_ok && j <= i && j < kend;
          const int bp = pos_bucket((int)(i - j), a.P);
          float z = s[r] + rps[bp];
          if (has_ts) z += rts[tbucket(tq - tks[buf][jr], a.T)];
          float p, dsl;
          silu2(z, a.inv_n, p, dsl);
          pz[r >> 3][r & 7] = (bf16)(vis ? dp[r] * dsl : 0.f);
        }
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int c = 0; c < NC; ++c) dq[c] = mfma(pz[s2], trfrag<D>(Kt, 32 * kb + 16 * s2, c, lane), dq[c]);
    }
    if (more) {
      st.store(Ks[buf ^ 1], Vs[buf ^ 1]);
      store_ts(nf, buf ^ 1);
    }
    __syncthreads();
  }
  if (!wave_live) return;
  bf16* dqo = (bf16*)a.dq;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = q0w + acc_row(r, hl);
      if (row < t.n) dqo[(t.base + row) * a.ld_dq + (int64_t)h * D + 32 * c + l32] = (bf16)dq[c][r];
    }
}

// ------------------------------------------------------------------ key side
template <int D>
__global__ __launch_bounds__(256, D <= 64 ? 2 : 1) void attn_bwd_kv_mfma(AttnBwdArgs a) {
  constexpr int NKK = D / 16, NC = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 Qs[2][TR * (D + 8)];
  __shared__ __attribute__((aligned(16))) bf16 Gs[2][TR * (D + 8)];
  __shared__ int64_t tqs[2][TR];
  __shared__ uint32_t tqs32[2][TR];  // low words, for the two-bucket test
  __shared__ KeyRange qrs[2][2];     // timestamp ranges of the tile's two query blocks
  __shared__ float rps[kMaxPosB];
  __shared__ float rts[kTimeB];
  extern __shared__ float bins[];  // [4][P + TT] when bias_partial is set

  const int item = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hl = lane >> 5;
  const bool has_ts = a.ts != nullptr;
  const int TT = a.T < kTimeB ? a.T : kTimeB;
  const int nbl = a.P + TT;  // LDS bins per wavefront
  float* my_bins = bins + w * nbl;
  if (a.bias_partial)
    for (int x = tid; x < 4 * nbl; x += 256) bins[x] = 0.f;
  const WTile t = wdecode(a, item, true);
  if (t.valid) {
    const bf16* q = (const bf16*)a.q;
    const bf16* k = (const bf16*)a.k;
    const bf16* v = (const bf16*)a.v;
    const bf16* g = (const bf16*)a.dout;
    for (int x = tid; x < a.P; x += 256) rps[x] = a.rab_pos ? a.rab_pos[(int64_t)h * a.P + x] : 0.f;
    for (int x = tid; x < TT; x += 256)
      rts[x] = (a.rab_time && has_ts) ? a.rab_time[(int64_t)h * a.T + x] : 0.f;

    const int64_t k0w = t.r0 + 32 * w;  // this wavefront's first key
    const bool wave_live = k0w < t.n;
    const int64_t j = k0w + l32;        // this lane's key
    const bool key_ok = j < t.n;
    bf16x8 kf[NKK], vf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int64_t off = (t.base + j) * a.ld_k + (int64_t)h * D + 16 * kk + 8 * hl;
      const int64_t offv = (t.base + j) * a.ld_v + (int64_t)h * D + 16 * kk + 8 * hl;
      kf[kk] = key_ok ? ld8(k + off) : bf16x8{};
      vf[kk] = key_ok ? ld8(v + offv) : bf16x8{};
    }
    const int64_t tk = (has_ts && key_ok) ? a.ts[t.base + j] : 0;
    KeyRange kr{0, 0};
    if (has_ts && wave_live) kr = block_range(a, t, k0w);
    f32x16 dk[NC], dv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) dk[c] = dv[c] = f32x16{};
    float bin_clamp = 0.f;  // this lane's share of dz in position bucket P-1 over constant blocks
    // Time-bucket sums of constant and two-bucket blocks: this lane's running sums for
    // buckets cur_b and cur_b + 1 (cur_b wavefront-uniform). Queries arrive in time
    // order for typical data, so a wavefront reduction is needed only when the bucket
    // moves on, not per block.
    int cur_b = -1;
    float acc0 = 0.f, acc1 = 0.f;
    auto flush_bin = [&](int b, float v) {
      const float tot = wave_sum64(v);
      if (lane == 0) my_bins[a.P + b] += tot;  // lane 0 alone writes its wavefront's bins here
    };
    auto flush_all = [&]() {
      if (cur_b >= 0) {
        flush_bin(cur_b, acc0);
        if (cur_b + 1 < TT) flush_bin(cur_b + 1, acc1);  // acc1 is 0 when cur_b is the top bucket
      }
      acc0 = acc1 = 0.f;
    };
    // add this lane's dz sums of a block in buckets b (zl) and b + 1 (zh)
    auto add_bins = [&](int b, float zl, float zh) {
      if (b == cur_b) {
        acc0 += zl;
        acc1 += zh;
      } else if (b == cur_b + 1) {
        flush_bin(cur_b, acc0);
        acc0 = acc1 + zl;
        acc1 = zh;
        cur_b = b;
      } else {
        flush_all();
        acc0 = zl;
        acc1 = zh;
        cur_b = b;
      }
    };

    const int64_t qbeg = t.r0;  // the first query that sees any key of the tile
    const int nqt = (int)((t.n - qbeg + TR - 1) / TR);
    TileStage<D> st;
    auto load_tile = [&](int qt) {
      const int64_t q0 = qbeg + (int64_t)qt * TR;
      const int rows = (int)(t.n - q0 < TR ? t.n - q0 : TR);
      st.load(q, a.ld_q, g, a.ld_do, t.base + q0, rows, h * D);
    };
    auto fetch_ts = [&](int qt) {
      const int64_t q0 = qbeg + (int64_t)qt * TR;
      SideTs f{0, {0, 0}};
      if (has_ts && tid < TR && q0 + tid < t.n) f.tv = a.ts[t.base + q0 + tid];
      if (has_ts && tid < 2 && q0 + 32 * tid < t.n)
        f.r = a.key_ranges[key_range_slot(t.base, t.seq) + q0 / 32 + tid];
      return f;
    };
    auto store_ts = [&](const SideTs& f, int buf) {
      if (tid < TR) {
        tqs[buf][tid] = f.tv;
        tqs32[buf][tid] = (uint32_t)f.tv;
      }
      if (tid < 2) qrs[buf][tid] = f.r;
    };
    load_tile(0);
    st.store(Qs[0], Gs[0]);
    store_ts(fetch_ts(0), 0);
    __syncthreads();

    for (int qt = 0; qt < nqt; ++qt) {
      const int buf = qt & 1;
      const bool more = qt + 1 < nqt;
      SideTs nf{0, {0, 0}};
      if (more) {
        load_tile(qt + 1);
        nf = fetch_ts(qt + 1);
      }
      const bf16* Qt = Qs[buf];
      const bf16* Gt = Gs[buf];
#pragma unroll 1
      for (int qb = 0; qb < 2; ++qb) {
        const int64_t q0b = qbeg + (int64_t)qt * TR + 32 * qb;
        if (!wave_live || q0b + 31 < k0w || q0b >= t.n) continue;  // uniform
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          s = mfma(ld8(&Qt[toff<D>(32 * qb + l32, 16 * kk + 8 * hl)]), kf[kk], s);
          dp = mfma(ld8(&Gt[toff<D>(32 * qb + l32, 16 * kk + 8 * hl)]), vf[kk], dp);
        }
        const bool full = q0b >= k0w + 31 && q0b + 31 < t.n && k0w + 31 < t.n;
        const bool posc = q0b - (k0w + 31) >= a.P - 1;
        int blo = 0, bhi = 0;
        bool fits32 = true;
        if (has_ts) {
          const KeyRange qr = qrs[buf][qb];
          blo = tbucket(qr.lo - kr.hi, a.T);
          bhi = tbucket(qr.hi - kr.lo, a.T);
          fits32 = time_fast_ok(qr.lo, qr.hi, kr.lo, kr.hi);
        }
        bf16x8 pp[2], pz[2];
        if (full && posc && blo == bhi) {
          const float bias = rps[a.P - 1] + rts[blo];
          float zsum = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float p, dsl;
            silu2(s[r] + bias, a.inv_n, p, dsl);
            const float dz = dp[r] * dsl;
            pp[r >> 3][r & 7] = (bf16)p;
            pz[r >> 3][r & 7] = (bf16)dz;
            zsum += dz;
          }
          if (a.bias_partial) {
            bin_clamp += zsum;
            if (has_ts) add_bins(blo, zsum, 0.f);
          }
        } else if (full && posc && bhi == blo + 1 && fits32) {
          // two adjacent time buckets (see the query side)
          const float b_lo = rps[a.P - 1] + rts[blo], b_hi = rps[a.P - 1] + rts[bhi];
          const int thr = 1 << bhi;
          const uint32_t tk32 = (uint32_t)tk;
          float zlo = 0.f, zhi = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int d = (int)(tqs32[buf][32 * qb + acc_row(r, hl)] + 1u - tk32);
            const bool up = d >= thr;
            float p, dsl;
            silu2(s[r] + (up ? b_hi : b_lo), a.inv_n, p, dsl);
            const float dz = dp[r] * dsl;
            pp[r >> 3][r & 7] = (bf16)p;
            pz[r >> 3][r & 7] = (bf16)dz;
            zhi += up ? dz : 0.f;
            zlo += up ? 0.f : dz;
          }
          if (a.bias_partial) {
            bin_clamp += zlo + zhi;
            add_bins(blo, zlo, zhi);
          }
        } else {
          // positions within a sequence fit in 32 bits
          const int i0 = (int)(qbeg + (int64_t)qt * TR), n32 = (int)t.n, j32 = (int)j;
          const uint32_t tk32 = (uint32_t)tk;
          float csum = 0.f;                   // this lane's dz in position bucket P-1
          float zb[4] = {0.f, 0.f, 0.f, 0.f};  // ... in time buckets blo .. blo+3
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ir = 32 * qb + acc_row(r, hl);  // query row within the tile
            const int i = i0 + ir;
            const bool vis = key_ok && i < n32 && j32 <= i;
            const int bp = pos_bucket(i - j32, a.P);
            int bt = 0;
            if (has_ts) {
              if (fits32) {  // t_i + 1 - t_j fits 32 bits; it is <= 0 for negative elapsed times
                const int d1 = (int)(tqs32[buf][ir] + 1u - tk32);
                bt = d1 <= 0 ? 0 : 31 - __builtin_clz((uint32_t)d1);
                bt = bt < a.T - 1 ? bt : a.T - 1;
              } else {
                bt = tbucket(tqs[buf][ir] - tk, a.T);
              }
            }
            const float z = s[r] + rps[bp] + rts[bt];
            float p, dsl;
            silu2(z, a.inv_n, p, dsl);
            const float dz = vis ? dp[r] * dsl : 0.f;
            pp[r >> 3][r & 7] = (bf16)(vis ? p : 0.f);
            pz[r >> 3][r & 7] = (bf16)dz;
            // below the clamp, the lanes of one slot (one query, 32 keys) hold distinct
            // buckets, so these atomics do not collide
            if (a.bias_partial) {
              if (bp == a.P - 1)
                csum += dz;
              else if (vis)
                atomicAdd(&my_bins[bp], dz);
              if (has_ts) {  // every visible pair's time bucket lies in [blo, bhi]
                const int kb = bt - blo;
#pragma unroll
                for (int q = 0; q < 4; ++q) zb[q] += kb == q ? dz : 0.f;
                if (kb >= 4 && vis) atomicAdd(&my_bins[a.P + bt], dz);  // spans past 4 buckets
              }
            }
          }
          if (a.bias_partial) {
            bin_clamp += csum;
            if (has_ts)  // one reduction per bucket
              for (int q = 0; q < 4 && blo + q <= bhi; ++q) {
                const float tb = wave_sum64(zb[q]);
                if (lane == 0) my_bins[a.P + blo + q] += tb;
              }
          }
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            dv[c] = mfma(pp[s2], trfrag<D>(Gt, 32 * qb + 16 * s2, c, lane), dv[c]);
            dk[c] = mfma(pz[s2], trfrag<D>(Qt, 32 * qb + 16 * s2, c, lane), dk[c]);
          }
      }
      if (more) {
        st.store(Qs[buf ^ 1], Gs[buf ^ 1]);
        store_ts(nf, buf ^ 1);
      }
      __syncthreads();
    }
    if (a.bias_partial) {
      if (has_ts) flush_all();
      const float tot = wave_sum64(bin_clamp);
      if (lane == 0) my_bins[a.P - 1] += tot;
    }
    if (wave_live) {
      bf16* dko = (bf16*)a.dk;
      bf16* dvo = (bf16*)a.dv;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = k0w + acc_row(r, hl);
          if (row < t.n) {
            const int64_t rr = t.base + row;
            dko[rr * a.ld_dk + (int64_t)h * D + 32 * c + l32] = (bf16)dk[c][r];
            dvo[rr * a.ld_dv + (int64_t)h * D + 32 * c + l32] = (bf16)dv[c][r];
          }
        }
    }
  }
  if (a.bias_partial) {  // this work item's bucket sums, waves added in a fixed order
    __syncthreads();
    const int nb = a.P + a.T;
    float* out = a.bias_partial + ((int64_t)item * a.H + h) * nb;
    for (int x = tid; x < nb; x += 256) {
      float s = 0.f;
      if (x < nbl)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) s += bins[qq * nbl + x];
      out[x] = s;
    }
  }
}

template <int D>
static void launch_bwd_mfma_d(const AttnBwdArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.n_items * (unsigned)a.H);
  const int TT = a.T < kTimeB ? a.T : kTimeB;
  const size_t bins = a.bias_partial ? (size_t)4 * (a.P + TT) * sizeof(float) : 0;
  hipLaunchKernelGGL((attn_bwd_kv_mfma<D>), grid, dim3(256), bins, s, a);
  hipLaunchKernelGGL((attn_bwd_q_mfma<D>), grid, dim3(256), 0, s, a);
}

hipError_t launch_attn_bwd_mfma(const AttnBwdArgs& a, hipStream_t s) {
  if (a.n_items <= 0 || a.H <= 0) return hipSuccess;
  if (a.ts && !a.key_ranges) return hipErrorInvalidValue;
  switch (a.d_qk) {
    case 32: launch_bwd_mfma_d<32>(a, s); break;
    case 64: launch_bwd_mfma_d<64>(a, s); break;
    case 128: launch_bwd_mfma_d<128>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hstu
