// Internal launch interface between the C-ABI host layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

// Smallest and largest timestamp of one 32-key block of a sequence. Block j of
// sequence b (keys 32j .. 32j+31, clipped to the sequence) sits at slot
// key_range_slot(offsets[b], b) + j; distinct sequences never share a slot.
struct KeyRange {
  int64_t lo, hi;
};
__host__ __device__ inline int64_t key_range_slot(int64_t seq_start, int seq) {
  return seq_start / 32 + seq;
}
// Slots needed for `total` keys in `batch` sequences.
inline int64_t key_range_slots(int64_t total, int batch) { return total / 32 + batch + 1; }

// One attention launch. Row strides (ld_*) are in elements. Tensor bases point
// at head 0 of row 0; head h sits at column h * d within each row.
// -log2(e): the factor the library's f1 projection applies to the queries it stores for
// the MFMA attention in candidate mode and in layers (split scores)
constexpr float kQueryPrescale = -1.4426950408889634f;

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;          // bf16 or f32 (out_f32), [rows, H, d_v] with stride ld_o
  int64_t ld_q, ld_k, ld_v, ld_o;
  const int64_t* q_offsets;   // causal: sequence offsets; candidate mode: candidate offsets
  const int64_t* k_offsets;   // causal: same as q_offsets; candidate mode: history offsets
  const int64_t* ts_q;        // per query row, or NULL
  const int64_t* ts_k;        // per key row, or NULL
  const float* rab_pos;       // [H][P] or NULL
  const float* rab_time;      // [H][T] or NULL
  const KeyRange* key_ranges; // per 32-key block timestamp ranges of the keys (with ts_k), else NULL
  int batch;                  // number of sequences (causal) or users (candidate mode)
  int H, d_qk, d_v, P, T;
  float inv_n;
  int out_f32;
  // causal mode: work list of (sequence, query tile), longest first
  const int2* items;
  int n_items;
  // candidate mode: candidates' own K and V rows (the self term), the global
  // candidate row range of this microbatch and the users overlapping it
  const void* kc;
  const void* vc;
  int64_t ld_kc, ld_vc;
  int64_t row_begin, row_end;
  int user_begin, n_users;
  int64_t max_user_rows;      // most candidate rows any one user has in this microbatch
  // candidate mode only: the history is split into kv_splits key ranges of
  // keys_per_split (a multiple of 64); split s writes its partial output (already
  // scaled by 1/N; split 0 also adds the self term) at out + s * part_stride
  int kv_splits;
  int64_t keys_per_split;
  int64_t part_stride;
  // causal mode, MFMA kernel, optional: the lo parts of q and k (same strides as q and k),
  // so that each score is formed from ~16-bit queries and keys (hi.hi + lo.hi + hi.lo).
  // The MFMA kernel in candidate mode and with these lo parts takes queries pre-scaled by
  // kQueryPrescale (see attn_mfma.hip); the f1 projection stores them so.
  const void* q_lo;
  const void* k_lo;
  // candidate mode, MFMA kernel: where split 0 writes each candidate's self weight
  // SiLU(q_c.k_c + rab_pos[0] + rab_time[0]) / N, [microbatch rows][H], for the LN gate to
  // add self_w * v_c (the vector-ALU kernel adds the self term itself and ignores this)
  float* self_w;
};

// Tile sizes (query rows per work item) of the two attention kernels.
constexpr int kMfmaRows = 128;
constexpr int kSimpleRows = 64;

// True when the MFMA kernel handles this shape (bf16, d_qk == d_v in {32,64,128}
// and the bias tables fit its LDS).
bool attn_mfma_supported(int dtype_bf16, int d_qk, int d_v, int P, int T);
// True when the MFMA kernel can take these row strides (K and V strides equal).
bool attn_mfma_strides_ok(const AttnArgs& a);

// Causal work list (sequence, query tile of tile_rows), longest first, and, when ts and kr
// are set, the per-32-key timestamp ranges of the B jagged sequences (see KeyRange); one
// launch.
hipError_t launch_plan(const int64_t* offsets, int B, int tile_rows, int max_tiles, int2* items,
                       int n_items, const int64_t* ts, int64_t max_len, KeyRange* kr,
                       hipStream_t s);
hipError_t launch_attn_simple(const AttnArgs& a, int use_bf16, bool cand, hipStream_t s);
// Causal softmax attention (the softmax ablation of the pointwise kernel): bf16,
// d_qk == d_v in {32,64,128}, P <= 1024; items from the planner with 128-row tiles,
// key ranges whenever ts_q is set; out is bf16 [rows, H, d_v] with stride ld_o.
bool attn_softmax_supported(int dtype_bf16, int d_qk, int d_v, int P);
hipError_t launch_attn_softmax(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_mfma(const AttnArgs& a, bool cand, hipStream_t s);

// One attention backward launch (causal mode). Row strides (ld_*) are in elements;
// head h sits at column h * d within each row.
struct AttnBwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;           // dL/d(attention output) [rows, H, d_v]
  void* dq;
  void* dk;
  void* dv;
  int64_t ld_q, ld_k, ld_v, ld_do, ld_dq, ld_dk, ld_dv;
  const int64_t* offsets;
  const int64_t* ts;          // NULL: no time term (and a zero time-table gradient)
  const float* rab_pos;       // [H][P] or NULL (= 0)
  const float* rab_time;      // [H][T] or NULL (= 0)
  float* bias_partial;        // [n_items][H][P + T] bucket sums of dz per work item, or NULL
  const KeyRange* key_ranges; // per 32-row timestamp ranges (MFMA kernels, with ts), else NULL
  const int2* items;          // (sequence, tile) list from the planner (64-row tiles for the
                              // vector-ALU kernels, 128-row tiles for the MFMA kernels)
  int n_items;
  int batch, H, d_qk, d_v, P, T;
  float inv_n;
};

hipError_t launch_attn_bwd_simple(const AttnBwdArgs& a, int use_bf16, hipStream_t s);
// True when the MFMA backward handles this shape (bf16, d_qk == d_v in {32,64,128}, P <= 1024).
bool attn_bwd_mfma_supported(int dtype_bf16, int d_qk, int d_v, int P);
hipError_t launch_attn_bwd_mfma(const AttnBwdArgs& a, hipStream_t s);
// d_rab_pos[h][p] / d_rab_time[h][t] = fixed-order sums of the per-item partials
// (partial may be NULL when n_items is 0; the outputs are then zeros).
hipError_t launch_bias_grad_reduce(const float* partial, int n_items, int H, int P, int T,
                                   float* d_rab_pos, float* d_rab_time, hipStream_t s);

// out[r, :] = (LN(o[r, :]) * gamma + beta) (.) u[r, :], width w, over `rows` rows, where
// o[r, :] is the sum of nsplit partial rows o + s * split_stride (s = 0..nsplit-1, in order).
hipError_t launch_ln_gate(const float* o, int64_t ld_o, int nsplit, int64_t split_stride,
                          const void* u, int64_t ld_u, const float* gamma, const float* beta,
                          float eps, void* out, int64_t ld_out, int64_t rows, int w, int use_bf16,
                          hipStream_t s, const float* self_w = nullptr,
                          const void* vself = nullptr, int64_t ld_vself = 0, int dv = 0);

// The LN gate and f2 in one launch (bf16): y[r, :] = g[r, :] W2^T + b2 (+ R[r, :]) with g the
// bf16 rounding of launch_ln_gate's output, never stored. K = H*d_v is the gated width and N
// the model width (W2 is [N, K], row stride ldw). ln_gate_f2_supported: the shapes with a
// one-kernel form, and W2, gamma and beta (NULL allowed for the last two) 16-byte aligned;
// the caller runs launch_ln_gate and launch_gemm otherwise.
bool ln_gate_f2_supported(int K, int N, int use_bf16, const void* w2, const float* gamma,
                          const float* beta);
hipError_t launch_ln_gate_f2(const float* o, int64_t ld_o, int nsplit, int64_t split_stride,
                             const void* u, int64_t ld_u, const float* gamma, const float* beta,
                             float eps, const void* w2, int64_t ldw, const float* b2, const void* R,
                             int64_t ldr, void* y, int64_t ldy, int64_t rows, int K, int N,
                             hipStream_t s, const float* self_w = nullptr,
                             const void* vself = nullptr, int64_t ld_vself = 0, int dv = 0);

// C[M,N] = epi(A[M,K] W[N,K]^T + bias[N]); epi = SiLU when silu, + R[M,N] when R.
// lo (bf16 output only): for columns n >= lo_c0 (a multiple of 8) also writes
// lo[m, n] = bf16(y - bf16(y)), the part of the fp32 result y that the bf16 C drops, with
// C's leading dimension; C + lo then carries y to about 16 significant bits.
// Columns [sc_c0, sc_c1) (multiples of 8; bf16 output only) are stored as sc * y (the
// remainder then belongs to the scaled value).
hipError_t launch_gemm(const void* A, int64_t lda, const void* W, int64_t ldw,
                       const float* bias, const void* R, int64_t ldr, void* C, int64_t ldc,
                       int64_t M, int N, int K, int silu, int use_bf16, hipStream_t s,
                       void* lo = nullptr, int lo_c0 = 0, int sc_c0 = 0, int sc_c1 = 0,
                       float sc = 1.f);

// launch_gemm (bf16, no residual) computing only two column windows of C: columns
// [c0, c0 + len0) and [c1, c1 + len1), from the same rows of W and bias. Returns
// hipErrorInvalidValue, launching nothing, when len0 is not a multiple of the tile width
// the size selects (the caller then computes every column).
hipError_t launch_gemm_2cols(const void* A, int64_t lda, const void* W, int64_t ldw,
                             const float* bias, void* C, int64_t ldc, int64_t M, int K, int silu,
                             int c0, int len0, int c1, int len1, hipStream_t s);

// launch_gemm with an fp32 output (bf16 inputs; fp32 inputs always write fp32) and
// split-K: grid dimension y = splits, split y covers K range [y*ksplit, (y+1)*ksplit)
// (ksplit a multiple of 64) and writes C + y*c_split; splits > 1 takes no bias,
// residual or SiLU. act (bf16 inputs, fp32 output, one split, no SiLU, else NULL) also
// receives SiLU(C) in bf16, same leading dimension, rounded as launch_silu_act rounds.
// lo as for launch_gemm: the bf16 remainder of C (bf16 output) or, with act, of SiLU(C).
hipError_t launch_gemm_ex(const void* A, int64_t lda, const void* W, int64_t ldw, const float* bias,
                          const void* R, int64_t ldr, void* C, int64_t ldc, int64_t M, int N, int K,
                          int silu, int use_bf16, int out_f32, int splits, int64_t ksplit,
                          int64_t c_split, void* act, hipStream_t s, void* lo = nullptr,
                          int lo_c0 = 0, int sc_c0 = 0, int sc_c1 = 0, float sc = 1.f);

// C[M,N] = sum_k A[k,m] B[k,n] (bf16 A [K, lda] and B [K, ldb] row-major, fp32 C): the
// weight-gradient form, contraction over rows. M, N and both leading dimensions multiples
// of 8. Split-K as launch_gemm_ex over rows: split y covers rows [y*ksplit, (y+1)*ksplit)
// (ksplit a multiple of 64) and writes C + y*c_split.
hipError_t launch_gemm_tn(const void* A, int64_t lda, const void* B, int64_t ldb, float* C,
                          int64_t ldc, int M, int N, int64_t K, int splits, int64_t ksplit,
                          int64_t c_split, hipStream_t s);

// logit[r] = sum_c y[r, c] * w[c] (fp32 accumulate).
hipError_t launch_rowdot(const void* y, int64_t ld_y, const float* w, float* logit, int64_t rows,
                         int d, int use_bf16, hipStream_t s);

// Stochastic Length: src[new_off[b] + i] = input row of the i-th kept action of
// sequence b (whole when its new length equals its length, else the positions of
// the smallest (key, position) pairs), then the optional row and timestamp gather.
hipError_t launch_sl_select(const int64_t* off, const int64_t* new_off, int B,
                            const uint32_t* keys, int64_t* src, hipStream_t s);
hipError_t launch_sl_gather(const int64_t* src, int64_t rows, const void* x, int64_t row_bytes,
                            const int64_t* ts, void* out_x, int64_t* out_ts, hipStream_t s);

// Layer backward helpers (layer_bwd.hip).
// out[c][r] = in[r][c] (r < R), 0 for R <= r < Rpad; rows of `in` stride ld_in.
hipError_t launch_transpose(const void* in, int64_t ld_in, void* out, int64_t ld_out, int64_t R,
                            int64_t Rpad, int C, int use_bf16, hipStream_t s);
// out[c] = sum over rows of x[r][c], fixed order; partial holds colsum_chunks(R) * C floats.
int colsum_chunks(int64_t R);
hipError_t launch_colsum(const void* x, int64_t ld, int64_t R, int C, int use_bf16, float* partial,
                         float* out, hipStream_t s);
// out[c] = sum_{k < n} partial[k * stride + c] in order of k (zeros when n == 0).
hipError_t launch_sum_rows(const float* partial, int64_t stride, int n, int64_t C, float* out,
                           hipStream_t s);
// act = SiLU(z) in the activation type, rounded as the f1 GEMM epilogue rounds.
hipError_t launch_silu_act(const float* z, int64_t ld_z, void* act, int64_t ld_a, int64_t R, int C,
                           int use_bf16, hipStream_t s);
// d *= SiLU'(z), in place.
hipError_t launch_silu_grad(const float* z, int64_t ld_z, void* d, int64_t ld_d, int64_t R, int C,
                            int use_bf16, hipStream_t s);
// Backward of out = (LN(o) gamma + beta) (.) u for width w <= 1024: writes d_o and du, and
// ln_gate_bwd_blocks(rows) partial rows of dgamma and dbeta.
int ln_gate_bwd_blocks(int64_t rows);
hipError_t launch_ln_gate_bwd(const float* o, int64_t ld_o, const void* u, int64_t ld_u,
                              const float* gamma, const float* beta, float eps, const void* g,
                              int64_t ld_g, void* d_o, int64_t ld_do, void* du, int64_t ld_du,
                              float* part_gamma, float* part_beta, int64_t rows, int w,
                              int use_bf16, hipStream_t s);

hipError_t launch_debug_buckets(const int64_t* offsets, const int64_t* ts, int seq, int n, int P,
                                int T, int32_t* pos_bucket, int32_t* time_bucket, hipStream_t s);

}  // namespace hstu
