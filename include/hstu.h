/*
 * libhstu: HSTU pointwise attention over jagged user-action sequences, for
 * AMD Instinct MI355X (gfx950).
 *
 * The operations follow the HSTU layer as the chenhuiyu.github.io HSTU chapter
 * states it ("What an HSTU layer changes", equations 1-3):
 *
 *   U, V, Q, K = Split(SiLU(f1(X)))                                  (eq. 1)
 *   A(X) V     = SiLU(Q K^T + rab^{p,t}) V, scaled by 1/N, no softmax (eq. 2)
 *   Y          = f2(LayerNorm(A(X) V) (.) U)                          (eq. 3)
 *
 * The same chapter ("Three more scaling components") asks for ragged kernels
 * with no padding. Its "M-FALCON" section scores candidates in microbatches
 * against a history computed once. The praveentn.live note ("What HSTU actually
 * changed") adds that candidates are masked from one another.
 *
 * Conventions for every entry point
 * ---------------------------------
 * Memory.  Pointer arguments named *_host point to host memory. All other
 *   tensor pointers are device memory. The caller allocates and owns all of
 *   it. The library never allocates or frees device memory and keeps no
 *   pointer after it returns. It needs scratch device memory only through the
 *   caller's `workspace` (256-byte aligned, at least the size that the
 *   matching *_workspace_size call reports). The caller keeps the workspace
 *   alive until the stream has passed the call. The one exception is
 *   hstu_attn_fwd_noalloc, whose scratch is a fixed device array inside the
 *   library.
 * Streams.  `stream` is a hipStream_t (NULL for the null stream). Every call
 *   only enqueues work on it and never synchronises the device. HSTU_OK means
 *   "validated and enqueued".
 * Jagged batches.  Sequence b occupies rows [offsets[b], offsets[b+1]) of
 *   every per-token tensor. offsets has B+1 int64 entries, with offsets[0] = 0
 *   and the entries non-decreasing. Empty sequences are allowed, and B = 0 is
 *   a no-op. The host copy (*_offsets_host) must hold the same values as the
 *   device copy. The library uses the host copy to validate and size the
 *   launch, so it never copies from device to host.
 * Layouts.  Row-major and contiguous:
 *   Q, K [T_tot, H, d_qk]; V, U and the attention output [T_tot, H, d_v];
 *   X, Y [T_tot, d_model].
 *   f1 weight w1 [2H(d_v+d_qk), d_model], stored out x in. Its row blocks are
 *   U, V, Q, K, in that order, and within each block head h owns rows
 *   h*d .. h*d+d-1. f2 weight w2 [d_model, H*d_v], stored out x in.
 *   Tensor elements have the descriptor's dtype. Biases, rab tables and the
 *   LayerNorm gamma/beta are always fp32. Timestamps are int64 seconds.
 * Bias.  bias(i, j) = rab_pos[h][min(i-j, P-1)]
 *                   + rab_time[h][min(floor(log2(max(t_i - t_j, 0) + 1)), T-1)]
 *   This is the relative position and elapsed time bias of eq. 2. The bucket
 *   indices are computed in exact integer arithmetic. A NULL table (or NULL
 *   timestamps, for the time term) contributes 0.
 * Scale.  Each score is SiLU(q.k + bias) / N, with N = desc->max_seq_len.
 *   There is no 1/sqrt(d). Key j is visible to query i iff j <= i (causal).
 *   A hidden pair contributes exactly 0.
 * Errors.  Every call returns an hstu_status. On any status other than
 *   HSTU_OK and HSTU_DEVICE_ERROR nothing has been launched or written.
 *   HSTU_DEVICE_ERROR reports a HIP launch failure. hstu_last_error() returns
 *   a message for the calling thread's last failure.
 * Support.  d_qk and d_v in {32, 64, 128}; dtype HSTU_F32 or HSTU_BF16.
 */
#ifndef HSTU_H_
#define HSTU_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSTU_VERSION 100 /* 1.0.0 */

typedef enum {
  HSTU_OK = 0,
  HSTU_INVALID_ARGUMENT = 1,
  HSTU_UNSUPPORTED = 2,
  HSTU_WORKSPACE_TOO_SMALL = 3,
  HSTU_DEVICE_ERROR = 4
} hstu_status;

typedef enum { HSTU_F32 = 0, HSTU_BF16 = 1 } hstu_dtype;

/* Shape of one attention call. */
typedef struct {
  int32_t batch;            /* B, number of sequences (>= 0) */
  int32_t num_heads;        /* H (>= 1) */
  int32_t d_qk;             /* per-head query/key width: 32, 64 or 128 */
  int32_t d_v;              /* per-head value width: 32, 64 or 128 */
  int32_t max_seq_len;      /* N (>= 1). Scores are scaled by 1/N. Must be >= every sequence length */
  int32_t num_pos_buckets;  /* P (>= 1), columns of rab_pos */
  int32_t num_time_buckets; /* T (>= 1), columns of rab_time */
  hstu_dtype dtype;         /* element type of q, k, v, u and out */
  float ln_eps;             /* LayerNorm epsilon (> 0) when the gated output is requested */
} hstu_attn_desc;

/* One HSTU layer (eqs. 1-3), or a stack of num_layers of them. */
typedef struct {
  hstu_attn_desc attn;
  int32_t d_model;          /* width of X and Y (>= 1, multiple of 8) */
  int32_t residual;         /* 0: Y = f2(...); 1: Y = f2(...) + X */
  int32_t num_layers;       /* >= 1; layer l reads layer l-1's output */
} hstu_layer_desc;

/* Device pointers of one layer's parameters (host struct). */
typedef struct {
  const void* w1;           /* [2H(d_v+d_qk), d_model], dtype */
  const float* b1;          /* [2H(d_v+d_qk)] or NULL (= 0) */
  const float* rab_pos;     /* [H][P] or NULL */
  const float* rab_time;    /* [H][T] or NULL */
  const float* ln_gamma;    /* [H*d_v] or NULL (= 1) */
  const float* ln_beta;     /* [H*d_v] or NULL (= 0) */
  const void* w2;           /* [d_model, H*d_v], dtype */
  const float* b2;          /* [d_model] or NULL (= 0) */
} hstu_layer_weights;

/* M-FALCON candidate scoring. */
typedef struct {
  hstu_layer_desc layer;    /* batch = number of users; max_seq_len = N for every user */
  int32_t microbatch;       /* candidates per pass through the layer stack (>= 1) */
} mfalcon_desc;

int hstu_version(void);
const char* hstu_status_string(hstu_status status);
/* Message for the calling thread's most recent failed call ("" if none). */
const char* hstu_last_error(void);

/* ------------------------------------------------------------------------
 * hstu_attn_fwd: jagged causal HSTU attention (eq. 2), with an optional
 * gated norm (the Norm(AV) (.) U part of eq. 3).
 *
 *   out[i,h,:] = sum_{j<=i} SiLU(q_i.k_j + bias_h(i,j)) / N * v_j   (u == NULL)
 *   out[i,:,:] = (LN(AV_i) * gamma + beta) (.) u_i                  (u != NULL)
 *
 * The LayerNorm runs over all H*d_v values of a row, with the biased
 * variance and eps = desc->ln_eps. It is computed in fp32.
 * seq_offsets_host [B+1] (host), seq_offsets [B+1] (device).
 * timestamps [T_tot] (device, int64 seconds) or NULL.
 * q, k [T_tot,H,d_qk]; v, u, out [T_tot,H,d_v] (device, dtype).
 * rab_pos [H][P], rab_time [H][T], ln_gamma, ln_beta [H*d_v]: device fp32 or NULL.
 * out must not overlap any input.
 * ---------------------------------------------------------------------- */
hstu_status hstu_attn_workspace_size(const hstu_attn_desc* desc, const int64_t* seq_offsets_host,
                                     size_t* bytes);
hstu_status hstu_attn_fwd(const hstu_attn_desc* desc, const int64_t* seq_offsets_host,
                          const int64_t* seq_offsets, const int64_t* timestamps, const void* q,
                          const void* k, const void* v, const float* rab_pos,
                          const float* rab_time, const void* u, const float* ln_gamma,
                          const float* ln_beta, void* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * hstu_attn_fwd_noalloc: hstu_attn_fwd without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). It runs the same
 * kernels and returns the same results bit for bit. Arguments are those of
 * hstu_attn_fwd minus workspace and workspace_bytes.
 * Its scratch is a device array inside the library, of
 * hstu_attn_noalloc_scratch_bytes() bytes (64 MiB): every device that the
 * library runs on holds one copy until the process ends. The call allocates
 * nothing (no hipMalloc, no hipFree, no allocating library routine); its first
 * call on a device looks up that device's copy once. A call whose scratch need
 * (hstu_attn_workspace_size) exceeds the array returns HSTU_UNSUPPORTED before
 * anything is launched. All calls on one device share its array, so calls
 * that overlap on one device (several streams or host threads) race: order
 * them on one stream. Nothing in the scratch needs to start at zero; each call
 * rewrites what it reads.
 * ---------------------------------------------------------------------- */
size_t hstu_attn_noalloc_scratch_bytes(void);
hstu_status hstu_attn_fwd_noalloc(const hstu_attn_desc* desc, const int64_t* seq_offsets_host,
                                  const int64_t* seq_offsets, const int64_t* timestamps,
                                  const void* q, const void* k, const void* v,
                                  const float* rab_pos, const float* rab_time, const void* u,
                                  const float* ln_gamma, const float* ln_beta, void* out,
                                  void* stream);

/* ------------------------------------------------------------------------
 * hstu_layer_fwd: num_layers HSTU layers over a jagged batch (eqs. 1-3):
 *   [U|V|Q|K] = SiLU(X w1^T + b1); G = LN(causal attention)*gamma+beta (.) U;
 *   Y = G w2^T + b2 (+ X if residual). Layer l + 1 reads layer l's Y.
 * x, y [T_tot, d_model] (device, dtype); x and y may not overlap.
 * weights: host array [num_layers] of device-pointer structs.
 * Intermediates are stored in the dtype (bf16 for HSTU_BF16). Accumulation
 * and the LayerNorm statistics are fp32.
 * ---------------------------------------------------------------------- */
hstu_status hstu_layer_workspace_size(const hstu_layer_desc* desc,
                                      const int64_t* seq_offsets_host, size_t* bytes);
hstu_status hstu_layer_fwd(const hstu_layer_desc* desc, const int64_t* seq_offsets_host,
                           const int64_t* seq_offsets, const int64_t* timestamps, const void* x,
                           const hstu_layer_weights* weights, void* y, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * mfalcon_score: M-FALCON ranking over candidate microbatches.
 * User b has history rows [hist_offsets[b], hist_offsets[b+1]) and candidate
 * rows [cand_offsets[b], cand_offsets[b+1]). A candidate sits at position
 * n_h(b), right after its user's history, with its own timestamp cand_ts[c].
 * At every layer it attends to all of its user's history keys
 * (bias position n_h - j, elapsed time t_c - t_j) and to its own key
 * (position 0, elapsed time 0), never to another candidate. Its output
 * therefore equals the last row of hstu_layer_fwd run on
 * (history, candidate). The history pass runs once per call. The candidates
 * are then processed desc->microbatch at a time (in global candidate order)
 * through all layers, reusing the cached history keys and values. Up to 16
 * microbatches (at most 65,536 rows, at least one microbatch) are in flight at
 * once: their work is issued together, one launch per step for the group,
 * which is what the workspace is sized for.
 * A candidate's result does not depend on the microbatch size or on the
 * other candidates, bit for bit.
 * hist_x [n_hist_tot, d_model], cand_x and cand_out [C_tot, d_model] (dtype).
 * hist_ts and cand_ts are both NULL or both set.
 * w_head [d_model] fp32 or NULL; cand_logit [C_tot] fp32 = cand_out . w_head,
 * or NULL.
 * ---------------------------------------------------------------------- */
hstu_status mfalcon_workspace_size(const mfalcon_desc* desc, const int64_t* hist_offsets_host,
                                   const int64_t* cand_offsets_host, size_t* bytes);
hstu_status mfalcon_score(const mfalcon_desc* desc, const int64_t* hist_offsets_host,
                          const int64_t* hist_offsets, const int64_t* hist_ts, const void* hist_x,
                          const int64_t* cand_offsets_host, const int64_t* cand_offsets,
                          const int64_t* cand_ts, const void* cand_x,
                          const hstu_layer_weights* weights, const float* w_head,
                          void* cand_out, float* cand_logit, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * A persistent M-FALCON history cache, for serving several requests (candidate
 * sets) against the same users' histories (HSTU chapter, "M-FALCON": the
 * history's keys and values are computed once and reused, as a KV cache).
 *
 * mfalcon_history runs the history pass of mfalcon_score and stores what the
 * candidate pass needs in `cache` (caller-owned device memory, 256-byte
 * aligned, at least mfalcon_cache_size bytes): per layer the f1 output over
 * the history, and the per-32-key timestamp ranges of the history keys.
 * `workspace` (mfalcon_history_workspace_size bytes) is scratch for the call
 * only.
 *
 * mfalcon_score_cached runs the candidate pass against such a cache. Its
 * results equal mfalcon_score's bit for bit when the descriptor, the history
 * offsets and timestamps, and the weights are the ones the cache was built
 * with; the library cannot check that the cache matches (it keeps no state),
 * so that is the caller's contract. The cache is only read, so calls with
 * different candidate sets may share it. `workspace` is
 * mfalcon_cached_workspace_size bytes.
 * ---------------------------------------------------------------------- */
hstu_status mfalcon_cache_size(const mfalcon_desc* desc, const int64_t* hist_offsets_host,
                               size_t* bytes);
hstu_status mfalcon_history_workspace_size(const mfalcon_desc* desc,
                                           const int64_t* hist_offsets_host, size_t* bytes);
hstu_status mfalcon_history(const mfalcon_desc* desc, const int64_t* hist_offsets_host,
                            const int64_t* hist_offsets, const int64_t* hist_ts,
                            const void* hist_x, const hstu_layer_weights* weights, void* cache,
                            size_t cache_bytes, void* workspace, size_t workspace_bytes,
                            void* stream);
hstu_status mfalcon_cached_workspace_size(const mfalcon_desc* desc,
                                          const int64_t* hist_offsets_host,
                                          const int64_t* cand_offsets_host, size_t* bytes);
hstu_status mfalcon_score_cached(const mfalcon_desc* desc, const int64_t* hist_offsets_host,
                                 const int64_t* hist_offsets, const int64_t* hist_ts,
                                 const void* cache, size_t cache_bytes,
                                 const int64_t* cand_offsets_host, const int64_t* cand_offsets,
                                 const int64_t* cand_ts, const void* cand_x,
                                 const hstu_layer_weights* weights, const float* w_head,
                                 void* cand_out, float* cand_logit, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * hstu_attn_bwd: gradients of hstu_attn_fwd without the gate (eq. 2), for
 * training (the HSTU chapter trains the model generatively). With g = d_out,
 * the gradient of a loss with respect to the attention output [T_tot, H, d_v]:
 *   z_ij = q_i.k_j + bias(i, j), a_ij = SiLU(z_ij) / N        (visible j <= i)
 *   dv_j = sum_i a_ij g_i
 *   dz_ij = (g_i.v_j) SiLU'(z_ij) / N
 *   dq_i = sum_j dz_ij k_j,  dk_j = sum_i dz_ij q_i
 *   d_rab_pos[h][p]  = sum of dz_ij over the pairs of head h in position bucket p
 *   d_rab_time[h][t] = sum of dz_ij over the pairs of head h in time bucket t
 * Inputs are those of the forward call (same layouts and dtype). dq, dk, dv
 * (same shapes and dtype as q, k, v) are overwritten. d_rab_pos [H][P] and
 * d_rab_time [H][T] are fp32 and overwritten. Pass NULL for either to skip
 * it. A NULL table still gets its gradient. So does the time table without
 * timestamps, which is then zero. The table gradients need P + T <= 2048
 * (HSTU_UNSUPPORTED otherwise). dq, dk and dv are summed in a fixed order, so
 * they repeat bit for bit. The table gradients are summed per workgroup with
 * LDS atomics, so they can differ run to run in the last bits.
 * `workspace` is hstu_attn_bwd_workspace_size bytes.
 * ---------------------------------------------------------------------- */
hstu_status hstu_attn_bwd_workspace_size(const hstu_attn_desc* desc,
                                         const int64_t* seq_offsets_host, size_t* bytes);
hstu_status hstu_attn_bwd(const hstu_attn_desc* desc, const int64_t* seq_offsets_host,
                          const int64_t* seq_offsets, const int64_t* timestamps, const void* q,
                          const void* k, const void* v, const float* rab_pos,
                          const float* rab_time, const void* d_out, void* dq, void* dk, void* dv,
                          float* d_rab_pos, float* d_rab_time, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * hstu_layer_bwd: gradients of hstu_layer_fwd (a stack of num_layers layers,
 * eqs. 1-3) for training. Given d_y = dL/dY of the stack's output, it writes
 * d_x = dL/dX (activation dtype; NULL to skip) and, for each layer l,
 * grads[l] (host array of num_layers structs; NULL, or any NULL pointer in
 * it, skips that gradient). Every gradient is overwritten, not accumulated.
 * Parameter gradients are fp32 and laid out like the parameters. The bias
 * tables of a layer get the sums of dL/dz over their buckets, as in
 * hstu_attn_bwd.
 * The forward pass is recomputed inside the call from x and the weights (the
 * inputs of layers 1..L-1 are kept in the workspace), so the caller stores no
 * activations. With g = dL/dY of a layer, z1 = X w1^T + b1 and
 * G = (LN(O) gamma + beta) (.) U:
 *   dW2 = g^T G, db2 = column sums of g, dG = g W2,
 *   (dO, dU, dgamma, dbeta) from the LayerNorm-gate backward,
 *   (dQ, dK, dV, table gradients) from the attention backward,
 *   dz1 = d[U|V|Q|K] (.) SiLU'(z1), dW1 = dz1^T X, db1 = column sums of dz1,
 *   dX = dz1 W1 (+ g when residual).
 * Sums over tokens run in a fixed order, so the results repeat bit for bit,
 * except the bias-table gradients (see hstu_attn_bwd).
 * Support: H*d_v <= 1024. `workspace` is hstu_layer_bwd_workspace_size bytes.
 * ---------------------------------------------------------------------- */
typedef struct {
  float* dw1;               /* [2H(d_v+d_qk), d_model] */
  float* db1;               /* [2H(d_v+d_qk)] */
  float* d_rab_pos;         /* [H][P] */
  float* d_rab_time;        /* [H][T] */
  float* d_ln_gamma;        /* [H*d_v] */
  float* d_ln_beta;         /* [H*d_v] */
  float* dw2;               /* [d_model, H*d_v] */
  float* db2;               /* [d_model] */
} hstu_layer_grads;

hstu_status hstu_layer_bwd_workspace_size(const hstu_layer_desc* desc,
                                          const int64_t* seq_offsets_host, size_t* bytes);
hstu_status hstu_layer_bwd(const hstu_layer_desc* desc, const int64_t* seq_offsets_host,
                           const int64_t* seq_offsets, const int64_t* timestamps, const void* x,
                           const hstu_layer_weights* weights, const void* d_y, void* d_x,
                           const hstu_layer_grads* grads, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * hstu_softmax_attn_fwd: the softmax variant of hstu_attn_fwd (u == NULL), the
 * ablation of the HSTU chapter ("No sequence-wise softmax") that replaces the
 * pointwise activation with a softmax over each query's visible keys:
 *   out[i,h,:] = sum_{j<=i} exp(z_ij) v_j / sum_{j<=i} exp(z_ij),
 *   z_ij = q_i.k_j + bias_h(i,j)   (the same scores, buckets and tables; no 1/sqrt(d)).
 * It is the in-house softmax-attention baseline for the pointwise kernel. Arguments
 * and layouts as hstu_attn_fwd. Support: dtype HSTU_BF16 (fp32 accumulation),
 * d_qk == d_v in {32, 64, 128}, num_pos_buckets <= 1024 (HSTU_UNSUPPORTED otherwise).
 * `workspace` is hstu_softmax_attn_workspace_size bytes.
 * ---------------------------------------------------------------------- */
hstu_status hstu_softmax_attn_workspace_size(const hstu_attn_desc* desc,
                                             const int64_t* seq_offsets_host, size_t* bytes);
hstu_status hstu_softmax_attn_fwd(const hstu_attn_desc* desc, const int64_t* seq_offsets_host,
                                  const int64_t* seq_offsets, const int64_t* timestamps,
                                  const void* q, const void* k, const void* v,
                                  const float* rab_pos, const float* rab_time, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stochastic Length (HSTU chapter, "Three more scaling components",
 * Stochastic Length): training keeps the full history of short users and of a
 * few long ones, and cuts the rest to a random subsequence of the target
 * length L = floor(N^(alpha/2)), so that alpha = 1.6 takes N = 4096 to 776.
 * The page leaves the rule open. These calls take one reading of it:
 *   - a sequence of n <= L actions is kept whole;
 *   - a longer one is kept whole iff u_keep[b] < (L/n)^2, which bounds the
 *     expected n^2 attention cost of a user by 2 L^2;
 *   - otherwise it keeps exactly L actions, in their original order. These
 *     are the L positions whose (keys[row], position) pairs are smallest,
 *     comparing keys as unsigned 32-bit integers and breaking ties by the
 *     smaller position.
 * With uniform random u_keep (in [0, 1)) and keys, the kept subsequence is
 * uniformly random. The random numbers are inputs, so every call is
 * deterministic.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t batch;            /* B, number of sequences (>= 0) */
  int32_t max_seq_len;      /* N (>= 1): the length the target L is derived from */
  float alpha;              /* in [0, 2]; L = floor(N^(alpha/2)), in double precision */
} hstu_sl_desc;

/* hstu_sl_lengths (host memory only; no device work): fills new_offsets_host
 * [B+1] with the offsets after sampling, given the input offsets_host [B+1]
 * and one float u_keep_host[b] per sequence. Sequence b keeps n_b or L
 * actions, by the rule above. L itself is written to *target_len when that
 * pointer is not NULL. */
hstu_status hstu_sl_lengths(const hstu_sl_desc* desc, const int64_t* offsets_host,
                            const float* u_keep_host, int64_t* new_offsets_host,
                            int64_t* target_len);

/* hstu_sl_sample: picks and gathers the kept actions on the device.
 *   offsets/offsets_host         [B+1] input offsets (device and host copy)
 *   new_offsets/new_offsets_host [B+1] output offsets, for instance from
 *       hstu_sl_lengths. Each new length m_b must satisfy 0 <= m_b <= n_b.
 *       m_b == n_b keeps the sequence whole; a smaller m_b keeps the m_b
 *       positions with the smallest (key, position) pairs.
 *   keys       device uint32 [T_in], one random key per input row
 *              (read only for cut sequences; may be NULL if none is cut)
 *   src_index  device int64 [T_out] (T_out = new_offsets_host[B]): the global
 *              input row of output row r, increasing within each sequence
 *   x, row_bytes, out_x  optional rows to gather: out_x[r] = x[src_index[r]].
 *              Each row is row_bytes bytes (a multiple of 16). x and out_x
 *              must be 16-byte aligned. Pass NULL for x and out_x to skip.
 *   ts, out_ts optional int64 timestamps to gather the same way (NULL: skip)
 * The device offsets must hold the same values as the host copies. The
 * scratch needs fit in LDS, so there is no workspace. */
hstu_status hstu_sl_sample(int32_t batch, const int64_t* offsets_host,
                           const int64_t* new_offsets_host, const int64_t* offsets,
                           const int64_t* new_offsets, const uint32_t* keys, int64_t* src_index,
                           const void* x, int64_t row_bytes, void* out_x, const int64_t* ts,
                           int64_t* out_ts, void* stream);

/* ------------------------------------------------------------------------
 * hstu_debug_buckets (test support): writes the position and time bucket
 * indices that the attention kernels use for sequence `seq`, as int32
 * [n][n] matrices (row i = query, column j = key). Entries with j > i are
 * written as -1. It uses the same device functions as the kernels.
 * pos_bucket and time_bucket are device int32 [n*n], where n is the length
 * of sequence `seq`.
 * ---------------------------------------------------------------------- */
hstu_status hstu_debug_buckets(const hstu_attn_desc* desc, const int64_t* seq_offsets_host,
                               const int64_t* seq_offsets, const int64_t* timestamps, int32_t seq,
                               int32_t* pos_bucket, int32_t* time_bucket, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* HSTU_H_ */
