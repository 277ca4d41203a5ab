// C-ABI host layer of libhstu: argument validation (host data only, so every
// rejection happens before any HIP call), workspace carving and launch order.
// The operations are the HSTU layer's eqs. 1-3 ("What an HSTU layer changes",
// HSTU chapter) and M-FALCON candidate scoring (same chapter, "M-FALCON").
#include "hstu.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "kernels.h"

using namespace hstu;

namespace {

thread_local std::string g_err;

hstu_status fail(hstu_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

hstu_status device_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return HSTU_OK;
  return fail(HSTU_DEVICE_ERROR, "%s: %s", where, hipGetErrorString(e));
}

#define HSTU_TRY(expr, where)                                   \
  do {                                                          \
    hstu_status st_ = device_status((expr), (where));           \
    if (st_ != HSTU_OK) return st_;                             \
  } while (0)

constexpr size_t kAlign = 256;
constexpr int64_t kMaxRows = int64_t(1) << 30;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t elt_size(hstu_dtype t) { return t == HSTU_BF16 ? 2 : 4; }

// Sequential carving of the caller's workspace.
struct Carver {
  char* base;
  size_t off = 0;
  void* take(size_t bytes) {  // NULL for an empty buffer
    void* p = (base && bytes) ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  }
};

struct Jagged {
  int64_t total = 0;    // rows
  int64_t max_len = 0;  // longest sequence
  int64_t items = 0;    // query tiles for the chosen kernel
  int max_tiles = 0;    // query tiles of the longest sequence
};

hstu_status check_offsets(const int64_t* off, int B, int64_t limit_len, int tile_rows,
                          const char* name, Jagged* j) {
  *j = Jagged{};
  if (B < 0) return fail(HSTU_INVALID_ARGUMENT, "%s: batch must be >= 0 (got %d)", name, B);
  if (B == 0) return HSTU_OK;
  if (!off) return fail(HSTU_INVALID_ARGUMENT, "%s: host offsets are NULL", name);
  if (off[0] != 0) return fail(HSTU_INVALID_ARGUMENT, "%s: offsets[0] must be 0", name);
  for (int b = 0; b < B; ++b) {
    const int64_t n = off[b + 1] - off[b];
    if (n < 0) return fail(HSTU_INVALID_ARGUMENT, "%s: offsets decrease at %d", name, b);
    if (limit_len >= 0 && n > limit_len)
      return fail(HSTU_INVALID_ARGUMENT, "%s: sequence %d has length %lld > max_seq_len %lld",
                  name, b, (long long)n, (long long)limit_len);
    j->max_len = std::max(j->max_len, n);
    j->items += (n + tile_rows - 1) / tile_rows;
  }
  j->total = off[B];
  if (j->total > kMaxRows)
    return fail(HSTU_UNSUPPORTED, "%s: %lld rows exceed the supported 2^30", name,
                (long long)j->total);
  j->max_tiles = (int)((j->max_len + tile_rows - 1) / tile_rows);
  return HSTU_OK;
}

hstu_status check_attn_desc(const hstu_attn_desc* d) {
  if (!d) return fail(HSTU_INVALID_ARGUMENT, "descriptor is NULL");
  if (d->batch < 0) return fail(HSTU_INVALID_ARGUMENT, "batch must be >= 0");
  if (d->num_heads < 1 || d->num_heads > 1024)
    return fail(HSTU_INVALID_ARGUMENT, "num_heads must be in [1, 1024] (got %d)", d->num_heads);
  auto okd = [](int x) { return x == 32 || x == 64 || x == 128; };
  if (!okd(d->d_qk) || !okd(d->d_v))
    return fail(HSTU_UNSUPPORTED, "d_qk and d_v must be 32, 64 or 128 (got %d, %d)", d->d_qk,
                d->d_v);
  if (d->max_seq_len < 1) return fail(HSTU_INVALID_ARGUMENT, "max_seq_len (N) must be >= 1");
  if (d->num_pos_buckets < 1 || d->num_time_buckets < 1)
    return fail(HSTU_INVALID_ARGUMENT, "bucket counts must be >= 1");
  // a C caller may store any int in the enum field; read it as its bytes, since loading an
  // out-of-range value as the enum type is undefined in C++
  int32_t dtype_raw;
  static_assert(sizeof(dtype_raw) == sizeof(d->dtype), "hstu_dtype is a 32-bit field");
  std::memcpy(&dtype_raw, &d->dtype, sizeof(dtype_raw));
  if (dtype_raw != HSTU_F32 && dtype_raw != HSTU_BF16)
    return fail(HSTU_UNSUPPORTED, "dtype must be HSTU_F32 or HSTU_BF16 (got %d)", dtype_raw);
  return HSTU_OK;
}

hstu_status check_eps(float eps) {
  if (!(eps > 0.f) || !std::isfinite(eps))
    return fail(HSTU_INVALID_ARGUMENT, "ln_eps must be finite and > 0");
  return HSTU_OK;
}

bool uses_mfma(const hstu_attn_desc* d);
int attn_tile_rows(const hstu_attn_desc* d) { return uses_mfma(d) ? kMfmaRows : kSimpleRows; }

bool uses_mfma(const hstu_attn_desc* d) {
  return attn_mfma_supported(d->dtype == HSTU_BF16, d->d_qk, d->d_v, d->num_pos_buckets,
                             d->num_time_buckets);
}

// Workspace bytes of the per-32-key timestamp ranges (MFMA kernel only).
size_t key_range_bytes(const hstu_attn_desc* d, int64_t total_keys) {
  return uses_mfma(d) ? (size_t)key_range_slots(total_keys, d->batch) * sizeof(KeyRange) : 0;
}

hipError_t run_attention(const hstu_attn_desc* d, const AttnArgs& a, bool cand, hipStream_t s) {
  if (!uses_mfma(d)) return launch_attn_simple(a, d->dtype == HSTU_BF16, cand, s);
  // work items were planned for the MFMA kernel's tile; every caller here passes
  // equal K and V strides (d_qk == d_v), which that kernel's key-tile DMA needs,
  // and the key ranges whenever the time bias is on
  if (!attn_mfma_strides_ok(a)) return hipErrorInvalidValue;
  if (a.rab_time && a.ts_q && a.ts_k && !a.key_ranges) return hipErrorInvalidValue;
  return launch_attn_mfma(a, cand, s);
}

AttnArgs base_args(const hstu_attn_desc* d) {
  AttnArgs a{};
  a.batch = d->batch;
  a.H = d->num_heads;
  a.d_qk = d->d_qk;
  a.d_v = d->d_v;
  a.P = d->num_pos_buckets;
  a.T = d->num_time_buckets;
  a.inv_n = 1.0f / (float)d->max_seq_len;
  return a;
}

// ---------------------------------------------------------------- attention
struct AttnPlan {
  Jagged j;
  size_t ws = 0;
};

hstu_status plan_attn(const hstu_attn_desc* d, const int64_t* off_host, bool gated, AttnPlan* p) {
  hstu_status st = check_attn_desc(d);
  if (st) return st;
  st = check_offsets(off_host, d->batch, d->max_seq_len, attn_tile_rows(d), "seq_offsets", &p->j);
  if (st) return st;
  if ((int64_t)p->j.items * d->num_heads >= (int64_t(1) << 31))
    return fail(HSTU_UNSUPPORTED, "too many query tiles for one launch");
  Carver c{nullptr};
  c.take((size_t)p->j.items * sizeof(int2));
  c.take(key_range_bytes(d, p->j.total));
  if (gated) c.take((size_t)p->j.total * d->num_heads * d->d_v * sizeof(float));
  p->ws = c.off;
  return HSTU_OK;
}

// ---------------------------------------------------------------- attention backward
constexpr int kMaxBiasBins = 2048;      // P + T limit of the bias-table gradient

bool bwd_uses_mfma(const hstu_attn_desc* d) {
  return attn_bwd_mfma_supported(d->dtype == HSTU_BF16, d->d_qk, d->d_v, d->num_pos_buckets);
}
int bwd_tile_rows(const hstu_attn_desc* d) { return bwd_uses_mfma(d) ? kMfmaRows : kSimpleRows; }

struct AttnBwdPlan {
  Jagged j;
  bool mfma = false;
  size_t items = 0, ranges = 0, partial = 0, ws = 0;
};

hstu_status plan_attn_bwd(const hstu_attn_desc* d, const int64_t* off_host, AttnBwdPlan* p) {
  hstu_status st = check_attn_desc(d);
  if (st) return st;
  p->mfma = bwd_uses_mfma(d);
  st = check_offsets(off_host, d->batch, d->max_seq_len, bwd_tile_rows(d), "seq_offsets", &p->j);
  if (st) return st;
  if ((int64_t)p->j.items * d->num_heads >= (int64_t(1) << 31))
    return fail(HSTU_UNSUPPORTED, "too many tiles for one launch");
  p->items = (size_t)p->j.items * sizeof(int2);
  p->ranges = p->mfma ? (size_t)key_range_slots(p->j.total, d->batch) * sizeof(KeyRange) : 0;
  const int64_t bins = (int64_t)d->num_pos_buckets + d->num_time_buckets;
  p->partial = bins <= kMaxBiasBins ? (size_t)p->j.items * d->num_heads * bins * sizeof(float) : 0;
  p->ws = align_up(p->items) + align_up(p->ranges) + align_up(p->partial);
  return HSTU_OK;
}

// ---------------------------------------------------------------- layer
struct LayerPlan {
  Jagged j;
  size_t ws = 0;
  int64_t f1_cols = 0;
};

hstu_status check_layer_desc(const hstu_layer_desc* d) {
  if (!d) return fail(HSTU_INVALID_ARGUMENT, "descriptor is NULL");
  hstu_status st = check_attn_desc(&d->attn);
  if (st) return st;
  if (d->d_model < 8 || d->d_model % 8 != 0 || d->d_model > 65536)
    return fail(HSTU_UNSUPPORTED, "d_model must be a multiple of 8 in [8, 65536] (got %d)",
                d->d_model);
  if (d->residual != 0 && d->residual != 1)
    return fail(HSTU_INVALID_ARGUMENT, "residual must be 0 or 1");
  if (d->num_layers < 1 || d->num_layers > 4096)
    return fail(HSTU_INVALID_ARGUMENT, "num_layers must be in [1, 4096]");
  return check_eps(d->attn.ln_eps);
}

hstu_status check_weights(const hstu_layer_weights* w, int L) {
  if (!w) return fail(HSTU_INVALID_ARGUMENT, "weights array is NULL");
  for (int l = 0; l < L; ++l) {
    if (!w[l].w1 || !w[l].w2)
      return fail(HSTU_INVALID_ARGUMENT, "layer %d: w1 and w2 are required", l);
    if (!aligned16(w[l].w1) || !aligned16(w[l].w2))
      return fail(HSTU_INVALID_ARGUMENT, "layer %d: w1 and w2 must be 16-byte aligned", l);
  }
  return HSTU_OK;
}

struct LayerBufs {
  int2* items;
  KeyRange* kr;  // per 32-key timestamp ranges (MFMA kernel), else NULL
  void* uvqk;
  float* o;
  void* g;
  void* tmp;
  // bf16 MFMA path: the lo parts of the f1 output's Q and K columns (same layout as uvqk),
  // so that the causal attention forms its scores from ~16-bit Q and K; NULL otherwise
  void* qk_lo;
};

// Whether a layer's causal attention takes split (hi + lo) Q and K: the bf16 MFMA kernel.
bool layer_splits_qk(const hstu_attn_desc& a) { return uses_mfma(&a); }

void carve_layer(Carver& c, const hstu_layer_desc* d, int64_t rows, int64_t items, LayerBufs* b) {
  const hstu_attn_desc& a = d->attn;
  const size_t es = elt_size(a.dtype);
  const int64_t f1 = 2LL * a.num_heads * (a.d_v + a.d_qk);
  const int64_t hv = (int64_t)a.num_heads * a.d_v;
  b->items = (int2*)c.take((size_t)items * sizeof(int2));
  b->kr = (KeyRange*)c.take(key_range_bytes(&a, rows));
  b->uvqk = c.take((size_t)rows * f1 * es);
  b->o = (float*)c.take((size_t)rows * hv * sizeof(float));
  b->g = c.take((size_t)rows * hv * es);
  b->tmp = d->num_layers > 1 ? c.take((size_t)rows * d->d_model * es) : nullptr;
  b->qk_lo = layer_splits_qk(a) ? c.take((size_t)rows * f1 * es) : nullptr;
}

hstu_status plan_layer(const hstu_layer_desc* d, const int64_t* off_host, LayerPlan* p) {
  hstu_status st = check_layer_desc(d);
  if (st) return st;
  st = check_offsets(off_host, d->attn.batch, d->attn.max_seq_len, attn_tile_rows(&d->attn),
                     "seq_offsets", &p->j);
  if (st) return st;
  if ((int64_t)p->j.items * d->attn.num_heads >= (int64_t(1) << 31))
    return fail(HSTU_UNSUPPORTED, "too many query tiles for one launch");
  Carver c{nullptr};
  LayerBufs b;
  carve_layer(c, d, p->j.total, p->j.items, &b);
  p->ws = c.off;
  p->f1_cols = 2LL * d->attn.num_heads * (d->attn.d_v + d->attn.d_qk);
  return HSTU_OK;
}

// Views into the f1 output [rows, U|V|Q|K].
struct UVQK {
  const char* u;
  const char* v;
  const char* q;
  const char* k;
  int64_t ld;
};
UVQK split_view(const void* base, const hstu_attn_desc& a) {
  const size_t es = elt_size(a.dtype);
  const int64_t hv = (int64_t)a.num_heads * a.d_v, hq = (int64_t)a.num_heads * a.d_qk;
  const char* p = (const char*)base;
  return UVQK{p, p + hv * es, p + 2 * hv * es, p + (2 * hv + hq) * es, 2 * hv + 2 * hq};
}

// Work items and key ranges of the causal attention; they depend on the offsets
// and timestamps only, so one call serves every layer.
hstu_status plan_causal(const hstu_attn_desc& a, const int64_t* off_dev, const int64_t* ts,
                        const Jagged& j, const LayerBufs& b, hipStream_t s) {
  HSTU_TRY(launch_plan(off_dev, a.batch, attn_tile_rows(&a), j.max_tiles, b.items, (int)j.items,
                       ts && b.kr ? ts : nullptr, j.max_len, b.kr, s),
           "tile planner and key ranges");
  return HSTU_OK;
}

// One layer over `rows` jagged rows: f1 -> causal attention -> LN gate -> f2.
// The work items and key ranges in b come from plan_causal.
hstu_status layer_once(const hstu_layer_desc* d, const int64_t* off_dev, const int64_t* ts,
                       const Jagged& j, const void* x, const hstu_layer_weights& w, void* y,
                       const LayerBufs& b, hipStream_t s, bool f1_only) {
  const hstu_attn_desc& a = d->attn;
  const int bf = a.dtype == HSTU_BF16;
  const int64_t rows = j.total;
  const int64_t f1 = 2LL * a.num_heads * (a.d_v + a.d_qk);
  const int hv = a.num_heads * a.d_v;
  const int hq = a.num_heads * a.d_qk;
  void* lo = f1_only ? nullptr : b.qk_lo;
  // f1 alone (the last history layer of M-FALCON): the candidates read only its keys and
  // values, so only the V and K columns are computed where they are whole GEMM tiles
  if (f1_only && bf &&
      launch_gemm_2cols(x, d->d_model, w.w1, d->d_model, w.b1, b.uvqk, f1, rows, d->d_model, 1,
                        hv, hv, 2 * hv + hq, hq, s) == hipSuccess)
    return HSTU_OK;
  // with split scores the attention takes its queries pre-scaled (kQueryPrescale)
  const int q_c1 = lo ? 2 * hv + hq : 0;
  HSTU_TRY(launch_gemm(x, d->d_model, w.w1, d->d_model, w.b1, nullptr, 0, b.uvqk, f1, rows, (int)f1,
                       d->d_model, 1, bf, s, lo, 2 * hv, 2 * hv, q_c1, kQueryPrescale),
           "f1 projection");
  if (f1_only) return HSTU_OK;
  const UVQK vw = split_view(b.uvqk, a);
  AttnArgs aa = base_args(&a);
  aa.q = vw.q;
  aa.k = vw.k;
  aa.v = vw.v;
  if (lo) {
    const UVQK lw = split_view(lo, a);
    aa.q_lo = lw.q;
    aa.k_lo = lw.k;
  }
  aa.ld_q = aa.ld_k = aa.ld_v = vw.ld;
  aa.out = b.o;
  aa.ld_o = hv;
  aa.out_f32 = 1;
  aa.q_offsets = aa.k_offsets = off_dev;
  aa.ts_q = aa.ts_k = ts;
  aa.rab_pos = w.rab_pos;
  aa.rab_time = w.rab_time;
  aa.key_ranges = (ts && w.rab_time) ? b.kr : nullptr;
  aa.items = b.items;
  aa.n_items = (int)j.items;
  HSTU_TRY(run_attention(&a, aa, false, s), "attention");
  if (ln_gate_f2_supported(hv, d->d_model, bf, w.w2, w.ln_gamma, w.ln_beta)) {
    // narrow layers: the gated rows stay in LDS
    HSTU_TRY(launch_ln_gate_f2(b.o, hv, 1, 0, vw.u, vw.ld, w.ln_gamma, w.ln_beta, a.ln_eps, w.w2,
                               hv, w.b2, d->residual ? x : nullptr, d->d_model, y, d->d_model,
                               rows, hv, d->d_model, s),
             "layer norm gate and f2 projection");
    return HSTU_OK;
  }
  HSTU_TRY(launch_ln_gate(b.o, hv, 1, 0, vw.u, vw.ld, w.ln_gamma, w.ln_beta, a.ln_eps, b.g, hv, rows,
                          hv, bf, s),
           "layer norm gate");
  HSTU_TRY(launch_gemm(b.g, hv, w.w2, hv, w.b2, d->residual ? x : nullptr, d->d_model, y,
                       d->d_model, rows, d->d_model, hv, 0, bf, s),
           "f2 projection");
  return HSTU_OK;
}

// ---------------------------------------------------------------- M-FALCON
// The history pass of M-FALCON produces a cache that the candidate pass reads:
// per layer, the f1 output over the history (its K and V columns are the keys
// and values the candidates attend to), and the per-32-key timestamp ranges.
// mfalcon_score runs both passes with the cache inside its workspace;
// mfalcon_history and mfalcon_score_cached let a caller keep the cache across
// requests for the same users.
struct MfPlan {
  Jagged hist;
  int64_t cand_total = 0;
  int kv_splits = 1;          // key-range splits of the candidate attention (MFMA kernel only)
  int64_t keys_per_split = 0;
  size_t cache = 0;           // bytes of the history cache
  size_t hist_ws = 0;         // history-pass workspace
  size_t cand_ws = 0;         // candidate-pass workspace
};

constexpr int64_t kKeysPerSplit = 2048;  // history keys per candidate-attention workgroup
constexpr int kMaxSplits = 16;

struct MfCache {
  std::vector<void*> uvqk;  // per layer f1 output over the history [n_h, f1] (K/V cache)
  KeyRange* kr;             // timestamp ranges of the history keys (MFMA kernel), else NULL
};
struct MfHistBufs {
  int2* items;
  float* o;
  void* g;
  void* hx[2];
  void* qk_lo;  // lo parts of Q and K for the history's full layers (0..L-2)
};
struct MfCandBufs {
  void* c_uvqk;
  float* c_o;
  float* c_self;  // self weights of the candidates, [rows][H] (MFMA attention kernel)
  void* c_g;
  void* cx[2];
};

void carve_cache(Carver& c, const mfalcon_desc* d, const MfPlan& p, MfCache* b) {
  const hstu_layer_desc& ld = d->layer;
  const hstu_attn_desc& a = ld.attn;
  const int64_t f1 = 2LL * a.num_heads * (a.d_v + a.d_qk);
  const int64_t nh = p.hist.total;
  b->uvqk.assign(ld.num_layers, nullptr);
  for (int l = 0; l < ld.num_layers; ++l) b->uvqk[l] = c.take((size_t)nh * f1 * elt_size(a.dtype));
  b->kr = (KeyRange*)c.take(key_range_bytes(&a, nh));
}

void carve_hist_ws(Carver& c, const mfalcon_desc* d, const MfPlan& p, MfHistBufs* b) {
  const hstu_layer_desc& ld = d->layer;
  const hstu_attn_desc& a = ld.attn;
  const size_t es = elt_size(a.dtype);
  const int64_t hv = (int64_t)a.num_heads * a.d_v;
  const int64_t nh = p.hist.total;
  b->items = (int2*)c.take((size_t)p.hist.items * sizeof(int2));
  b->o = (float*)c.take((size_t)nh * hv * sizeof(float));
  b->g = c.take((size_t)nh * hv * es);
  b->hx[0] = ld.num_layers > 1 ? c.take((size_t)nh * ld.d_model * es) : nullptr;
  b->hx[1] = ld.num_layers > 2 ? c.take((size_t)nh * ld.d_model * es) : nullptr;
  const int64_t f1 = 2LL * a.num_heads * (a.d_v + a.d_qk);
  b->qk_lo = ld.num_layers > 1 && layer_splits_qk(a) ? c.take((size_t)nh * f1 * es) : nullptr;
}

// The candidate pass keeps up to kInFlight microbatches in flight (fewer when they would
// exceed kGroupRowCap rows, never less than one): their work is issued together, one
// launch per step for all of them (the rows of one group, in global candidate order), on
// the caller's stream. Each microbatch's candidates are computed exactly as they would be
// alone (every output row has its own fixed reduction order), so the grouping only sets
// how much work one launch holds: one microbatch of ~1k candidates leaves most of the
// device idle in every step, and a group of 16 lets each launch run several rounds of
// workgroups, so that the tail of one round is a small part of it (4 -> 16 in flight:
// 0.389 -> 0.309 ms on 16,384 candidates against a 4,096-key history). The workspace
// holds the working set of one group (~10 KB per candidate row at d_model 512, 8 heads).
constexpr int kInFlight = 16;
constexpr int64_t kGroupRowCap = 65536;
int64_t group_rows(const mfalcon_desc* d, const MfPlan& p) {
  const int64_t mb = d->microbatch;
  const int64_t n = std::max<int64_t>(1, std::min<int64_t>(kInFlight, kGroupRowCap / mb));
  return std::max<int64_t>(1, std::min<int64_t>(mb * n, p.cand_total));
}

void carve_cand_ws(Carver& c, const mfalcon_desc* d, const MfPlan& p, MfCandBufs* b) {
  const hstu_layer_desc& ld = d->layer;
  const hstu_attn_desc& a = ld.attn;
  const size_t es = elt_size(a.dtype);
  const int64_t f1 = 2LL * a.num_heads * (a.d_v + a.d_qk);
  const int64_t hv = (int64_t)a.num_heads * a.d_v;
  const int64_t m = group_rows(d, p);
  b->c_uvqk = c.take((size_t)m * f1 * es);
  b->c_o = (float*)c.take((size_t)p.kv_splits * m * hv * sizeof(float));
  b->c_self = uses_mfma(&a) ? (float*)c.take((size_t)m * a.num_heads * sizeof(float)) : nullptr;
  b->c_g = c.take((size_t)m * hv * es);
  b->cx[0] = ld.num_layers > 1 ? c.take((size_t)m * ld.d_model * es) : nullptr;
  b->cx[1] = ld.num_layers > 2 ? c.take((size_t)m * ld.d_model * es) : nullptr;
}

// The history half of the plan (cand offsets may be NULL: then no candidate sizes).
hstu_status plan_mfalcon(const mfalcon_desc* d, const int64_t* hoff, const int64_t* coff,
                         MfPlan* p) {
  if (!d) return fail(HSTU_INVALID_ARGUMENT, "descriptor is NULL");
  hstu_status st = check_layer_desc(&d->layer);
  if (st) return st;
  if (d->microbatch < 1) return fail(HSTU_INVALID_ARGUMENT, "microbatch must be >= 1");
  const hstu_attn_desc& a = d->layer.attn;
  st = check_offsets(hoff, a.batch, a.max_seq_len, attn_tile_rows(&a), "hist_offsets", &p->hist);
  if (st) return st;
  if (coff) {
    Jagged cj;
    st = check_offsets(coff, a.batch, -1, 1, "cand_offsets", &cj);
    if (st) return st;
    for (int b = 0; b < a.batch; ++b) {
      const int64_t nh = hoff[b + 1] - hoff[b], nc = coff[b + 1] - coff[b];
      if (nc > 0 && nh + 1 > a.max_seq_len)
        return fail(HSTU_INVALID_ARGUMENT,
                    "user %d: history %lld plus the candidate exceeds max_seq_len %d", b,
                    (long long)nh, a.max_seq_len);
    }
    p->cand_total = cj.total;
  }
  // The MFMA kernel splits the history into key ranges of kKeysPerSplit (more when
  // the history is long), so that a microbatch of ~1k candidates still fills the
  // device. The geometry depends on the history lengths only.
  if (uses_mfma(&a) && p->hist.max_len > kKeysPerSplit) {
    p->kv_splits = (int)std::min<int64_t>(kMaxSplits,
                                          (p->hist.max_len + kKeysPerSplit - 1) / kKeysPerSplit);
    p->keys_per_split = ((p->hist.max_len + p->kv_splits - 1) / p->kv_splits + 63) / 64 * 64;
  }
  if ((int64_t)p->hist.items * a.num_heads >= (int64_t(1) << 31))
    return fail(HSTU_UNSUPPORTED, "too many history tiles for one launch");
  Carver c{nullptr};
  MfCache cb;
  carve_cache(c, d, *p, &cb);
  p->cache = c.off;
  Carver h{nullptr};
  MfHistBufs hb;
  carve_hist_ws(h, d, *p, &hb);
  p->hist_ws = h.off;
  Carver k{nullptr};
  MfCandBufs kb;
  carve_cand_ws(k, d, *p, &kb);
  p->cand_ws = k.off;
  return HSTU_OK;
}

hstu_status check_ws(const void* ws, size_t have, size_t need, const char* what) {
  if (have < need || (!ws && need))
    return fail(HSTU_WORKSPACE_TOO_SMALL, "%s needs %zu bytes (got %zu)", what, need, have);
  if (((uintptr_t)ws & (kAlign - 1)) != 0)
    return fail(HSTU_INVALID_ARGUMENT, "%s must be 256-byte aligned", what);
  return HSTU_OK;
}

// History pass: layers 0..L-2 in full; layer L-1 only needs its K and V. Every
// layer's f1 output stays in the cache.
hstu_status run_history(const mfalcon_desc* d, const MfPlan& p, const int64_t* hist_offsets,
                        const int64_t* hist_ts, const void* hist_x,
                        const hstu_layer_weights* weights, const MfCache& cache,
                        const MfHistBufs& hb, hipStream_t s) {
  if (p.hist.total == 0) return HSTU_OK;
  const hstu_layer_desc& ld = d->layer;
  const int L = ld.num_layers;
  LayerBufs lb{};
  lb.items = hb.items;
  lb.kr = cache.kr;
  lb.o = hb.o;
  lb.g = hb.g;
  lb.qk_lo = hb.qk_lo;
  // the history's work items (layers 0..L-2) and key ranges (every layer, candidates included)
  hstu_status st = plan_causal(ld.attn, hist_offsets, hist_ts, p.hist, lb, s);
  if (st) return st;
  const void* in = hist_x;
  for (int l = 0; l < L; ++l) {
    lb.uvqk = cache.uvqk[l];
    void* out = (l < L - 1) ? hb.hx[l % 2] : nullptr;
    st = layer_once(&ld, hist_offsets, hist_ts, p.hist, in, weights[l], out, lb, s, l == L - 1);
    if (st) return st;
    in = out;
  }
  return HSTU_OK;
}

// Candidate microbatches, in global candidate order, against a history cache.
hstu_status run_candidates(const mfalcon_desc* d, const MfPlan& p, const int64_t* hist_offsets,
                           const int64_t* hist_ts, const MfCache& cache,
                           const int64_t* cand_offsets_host, const int64_t* cand_offsets,
                           const int64_t* cand_ts, const void* cand_x,
                           const hstu_layer_weights* weights, const float* w_head, void* cand_out,
                           float* cand_logit, const MfCandBufs* bufs, hipStream_t s0) {
  const hstu_layer_desc& ld = d->layer;
  const hstu_attn_desc& a = ld.attn;
  const int L = ld.num_layers;
  const int bf = a.dtype == HSTU_BF16;
  const size_t es = elt_size(a.dtype);
  const int hv = a.num_heads * a.d_v;
  const int dm = ld.d_model;
  const int B = a.batch;
  const int64_t gm = group_rows(d, p);
  const hipStream_t s = s0;
  const MfCandBufs& b = *bufs;
  for (int64_t m0 = 0; m0 < p.cand_total; m0 += gm) {
    const int64_t m1 = std::min(m0 + gm, p.cand_total);
    const int64_t rows = m1 - m0;
    // users whose candidate range overlaps [m0, m1)
    int ub = (int)(std::upper_bound(cand_offsets_host, cand_offsets_host + B + 1, m0) -
                   cand_offsets_host) - 1;
    int ue = (int)(std::lower_bound(cand_offsets_host, cand_offsets_host + B + 1, m1) -
                   cand_offsets_host);  // one past the last overlapping user
    ub = std::max(ub, 0);
    ue = std::min(ue, B);
    int64_t max_rows = 0;
    for (int u = ub; u < ue; ++u) {
      const int64_t cs = std::max(cand_offsets_host[u], m0);
      const int64_t ce = std::min(cand_offsets_host[u + 1], m1);
      max_rows = std::max(max_rows, ce - cs);
    }
    const void* in = (const char*)cand_x + (size_t)m0 * dm * es;
    for (int l = 0; l < L; ++l) {
      const hstu_layer_weights& w = weights[l];
      void* out = (l == L - 1) ? (void*)((char*)cand_out + (size_t)m0 * dm * es) : b.cx[l % 2];
      const int64_t f1 = 2LL * a.num_heads * (a.d_v + a.d_qk);
      // the MFMA kernel's candidate mode takes its queries pre-scaled (kQueryPrescale)
      const int q_c1 = uses_mfma(&a) ? 2 * hv + a.num_heads * a.d_qk : 0;
      HSTU_TRY(launch_gemm(in, dm, w.w1, dm, w.b1, nullptr, 0, b.c_uvqk, f1, rows, (int)f1, dm, 1,
                           bf, s, nullptr, 0, 2 * hv, q_c1, kQueryPrescale),
               "candidate f1 projection");
      const UVQK cv = split_view(b.c_uvqk, a);
      const UVQK hvw = split_view(cache.uvqk[l], a);
      AttnArgs aa = base_args(&a);
      aa.q = cv.q;
      aa.ld_q = cv.ld;
      aa.kc = cv.k;
      aa.vc = cv.v;
      aa.ld_kc = aa.ld_vc = cv.ld;
      aa.k = hvw.k;
      aa.v = hvw.v;
      aa.ld_k = aa.ld_v = hvw.ld;
      aa.out = b.c_o;
      aa.ld_o = hv;
      aa.out_f32 = 1;
      aa.q_offsets = cand_offsets;
      aa.k_offsets = hist_offsets;
      aa.ts_q = cand_ts;
      aa.ts_k = hist_ts;
      aa.rab_pos = w.rab_pos;
      aa.rab_time = w.rab_time;
      aa.key_ranges = (hist_ts && w.rab_time) ? cache.kr : nullptr;  // unread when no history
      aa.row_begin = m0;
      aa.row_end = m1;
      aa.max_user_rows = max_rows;
      // key-range splits of the history: fixed by the history lengths alone, so a
      // candidate's reduction order never depends on the rows around it
      aa.kv_splits = p.kv_splits;
      aa.keys_per_split = p.keys_per_split;
      aa.part_stride = rows * hv;
      // the MFMA kernel leaves the candidates' own values to the layer norm
      aa.self_w = b.c_self;
      for (int u0 = ub; u0 < ue; u0 += 65535) {
        aa.user_begin = u0;
        aa.n_users = std::min(ue - u0, 65535);
        HSTU_TRY(run_attention(&a, aa, true, s), "candidate attention");
      }
      if (ln_gate_f2_supported(hv, dm, bf, w.w2, w.ln_gamma, w.ln_beta)) {
        HSTU_TRY(launch_ln_gate_f2(b.c_o, hv, aa.kv_splits, aa.part_stride, cv.u, cv.ld,
                                   w.ln_gamma, w.ln_beta, a.ln_eps, w.w2, hv, w.b2,
                                   ld.residual ? in : nullptr, dm, out, dm, rows, hv, dm, s,
                                   aa.self_w, cv.v, cv.ld, a.d_v),
                 "candidate layer norm gate and f2 projection");
      } else {
        HSTU_TRY(launch_ln_gate(b.c_o, hv, aa.kv_splits, aa.part_stride, cv.u, cv.ld, w.ln_gamma,
                                w.ln_beta, a.ln_eps, b.c_g, hv, rows, hv, bf, s, aa.self_w, cv.v,
                                cv.ld, a.d_v),
                 "candidate layer norm gate");
        HSTU_TRY(launch_gemm(b.c_g, hv, w.w2, hv, w.b2, ld.residual ? in : nullptr, dm, out, dm,
                             rows, dm, hv, 0, bf, s),
                 "candidate f2 projection");
      }
      in = out;
    }
  }
  // the logits of every candidate in one launch (each row's dot product is independent
  // of the microbatch it was scored in)
  if (cand_logit)
    HSTU_TRY(launch_rowdot(cand_out, dm, w_head, cand_logit, p.cand_total, dm, bf, s0),
             "candidate logit");
  return HSTU_OK;
}

hstu_status check_history_args(const hstu_layer_weights* weights, int L, const MfPlan& p,
                               const void* hist_offsets, const void* hist_x) {
  hstu_status st = check_weights(weights, L);
  if (st) return st;
  if (p.hist.total > 0 && (!hist_offsets || !hist_x))
    return fail(HSTU_INVALID_ARGUMENT, "hist_offsets and hist_x are required");
  if (hist_x && !aligned16(hist_x))
    return fail(HSTU_INVALID_ARGUMENT, "activation pointers must be 16-byte aligned");
  return HSTU_OK;
}

hstu_status check_candidate_args(const MfPlan& p, const int64_t* hist_offsets,
                                 const int64_t* hist_ts, const int64_t* cand_offsets,
                                 const int64_t* cand_ts, const void* cand_x, const void* cand_out,
                                 const float* cand_logit, const float* w_head) {
  if ((hist_ts == nullptr) != (cand_ts == nullptr))
    return fail(HSTU_INVALID_ARGUMENT, "hist_ts and cand_ts must both be set or both be NULL");
  if (!hist_offsets || !cand_offsets)
    return fail(HSTU_INVALID_ARGUMENT, "device offsets are required");
  if (!cand_x || !cand_out) return fail(HSTU_INVALID_ARGUMENT, "cand_x and cand_out are required");
  if (!aligned16(cand_x) || !aligned16(cand_out))
    return fail(HSTU_INVALID_ARGUMENT, "activation pointers must be 16-byte aligned");
  if (cand_logit && !w_head) return fail(HSTU_INVALID_ARGUMENT, "cand_logit needs w_head");
  (void)p;
  return HSTU_OK;
}

// ---------------------------------------------------------------- layer backward
// Gradients of a stack of HSTU layers (eqs. 1-3). The forward pass is recomputed:
// the inputs of layers 1..L-1 are kept in the workspace, and each layer's f1
// pre-activation, attention output and gate are recomputed just before its
// backward. The weight gradients reduce over tokens; they are GEMMs of transposed
// row-major activations, split over the token range when the output has few tiles
// (fp32 partials added in a fixed order).
struct LayerBwdPlan {
  Jagged j;
  int64_t Tp = 0;                // rows padded to a multiple of 32
  int split1 = 1, split2 = 1;    // split-K of dW1 and dW2
  int64_t ks1 = 0, ks2 = 0;
  int ln_blocks = 0;
  bool bias_ok = false;          // P + T small enough for the bias-table gradient
  size_t ws = 0;
};

struct LayerBwdBufs {
  int2* items;
  KeyRange* kr;
  char* xs;       // inputs of layers 1..L-1
  float* z1;      // f1 pre-activation (fp32)
  void* uvqk;     // SiLU(z1)
  float* o;       // attention output (fp32)
  void* g;        // gated value G
  void* dg;       // dL/dG
  void* d_o;      // dL/d(attention output)
  void* dact;     // dL/d[U|V|Q|K], then dL/dz1 in place
  void* dyb[2];   // dL/dX of inner layers (ping-pong)
  void* ta;       // transposed operands of the weight-gradient GEMMs
  void* tb;
  void* w1t;
  void* w2t;
  float* wpart;   // split-K partials
  float* bpart;   // bias-table partials
  float* lnpart;  // dgamma, dbeta partials
  float* cpart;   // column-sum partials
};

void split_k(int64_t M, int64_t N, int64_t K, bool bf, int* splits, int64_t* ks) {
  if (!bf || K <= 0) {
    *splits = 1;
    *ks = K;
    return;
  }
  const int64_t tiles = ((M + 63) / 64) * ((N + 63) / 64);
  int64_t sp = std::max<int64_t>(1, 512 / std::max<int64_t>(tiles, 1));
  sp = std::min<int64_t>(sp, std::max<int64_t>(1, K / 256));
  int64_t k = (K + sp - 1) / sp;
  k = (k + 63) / 64 * 64;  // whole pipeline stages of either GEMM tile shape
  *splits = (int)((K + k - 1) / k);
  *ks = k;
}

void carve_layer_bwd(Carver& c, const hstu_layer_desc* d, const LayerBwdPlan& p, LayerBwdBufs* b) {
  const hstu_attn_desc& a = d->attn;
  const size_t es = elt_size(a.dtype);
  const int64_t T = p.j.total, F1 = 2LL * a.num_heads * (a.d_v + a.d_qk);
  const int64_t hv = (int64_t)a.num_heads * a.d_v, dm = d->d_model;
  const bool bf = a.dtype == HSTU_BF16;
  b->items = (int2*)c.take((size_t)p.j.items * sizeof(int2));
  b->kr = (KeyRange*)c.take(key_range_bytes(&a, T));
  b->xs = (char*)c.take((size_t)(d->num_layers - 1) * T * dm * es);
  b->z1 = (float*)c.take((size_t)T * F1 * 4);
  b->uvqk = c.take((size_t)T * F1 * es);
  b->o = (float*)c.take((size_t)T * hv * 4);
  b->g = c.take((size_t)T * hv * es);
  b->dg = c.take((size_t)T * hv * es);
  b->d_o = c.take((size_t)T * hv * es);
  b->dact = c.take((size_t)T * F1 * es);
  for (int i = 0; i < 2; ++i) b->dyb[i] = c.take(d->num_layers > 1 ? (size_t)T * dm * es : 0);
  // transposed activations: only the fp32 weight gradients use them (bf16 reads rows)
  b->ta = c.take(bf ? 0 : (size_t)std::max(dm, F1) * p.Tp * es);
  b->tb = c.take(bf ? 0 : (size_t)std::max(hv, dm) * p.Tp * es);
  b->w1t = c.take((size_t)dm * F1 * es);
  b->w2t = c.take((size_t)hv * dm * es);
  const int64_t wp = std::max<int64_t>(p.split1 > 1 ? p.split1 * F1 * dm : 0,
                                       p.split2 > 1 ? p.split2 * dm * hv : 0);
  b->wpart = (float*)c.take(bf ? (size_t)wp * 4 : 0);
  b->bpart = (float*)c.take(p.bias_ok ? (size_t)p.j.items * a.num_heads *
                                            (a.num_pos_buckets + a.num_time_buckets) * 4
                                      : 0);
  b->lnpart = (float*)c.take((size_t)2 * p.ln_blocks * hv * 4);
  b->cpart = (float*)c.take((size_t)colsum_chunks(T) * std::max(F1, dm) * 4);
}

hstu_status plan_layer_bwd(const hstu_layer_desc* d, const int64_t* off_host, LayerBwdPlan* p) {
  hstu_status st = check_layer_desc(d);
  if (st) return st;
  const hstu_attn_desc& a = d->attn;
  if ((int64_t)a.num_heads * a.d_v > 1024)
    return fail(HSTU_UNSUPPORTED, "the layer backward needs H*d_v <= 1024");
  if (attn_tile_rows(&a) != bwd_tile_rows(&a))
    return fail(HSTU_UNSUPPORTED, "attention forward and backward disagree on the tile");
  st = check_offsets(off_host, a.batch, a.max_seq_len, attn_tile_rows(&a), "seq_offsets", &p->j);
  if (st) return st;
  if ((int64_t)p->j.items * a.num_heads >= (int64_t(1) << 31))
    return fail(HSTU_UNSUPPORTED, "too many query tiles for one launch");
  const bool bf = a.dtype == HSTU_BF16;
  const int64_t T = p->j.total, F1 = 2LL * a.num_heads * (a.d_v + a.d_qk);
  const int64_t hv = (int64_t)a.num_heads * a.d_v, dm = d->d_model;
  p->Tp = (T + 31) / 32 * 32;
  split_k(F1, dm, bf ? T : p->Tp, bf, &p->split1, &p->ks1);
  split_k(dm, hv, bf ? T : p->Tp, bf, &p->split2, &p->ks2);
  p->ln_blocks = ln_gate_bwd_blocks(T);
  p->bias_ok = (int64_t)a.num_pos_buckets + a.num_time_buckets <= kMaxBiasBins;
  Carver c{nullptr};
  LayerBwdBufs b;
  carve_layer_bwd(c, d, *p, &b);
  p->ws = c.off;
  return HSTU_OK;
}

// dW [M, N] (fp32) = A [M, K] W [N, K]^T, both operands transposed activations.
// dW[M, N] = sum over the T rows of A[t, m] B[t, n] (bf16 row-major activations),
// split over rows into fp32 partials added in a fixed order when splits > 1
hstu_status weight_grad_tn(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M,
                           int N, int64_t T, int splits, int64_t ks, float* wpart, float* out,
                           hipStream_t s) {
  if (splits <= 1) {
    HSTU_TRY(launch_gemm_tn(A, lda, B, ldb, out, N, (int)M, N, T, 1, T, 0, s), "weight gradient");
    return HSTU_OK;
  }
  HSTU_TRY(launch_gemm_tn(A, lda, B, ldb, wpart, N, (int)M, N, T, splits, ks, M * N, s),
           "weight gradient");
  HSTU_TRY(launch_sum_rows(wpart, M * N, splits, M * N, out, s), "split-K sum");
  return HSTU_OK;
}

// The same from transposed copies (fp32: A [M, K] and W [N, K], K contiguous).
hstu_status weight_grad(const void* A, const void* W, int64_t M, int N, int64_t K, int splits,
                        int64_t ks, bool bf, float* wpart, float* out, hipStream_t s) {
  if (splits <= 1) {
    HSTU_TRY(launch_gemm_ex(A, K, W, K, nullptr, nullptr, 0, out, N, M, N, (int)K, 0, bf, 1, 1, K, 0,
                            nullptr, s),
             "weight gradient");
    return HSTU_OK;
  }
  HSTU_TRY(launch_gemm_ex(A, K, W, K, nullptr, nullptr, 0, wpart, N, M, N, (int)K, 0, bf, 1, splits,
                          ks, M * N, nullptr, s),
           "weight gradient");
  HSTU_TRY(launch_sum_rows(wpart, M * N, splits, M * N, out, s), "split-K sum");
  return HSTU_OK;
}

// Zero gradients of one layer (no tokens).
hstu_status zero_layer_grads(const hstu_layer_desc* d, const hstu_layer_grads* g, hipStream_t s) {
  const hstu_attn_desc& a = d->attn;
  const int64_t F1 = 2LL * a.num_heads * (a.d_v + a.d_qk);
  const int64_t hv = (int64_t)a.num_heads * a.d_v, dm = d->d_model;
  const std::pair<float*, int64_t> all[] = {{g->dw1, F1 * dm}, {g->db1, F1}, {g->dw2, dm * hv},
                                            {g->db2, dm}, {g->d_ln_gamma, hv}, {g->d_ln_beta, hv}};
  for (const auto& z : all) HSTU_TRY(launch_sum_rows(nullptr, 0, 0, z.second, z.first, s), "zero");
  HSTU_TRY(launch_bias_grad_reduce(nullptr, 0, a.num_heads, a.num_pos_buckets, a.num_time_buckets,
                                   g->d_rab_pos, g->d_rab_time, s),
           "zero");
  return HSTU_OK;
}

// Backward of one layer: reads its input xl and dL/dY, writes dL/dX (if dX) and the
// parameter gradients in g (each pointer optional).
hstu_status layer_bwd_once(const hstu_layer_desc* d, const LayerBwdPlan& p, const int64_t* off,
                           const int64_t* ts, const void* xl, const hstu_layer_weights& w,
                           const hstu_layer_grads* g, const void* dY, void* dX,
                           const LayerBwdBufs& b, hipStream_t s) {
  const hstu_attn_desc& a = d->attn;
  const int bf = a.dtype == HSTU_BF16;
  const int64_t T = p.j.total, F1 = 2LL * a.num_heads * (a.d_v + a.d_qk);
  const int hv = a.num_heads * a.d_v, dm = d->d_model;
  const hstu_layer_grads none{};
  if (!g) g = &none;
  // forward pieces: z1, SiLU(z1), attention output, gate
  // (bf16: the GEMM writes SiLU(z1) too)
  // (the attention here takes bf16 scores: the attention backward reads the same Q and K)
  HSTU_TRY(launch_gemm_ex(xl, dm, w.w1, dm, w.b1, nullptr, 0, b.z1, F1, T, (int)F1, dm, 0, bf, 1, 1,
                          dm, 0, bf ? b.uvqk : nullptr, s),
           "f1 pre-activation");
  if (!bf) HSTU_TRY(launch_silu_act(b.z1, F1, b.uvqk, F1, T, (int)F1, bf, s), "f1 activation");
  const UVQK vw = split_view(b.uvqk, a);
  AttnArgs aa = base_args(&a);
  aa.q = vw.q;
  aa.k = vw.k;
  aa.v = vw.v;
  aa.ld_q = aa.ld_k = aa.ld_v = vw.ld;
  aa.out = b.o;
  aa.ld_o = hv;
  aa.out_f32 = 1;
  aa.q_offsets = aa.k_offsets = off;
  aa.ts_q = aa.ts_k = ts;
  aa.rab_pos = w.rab_pos;
  aa.rab_time = w.rab_time;
  aa.key_ranges = (ts && w.rab_time) ? b.kr : nullptr;
  aa.items = b.items;
  aa.n_items = (int)p.j.items;
  HSTU_TRY(run_attention(&a, aa, false, s), "attention");
  HSTU_TRY(launch_ln_gate(b.o, hv, 1, 0, vw.u, vw.ld, w.ln_gamma, w.ln_beta, a.ln_eps, b.g, hv, T,
                          hv, bf, s),
           "layer norm gate");
  // f2: dG = dY W2, dW2 = dY^T G, db2 = column sums of dY
  HSTU_TRY(launch_transpose(w.w2, hv, b.w2t, dm, dm, dm, hv, bf, s), "transpose");
  HSTU_TRY(launch_gemm_ex(dY, dm, b.w2t, dm, nullptr, nullptr, 0, b.dg, hv, T, hv, dm, 0, bf, 0, 1,
                          dm, 0, nullptr, s),
           "dG");
  hstu_status st;
  if (g->dw2 && bf) {
    if ((st = weight_grad_tn(dY, dm, b.g, hv, dm, hv, T, p.split2, p.ks2, b.wpart, g->dw2, s)))
      return st;
  } else if (g->dw2) {
    HSTU_TRY(launch_transpose(dY, dm, b.ta, p.Tp, T, p.Tp, dm, bf, s), "transpose");
    HSTU_TRY(launch_transpose(b.g, hv, b.tb, p.Tp, T, p.Tp, hv, bf, s), "transpose");
    if ((st = weight_grad(b.ta, b.tb, dm, hv, p.Tp, p.split2, p.ks2, bf, b.wpart, g->dw2, s)))
      return st;
  }
  HSTU_TRY(launch_colsum(dY, dm, T, dm, bf, b.cpart, g->db2, s), "db2");
  // gate and norm
  const UVQK dw = split_view(b.dact, a);
  float* pg = b.lnpart;
  float* pb = b.lnpart + (size_t)p.ln_blocks * hv;
  HSTU_TRY(launch_ln_gate_bwd(b.o, hv, vw.u, vw.ld, w.ln_gamma, w.ln_beta, a.ln_eps, b.dg, hv, b.d_o,
                              hv, const_cast<char*>(dw.u), dw.ld, pg, pb, T, hv, bf, s),
           "gate backward");
  HSTU_TRY(launch_sum_rows(pg, hv, p.ln_blocks, hv, g->d_ln_gamma, s), "dgamma");
  HSTU_TRY(launch_sum_rows(pb, hv, p.ln_blocks, hv, g->d_ln_beta, s), "dbeta");
  // attention
  const bool want_bias = g->d_rab_pos || g->d_rab_time;
  if (want_bias && !p.bias_ok)
    return fail(HSTU_UNSUPPORTED, "bias-table gradients need P + T <= %d", kMaxBiasBins);
  AttnBwdArgs ba{};
  ba.q = vw.q;
  ba.k = vw.k;
  ba.v = vw.v;
  ba.dout = b.d_o;
  ba.dq = const_cast<char*>(dw.q);
  ba.dk = const_cast<char*>(dw.k);
  ba.dv = const_cast<char*>(dw.v);
  ba.ld_q = ba.ld_k = ba.ld_v = ba.ld_dq = ba.ld_dk = ba.ld_dv = vw.ld;
  ba.ld_do = hv;
  ba.offsets = off;
  ba.ts = ts;
  ba.rab_pos = w.rab_pos;
  ba.rab_time = w.rab_time;
  ba.bias_partial = want_bias ? b.bpart : nullptr;
  ba.key_ranges = (bwd_uses_mfma(&a) && ts) ? b.kr : nullptr;
  ba.items = b.items;
  ba.n_items = (int)p.j.items;
  ba.batch = a.batch;
  ba.H = a.num_heads;
  ba.d_qk = a.d_qk;
  ba.d_v = a.d_v;
  ba.P = a.num_pos_buckets;
  ba.T = a.num_time_buckets;
  ba.inv_n = 1.0f / (float)a.max_seq_len;
  if (bwd_uses_mfma(&a))
    HSTU_TRY(launch_attn_bwd_mfma(ba, s), "attention backward");
  else
    HSTU_TRY(launch_attn_bwd_simple(ba, bf, s), "attention backward");
  if (want_bias)
    HSTU_TRY(launch_bias_grad_reduce(b.bpart, ba.n_items, ba.H, ba.P, ba.T, g->d_rab_pos,
                                     g->d_rab_time, s),
             "bias gradient");
  // f1: dz1 = d[U|V|Q|K] SiLU'(z1), db1, dW1 = dz1^T X, dX = dz1 W1 (+ dY)
  HSTU_TRY(launch_silu_grad(b.z1, F1, b.dact, F1, T, (int)F1, bf, s), "SiLU backward");
  HSTU_TRY(launch_colsum(b.dact, F1, T, (int)F1, bf, b.cpart, g->db1, s), "db1");
  if (g->dw1 && bf) {
    if ((st = weight_grad_tn(b.dact, F1, xl, dm, F1, dm, T, p.split1, p.ks1, b.wpart, g->dw1, s)))
      return st;
  } else if (g->dw1) {
    HSTU_TRY(launch_transpose(b.dact, F1, b.ta, p.Tp, T, p.Tp, (int)F1, bf, s), "transpose");
    HSTU_TRY(launch_transpose(xl, dm, b.tb, p.Tp, T, p.Tp, dm, bf, s), "transpose");
    if ((st = weight_grad(b.ta, b.tb, F1, dm, p.Tp, p.split1, p.ks1, bf, b.wpart, g->dw1, s)))
      return st;
  }
  if (dX) {
    HSTU_TRY(launch_transpose(w.w1, dm, b.w1t, F1, F1, F1, dm, bf, s), "transpose");
    HSTU_TRY(launch_gemm_ex(b.dact, F1, b.w1t, F1, nullptr, d->residual ? dY : nullptr, dm, dX, dm,
                            T, dm, (int)F1, 0, bf, 0, 1, F1, 0, nullptr, s),
             "dX");
  }
  return HSTU_OK;
}

// ---------------------------------------------------------------- attention entry
// Host-only checks of an hstu_attn_fwd call (nothing is launched), then the launches.
hstu_status check_attn_fwd(const hstu_attn_desc* desc, const int64_t* off_host,
                           const int64_t* seq_offsets, const void* q, const void* k,
                           const void* v, const void* u, const void* out, AttnPlan* p) {
  hstu_status st = plan_attn(desc, off_host, u != nullptr, p);
  if (st) return st;
  if (u && (st = check_eps(desc->ln_eps))) return st;
  if (p->j.total == 0) return HSTU_OK;
  if (!seq_offsets) return fail(HSTU_INVALID_ARGUMENT, "device seq_offsets is NULL");
  if (!q || !k || !v || !out) return fail(HSTU_INVALID_ARGUMENT, "q, k, v and out are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || (u && !aligned16(u)))
    return fail(HSTU_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  return HSTU_OK;
}

hstu_status enqueue_attn_fwd(const hstu_attn_desc* desc, const AttnPlan& p,
                             const int64_t* seq_offsets, const int64_t* timestamps, const void* q,
                             const void* k, const void* v, const float* rab_pos,
                             const float* rab_time, const void* u, const float* ln_gamma,
                             const float* ln_beta, void* out, void* workspace, hipStream_t s) {
  Carver c{(char*)workspace};
  int2* items = (int2*)c.take((size_t)p.j.items * sizeof(int2));
  KeyRange* kr = (KeyRange*)c.take(key_range_bytes(desc, p.j.total));
  float* o32 = u ? (float*)c.take((size_t)p.j.total * desc->num_heads * desc->d_v * 4) : nullptr;
  const bool timed = rab_time && timestamps && kr;
  HSTU_TRY(launch_plan(seq_offsets, desc->batch, attn_tile_rows(desc), p.j.max_tiles, items,
                       (int)p.j.items, timed ? timestamps : nullptr, p.j.max_len, kr, s),
           "tile planner and key ranges");
  AttnArgs a = base_args(desc);
  a.q = q;
  a.k = k;
  a.v = v;
  a.ld_q = a.ld_k = (int64_t)desc->num_heads * desc->d_qk;
  a.ld_v = (int64_t)desc->num_heads * desc->d_v;
  a.out = u ? (void*)o32 : out;
  a.ld_o = (int64_t)desc->num_heads * desc->d_v;
  a.out_f32 = u ? 1 : (desc->dtype == HSTU_F32);
  a.q_offsets = a.k_offsets = seq_offsets;
  a.ts_q = a.ts_k = timestamps;
  a.rab_pos = rab_pos;
  a.rab_time = rab_time;
  a.key_ranges = timed ? kr : nullptr;
  a.items = items;
  a.n_items = (int)p.j.items;
  HSTU_TRY(run_attention(desc, a, false, s), "attention");
  if (u) {
    const int hv = desc->num_heads * desc->d_v;
    HSTU_TRY(launch_ln_gate(o32, hv, 1, 0, u, hv, ln_gamma, ln_beta, desc->ln_eps, out, hv,
                            p.j.total, hv, desc->dtype == HSTU_BF16, s),
             "layer norm gate");
  }
  return HSTU_OK;
}

// ---------------------------------------------------------------- allocation-free scratch
// The scratch of hstu_attn_fwd_noalloc: a file-scope device array. Every device the
// library runs on holds its own copy until the process ends. Host code never passes the
// array's name to a kernel or a copy (on the host that name is a stand-in, not a device
// address): the device address comes from hipGetSymbolAddress, taken once per device
// with that device current, and kept below.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hstu_status noalloc_scratch(void** out) {
  int dev = 0;
  HSTU_TRY(hipGetDevice(&dev), "current device");
  if (dev < 0 || dev >= kMaxDevices) return fail(HSTU_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    HSTU_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "scratch address");
    if (!ptr || ((uintptr_t)ptr & (kAlign - 1)) != 0)
      return fail(HSTU_DEVICE_ERROR, "scratch address is NULL or not 256-byte aligned");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return HSTU_OK;
}

}  // namespace

// =========================================================================
extern "C" {

int hstu_version(void) { return HSTU_VERSION; }

const char* hstu_status_string(hstu_status s) {
  switch (s) {
    case HSTU_OK: return "HSTU_OK";
    case HSTU_INVALID_ARGUMENT: return "HSTU_INVALID_ARGUMENT";
    case HSTU_UNSUPPORTED: return "HSTU_UNSUPPORTED";
    case HSTU_WORKSPACE_TOO_SMALL: return "HSTU_WORKSPACE_TOO_SMALL";
    case HSTU_DEVICE_ERROR: return "HSTU_DEVICE_ERROR";
  }
  return "unknown hstu_status";
}

const char* hstu_last_error(void) { return g_err.c_str(); }

hstu_status hstu_attn_workspace_size(const hstu_attn_desc* desc, const int64_t* seq_offsets_host,
                                     size_t* bytes) {
  if (!bytes) return fail(HSTU_INVALID_ARGUMENT, "bytes is NULL");
  AttnPlan p;
  hstu_status st = plan_attn(desc, seq_offsets_host, true, &p);
  if (st) return st;
  *bytes = p.ws;
  return HSTU_OK;
}

hstu_status hstu_attn_fwd(const hstu_attn_desc* desc, const int64_t* seq_offsets_host,
                          const int64_t* seq_offsets, const int64_t* timestamps, const void* q,
                          const void* k, const void* v, const float* rab_pos,
                          const float* rab_time, const void* u, const float* ln_gamma,
                          const float* ln_beta, void* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  AttnPlan p;
  hstu_status st = check_attn_fwd(desc, seq_offsets_host, seq_offsets, q, k, v, u, out, &p);
  if (st || p.j.total == 0) return st;
  if (workspace_bytes < p.ws || (!workspace && p.ws))
    return fail(HSTU_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes (got %zu)", p.ws,
                workspace_bytes);
  if (((uintptr_t)workspace & (kAlign - 1)) != 0)
    return fail(HSTU_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  return enqueue_attn_fwd(desc, p, seq_offsets, timestamps, q, k, v, rab_pos, rab_time, u,
                          ln_gamma, ln_beta, out, workspace, (hipStream_t)stream);
}

size_t hstu_attn_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

hstu_status hstu_attn_fwd_noalloc(const hstu_attn_desc* desc, const int64_t* seq_offsets_host,
                                  const int64_t* seq_offsets, const int64_t* timestamps,
                                  const void* q, const void* k, const void* v,
                                  const float* rab_pos, const float* rab_time, const void* u,
                                  const float* ln_gamma, const float* ln_beta, void* out,
                                  void* stream) {
  AttnPlan p;
  hstu_status st = check_attn_fwd(desc, seq_offsets_host, seq_offsets, q, k, v, u, out, &p);
  if (st || p.j.total == 0) return st;
  if (p.ws > kNoAllocScratchBytes)
    return fail(HSTU_UNSUPPORTED,
                "this call needs %zu bytes of scratch; the allocation-free entry point has %zu "
                "(use hstu_attn_fwd with a workspace)",
                p.ws, kNoAllocScratchBytes);
  void* ws = nullptr;
  if ((st = noalloc_scratch(&ws))) return st;
  return enqueue_attn_fwd(desc, p, seq_offsets, timestamps, q, k, v, rab_pos, rab_time, u,
                          ln_gamma, ln_beta, out, ws, (hipStream_t)stream);
}

hstu_status hstu_layer_workspace_size(const hstu_layer_desc* desc,
                                      const int64_t* seq_offsets_host, size_t* bytes) {
  if (!bytes) return fail(HSTU_INVALID_ARGUMENT, "bytes is NULL");
  LayerPlan p;
  hstu_status st = plan_layer(desc, seq_offsets_host, &p);
  if (st) return st;
  *bytes = p.ws;
  return HSTU_OK;
}

hstu_status hstu_layer_fwd(const hstu_layer_desc* desc, const int64_t* seq_offsets_host,
                           const int64_t* seq_offsets, const int64_t* timestamps, const void* x,
                           const hstu_layer_weights* weights, void* y, void* workspace,
                           size_t workspace_bytes, void* stream) {
  LayerPlan p;
  hstu_status st = plan_layer(desc, seq_offsets_host, &p);
  if (st) return st;
  if ((st = check_weights(weights, desc->num_layers))) return st;
  if (p.j.total == 0) return HSTU_OK;
  if (!seq_offsets) return fail(HSTU_INVALID_ARGUMENT, "device seq_offsets is NULL");
  if (!x || !y) return fail(HSTU_INVALID_ARGUMENT, "x and y are required");
  if (!aligned16(x) || !aligned16(y))
    return fail(HSTU_INVALID_ARGUMENT, "x and y must be 16-byte aligned");
  if (workspace_bytes < p.ws || (!workspace && p.ws))
    return fail(HSTU_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes (got %zu)", p.ws,
                workspace_bytes);
  if (((uintptr_t)workspace & (kAlign - 1)) != 0)
    return fail(HSTU_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  Carver c{(char*)workspace};
  LayerBufs b;
  carve_layer(c, desc, p.j.total, p.j.items, &b);
  const int L = desc->num_layers;
  if ((st = plan_causal(desc->attn, seq_offsets, timestamps, p.j, b, s))) return st;
  const void* in = x;
  for (int l = 0; l < L; ++l) {
    // layer outputs alternate between y and tmp so that the last one lands in y
    void* out = ((L - 1 - l) % 2 == 0) ? y : b.tmp;
    st = layer_once(desc, seq_offsets, timestamps, p.j, in, weights[l], out, b, s, false);
    if (st) return st;
    in = out;
  }
  return HSTU_OK;
}

hstu_status hstu_layer_bwd_workspace_size(const hstu_layer_desc* desc,
                                          const int64_t* seq_offsets_host, size_t* bytes) {
  if (!bytes) return fail(HSTU_INVALID_ARGUMENT, "bytes is NULL");
  LayerBwdPlan p;
  hstu_status st = plan_layer_bwd(desc, seq_offsets_host, &p);
  if (st) return st;
  *bytes = p.ws;
  return HSTU_OK;
}

hstu_status hstu_layer_bwd(const hstu_layer_desc* desc, const int64_t* seq_offsets_host,
                           const int64_t* seq_offsets, const int64_t* timestamps, const void* x,
                           const hstu_layer_weights* weights, const void* d_y, void* d_x,
                           const hstu_layer_grads* grads, void* workspace,
                           size_t workspace_bytes, void* stream) {
  LayerBwdPlan p;
  hstu_status st = plan_layer_bwd(desc, seq_offsets_host, &p);
  if (st) return st;
  if ((st = check_weights(weights, desc->num_layers))) return st;
  const int L = desc->num_layers;
  if (grads && !p.bias_ok)
    for (int l = 0; l < L; ++l)
      if (grads[l].d_rab_pos || grads[l].d_rab_time)
        return fail(HSTU_UNSUPPORTED, "bias-table gradients need P + T <= %d", kMaxBiasBins);
  hipStream_t s = (hipStream_t)stream;
  if (p.j.total == 0) {
    if (grads)
      for (int l = 0; l < L; ++l)
        if ((st = zero_layer_grads(desc, &grads[l], s))) return st;
    return HSTU_OK;
  }
  if (!seq_offsets) return fail(HSTU_INVALID_ARGUMENT, "device seq_offsets is NULL");
  if (!x || !d_y) return fail(HSTU_INVALID_ARGUMENT, "x and d_y are required");
  if (!aligned16(x) || !aligned16(d_y) || (d_x && !aligned16(d_x)))
    return fail(HSTU_INVALID_ARGUMENT, "x, d_y and d_x must be 16-byte aligned");
  if ((st = check_ws(workspace, workspace_bytes, p.ws, "workspace"))) return st;
  Carver c{(char*)workspace};
  LayerBwdBufs b;
  carve_layer_bwd(c, desc, p, &b);
  const hstu_attn_desc& a = desc->attn;
  const size_t xbytes = (size_t)p.j.total * desc->d_model * elt_size(a.dtype);
  // forward: inputs of layers 1..L-1
  // the forward recompute borrows dact (not used until the backward part) for the lo parts
  LayerBufs lb{b.items, b.kr, b.uvqk, b.o, b.g, nullptr,
               layer_splits_qk(a) ? b.dact : nullptr};
  if ((st = plan_causal(a, seq_offsets, timestamps, p.j, lb, s))) return st;
  for (int l = 0; l + 1 < L; ++l) {
    const void* in = l == 0 ? x : (const void*)(b.xs + (l - 1) * xbytes);
    if ((st = layer_once(desc, seq_offsets, timestamps, p.j, in, weights[l], b.xs + l * xbytes, lb, s,
                         false)))
      return st;
  }
  // backward, last layer first; dL/dX of layer l is dL/dY of layer l - 1
  const void* dY = d_y;
  for (int l = L - 1; l >= 0; --l) {
    const void* xl = l == 0 ? x : (const void*)(b.xs + (l - 1) * xbytes);
    void* dX = l == 0 ? d_x : b.dyb[l & 1];
    if ((st = layer_bwd_once(desc, p, seq_offsets, timestamps, xl, weights[l],
                             grads ? &grads[l] : nullptr, dY, dX, b, s)))
      return st;
    dY = dX;
  }
  return HSTU_OK;
}

hstu_status mfalcon_workspace_size(const mfalcon_desc* desc, const int64_t* hist_offsets_host,
                                   const int64_t* cand_offsets_host, size_t* bytes) {
  if (!bytes) return fail(HSTU_INVALID_ARGUMENT, "bytes is NULL");
  if (!cand_offsets_host) return fail(HSTU_INVALID_ARGUMENT, "cand_offsets_host is NULL");
  MfPlan p;
  hstu_status st = plan_mfalcon(desc, hist_offsets_host, cand_offsets_host, &p);
  if (st) return st;
  *bytes = align_up(p.cache) + align_up(p.hist_ws) + align_up(p.cand_ws);
  return HSTU_OK;
}

hstu_status mfalcon_score(const mfalcon_desc* desc, const int64_t* hist_offsets_host,
                          const int64_t* hist_offsets, const int64_t* hist_ts, const void* hist_x,
                          const int64_t* cand_offsets_host, const int64_t* cand_offsets,
                          const int64_t* cand_ts, const void* cand_x,
                          const hstu_layer_weights* weights, const float* w_head,
                          void* cand_out, float* cand_logit, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!cand_offsets_host) return fail(HSTU_INVALID_ARGUMENT, "cand_offsets_host is NULL");
  MfPlan p;
  hstu_status st = plan_mfalcon(desc, hist_offsets_host, cand_offsets_host, &p);
  if (st) return st;
  if ((st = check_weights(weights, desc->layer.num_layers))) return st;
  if (p.cand_total == 0) {
    if ((hist_ts == nullptr) != (cand_ts == nullptr))
      return fail(HSTU_INVALID_ARGUMENT, "hist_ts and cand_ts must both be set or both be NULL");
    return HSTU_OK;
  }
  if ((st = check_candidate_args(p, hist_offsets, hist_ts, cand_offsets, cand_ts, cand_x, cand_out,
                                 cand_logit, w_head)))
    return st;
  if ((st = check_history_args(weights, desc->layer.num_layers, p, hist_offsets, hist_x))) return st;
  const size_t need = align_up(p.cache) + align_up(p.hist_ws) + align_up(p.cand_ws);
  if ((st = check_ws(workspace, workspace_bytes, need, "workspace"))) return st;
  hipStream_t s = (hipStream_t)stream;
  Carver c{(char*)workspace};
  MfCache cache;
  carve_cache(c, desc, p, &cache);
  c.off = align_up(p.cache);
  MfHistBufs hb;
  carve_hist_ws(c, desc, p, &hb);
  c.off = align_up(p.cache) + align_up(p.hist_ws);
  MfCandBufs cb;
  carve_cand_ws(c, desc, p, &cb);
  if ((st = run_history(desc, p, hist_offsets, hist_ts, hist_x, weights, cache, hb, s))) return st;
  return run_candidates(desc, p, hist_offsets, hist_ts, cache, cand_offsets_host, cand_offsets,
                        cand_ts, cand_x, weights, w_head, cand_out, cand_logit, &cb, s);
}

hstu_status mfalcon_cache_size(const mfalcon_desc* desc, const int64_t* hist_offsets_host,
                               size_t* bytes) {
  if (!bytes) return fail(HSTU_INVALID_ARGUMENT, "bytes is NULL");
  MfPlan p;
  hstu_status st = plan_mfalcon(desc, hist_offsets_host, nullptr, &p);
  if (st) return st;
  *bytes = p.cache;
  return HSTU_OK;
}

hstu_status mfalcon_history_workspace_size(const mfalcon_desc* desc,
                                           const int64_t* hist_offsets_host, size_t* bytes) {
  if (!bytes) return fail(HSTU_INVALID_ARGUMENT, "bytes is NULL");
  MfPlan p;
  hstu_status st = plan_mfalcon(desc, hist_offsets_host, nullptr, &p);
  if (st) return st;
  *bytes = p.hist_ws;
  return HSTU_OK;
}

hstu_status mfalcon_history(const mfalcon_desc* desc, const int64_t* hist_offsets_host,
                            const int64_t* hist_offsets, const int64_t* hist_ts,
                            const void* hist_x, const hstu_layer_weights* weights, void* cache,
                            size_t cache_bytes, void* workspace, size_t workspace_bytes,
                            void* stream) {
  MfPlan p;
  hstu_status st = plan_mfalcon(desc, hist_offsets_host, nullptr, &p);
  if (st) return st;
  if ((st = check_history_args(weights, desc->layer.num_layers, p, hist_offsets, hist_x))) return st;
  if ((st = check_ws(cache, cache_bytes, p.cache, "cache"))) return st;
  if ((st = check_ws(workspace, workspace_bytes, p.hist_ws, "workspace"))) return st;
  Carver c{(char*)cache};
  MfCache cb;
  carve_cache(c, desc, p, &cb);
  Carver w{(char*)workspace};
  MfHistBufs hb;
  carve_hist_ws(w, desc, p, &hb);
  return run_history(desc, p, hist_offsets, hist_ts, hist_x, weights, cb, hb, (hipStream_t)stream);
}

hstu_status mfalcon_cached_workspace_size(const mfalcon_desc* desc,
                                          const int64_t* hist_offsets_host,
                                          const int64_t* cand_offsets_host, size_t* bytes) {
  if (!bytes) return fail(HSTU_INVALID_ARGUMENT, "bytes is NULL");
  if (!cand_offsets_host) return fail(HSTU_INVALID_ARGUMENT, "cand_offsets_host is NULL");
  MfPlan p;
  hstu_status st = plan_mfalcon(desc, hist_offsets_host, cand_offsets_host, &p);
  if (st) return st;
  *bytes = p.cand_ws;
  return HSTU_OK;
}

hstu_status mfalcon_score_cached(const mfalcon_desc* desc, const int64_t* hist_offsets_host,
                                 const int64_t* hist_offsets, const int64_t* hist_ts,
                                 const void* cache, size_t cache_bytes,
                                 const int64_t* cand_offsets_host, const int64_t* cand_offsets,
                                 const int64_t* cand_ts, const void* cand_x,
                                 const hstu_layer_weights* weights, const float* w_head,
                                 void* cand_out, float* cand_logit, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!cand_offsets_host) return fail(HSTU_INVALID_ARGUMENT, "cand_offsets_host is NULL");
  MfPlan p;
  hstu_status st = plan_mfalcon(desc, hist_offsets_host, cand_offsets_host, &p);
  if (st) return st;
  if ((st = check_weights(weights, desc->layer.num_layers))) return st;
  if ((hist_ts == nullptr) != (cand_ts == nullptr))
    return fail(HSTU_INVALID_ARGUMENT, "hist_ts and cand_ts must both be set or both be NULL");
  if (p.cand_total == 0) return HSTU_OK;
  if ((st = check_candidate_args(p, hist_offsets, hist_ts, cand_offsets, cand_ts, cand_x, cand_out,
                                 cand_logit, w_head)))
    return st;
  if ((st = check_ws(cache, cache_bytes, p.cache, "cache"))) return st;
  if ((st = check_ws(workspace, workspace_bytes, p.cand_ws, "workspace"))) return st;
  Carver c{(char*)const_cast<void*>(cache)};
  MfCache cb;
  carve_cache(c, desc, p, &cb);
  Carver w{(char*)workspace};
  MfCandBufs kb;
  carve_cand_ws(w, desc, p, &kb);
  return run_candidates(desc, p, hist_offsets, hist_ts, cb, cand_offsets_host, cand_offsets,
                        cand_ts, cand_x, weights, w_head, cand_out, cand_logit, &kb,
                        (hipStream_t)stream);
}

hstu_status hstu_attn_bwd_workspace_size(const hstu_attn_desc* desc,
                                         const int64_t* seq_offsets_host, size_t* bytes) {
  if (!bytes) return fail(HSTU_INVALID_ARGUMENT, "bytes is NULL");
  AttnBwdPlan p;
  hstu_status st = plan_attn_bwd(desc, seq_offsets_host, &p);
  if (st) return st;
  *bytes = p.ws;
  return HSTU_OK;
}

// Gradients of hstu_attn_fwd without the gate (HSTU chapter, eq. 2).
hstu_status hstu_attn_bwd(const hstu_attn_desc* desc, const int64_t* seq_offsets_host,
                          const int64_t* seq_offsets, const int64_t* timestamps, const void* q,
                          const void* k, const void* v, const float* rab_pos,
                          const float* rab_time, const void* d_out, void* dq, void* dk, void* dv,
                          float* d_rab_pos, float* d_rab_time, void* workspace,
                          size_t workspace_bytes, void* stream) {
  AttnBwdPlan p;
  hstu_status st = plan_attn_bwd(desc, seq_offsets_host, &p);
  if (st) return st;
  const bool want_bias = d_rab_pos || d_rab_time;
  if (want_bias && desc->num_pos_buckets + desc->num_time_buckets > kMaxBiasBins)
    return fail(HSTU_UNSUPPORTED, "bias-table gradients need P + T <= %d", kMaxBiasBins);
  hipStream_t s = (hipStream_t)stream;
  if (p.j.total == 0) {  // no pairs: the table gradients are zero
    HSTU_TRY(launch_bias_grad_reduce(nullptr, 0, desc->num_heads, desc->num_pos_buckets,
                                     desc->num_time_buckets, d_rab_pos, d_rab_time, s),
             "bias gradient");
    return HSTU_OK;
  }
  if (!seq_offsets) return fail(HSTU_INVALID_ARGUMENT, "device seq_offsets is NULL");
  if (!q || !k || !v || !d_out || !dq || !dk || !dv)
    return fail(HSTU_INVALID_ARGUMENT, "q, k, v, d_out, dq, dk and dv are required");
  for (const void* t : {q, k, v, d_out, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned16(t)) return fail(HSTU_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  if ((st = check_ws(workspace, workspace_bytes, p.ws, "workspace"))) return st;
  Carver c{(char*)workspace};
  int2* items = (int2*)c.take(p.items);
  KeyRange* kr = (KeyRange*)c.take(p.ranges);
  float* partial = (float*)c.take(p.partial);
  HSTU_TRY(launch_plan(seq_offsets, desc->batch, bwd_tile_rows(desc), p.j.max_tiles, items,
                       (int)p.j.items, p.mfma && timestamps ? timestamps : nullptr, p.j.max_len,
                       kr, s),
           "tile planner and key ranges");
  AttnBwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = d_out;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.ld_q = a.ld_k = a.ld_dq = a.ld_dk = (int64_t)desc->num_heads * desc->d_qk;
  a.ld_v = a.ld_do = a.ld_dv = (int64_t)desc->num_heads * desc->d_v;
  a.offsets = seq_offsets;
  a.ts = timestamps;
  a.rab_pos = rab_pos;
  a.rab_time = rab_time;
  a.bias_partial = want_bias ? partial : nullptr;
  a.key_ranges = (p.mfma && timestamps) ? kr : nullptr;
  a.items = items;
  a.n_items = (int)p.j.items;
  a.batch = desc->batch;
  a.H = desc->num_heads;
  a.d_qk = desc->d_qk;
  a.d_v = desc->d_v;
  a.P = desc->num_pos_buckets;
  a.T = desc->num_time_buckets;
  a.inv_n = 1.0f / (float)desc->max_seq_len;
  if (p.mfma)
    HSTU_TRY(launch_attn_bwd_mfma(a, s), "attention backward");
  else
    HSTU_TRY(launch_attn_bwd_simple(a, desc->dtype == HSTU_BF16, s), "attention backward");
  if (want_bias)
    HSTU_TRY(launch_bias_grad_reduce(partial, a.n_items, a.H, a.P, a.T, d_rab_pos, d_rab_time, s),
             "bias gradient");
  return HSTU_OK;
}

hstu_status hstu_softmax_attn_workspace_size(const hstu_attn_desc* desc,
                                             const int64_t* seq_offsets_host, size_t* bytes) {
  if (!bytes) return fail(HSTU_INVALID_ARGUMENT, "bytes is NULL");
  hstu_status st = check_attn_desc(desc);
  if (st) return st;
  if (!attn_softmax_supported(desc->dtype == HSTU_BF16, desc->d_qk, desc->d_v,
                              desc->num_pos_buckets))
    return fail(HSTU_UNSUPPORTED, "softmax attention needs bf16, d_qk == d_v and P <= 1024");
  Jagged j;
  if ((st = check_offsets(seq_offsets_host, desc->batch, desc->max_seq_len, kMfmaRows,
                          "seq_offsets", &j)))
    return st;
  *bytes = align_up((size_t)j.items * sizeof(int2)) +
           align_up((size_t)key_range_slots(j.total, desc->batch) * sizeof(KeyRange));
  return HSTU_OK;
}

// The softmax ablation of hstu_attn_fwd (HSTU chapter, "No sequence-wise softmax").
hstu_status hstu_softmax_attn_fwd(const hstu_attn_desc* desc, const int64_t* seq_offsets_host,
                                  const int64_t* seq_offsets, const int64_t* timestamps,
                                  const void* q, const void* k, const void* v,
                                  const float* rab_pos, const float* rab_time, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  size_t need = 0;
  hstu_status st = hstu_softmax_attn_workspace_size(desc, seq_offsets_host, &need);
  if (st) return st;
  Jagged j;
  check_offsets(seq_offsets_host, desc->batch, desc->max_seq_len, kMfmaRows, "seq_offsets", &j);
  if ((int64_t)j.items * desc->num_heads >= (int64_t(1) << 31))
    return fail(HSTU_UNSUPPORTED, "too many query tiles for one launch");
  if (j.total == 0) return HSTU_OK;
  if (!seq_offsets) return fail(HSTU_INVALID_ARGUMENT, "device seq_offsets is NULL");
  if (!q || !k || !v || !out) return fail(HSTU_INVALID_ARGUMENT, "q, k, v and out are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(HSTU_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  if ((st = check_ws(workspace, workspace_bytes, need, "workspace"))) return st;
  hipStream_t s = (hipStream_t)stream;
  Carver c{(char*)workspace};
  int2* items = (int2*)c.take((size_t)j.items * sizeof(int2));
  KeyRange* kr = (KeyRange*)c.take((size_t)key_range_slots(j.total, desc->batch) * sizeof(KeyRange));
  HSTU_TRY(launch_plan(seq_offsets, desc->batch, kMfmaRows, j.max_tiles, items, (int)j.items,
                       timestamps, j.max_len, kr, s),
           "tile planner and key ranges");
  AttnArgs a = base_args(desc);
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.ld_q = a.ld_k = (int64_t)desc->num_heads * desc->d_qk;
  a.ld_v = a.ld_o = (int64_t)desc->num_heads * desc->d_v;
  a.q_offsets = a.k_offsets = seq_offsets;
  a.ts_q = a.ts_k = timestamps;
  a.rab_pos = rab_pos;
  a.rab_time = rab_time;
  a.key_ranges = timestamps ? kr : nullptr;
  a.items = items;
  a.n_items = (int)j.items;
  HSTU_TRY(launch_attn_softmax(a, s), "softmax attention");
  return HSTU_OK;
}

// Stochastic Length (HSTU chapter, "Three more scaling components"): the
// target length and the keep-whole decision, in double precision on the host.
hstu_status hstu_sl_lengths(const hstu_sl_desc* desc, const int64_t* offsets_host,
                            const float* u_keep_host, int64_t* new_offsets_host,
                            int64_t* target_len) {
  if (!desc) return fail(HSTU_INVALID_ARGUMENT, "descriptor is NULL");
  if (desc->max_seq_len < 1) return fail(HSTU_INVALID_ARGUMENT, "max_seq_len (N) must be >= 1");
  if (!(desc->alpha >= 0.f && desc->alpha <= 2.f))
    return fail(HSTU_INVALID_ARGUMENT, "alpha must be in [0, 2]");
  Jagged j;
  hstu_status st = check_offsets(offsets_host, desc->batch, -1, 1, "offsets", &j);
  if (st) return st;
  const int64_t L = (int64_t)std::floor(
      std::pow((double)desc->max_seq_len, (double)desc->alpha / 2.0) + 1e-9);
  if (target_len) *target_len = L;
  if (desc->batch == 0) {
    if (new_offsets_host) new_offsets_host[0] = 0;
    return HSTU_OK;
  }
  if (!u_keep_host || !new_offsets_host)
    return fail(HSTU_INVALID_ARGUMENT, "u_keep_host and new_offsets_host are required");
  int64_t acc = 0;
  new_offsets_host[0] = 0;
  for (int b = 0; b < desc->batch; ++b) {
    const int64_t n = offsets_host[b + 1] - offsets_host[b];
    const bool whole =
        n <= L || (double)u_keep_host[b] < ((double)L * (double)L) / ((double)n * (double)n);
    acc += whole ? n : L;
    new_offsets_host[b + 1] = acc;
  }
  return HSTU_OK;
}

hstu_status hstu_sl_sample(int32_t batch, const int64_t* offsets_host,
                           const int64_t* new_offsets_host, const int64_t* offsets,
                           const int64_t* new_offsets, const uint32_t* keys, int64_t* src_index,
                           const void* x, int64_t row_bytes, void* out_x, const int64_t* ts,
                           int64_t* out_ts, void* stream) {
  Jagged j;
  hstu_status st = check_offsets(offsets_host, batch, -1, 1, "offsets", &j);
  if (st) return st;
  if (batch == 0) return HSTU_OK;
  if (!new_offsets_host) return fail(HSTU_INVALID_ARGUMENT, "new_offsets_host is NULL");
  if (new_offsets_host[0] != 0) return fail(HSTU_INVALID_ARGUMENT, "new_offsets[0] must be 0");
  bool cut = false;
  for (int b = 0; b < batch; ++b) {
    const int64_t n = offsets_host[b + 1] - offsets_host[b];
    const int64_t m = new_offsets_host[b + 1] - new_offsets_host[b];
    if (m < 0 || m > n)
      return fail(HSTU_INVALID_ARGUMENT,
                  "sequence %d: new length %lld must be in [0, %lld]", b, (long long)m,
                  (long long)n);
    cut |= m > 0 && m < n;
  }
  const int64_t rows = new_offsets_host[batch];
  if (rows == 0) return HSTU_OK;
  if (!offsets || !new_offsets || !src_index)
    return fail(HSTU_INVALID_ARGUMENT, "offsets, new_offsets and src_index are required");
  if (cut && !keys) return fail(HSTU_INVALID_ARGUMENT, "keys are required to cut a sequence");
  if ((x == nullptr) != (out_x == nullptr))
    return fail(HSTU_INVALID_ARGUMENT, "x and out_x must both be set or both be NULL");
  if ((ts == nullptr) != (out_ts == nullptr))
    return fail(HSTU_INVALID_ARGUMENT, "ts and out_ts must both be set or both be NULL");
  if (x) {
    if (row_bytes <= 0 || row_bytes % 16)
      return fail(HSTU_INVALID_ARGUMENT, "row_bytes must be a positive multiple of 16");
    if (row_bytes > (int64_t(1) << 24))
      return fail(HSTU_UNSUPPORTED, "row_bytes above 16 MiB");
    if (!aligned16(x) || !aligned16(out_x))
      return fail(HSTU_INVALID_ARGUMENT, "x and out_x must be 16-byte aligned");
  }
  hipStream_t s = (hipStream_t)stream;
  HSTU_TRY(launch_sl_select(offsets, new_offsets, batch, keys, src_index, s), "sl select");
  HSTU_TRY(launch_sl_gather(src_index, rows, x, row_bytes, ts, out_x, out_ts, s), "sl gather");
  return HSTU_OK;
}

hstu_status hstu_debug_buckets(const hstu_attn_desc* desc, const int64_t* seq_offsets_host,
                               const int64_t* seq_offsets, const int64_t* timestamps, int32_t seq,
                               int32_t* pos_bucket, int32_t* time_bucket, void* stream) {
  hstu_status st = check_attn_desc(desc);
  if (st) return st;
  Jagged j;
  st = check_offsets(seq_offsets_host, desc->batch, desc->max_seq_len, 1, "seq_offsets", &j);
  if (st) return st;
  if (seq < 0 || seq >= desc->batch) return fail(HSTU_INVALID_ARGUMENT, "seq out of range");
  const int64_t n = seq_offsets_host[seq + 1] - seq_offsets_host[seq];
  if (n > 46340) return fail(HSTU_UNSUPPORTED, "sequence too long for the n x n export");
  if (n == 0) return HSTU_OK;
  if (!seq_offsets || !pos_bucket || !time_bucket)
    return fail(HSTU_INVALID_ARGUMENT, "device pointers are required");
  HSTU_TRY(launch_debug_buckets(seq_offsets, timestamps, seq, (int)n, desc->num_pos_buckets,
                                desc->num_time_buckets, pos_bucket, time_bucket,
                                (hipStream_t)stream),
           "bucket export");
  return HSTU_OK;
}

}  // extern "C"
