// Norm(AV) (.) U, the gating of eq. 3 of the HSTU layer ("What an HSTU layer
// changes" and "Gating instead of a separate FFN", HSTU chapter). The pooled
// value of each token, all H*d_v attention outputs of the row, is
// layer-normalised (biased variance, fp32 statistics), then scaled by gamma,
// shifted by beta and multiplied elementwise by the gate U.
//
// This step is bound by HBM bandwidth. One wavefront owns one row. When the row
// is at most 64 * 16 values wide it stays in registers, so it is read once;
// otherwise three passes reread it (from L2). The statistics use two passes
// over the values (mean, then squared deviations), not E[x^2] - E[x]^2.
// The row may arrive as nsplit partial rows (attention split over key ranges),
// which are summed here in split order, so the result never depends on timing.
// For M-FALCON candidates the pooled value also holds the candidate's own value
// v_c weighted by its self score, which the attention stores per row and head;
// it is added to the row before the partial rows.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace hstu {

// The self term of a candidate row: x[c] += w[row * H + c / dv] * v[row * ld_v + c] for
// the H = width / dv heads of the row; w == nullptr when there is none.
template <typename T>
struct SelfTerm {
  const float* w;
  const T* v;
  int64_t ld_v;
  int dv, H;
};

template <typename T, int NPL>
__global__ __launch_bounds__(256) void ln_gate_reg_kernel(const float* __restrict__ o, int64_t ld_o,
                                                          int nsplit, int64_t split_stride,
                                                          const T* __restrict__ u, int64_t ld_u,
                                                          const float* __restrict__ gamma,
                                                          const float* __restrict__ beta, float eps,
                                                          T* __restrict__ out, int64_t ld_out,
                                                          int64_t rows, int w, SelfTerm<T> st) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* orow = o + row * ld_o;
  float x[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int c = lane + 64 * i;
    x[i] = (st.w && c < w)
               ? st.w[row * st.H + c / st.dv] * to_f32<T>(st.v[row * st.ld_v + c])
               : 0.f;
  }
  // all loads of up to four splits are issued before any of them is summed
  for (int sp0 = 0; sp0 < nsplit; sp0 += 4) {
    float part[4][NPL];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* op = orow + (int64_t)(sp0 + q) * split_stride;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const int c = lane + 64 * i;
        part[q][i] = (sp0 + q < nsplit && c < w) ? op[c] : 0.f;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < NPL; ++i) x[i] += part[q][i];
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NPL; ++i) sum += x[i];
  const float mean = wave_sum(sum) / (float)w;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int c = lane + 64 * i;
    const float d = c < w ? x[i] - mean : 0.f;
    sq = fmaf(d, d, sq);
  }
  const float rstd = rsqrtf(wave_sum(sq) / (float)w + eps);
  const T* urow = u + row * ld_u;
  T* dst = out + row * ld_out;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int c = lane + 64 * i;
    if (c < w) {
      float y = (x[i] - mean) * rstd;
      if (gamma) y *= gamma[c];
      if (beta) y += beta[c];
      dst[c] = from_f32<T>(y * to_f32<T>(urow[c]));
    }
  }
}

// Vector form for rows whose width is a multiple of 4 with 16-byte aligned fp32 rows: a
// lane owns 4 adjacent columns per 4*LPR, so every load and store moves 16 (or 8) bytes.
// LPR lanes own a row: the whole wavefront (64), or for rows of at most 128 (64) values
// half (a quarter) of it, so that narrow rows keep every lane busy. The gate row, gamma
// and beta are requested first, then the partial rows of up to SB splits at once, so
// that a row's traffic is in flight together.
template <typename T, int NV, int LPR>
__global__ __launch_bounds__(256) void ln_gate_vec_kernel(const float* __restrict__ o, int64_t ld_o,
                                                          int nsplit, int64_t split_stride,
                                                          const T* __restrict__ u, int64_t ld_u,
                                                          const float* __restrict__ gamma,
                                                          const float* __restrict__ beta, float eps,
                                                          T* __restrict__ out, int64_t ld_out,
                                                          int64_t rows, int w, SelfTerm<T> st) {
  constexpr int SB = NV <= 1 ? 16 : 16 / NV;  // splits per batch of loads
  constexpr int RPW = 64 / LPR;               // rows per wavefront
  const int lane = threadIdx.x & 63, sl = lane % LPR;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const bool live = row < rows;  // no early exit: the row sums shuffle across lanes
  const float* orow = o + row * ld_o;
  const T* urow = u + row * ld_u;
  auto seg_sum = [](float v) {  // sum over the LPR lanes of this row (xor stays inside them)
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
  };
  f32x4 uv[NV], gv[NV], bv[NV], x[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int c = 4 * sl + 4 * LPR * v;
    const bool ok = live && c < w;
    if constexpr (std::is_same<T, float>::value) {
      uv[v] = ok ? *reinterpret_cast<const f32x4*>(urow + c) : f32x4{};
    } else {
      const bf16x4 ub = ok ? *reinterpret_cast<const bf16x4*>(urow + c) : bf16x4{};
#pragma unroll
      for (int e = 0; e < 4; ++e) uv[v][e] = (float)ub[e];
    }
    gv[v] = (ok && gamma) ? *reinterpret_cast<const f32x4*>(gamma + c) : f32x4{1.f, 1.f, 1.f, 1.f};
    bv[v] = (ok && beta) ? *reinterpret_cast<const f32x4*>(beta + c) : f32x4{};
    x[v] = f32x4{};
    if (st.w && ok) {  // the 4 columns lie in one head (dv % 4 == 0)
      const float sw = st.w[row * st.H + c / st.dv];
      const T* vp = st.v + row * st.ld_v + c;
      if constexpr (std::is_same<T, float>::value) {
        const f32x4 vv = *reinterpret_cast<const f32x4*>(vp);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[v][e] = sw * vv[e];
      } else {
        const bf16x4 vv = *reinterpret_cast<const bf16x4*>(vp);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[v][e] = sw * (float)vv[e];
      }
    }
  }
  for (int sp0 = 0; sp0 < nsplit; sp0 += SB) {
    f32x4 part[SB][NV];
#pragma unroll
    for (int q = 0; q < SB; ++q)
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int c = 4 * sl + 4 * LPR * v;
        part[q][v] = (live && sp0 + q < nsplit && c < w)
                         ? *reinterpret_cast<const f32x4*>(orow + (int64_t)(sp0 + q) * split_stride + c)
                         : f32x4{};
      }
#pragma unroll
    for (int q = 0; q < SB; ++q)  // in split order
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[v][e] += part[q][v][e];
  }
  float sum = 0.f;
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int e = 0; e < 4; ++e) sum += x[v][e];
  const float mean = seg_sum(sum) / (float)w;
  float sq = 0.f;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const bool ok = 4 * sl + 4 * LPR * v < w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float d = ok ? x[v][e] - mean : 0.f;
      sq = fmaf(d, d, sq);
    }
  }
  const float rstd = rsqrtf(seg_sum(sq) / (float)w + eps);
  if (!live) return;
  T* dst = out + row * ld_out;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int c = 4 * sl + 4 * LPR * v;
    if (c >= w) continue;
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = ((x[v][e] - mean) * rstd * gv[v][e] + bv[v][e]) * uv[v][e];
    if constexpr (std::is_same<T, float>::value) {
      *reinterpret_cast<f32x4*>(dst + c) = f32x4{y[0], y[1], y[2], y[3]};
    } else {
      bf16x4 ob;
#pragma unroll
      for (int e = 0; e < 4; ++e) ob[e] = (bf16)y[e];
      *reinterpret_cast<bf16x4*>(dst + c) = ob;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void ln_gate_loop_kernel(const float* __restrict__ o, int64_t ld_o,
                                                           int nsplit, int64_t split_stride,
                                                           const T* __restrict__ u, int64_t ld_u,
                                                           const float* __restrict__ gamma,
                                                           const float* __restrict__ beta, float eps,
                                                           T* __restrict__ out, int64_t ld_out,
                                                           int64_t rows, int w, SelfTerm<T> st) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* orow = o + row * ld_o;
  auto val = [&](int c) {
    float xv = st.w ? st.w[row * st.H + c / st.dv] * to_f32<T>(st.v[row * st.ld_v + c]) : 0.f;
    for (int sp = 0; sp < nsplit; ++sp) xv += orow[sp * split_stride + c];
    return xv;
  };
  float sum = 0.f;
  for (int c = lane; c < w; c += 64) sum += val(c);
  const float mean = wave_sum(sum) / (float)w;
  float sq = 0.f;
  for (int c = lane; c < w; c += 64) {
    const float d = val(c) - mean;
    sq = fmaf(d, d, sq);
  }
  const float rstd = rsqrtf(wave_sum(sq) / (float)w + eps);
  const T* urow = u + row * ld_u;
  T* dst = out + row * ld_out;
  for (int c = lane; c < w; c += 64) {
    float y = (val(c) - mean) * rstd;
    if (gamma) y *= gamma[c];
    if (beta) y += beta[c];
    dst[c] = from_f32<T>(y * to_f32<T>(urow[c]));
  }
}

template <typename T>
static hipError_t ln_dispatch(const float* o, int64_t ld_o, int nsplit, int64_t split_stride,
                              const void* u, int64_t ld_u,
                              const float* gamma, const float* beta, float eps, void* out,
                              int64_t ld_out, int64_t rows, int w, hipStream_t s,
                              const float* self_w, const void* vself, int64_t ld_vself, int dv) {
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  const T* uu = (const T*)u;
  T* oo = (T*)out;
  const SelfTerm<T> st{self_w, (const T*)vself, ld_vself, self_w ? dv : 1, self_w ? w / dv : 0};
  const int npl = (w + 63) / 64;
  // 16-byte fp32 rows, 8- (bf16) or 16-byte (fp32) gate and output rows
  auto al = [](const void* p, unsigned b) { return ((uintptr_t)p & (b - 1)) == 0; };
  const unsigned ub = (unsigned)(4 * sizeof(T));
  const bool vec = w % 4 == 0 && w <= 1024 && ld_o % 4 == 0 && split_stride % 4 == 0 &&
                   ld_u % 4 == 0 && ld_out % 4 == 0 && al(o, 16) && al(u, ub) && al(out, ub) &&
                   (!gamma || al(gamma, 16)) && (!beta || al(beta, 16)) &&
                   (!self_w || (dv % 4 == 0 && ld_vself % 4 == 0 && al(vself, ub)));
  if (vec) {
    const int nv = (w + 255) / 256;
    // rows of at most 64 or 128 values: 4 or 2 rows per wavefront
    const int lpr = w <= 64 ? 16 : w <= 128 ? 32 : 64;
    const dim3 vgrid((unsigned)((rows + 4 * (64 / lpr) - 1) / (4 * (64 / lpr))));
#define HSTU_LNV_CASE(N, L)                                                                      \
    if (nv <= N && lpr == L) {                                                                   \
      hipLaunchKernelGGL((ln_gate_vec_kernel<T, N, L>), vgrid, block, 0, s, o, ld_o, nsplit,     \
                         split_stride, uu, ld_u, gamma, beta, eps, oo, ld_out, rows, w, st);     \
      return hipGetLastError();                                                                  \
    }
    HSTU_LNV_CASE(1, 16) HSTU_LNV_CASE(1, 32) HSTU_LNV_CASE(1, 64) HSTU_LNV_CASE(2, 64)
    HSTU_LNV_CASE(4, 64)
#undef HSTU_LNV_CASE
  }
#define HSTU_LN_CASE(N)                                                                          \
  if (npl <= N) {                                                                                \
    hipLaunchKernelGGL((ln_gate_reg_kernel<T, N>), grid, block, 0, s, o, ld_o, nsplit,           \
                       split_stride, uu, ld_u, gamma, beta, eps, oo, ld_out, rows, w, st);       \
    return hipGetLastError();                                                                    \
  }
  HSTU_LN_CASE(1) HSTU_LN_CASE(2) HSTU_LN_CASE(4) HSTU_LN_CASE(8) HSTU_LN_CASE(16)
#undef HSTU_LN_CASE
  hipLaunchKernelGGL((ln_gate_loop_kernel<T>), grid, block, 0, s, o, ld_o, nsplit, split_stride, uu,
                     ld_u, gamma, beta, eps, oo, ld_out, rows, w, st);
  return hipGetLastError();
}

hipError_t launch_ln_gate(const float* o, int64_t ld_o, int nsplit, int64_t split_stride,
                          const void* u, int64_t ld_u, const float* gamma, const float* beta,
                          float eps, void* out, int64_t ld_out, int64_t rows, int w, int bf16flag,
                          hipStream_t s, const float* self_w, const void* vself, int64_t ld_vself,
                          int dv) {
  if (rows <= 0) return hipSuccess;
  if (self_w && (dv <= 0 || w % dv != 0 || !vself)) return hipErrorInvalidValue;
  nsplit = nsplit < 1 ? 1 : nsplit;
  return bf16flag ? ln_dispatch<bf16>(o, ld_o, nsplit, split_stride, u, ld_u, gamma, beta, eps, out,
                                      ld_out, rows, w, s, self_w, vself, ld_vself, dv)
                  : ln_dispatch<float>(o, ld_o, nsplit, split_stride, u, ld_u, gamma, beta, eps,
                                       out, ld_out, rows, w, s, self_w, vself, ld_vself, dv);
}

}  // namespace hstu
