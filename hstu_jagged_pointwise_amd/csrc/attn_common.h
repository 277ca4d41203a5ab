// Work decoding shared by the attention kernels.
#pragma once
#include "common.h"
#include "kernels.h"

namespace hstu {

struct TileDecode {
  int h;
  int seq;          // sequence (causal) or user (candidate mode)
  int64_t q_base;   // global row of tile row 0 (candidate mode: global candidate row)
  int64_t q_local;  // row index into q/out/kc/vc of tile row 0
  int rows;         // valid query rows in the tile
  int64_t k_base;   // global row of key 0
  int64_t nk;       // keys that hold data (causal: whole sequence; candidates: history)
  int64_t kbeg;     // first key of this work item (candidate splits), else 0
  int64_t kend;     // keys that can be visible (causal: up to the last row of the tile)
  int64_t qpos0;    // position of tile row 0 (causal) or of every candidate (n_h)
  bool valid;
};

template <bool CAND>
__device__ __forceinline__ TileDecode decode(const AttnArgs& a, int bm) {
  TileDecode d;
  d.valid = false;
  if (!CAND) {
    const int item = blockIdx.x / a.H;
    d.h = blockIdx.x % a.H;
    if (item >= a.n_items) return d;
    // the (sequence, tile) pair as one 64-bit scalar load
    const uint64_t raw = sload(reinterpret_cast<const uint64_t*>(a.items + item));
    const int2 it = make_int2((int)(uint32_t)raw, (int)(uint32_t)(raw >> 32));
    if (it.x < 0 || it.x >= a.batch || it.y < 0) return d;
    d.seq = it.x;
    const int64_t s0 = sload(a.q_offsets + it.x);
    const int64_t n = sload(a.q_offsets + it.x + 1) - s0;
    const int64_t r0 = (int64_t)it.y * bm;
    if (r0 >= n) return d;
    d.rows = (int)(n - r0 < bm ? n - r0 : bm);
    d.q_base = s0 + r0;
    d.q_local = d.q_base;
    d.k_base = s0;
    d.nk = n;
    d.kbeg = 0;
    d.kend = r0 + d.rows;
    d.qpos0 = r0;
  } else {
    d.h = blockIdx.x % a.H;
    const int tile = blockIdx.x / a.H;
    const int b = a.user_begin + blockIdx.y;
    d.seq = b;
    int64_t cs = sload(a.q_offsets + b), ce = sload(a.q_offsets + b + 1);
    cs = cs > a.row_begin ? cs : a.row_begin;
    ce = ce < a.row_end ? ce : a.row_end;
    const int64_t r0 = cs + (int64_t)tile * bm;
    if (r0 >= ce) return d;
    d.rows = (int)(ce - r0 < bm ? ce - r0 : bm);
    d.q_base = r0;
    d.q_local = r0 - a.row_begin;
    d.k_base = sload(a.k_offsets + b);
    d.nk = sload(a.k_offsets + b + 1) - d.k_base;
    d.kbeg = 0;
    d.kend = d.nk;
    d.qpos0 = d.nk;
    if (a.kv_splits > 1) {
      const int64_t lo = (int64_t)blockIdx.z * a.keys_per_split;
      d.kbeg = lo < d.nk ? lo : d.nk;
      d.kend = lo + a.keys_per_split < d.nk ? lo + a.keys_per_split : d.nk;
    }
  }
  d.valid = true;
  return d;
}

}  // namespace hstu
