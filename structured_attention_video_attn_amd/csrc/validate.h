// validate.h -- host-only argument checks and problem resolution (no HIP calls).
//
// Every public entry point runs these checks before it touches the HIP
// runtime, so a rejected call enqueues nothing.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/monarch_attn.h"
#include "group_addr.h"

namespace ma {

struct Problem {
  int64_t batch, heads, T, H, W, N, D;
  int32_t r_axes;
  int64_t b1, b2;
  int32_t tile_t, tile_h;   // 0,0 = untiled; otherwise clamped to (T, H)
  int32_t dtype;
  size_t elem_bytes;
  size_t tensor_bytes;      // bytes of one [batch, heads, N, D] tensor
  int64_t slice_elems;      // elements between (batch, head) slices: N * D, or the full
                            // buffer's when the grid is a frame range of a longer one
  bool empty;               // some extent is zero: nothing to do
  bool r_trivial;           // b2 == 1: Y = V
  bool l_trivial;           // every stage-L group has one member: O = Y
};

inline bool head_dim_supported(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool overlaps(const void *a, const void *b, size_t bytes) {
  if (a == nullptr || b == nullptr || bytes == 0) return false;
  uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bytes && y < x + bytes;
}

// [a, a + na) and [b, b + nb) intersect.
inline bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Shape checks shared by all Monarch entry points. tiled: tile_t/tile_h must be >= 1.
inline int resolve_grid(int32_t batch, int32_t heads, int32_t T, int32_t H, int32_t W,
                        int32_t r_axes, int32_t tile_t, int32_t tile_h, bool tiled,
                        int32_t head_dim, int32_t dtype, Problem *p) {
  if (batch < 0 || heads < 0 || T < 0 || H < 0 || W < 0) return MA_ERR_INVALID_ARG;
  if (r_axes < 0 || r_axes > 3) return MA_ERR_INVALID_ARG;
  if (tiled) {
    if (tile_t < 1 || tile_h < 1) return MA_ERR_INVALID_ARG;
    if (r_axes != 1) return MA_ERR_INVALID_ARG;
  } else if (tile_t != 0 || tile_h != 0) {
    return MA_ERR_INVALID_ARG;
  }
  if (dtype != MA_BF16 && dtype != MA_F32) return MA_ERR_UNSUPPORTED;
  if (!head_dim_supported(head_dim)) return MA_ERR_UNSUPPORTED;
  p->batch = batch;
  p->heads = heads;
  p->T = T;
  p->H = H;
  p->W = W;
  p->N = (int64_t)T * H * W;
  p->D = head_dim;
  p->r_axes = r_axes;
  p->dtype = dtype;
  p->elem_bytes = dtype == MA_BF16 ? 2 : 4;
  p->empty = (batch == 0 || heads == 0 || p->N == 0);
  // per-head element offsets are 32-bit inside the kernels
  if (p->N * p->D > (int64_t)INT32_MAX) return MA_ERR_UNSUPPORTED;
  if ((int64_t)batch * heads > (int64_t)INT32_MAX / 2) return MA_ERR_UNSUPPORTED;
  p->tensor_bytes = (size_t)batch * (size_t)heads * (size_t)p->N * (size_t)head_dim * p->elem_bytes;
  p->slice_elems = p->N * p->D;
  switch (r_axes) {
    case 0: p->b2 = 1; break;
    case 1: p->b2 = W; break;
    case 2: p->b2 = (int64_t)H * W; break;
    default: p->b2 = p->N; break;
  }
  p->b1 = p->b2 > 0 ? p->N / p->b2 : 0;
  if (tiled) {
    p->tile_t = tile_t < T ? tile_t : T;
    p->tile_h = tile_h < H ? tile_h : H;
  } else {
    p->tile_t = 0;
    p->tile_h = 0;
  }
  p->r_trivial = p->b2 <= 1;
  p->l_trivial = tiled ? ((int64_t)p->tile_t * p->tile_h <= 1) : (p->b1 <= 1);
  return MA_OK;
}

inline int check_tensor_ptrs(const void *q, const void *k, const void *v, const void *out,
                             size_t bytes) {
  if (!q || !k || !v || !out) return MA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return MA_ERR_ALIGNMENT;
  if (overlaps(out, q, bytes) || overlaps(out, k, bytes) || overlaps(out, v, bytes))
    return MA_ERR_INVALID_ARG;
  return MA_OK;
}

inline size_t workspace_needed(const Problem &p) {
  return (p.empty || p.r_trivial || p.l_trivial) ? 0 : p.tensor_bytes;
}

// Groups of stage R: blocks of b2 contiguous tokens.
inline GroupAddr stage_r_groups(const Problem &p) {
  GroupAddr a{};
  a.n_w = (int32_t)p.b1;
  a.stride_w = (int32_t)p.b2;
  a.n_bi = a.n_bo = 1;
  a.len_i = a.tile_i = (int32_t)p.b2;
  a.stride_in = 1;
  a.len_o = a.tile_o = 1;
  a.stride_out = 0;
  a.max_len = (int32_t)p.b2;
  a.n_groups = a.n_w;
  return a;
}

// Groups of stage L: stride-b2 token sets, or (tile_t x tile_h) boxes of them.
inline GroupAddr stage_l_groups(const Problem &p) {
  GroupAddr a{};
  if (p.tile_t == 0) {
    a.n_w = (int32_t)p.b2;
    a.stride_w = 1;
    a.n_bi = a.n_bo = 1;
    a.len_i = a.tile_i = (int32_t)p.b1;
    a.stride_in = (int32_t)p.b2;
    a.len_o = a.tile_o = 1;
    a.stride_out = 0;
    a.max_len = (int32_t)p.b1;
  } else {
    a.n_w = (int32_t)p.W;
    a.stride_w = 1;
    a.len_i = (int32_t)p.H;
    a.tile_i = p.tile_h;
    a.stride_in = (int32_t)p.W;
    a.len_o = (int32_t)p.T;
    a.tile_o = p.tile_t;
    a.stride_out = (int32_t)(p.H * p.W);
    a.n_bi = (int32_t)((p.H + p.tile_h - 1) / p.tile_h);
    a.n_bo = (int32_t)((p.T + p.tile_t - 1) / p.tile_t);
    a.max_len = p.tile_t * p.tile_h;
  }
  a.n_groups = a.n_w * a.n_bi * a.n_bo;
  return a;
}

// One group holding all N tokens (dense attention).
inline GroupAddr dense_groups(int32_t n) {
  GroupAddr a{};
  a.n_w = 1;
  a.stride_w = 0;
  a.n_bi = a.n_bo = 1;
  a.len_i = a.tile_i = n;
  a.stride_in = 1;
  a.len_o = a.tile_o = 1;
  a.stride_out = 0;
  a.max_len = n;
  a.n_groups = 1;
  return a;
}

}  // namespace ma
