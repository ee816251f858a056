// group_addr.h -- which tokens form one softmax group, for every kernel launch.
//
// Each stage of Monarch attention is softmax attention restricted to token
// groups (MonarchRT summaries: nl "Methodologie" -- permutation and
// block-diagonal factors; zh 2.2 -- blocks aligned to whole grid axes; zh 2.2
// "Tiled Monarch" -- a block split into tiles). All groups of one launch are
// described by one GroupAddr; a kernel maps (group g, member m) to a token
// index with integer arithmetic, so the stride permutation of stage L is pure
// addressing and no permuted copy of any tensor exists.
//
//   g = (bo * n_bi + bi) * n_w + w
//   base(g)   = w*stride_w + bi*tile_i*stride_in + bo*tile_o*stride_out
//   len_i(g)  = min(tile_i, len_i - bi*tile_i),  len_o(g) = min(tile_o, len_o - bo*tile_o)
//   token(g, m) = base(g) + (m / len_i(g))*stride_out + (m % len_i(g))*stride_in,
//   m in [0, len_i(g)*len_o(g)).
//
// Instances (b2 = intra-block length, b1 = number of blocks, N = b1*b2):
//   stage R blocks:   n_w = b1, stride_w = b2, len_i = tile_i = b2, stride_in = 1
//   stage L untiled:  n_w = b2, stride_w = 1,  len_i = tile_i = b1, stride_in = b2
//   stage L tiled:    n_w = W,  stride_w = 1,  (len_i, tile_i, stride_in) = (H, tile_h, W),
//                     (len_o, tile_o, stride_out) = (T, tile_t, H*W)
//   dense:            n_w = 1,  len_i = tile_i = N, stride_in = 1
// (unused outer axis: len_o = tile_o = 1).
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define MA_HD __host__ __device__ __forceinline__
#else
#define MA_HD inline
#endif

struct GroupAddr {
  int32_t n_w, n_bi, n_bo;
  int32_t stride_w, stride_in, stride_out;
  int32_t len_i, tile_i, len_o, tile_o;
  int32_t max_len;   // largest group, min(tile_i, len_i) * min(tile_o, len_o)
  int32_t n_groups;  // n_w * n_bi * n_bo
};

struct GroupGeom {
  int32_t base;
  int32_t len_i;    // members along the inner axis in this group
  int32_t len;      // members in this group
  int32_t two_level;   // len_o(g) > 1 (an int: GroupGeom has no padding bytes to copy)
  int32_t stride_in, stride_out;
};

MA_HD GroupGeom group_geom(const GroupAddr &a, int32_t g) {
  int32_t w = g % a.n_w;
  int32_t rest = g / a.n_w;
  int32_t bi = rest % a.n_bi;
  int32_t bo = rest / a.n_bi;
  int32_t li = a.len_i - bi * a.tile_i;
  li = li < a.tile_i ? li : a.tile_i;
  int32_t lo = a.len_o - bo * a.tile_o;
  lo = lo < a.tile_o ? lo : a.tile_o;
  GroupGeom r;
  r.base = w * a.stride_w + bi * a.tile_i * a.stride_in + bo * a.tile_o * a.stride_out;
  r.len_i = li;
  r.len = li * lo;
  r.two_level = lo > 1 ? 1 : 0;
  r.stride_in = a.stride_in;
  r.stride_out = a.stride_out;
  return r;
}

MA_HD int32_t member_token(const GroupGeom &gg, int32_t m) {
  if (!gg.two_level) return gg.base + m * gg.stride_in;
  int32_t o = m / gg.len_i;
  int32_t x = m - o * gg.len_i;
  return gg.base + o * gg.stride_out + x * gg.stride_in;
}

// MI355X dispatches consecutive workgroup ids round-robin over its 8 XCDs,
// each with a private L2. Remap so that ids adjacent in the logical order
// (the query tiles of one group, which read the same keys and values) land
// on the same XCD at about the same time. Bijective on [0, n).
MA_HD uint32_t xcd_remap(uint32_t b, uint32_t n) {
  constexpr uint32_t kXcd = 8;
  const uint32_t per = n / kXcd, rem = n % kXcd;
  const uint32_t xcd = b % kXcd, slot = b / kXcd;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}
