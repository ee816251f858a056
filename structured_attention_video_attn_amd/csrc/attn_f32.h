// attn_f32.h -- fp32 group softmax attention on the vector ALUs.
//
// The fp32 path at head_dim 16 (head_dim 32 to 128 take the matrix-core
// kernel of attn_f32_mfma.h): inputs, intermediate Y and output are fp32 and
// every product and exponential is evaluated in fp32. One thread owns one
// query of a group; keys and
// values of the group stream through LDS in tiles and every thread reads the
// same key row (an LDS broadcast). Online softmax (running max, rescaled sum)
// makes one pass over the keys for groups of any length.
#pragma once
#include "kernels_common.h"

namespace ma {

constexpr int kF32Threads = 64;   // one wavefront per workgroup, one query per lane
constexpr int kF32KeyTile = 32;

template <int D>
__global__ __launch_bounds__(kF32Threads) void group_attn_f32(AttnLaunch p) {
  __shared__ __align__(16) float ks[kF32KeyTile][D];
  __shared__ __align__(16) float vs[kF32KeyTile][D];

  const uint32_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int32_t qt = (int32_t)(bid % (uint32_t)p.n_qtiles);
  const uint32_t rest = bid / (uint32_t)p.n_qtiles;
  const int32_t g = (int32_t)(rest % (uint32_t)p.ga.n_groups);
  const int64_t bh = (int64_t)(rest / (uint32_t)p.ga.n_groups);
  const GroupGeom geo = group_geom(p.ga, g);
  if (qt * kF32Threads >= geo.len) return;   // uniform over the workgroup

  const float *qh = static_cast<const float *>(p.q) + bh * p.head_elems;
  const float *kh = static_cast<const float *>(p.k) + bh * p.head_elems;
  const float *vh = static_cast<const float *>(p.vals) + bh * p.head_elems;
  float *oh = static_cast<float *>(p.out) + bh * p.head_elems;

  const int lane = threadIdx.x;
  const int32_t qm = qt * kF32Threads + lane;
  const bool qvalid = qm < geo.len;
  const int32_t qtok = qvalid ? member_token(geo, qm) : 0;

  float q[D], o[D];
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    float4 x = qvalid ? *reinterpret_cast<const float4 *>(qh + (int64_t)qtok * D + d)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
    q[d] = x.x; q[d + 1] = x.y; q[d + 2] = x.z; q[d + 3] = x.w;
    o[d] = o[d + 1] = o[d + 2] = o[d + 3] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  constexpr int kChunks = kF32KeyTile * D / 4;   // float4 chunks per tile and tensor
  for (int32_t k0 = 0; k0 < geo.len; k0 += kF32KeyTile) {
    for (int c = lane; c < kChunks; c += kF32Threads) {
      const int r = c / (D / 4), cc = (c % (D / 4)) * 4;
      const int32_t km = k0 + r;
      float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
      if (km < geo.len) {
        const int64_t off = (int64_t)member_token(geo, km) * D + cc;
        kx = *reinterpret_cast<const float4 *>(kh + off);
        vx = *reinterpret_cast<const float4 *>(vh + off);
      }
      *reinterpret_cast<float4 *>(&ks[r][cc]) = kx;
      *reinterpret_cast<float4 *>(&vs[r][cc]) = vx;
    }
    __syncthreads();
    const int nk = min(kF32KeyTile, geo.len - k0);
    for (int kk = 0; kk < nk; ++kk) {
      float x = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) x = fmaf(q[d], ks[kk][d], x);
      x *= p.scale;
      const float m_new = fmaxf(m, x);
      const float corr = expf(m - m_new);
      const float e = expf(x - m_new);
      l = fmaf(l, corr, e);
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(o[d], corr, e * vs[kk][d]);
      m = m_new;
    }
    __syncthreads();
  }
  if (qvalid) {
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < D; d += 4)
      *reinterpret_cast<float4 *>(oh + (int64_t)qtok * D + d) =
          make_float4(o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv);
  }
}

}  // namespace ma
