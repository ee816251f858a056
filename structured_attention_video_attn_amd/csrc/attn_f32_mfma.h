// attn_f32_mfma.h -- fp32 group softmax attention on the gfx950 matrix cores.
//
// The fp32 path for head_dim >= 32: every product is an fp32 x fp32 product
// accumulated in fp32 (v_mfma_f32_32x32x2_f32, no reduced-precision mode),
// and the softmax is evaluated in fp32. A workgroup of NW waves owns 32*NW
// queries of one group and streams the group's keys and values through LDS in
// 32-key tiles with an online softmax (the same running max / lazy rescale as
// the bf16 kernel, at fp32 weights).
//
// Matrix-core formulation (C[32x32] += A[32x2] B[2x32]; lane l holds A row
// l%32 and B column l%32 at k-slot l/32; C element r of lane l sits at row
// 8*(r/4)+4*(l/32)+r%4, column l%32):
//   S^T = K Q^T     step j (of D/2): k-slot h -> head_dim h*D/2 + j. A = key
//                   rows from LDS (one 16-byte read feeds four steps), B = this
//                   lane's query, held in registers.
//   O^T += Y^T P^T  step i (of 16): k-slot h -> key 8(i/4) + 4h + i%4, the key
//                   of S^T element i in this lane, so B is the lane's own
//                   weight p[i]; A = the value tile stored transposed in LDS,
//                   where those four keys of one head_dim row are adjacent.
// Rows past the group are clamped duplicates of its last member (finite);
// their scores are masked to -inf and their outputs never stored.
#pragma once
#include "attn_bf16.h"   // kLazyRescale, swap_halves, f32x16_t
#include "kernels_common.h"

namespace ma {

constexpr int kF32MKeyTile = 32;
typedef float f32x4v_t __attribute__((ext_vector_type(4)));   // a native vector (HIP's float4 is a struct)

// LDS tiles. K: 32 key rows of D floats; Y^T: D head_dim rows of 32 keys.
// Each row is padded by 16 bytes, so the 16 rows one 16-byte read serves
// (consecutive rows, same column) start on 16 distinct groups of 4 banks (of
// 64): K rows are 132 banks apart, Y^T rows 36. Every lane's reads are then
// one base register plus immediates.
template <int D>
struct F32Geo {
  static_assert(D == 32 || D == 64 || D == 128, "fp32 matrix-core path: head_dim 32, 64 or 128");
  static constexpr int KROWB = 4 * D + 16;              // bytes per key row
  static constexpr int YROWB = 4 * kF32MKeyTile + 16;   // bytes per head_dim row of Y^T
  static constexpr int KTB = kF32MKeyTile * KROWB;      // K tile
  static constexpr int YTB = D * YROWB;                 // Y^T tile
  static constexpr int SETB = KTB + YTB;                // one buffer set
  static constexpr int CPR = D / 4;                     // 16-byte chunks per key row in HBM
  static constexpr int DB = D / 32;                     // 32-row head_dim blocks of O^T
};

// NW = 4: two buffer sets (the next tile is stored while the current one is
// read), two workgroups per CU. NW = 2 (groups of at most 64 members, two key
// tiles): one buffer set and four workgroups per CU; the second tile is loaded
// after the first has been used, while the other workgroups keep the CU busy.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void group_attn_f32_mfma(
    AttnLaunch p) {
  using G = F32Geo<D>;
  constexpr int NT = NW * 64;
  constexpr int kSets = NW == 2 ? 1 : 2;
  __shared__ __align__(1024) unsigned char lds[kSets * G::SETB];

  const uint32_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int32_t qt = (int32_t)(bid % (uint32_t)p.n_qtiles);
  const uint32_t rest = bid / (uint32_t)p.n_qtiles;
  const int32_t g = (int32_t)(rest % (uint32_t)p.ga.n_groups);
  const int64_t bh = (int64_t)(rest / (uint32_t)p.ga.n_groups);
  const GroupGeom geo = group_geom(p.ga, g);
  const int32_t qbase = qt * p.q_tile;
  if (qbase >= geo.len) return;   // uniform over the workgroup
  const int32_t qend = min(geo.len, qbase + p.q_tile);

  const float *qh = static_cast<const float *>(p.q) + bh * p.head_elems;
  const float *kh = static_cast<const float *>(p.k) + bh * p.head_elems;
  const float *vh = static_cast<const float *>(p.vals) + bh * p.head_elems;
  float *oh = static_cast<float *>(p.out) + bh * p.head_elems;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int32_t last = geo.len - 1;
  const int32_t n = (geo.len + kF32MKeyTile - 1) / kF32MKeyTile;

  // Tile loads: thread tid takes 16-byte chunks tid + NT*u of the tile (row
  // chunk / CPR, column chunk % CPR): consecutive threads read consecutive
  // bytes of a row. NW = 2 covers the tile in twice the chunks per thread.
  constexpr int UT = kF32MKeyTile * G::CPR / NT;   // chunks per thread per tensor
  static_assert(UT * NT == kF32MKeyTile * G::CPR, "whole chunks per thread");
  f32x4v_t kreg[UT], yreg[UT];
  auto load_tile = [&](int32_t k0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      const int c = tid + NT * u;
      const int r = c / G::CPR, cc = c % G::CPR;
      const int64_t off = (int64_t)member_token(geo, min(k0 + r, last)) * D + 4 * cc;
      kreg[u] = *reinterpret_cast<const f32x4v_t *>(kh + off);
      yreg[u] = *reinterpret_cast<const f32x4v_t *>(vh + off);
    }
  };
  auto store_tile = [&](int buf) __attribute__((always_inline)) {
    unsigned char *kt = lds + buf * G::SETB;
    unsigned char *yt = kt + G::KTB;
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      const int c = tid + NT * u;
      const int r = c / G::CPR, cc = c % G::CPR;
      *reinterpret_cast<f32x4v_t *>(kt + r * G::KROWB + 16 * cc) = kreg[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) *reinterpret_cast<float *>(yt + (4 * cc + e) * G::YROWB + 4 * r) = yreg[u][e];
    }
  };

  // This lane's query (row col of the wave's 32), head_dim [half*D/2, +D/2),
  // as the B operand of the D/2 score steps.
  const int32_t q0 = qbase + 32 * wave;
  const int32_t qm = q0 + col;
  const bool wave_active = q0 < qend;   // wave-uniform
  float qb[D / 2];
  {
    const float *qrow = qh + (int64_t)member_token(geo, min(qm, last)) * D + half * (D / 2);
#pragma unroll
    for (int j = 0; j < D / 2; j += 4) {
      const f32x4v_t x = *reinterpret_cast<const f32x4v_t *>(qrow + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) qb[j + e] = x[e];
    }
  }
  load_tile(0);
  store_tile(0);
  if (kSets == 2 && n > 1) load_tile(kF32MKeyTile);
  __syncthreads();

  // per-lane LDS bases: key reads (row col, head_dim half*D/2 + 4c: + 16c) and
  // value reads (head_dim row 32b + col, keys 8a + 4 half: + 32a)
  const uint32_t kbase = (uint32_t)(col * G::KROWB + half * 2 * D);
  const uint32_t ybase = (uint32_t)(col * G::YROWB + 16 * half);

  f32x16_t oacc[G::DB];
#pragma unroll
  for (int b = 0; b < G::DB; ++b) oacc[b] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;
  const float scale_log2 = p.scale_log2;

  for (int32_t t = 0; t < n; ++t) {
    const unsigned char *kt = lds + (t & (kSets - 1)) * G::SETB + kbase;
    const unsigned char *yt = lds + (t & (kSets - 1)) * G::SETB + G::KTB + ybase;
    if (wave_active) {
      // S^T = K Q^T: two accumulators (even and odd steps), summed at the end
      f32x16_t sa = {}, sb = {};
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        const f32x4v_t kf = *reinterpret_cast<const f32x4v_t *>(kt + 16 * c);
        sa = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[0], qb[4 * c], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[1], qb[4 * c + 1], sb, 0, 0, 0);
        sa = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[2], qb[4 * c + 2], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[3], qb[4 * c + 3], sb, 0, 0, 0);
      }
      f32x16_t s = sa + sb;
      // element r of this lane: key 8(r/4) + 4 half + r%4 of the tile
      const int32_t k0 = t * kF32MKeyTile;
      if (k0 + kF32MKeyTile > geo.len) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (k0 + 8 * (r / 4) + 4 * half + (r % 4) >= geo.len) s[r] = -INFINITY;
      }
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = fmaxf(mx, swap_halves(mx));   // the other 16 keys of the tile for this query
      const float tmax = mx * scale_log2;
      if (__any(tmax > m_run + kLazyRescale)) {
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < G::DB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
        m_run = m_new;
      }
      float pw[16];
      float lsum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pw[r] = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -m_run));
        lsum += pw[r];
      }
      l_run += lsum;
      // O^T += Y^T P^T
#pragma unroll
      for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int b = 0; b < G::DB; ++b) {
          const f32x4v_t yf = *reinterpret_cast<const f32x4v_t *>(yt + b * 32 * G::YROWB + 32 * a);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            oacc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(yf[e], pw[4 * a + e], oacc[b], 0, 0, 0);
        }
      }
    }
    if (t + 1 < n) {
      if constexpr (kSets == 2) {
        // buffer (t+1) % 2 was last read in step t-1, before the barrier that ended it
        store_tile((t + 1) & 1);
        if (t + 2 < n) load_tile((t + 2) * kF32MKeyTile);
      } else {
        __syncthreads();   // every wave is done with tile t
        load_tile((t + 1) * kF32MKeyTile);
        store_tile(0);
      }
      __syncthreads();
    }
  }
  if (!wave_active) return;
  // O^T element r of lane (col, half) in block b: head_dim 32b + 8(r/4) + 4 half + r%4
  const float inv = 1.f / (l_run + swap_halves(l_run));
  if (qm < qend) {
    float *orow = oh + (int64_t)member_token(geo, qm) * D;
#pragma unroll
    for (int b = 0; b < G::DB; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<f32x4v_t *>(orow + 32 * b + 8 * r4 + 4 * half) =
            f32x4v_t{oacc[b][4 * r4] * inv, oacc[b][4 * r4 + 1] * inv, oacc[b][4 * r4 + 2] * inv,
                     oacc[b][4 * r4 + 3] * inv};
  }
}

}  // namespace ma
