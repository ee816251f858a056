// attn_bf16.h -- bf16 group softmax attention on the gfx950 matrix cores.
//
// One kernel serves stage R (blocks of contiguous tokens), stage L (stride-b2
// token sets, untiled or cut into frame x row boxes) and dense attention: the
// token groups come from a GroupAddr, so stage L gathers its rows straight
// from the natural-order tensors and scatters its output to the same natural
// positions; no permuted copy is written (MonarchRT summaries, nl
// "Methodologie": a product of permutation and block-diagonal factors).
// Like FlashAttention the score matrix never leaves the chip (zh 2.2, custom
// kernels keep the work in on-chip memory): each workgroup owns up to 32*NW
// queries of one group and streams the group's keys and values through LDS
// in tiles of 64, keeping an online softmax.
//
// Matrix-core formulation (v_mfma_f32_32x32x16_bf16: C[32x32] += A[32x16] B[16x32];
// lane l holds A row l%32 and B column l%32, each with 8 consecutive
// k-slots 8*(l/32)+e; C element r of lane l sits at row 8*(r/4)+4*(l/32)+r%4,
// column l%32):
//   S^T = K Q^T      A = key tile from LDS, B = this wave's queries (registers)
//   O^T += Y^T P^T   A = value tile, transposed in LDS, B = P^T straight from S^T
// With queries on the column index, every per-query scalar (running max,
// running sum, rescale factor) is a per-lane scalar, and the S^T accumulator
// of a 32-key block is already the B operand of two PV steps. The
// k-slot -> head_dim (QK) and k-slot -> key (PV) assignments only have to
// agree between A and B, since each product sums over all k-slots; they are
// chosen so that every operand is one contiguous 16- or 8-byte read.
//
// Softmax: exp2 with the scale s*log2(e) folded into one FMA per score; the
// running max only moves (and the accumulator is only rescaled) when a tile's
// max exceeds it by more than 8 (log2 units), so unnormalised weights stay
// below 2^8 and the result is unchanged up to rounding.
#pragma once
#include "kernels_common.h"

namespace ma {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint16_t u16;

constexpr int kKeyTile = 64;       // keys per LDS tile
constexpr int kQueriesPerWave = 32;
constexpr float kLazyRescale = 8.f;

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void group_attn_bf16(AttnLaunch p) {
  constexpr int NT = NW * 64;
  constexpr int DK = D / 16;              // k-steps of 16 over head_dim for S^T
  constexpr int DB = (D + 31) / 32;       // 32-row blocks of O^T
  constexpr int DR = DB * 32;             // rows of the transposed value tile
  constexpr int KSTR = D + 8;             // bf16 per key-tile row (16 B pad: no bank conflicts)
  constexpr int YSTR = kKeyTile + 4;      // bf16 per transposed value row (8 B pad)
  constexpr int CPR = D / 8;              // 16-byte chunks per token row
  constexpr int NCH = kKeyTile * CPR;     // chunks per tile and tensor
  constexpr int CPT = (NCH + NT - 1) / NT;

  __shared__ __align__(16) u16 ks[kKeyTile * KSTR];
  __shared__ __align__(16) u16 yt[DR * YSTR];

  const uint32_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int32_t qt = (int32_t)(bid % (uint32_t)p.n_qtiles);
  const uint32_t rest = bid / (uint32_t)p.n_qtiles;
  const int32_t g = (int32_t)(rest % (uint32_t)p.ga.n_groups);
  const int64_t bh = (int64_t)(rest / (uint32_t)p.ga.n_groups);
  const GroupGeom geo = group_geom(p.ga, g);
  if (qt * (kQueriesPerWave * NW) >= geo.len) return;   // uniform over the workgroup

  const u16 *qh = static_cast<const u16 *>(p.q) + bh * p.head_elems;
  const u16 *kh = static_cast<const u16 *>(p.k) + bh * p.head_elems;
  const u16 *vh = static_cast<const u16 *>(p.vals) + bh * p.head_elems;
  u16 *oh = static_cast<u16 *>(p.out) + bh * p.head_elems;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;

  if constexpr (DR > D) {   // value rows past head_dim stay zero for the whole kernel
    for (int i = tid; i < (DR - D) * YSTR; i += NT) yt[D * YSTR + i] = 0;
  }

  // This lane's query (column of S^T), head_dim slots [D/2*half, D/2*half + D/2).
  const int32_t qm = qt * (kQueriesPerWave * NW) + wave * kQueriesPerWave + col;
  const bool qvalid = qm < geo.len;
  const int32_t qtok = qvalid ? member_token(geo, qm) : 0;
  bf16x8_t qb[DK];
  {
    const u16 *qrow = qh + (int64_t)qtok * D + (D / 2) * half;
#pragma unroll
    for (int j = 0; j < DK; ++j) {
      uint4 x = qvalid ? *reinterpret_cast<const uint4 *>(qrow + 8 * j) : make_uint4(0, 0, 0, 0);
      qb[j] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  f32x16_t oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[b] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

  uint4 kreg[CPT], yreg[CPT];
  auto load_tile = [&](int32_t k0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      kreg[i] = yreg[i] = make_uint4(0, 0, 0, 0);
      if (NCH % NT == 0 || c < NCH) {
        const int r = c / CPR, cc = c % CPR;
        const int32_t km = k0 + r;
        if (km < geo.len) {
          const int64_t off = (int64_t)member_token(geo, km) * D + cc * 8;
          kreg[i] = *reinterpret_cast<const uint4 *>(kh + off);
          yreg[i] = *reinterpret_cast<const uint4 *>(vh + off);
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (NCH % NT == 0 || c < NCH) {
        const int r = c / CPR, cc = c % CPR;
        *reinterpret_cast<uint4 *>(&ks[r * KSTR + cc * 8]) = kreg[i];
        const uint32_t w4[4] = {yreg[i].x, yreg[i].y, yreg[i].z, yreg[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          yt[(cc * 8 + 2 * e) * YSTR + r] = (u16)(w4[e] & 0xffffu);
          yt[(cc * 8 + 2 * e + 1) * YSTR + r] = (u16)(w4[e] >> 16);
        }
      }
    }
  };

  const int32_t ntiles = (geo.len + kKeyTile - 1) / kKeyTile;
  load_tile(0);
  for (int32_t t = 0; t < ntiles; ++t) {
    const int32_t k0 = t * kKeyTile;
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) load_tile(k0 + kKeyTile);

    // S^T for the two 32-key blocks of this tile.
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16_t{};
      const u16 *krow = &ks[(32 * kb + col) * KSTR + (D / 2) * half];
#pragma unroll
      for (int j = 0; j < DK; ++j) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(krow + 8 * j);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[j], s[kb], 0, 0, 0);
      }
    }
    if (k0 + kKeyTile > geo.len) {   // ragged last tile: keys past the group get -inf
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int32_t key = k0 + 32 * kb + 8 * (r / 4) + 4 * half + (r % 4);
          if (key >= geo.len) s[kb][r] = -INFINITY;
        }
    }

    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));          // the other 32 keys of this query
    const float tmax = mx * p.scale_log2;
    if (__any(tmax > m_run + kLazyRescale)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
      m_run = m_new;
    }

    bf16x8_t pb[2][2];
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = exp2f(fmaf(s[kb][r], p.scale_log2, -m_run));
        lsum += e;
        pb[kb][r / 8][r % 8] = (__bf16)e;
      }
    l_run += lsum;

    // O^T += Y^T P^T. Step (kb, h) covers keys 32kb+16h+[0,16); k-slot e of lane
    // half `half` is key 32kb + 16h + 8(e/4) + 4half + e%4, the key that S^T
    // element r = 8h + e of this lane holds.
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const u16 *yrow = &yt[(32 * b + col) * YSTR + 4 * half];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u16 *src = yrow + 32 * kb + 16 * h;
          const bf16x4_t lo = *reinterpret_cast<const bf16x4_t *>(src);
          const bf16x4_t hi = *reinterpret_cast<const bf16x4_t *>(src + 8);
          const bf16x8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][h], oacc[b], 0, 0, 0);
        }
    }
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qvalid) {
    const float inv = 1.f / l_tot;
    u16 *orow = oh + (int64_t)qtok * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * b + 8 * rq + 4 * half;
        if (d0 < D) {
          bf16x4_t v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (__bf16)(oacc[b][4 * rq + e] * inv);
          *reinterpret_cast<bf16x4_t *>(orow + d0) = v;
        }
      }
  }
}

}  // namespace ma
