// attn_bf16.h -- bf16 group softmax attention on the gfx950 matrix cores.
//
// One kernel serves stage R (blocks of contiguous tokens), stage L (stride-b2
// token sets, untiled or cut into frame x row boxes) and dense attention: the
// token groups come from a GroupAddr, so stage L gathers its rows straight
// from the natural-order tensors and scatters its output to the same natural
// positions; no permuted copy is written (MonarchRT summaries, nl
// "Methodologie": a product of permutation and block-diagonal factors).
// Like FlashAttention the score matrix never leaves the chip (zh 2.2: the
// custom kernels keep the work in on-chip memory): each workgroup owns up to
// 32*NW queries of one group and streams the group's keys and values through
// LDS in tiles of 64 rows, keeping an online softmax.
//
// Data movement. Key and value tiles go global -> LDS by direct-to-LDS DMA
// (global_load_lds_dwordx4: lane l of an instruction fills LDS bytes
// [16l, 16l+16) of that instruction's 1 KB window), row-major, 2*D bytes per
// row, with the 16-byte chunks of row r permuted by an XOR swizzle so that
// both read patterns below hit distinct LDS banks. With NBUF = 2 the DMA of
// tile t+1 runs while tile t is computed; one barrier per tile.
//
// Matrix-core formulation (v_mfma_f32_32x32x16_bf16: C[32x32] += A[32x16] B[16x32];
// lane l holds A row l%32 and B column l%32, each with 8 k-slots 8*(l/32)+e;
// C element r of lane l sits at row 8*(r/4)+4*(l/32)+r%4, column l%32):
//   S^T = K Q^T      A = key tile (16-byte LDS reads), B = this wave's queries
//   O^T += Y^T P^T   A = value tile read transposed, B = P^T straight from S^T
// With queries on the column index, every per-query scalar (running max,
// running sum, rescale factor) is a per-lane scalar, and the S^T accumulator
// of a 32-key block is already the B operand of two PV steps. The
// k-slot -> head_dim (QK) and k-slot -> key (PV) assignments only have to
// agree between A and B, since each product sums over all k-slots.
// The Y^T operand comes from ds_read_b64_tr_b16, which, inside each group of
// 16 lanes, hands lane j element j%4 of the 8-byte rows fetched by lanes
// j/4, 4+j/4, 8+j/4, 12+j/4 (as its elements 0..3): four source lanes that
// point at four keys and one 4-column run give the receiving lanes one
// head_dim column each across four keys.
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

#define MA_LDS __attribute__((address_space(3)))
#define MA_GLOBAL __attribute__((address_space(1)))

constexpr int kKeyTile = 64;       // keys per LDS tile
constexpr int kQueriesPerWave = 32;
constexpr float kLazyRescale = 8.f;

// Position of 16-byte chunk c of tile row r (CPR chunks per row, a power of 2).
template <int CPR>
__device__ __forceinline__ int swizzle_chunk(int r, int c) {
  constexpr int kBits = CPR >= 2 ? __builtin_ctz(CPR) : 0;
  const int s = ((r << 1) | ((r >> (kBits > 0 ? kBits - 1 : 0)) & 1)) & (CPR - 1);
  return c ^ s;
}

template <int D, int NW, int NBUF>
__global__ __launch_bounds__(NW * 64, 2) void group_attn_bf16(AttnLaunch p) {
  constexpr int NT = NW * 64;
  constexpr int DK = D / 16;              // k-steps of 16 over head_dim for S^T
  constexpr int DB = (D + 31) / 32;       // 32-row blocks of O^T
  constexpr int CPR = D / 8;              // 16-byte chunks per token row
  constexpr int ROWB = 2 * D;             // bytes per tile row
  constexpr int TILEB = kKeyTile * ROWB;  // bytes per tile and tensor
  constexpr int NINST = kKeyTile * CPR / 64;   // DMA instructions per tile and tensor

  // Two distinct LDS objects (not one array indexed by t % 2), so that the
  // compiler can prove the DMA into one buffer never aliases reads of the
  // other and does not wait for the prefetch before computing.
  __shared__ __align__(1024) unsigned char smem0[2 * TILEB];
  __shared__ __align__(1024) unsigned char smem1[NBUF > 1 ? 2 * TILEB : 16];

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
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;

  // DMA of one key tile and its value tile into buffer `buf`. Rows past the
  // group repeat its last member: finite data whose scores are masked to -inf.
  auto issue_tile = [&](int32_t k0, unsigned char *kb_lds) {
    unsigned char *vb_lds = kb_lds + TILEB;
#pragma unroll
    for (int ii = wave; ii < NINST; ii += NW) {
      const int slot = ii * 64 + lane;
      const int r = slot / CPR, pos = slot % CPR;
      const int c = swizzle_chunk<CPR>(r, pos);
      const int32_t km = min(k0 + r, geo.len - 1);
      const int64_t off = (int64_t)member_token(geo, km) * D + c * 8;
      __builtin_amdgcn_global_load_lds((MA_GLOBAL void *)(kh + off), (MA_LDS void *)(kb_lds + ii * 1024),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((MA_GLOBAL void *)(vh + off), (MA_LDS void *)(vb_lds + ii * 1024),
                                       16, 0, 0);
    }
  };

  const int32_t ntiles = (geo.len + kKeyTile - 1) / kKeyTile;
  issue_tile(0, smem0);

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

  // Transposed-read source coordinates of this lane (see the header comment).
  const int tr_grp = lane >> 4, tr_i = lane & 15;
  const int tr_key = 4 * half + (tr_i >> 2);                        // + 32kb + 16h (+8)
  const int tr_col = 16 * (tr_grp & 1) + 4 * (tr_i & 3);           // + 32b

  auto compute_tile = [&](int32_t k0, const unsigned char *ks) {
    const unsigned char *vs = ks + TILEB;
    // S^T for the two 32-key blocks of this tile.
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16_t{};
      const int r = 32 * kb + col;
      bf16x8_t a[DK];
#pragma unroll
      for (int j = 0; j < DK; ++j)
        a[j] = *reinterpret_cast<const bf16x8_t *>(
            ks + r * ROWB + 16 * swizzle_chunk<CPR>(r, (D / 16) * half + j));
#pragma unroll
      for (int j = 0; j < DK; ++j)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], qb[j], s[kb], 0, 0, 0);
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

    // O^T += Y^T P^T. Step (kb, h) covers keys 32kb+16h+[0,16); k-slot e of
    // lane half `half` is key 32kb + 16h + 8(e/4) + 4half + e%4, the key that
    // S^T element r = 8h + e of this lane holds.
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      // head_dim column of this lane's source run; past head_dim (D = 16 only)
      // the whole 16-lane group reads column 0 and feeds zero rows instead.
      const int cidx = 32 * b + tr_col;
      const bool dvalid = (DB * 32 == D) || cidx < D;
      const int cc = dvalid ? cidx : 0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r0 = 32 * kb + 16 * h + tr_key;
          const int r1 = r0 + 8;
          const unsigned char *p0 =
              vs + r0 * ROWB + 16 * swizzle_chunk<CPR>(r0, cc >> 3) + 2 * (cc & 7);
          const unsigned char *p1 =
              vs + r1 * ROWB + 16 * swizzle_chunk<CPR>(r1, cc >> 3) + 2 * (cc & 7);
          const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MA_LDS bf16x4_t *)p0);
          const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MA_LDS bf16x4_t *)p1);
          bf16x8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          if (!dvalid) a = bf16x8_t{};
          oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][h], oacc[b], 0, 0, 0);
        }
    }
  };

  // Tile t lives in smem0 for even t and in smem1 for odd t (NBUF = 2); the
  // DMA of tile t+1 is issued right after the barrier that opens tile t.
  for (int32_t t = 0; t < ntiles; t += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if constexpr (NBUF > 1) {
      if (t + 1 < ntiles) issue_tile((t + 1) * kKeyTile, smem1);
    }
    compute_tile(t * kKeyTile, smem0);
    if (t + 1 >= ntiles) break;
    if constexpr (NBUF > 1) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (t + 2 < ntiles) issue_tile((t + 2) * kKeyTile, smem0);
      compute_tile((t + 1) * kKeyTile, smem1);
    } else {   // single buffer: refill only after every wave is done with it
      __syncthreads();
      issue_tile((t + 1) * kKeyTile, smem0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      compute_tile((t + 1) * kKeyTile, smem0);
      if (t + 2 < ntiles) {
        __syncthreads();
        issue_tile((t + 2) * kKeyTile, smem0);
      }
    }
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
