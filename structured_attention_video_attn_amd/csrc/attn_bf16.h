// attn_bf16.h -- bf16 group softmax attention on the gfx950 matrix cores.
//
// Two kernels run softmax attention inside token groups described by a
// GroupAddr, so stage L gathers its rows straight from the natural-order
// tensors and scatters its output to the same natural positions; no permuted
// copy is written (MonarchRT summaries, nl "Methodologie": a product of
// permutation and block-diagonal factors). Like FlashAttention the score
// matrix never leaves the chip (zh 2.2: the custom kernels keep the work in
// on-chip memory).
//
//   group_attn_bf16  groups longer than 64 tokens (stage L, long stage-R
//                    blocks, dense): a workgroup of 4 waves owns up to 128
//                    queries of one group, 32 per wave (under chunk-causal
//                    spans each wave's 32 come from one span), and streams the
//                    group's keys and values through LDS in 64-row tiles with
//                    an online softmax; each tile runs in a fixed instruction
//                    order that keeps LDS reads ahead of the MFMAs and puts the
//                    second 32-key block's exponentials between the first
//                    block's PV MFMAs.
//   block_attn_bf16  groups of at most 64 tokens (stage R's W-row blocks,
//                    small tiles): persistent workgroups of 2 waves walk over
//                    the groups, one group at a time; four of them resident
//                    per CU keep HBM requests in flight while each computes.
//
// Data movement. Key and value tiles go global -> LDS by direct-to-LDS DMA
// (global_load_lds_dwordx4: lane l of an instruction fills LDS bytes
// [16l, 16l+16) of that instruction's 1 KB window), row-major, 2*D bytes per
// row, with the 16-byte chunks of row r permuted by an XOR swizzle so that
// both read patterns below hit distinct LDS banks. The block kernel's
// buffers are separate LDS objects, so the compiler can prove that its
// builtin DMAs in flight never alias the buffer being read; the streaming
// kernel issues its DMAs through an inline-asm wrapper the compiler does not
// track (see dma16) and orders them itself.
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
// Softmax: exp2 with the scale s*log2(e) folded into one FMA per score
// (v_exp_f32 directly: weights that would be denormal are negligible); the
// running max only moves (and the accumulator is only rescaled) when a
// tile's max exceeds it by more than 8 (log2 units), so unnormalised weights
// stay below 2^8 and the result is unchanged up to rounding.
#pragma once
#include <type_traits>

#include "kernels_common.h"

namespace ma {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint16_t u16;

#define MA_LDS __attribute__((address_space(3)))
#define MA_GLOBAL __attribute__((address_space(1)))

constexpr int kKeyTile = 64;       // keys per LDS tile
constexpr int kQueriesPerWave = 32;
constexpr int kBlockWaves = 2;     // waves per block_attn_bf16 workgroup
constexpr int kBlockResident = 4;  // resident block_attn_bf16 workgroups per CU (LDS 32 KB, <= 256 VGPRs)
constexpr float kLazyRescale = 8.f;

template <int D>
struct TileGeo {
  static constexpr int DK = D / 16;              // k-steps of 16 over head_dim for S^T
  static constexpr int DB = (D + 31) / 32;       // 32-row blocks of O^T
  static constexpr int CPR = D / 8;              // 16-byte chunks per token row
  static constexpr int ROWB = 2 * D;             // bytes per tile row
  static constexpr int TILEB = kKeyTile * ROWB;  // bytes per tile
  static constexpr int NINST = kKeyTile * CPR / 64;   // DMA instructions per tile
  static constexpr int ROWS_PER_INST = 64 / CPR;
};

// Position of 16-byte chunk c of tile row r (CPR chunks per row, a power of 2).
// The LDS serves 256 bytes (64 banks) per cycle: a 16-byte read of one chunk
// column serves 16 lanes, one tile row each, and an 8-byte transposed value
// read serves 32 lanes over four consecutive rows and a quarter of the
// columns each. Row r gets an XOR mask that depends on r mod 16 only, chosen
// so that neither read meets a bank twice (rows of 256 bytes fill a bank line
// at head_dim 128; at 64, 32 and 16 two, four and eight rows share one):
//   D = 128: row 4q + p gets 4p + q;      D = 64: bit 1 of r -> bit 2, bits 2-3 -> bits 0-1;
//   D = 32:  bits 2-3 of r;               D = 16: bit 3 of r.
template <int CPR>
__device__ __forceinline__ int swizzle_chunk(int r, int c) {
  if constexpr (CPR == 16) {
    return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  } else if constexpr (CPR == 8) {
    return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  } else if constexpr (CPR == 4) {
    return c ^ ((r >> 2) & 3);
  } else if constexpr (CPR == 2) {
    return c ^ ((r >> 3) & 1);
  } else {
    return c;
  }
}

__device__ __forceinline__ float swap_halves(float x) {   // value of lane l ^ 32
  auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? pr[0] : pr[1]);
}

// This lane's query as the B operand of S^T = K Q^T: head_dim slots
// [D/2*half + 8j, +8) for k-step j.
template <int D>
__device__ __forceinline__ void load_query(const u16 *qh, const GroupGeom &geo, int32_t qm, int half,
                                           bf16x8_t *qb) {
  const bool valid = qm < geo.len;
  const u16 *qrow = qh + (uint32_t)(valid ? member_token(geo, qm) : 0) * D + (D / 2) * half;
#pragma unroll
  for (int j = 0; j < D / 16; ++j) {
    const uint4 x = valid ? *reinterpret_cast<const uint4 *>(qrow + 8 * j) : make_uint4(0, 0, 0, 0);
    qb[j] = __builtin_bit_cast(bf16x8_t, x);
  }
}

// S^T for both 32-key blocks of an LDS key tile. The two accumulators are
// independent chains, interleaved so the matrix pipe never waits on a
// result; key operands are fetched in batches of 4 k-steps per block to
// bound register pressure. hook(i) runs after batch i (0 .. 2*DK/B - 1).
template <int D, typename Hook>
__device__ __forceinline__ void qk_tile(const unsigned char *ks, const bf16x8_t *qb, int col, int half,
                                        f32x16_t &s0, f32x16_t &s1, Hook &&hook) {
  using G = TileGeo<D>;
  constexpr int B = G::DK < 4 ? G::DK : 4;
  const int r0 = col, r1 = 32 + col;
  f32x16_t a0 = {}, a1 = {};
#pragma unroll
  for (int j0 = 0; j0 < G::DK; j0 += B) {
    bf16x8_t k0[B], k1[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int c = (D / 16) * half + j0 + j;
      k0[j] = *reinterpret_cast<const bf16x8_t *>(ks + r0 * G::ROWB + 16 * swizzle_chunk<G::CPR>(r0, c));
      k1[j] = *reinterpret_cast<const bf16x8_t *>(ks + r1 * G::ROWB + 16 * swizzle_chunk<G::CPR>(r1, c));
    }
#pragma unroll
    for (int j = 0; j < B; ++j) {
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0[j], qb[j0 + j], a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1[j], qb[j0 + j], a1, 0, 0, 0);
    }
    hook(2 * (j0 / B));
    hook(2 * (j0 / B) + 1);
  }
  s0 = a0;
  s1 = a1;
}

// Online-softmax update for one 32-key block of scores (keys k0.. of a group
// of len): mask, running max (lazy), exp2, running sum; returns P^T as the
// B operands of the block's two PV steps.
template <int DB>
__device__ __forceinline__ void softmax_block(f32x16_t &s, int32_t k0, int32_t len, int half,
                                              float scale_log2, float &m_run, float &l_run,
                                              f32x16_t *oacc, bf16x8_t (&pb)[2]) {
  if (k0 + 32 > len) {   // ragged block: keys past the group get -inf
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int32_t key = k0 + 8 * (r / 4) + 4 * half + (r % 4);
      if (key >= len) s[r] = -INFINITY;
    }
  }
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
  mx = fmaxf(mx, swap_halves(mx));   // the other 16 keys of this query
  const float tmax = mx * scale_log2;
  if (__any(tmax > m_run + kLazyRescale)) {
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
    m_run = m_new;
  }
  float lsum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const float e0 = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -m_run));
    const float e1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1], scale_log2, -m_run));
    lsum += e0 + e1;
    const bf16x2_t pr = __builtin_convertvector((f32x2_t){e0, e1}, bf16x2_t);   // v_cvt_pk_bf16_f32
    pb[r / 8][r % 8] = pr[0];
    pb[r / 8][r % 8 + 1] = pr[1];
  }
  l_run += lsum;
}

// O^T += Y^T P^T for 32-key block kb of an LDS value tile. Step h covers keys
// 32kb+16h+[0,16); k-slot e of lane half `half` is key 32kb + 16h + 8(e/4) +
// 4half + e%4, the key that S^T element r = 8h + e of this lane holds.
template <int D, typename Hook>
__device__ __forceinline__ void pv_block(const unsigned char *vs, const bf16x8_t (&pb)[2], int kb,
                                         f32x16_t *oacc, int tr_key, int tr_col, Hook &&hook) {
  using G = TileGeo<D>;
#pragma unroll
  for (int h = 0; h < 2; ++h) {   // k-step outer: the DB accumulators are independent chains
    const int r0 = 32 * kb + 16 * h + tr_key;
    const int r1 = r0 + 8;
#pragma unroll
    for (int b = 0; b < G::DB; ++b) {
      // head_dim column of this lane's source run; past head_dim (D = 16 only)
      // the whole 16-lane group reads column 0 and feeds zero rows instead.
      const int cidx = 32 * b + tr_col;
      const bool dvalid = (G::DB * 32 == D) || cidx < D;
      const int cc = dvalid ? cidx : 0;
      const unsigned char *p0 = vs + r0 * G::ROWB + 16 * swizzle_chunk<G::CPR>(r0, cc >> 3) + 2 * (cc & 7);
      const unsigned char *p1 = vs + r1 * G::ROWB + 16 * swizzle_chunk<G::CPR>(r1, cc >> 3) + 2 * (cc & 7);
      const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MA_LDS bf16x4_t *)p0);
      const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MA_LDS bf16x4_t *)p1);
      bf16x8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      if (!dvalid) a = bf16x8_t{};
      oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[h], oacc[b], 0, 0, 0);
      if (h == 1) hook(G::DB * kb + b);   // d-block index across the two 32-key blocks
    }
  }
}

// One 64-key tile: QK(block 1) is issued before the softmax of block 0 and
// PV(block 0) before the softmax of block 1, so matrix-core work is in
// flight while the vector ALUs run each softmax. `on_qk(i)` runs after each
// batch of QK MFMAs and `on_pv(i)` after each PV d-block; the streaming
// kernel issues its next DMA instructions there one at a time, so that no
// wave stalls behind a burst of its own memory instructions.
template <int D, typename FQ, typename FP>
__device__ __forceinline__ void attend_tile(const unsigned char *ks, const unsigned char *vs,
                                            const bf16x8_t *qb, int32_t k0, int32_t len, float scale_log2,
                                            float &m_run, float &l_run, f32x16_t *oacc, int col, int half,
                                            int tr_key, int tr_col, FQ &&on_qk, FP &&on_pv) {
  constexpr int DB = TileGeo<D>::DB;
  f32x16_t s0, s1;
  qk_tile<D>(ks, qb, col, half, s0, s1, on_qk);
  bf16x8_t pb[2];
  softmax_block<DB>(s0, k0, len, half, scale_log2, m_run, l_run, oacc, pb);
  pv_block<D>(vs, pb, 0, oacc, tr_key, tr_col, on_pv);
  softmax_block<DB>(s1, k0 + 32, len, half, scale_log2, m_run, l_run, oacc, pb);
  pv_block<D>(vs, pb, 1, oacc, tr_key, tr_col, on_pv);
}

template <int D>
__device__ __forceinline__ void attend_tile(const unsigned char *ks, const unsigned char *vs,
                                            const bf16x8_t *qb, int32_t k0, int32_t len, float scale_log2,
                                            float &m_run, float &l_run, f32x16_t *oacc, int col, int half,
                                            int tr_key, int tr_col) {
  attend_tile<D>(ks, vs, qb, k0, len, scale_log2, m_run, l_run, oacc, col, half, tr_key, tr_col,
                 [](int) {}, [](int) {});
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------
// Streaming kernel for groups longer than one key tile.
//
// A workgroup of NW waves owns up to 32*NW queries of one group (p.q_tile of
// them; waves whose queries all lie past that share skip the math but still
// take part in the DMA and the barriers). Every wave reads the workgroup's
// shared key/value tiles.
//
// Rings: key tiles in three LDS buffers (tile t in buffer t % 3), value tiles
// in two (t % 2). While computing tile t a wave issues the value windows of
// tile t+1 between its QK MFMAs and the key windows of tile t+2 between its
// PV MFMAs, one DMA instruction at a time. Vector-memory loads retire in
// order, so the wait that opens tile t can leave the newest key windows
// (tile t+1) in flight. DMAs for tiles past the group are issued anyway from
// clamped rows (the last member, one cache line per row) into buffers no wave
// reads again: the tile loop then has no data-dependent branches, and the
// per-wave count of outstanding DMAs is the same at every tile.

// Token of group member m for the DMA address: base + (m / len_i) * stride_out
// + (m % len_i) * stride_in. The quotient uses a double reciprocal: for
// 0 <= m < 2^31 the truncated product m * (1/len_i) is within 2^-21 of m/len_i
// relative to 1/len_i, so it is the exact quotient or, when len_i divides m,
// one less; the remainder test repairs that. One-level groups have
// len_i = len > m, so the quotient is 0 there.
struct RowMap {
  int32_t base, len_i, stride_in, stride_out, last;
  double rcp;
};

__device__ __forceinline__ RowMap row_map(const GroupGeom &g) {
  RowMap r;
  r.base = g.base;
  r.len_i = g.len_i;
  r.stride_in = g.stride_in;
  r.stride_out = g.stride_out;
  r.last = g.len - 1;
  r.rcp = 1.0 / (double)g.len_i;
  return r;
}

__device__ __forceinline__ uint32_t row_token(const RowMap &rm, int32_t m) {
  int32_t o = (int32_t)((double)m * rm.rcp);
  int32_t x = m - o * rm.len_i;
  const bool up = x >= rm.len_i;
  o += up ? 1 : 0;
  x -= up ? rm.len_i : 0;
  return (uint32_t)(rm.base + o * rm.stride_out + x * rm.stride_in);
}

// One global_load_lds_dwordx4 (lane l: 16 bytes from src + off_l to LDS
// lds_dst + 16 l), written as inline assembly. The compiler's wait insertion
// models the builtin form as a FLAT access that may also complete through the
// LDS counter, out of order, and then makes every wait for an LDS read a full
// lgkmcnt(0), which stalls each MFMA on the reads issued ahead for the next
// one. The streaming kernel orders its DMAs with explicit vmcnt waits and
// barriers instead, so the compiler need not see them. No register is
// written: the instruction only reads its address operands at issue.
__device__ __forceinline__ void dma16(const unsigned char *src, uint32_t off, unsigned char *lds_dst) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(MA_LDS unsigned char *)lds_dst;
  // s_nop: one wait state between the M0 write and the DMA that reads it
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(src), "{m0}"(lds_addr) : "memory");
}

// A workgroup-uniform pointer, held in scalar registers (the DMA's base operand).
__device__ __forceinline__ const unsigned char *uniform_ptr(const unsigned char *p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  // readfirstlane returns int: go through uint32_t so the low word is not sign-extended
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<const unsigned char *>((uintptr_t)((hi << 32) | lo));
}

// DMA window ii (1 KB: 64 lanes x 16 bytes) of the tile holding group rows
// [k0, k0 + 64); rows past the group repeat its last member.
template <int D>
__device__ __forceinline__ void dma_row_window(const unsigned char *src, unsigned char *dst, const RowMap &rm,
                                               int32_t k0, int ii, int lane) {
  using G = TileGeo<D>;
  const int slot = ii * 64 + lane;
  const int r = slot / G::CPR, pos = slot % G::CPR;
  const int c = swizzle_chunk<G::CPR>(r, pos);
  const int32_t km = min(k0 + r, rm.last);
  // offsets inside one (batch, head) slice fit in 32 bits (N * D < 2^31 elements)
  const uint32_t off = (row_token(rm, km) * D + c * 8) * 2u;
  dma16(src, off, dst + ii * 1024);
}

// Two softmax weights (scores s[r], s[r+1]) of this lane's query: exp2 of the
// scaled score minus the running max, packed to bf16 into the P^T operand and
// added to the running sum.
__device__ __forceinline__ void exp_pair(const f32x16_t &s, int r, float scale_log2, float m_run, float &lsum,
                                         bf16x8_t (&pb)[2]) {
  const float e0 = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -m_run));
  const float e1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1], scale_log2, -m_run));
  const bf16x2_t pr = __builtin_convertvector((f32x2_t){e0, e1}, bf16x2_t);   // v_cvt_pk_bf16_f32
  // running sum of the rounded weights (the values the PV MFMA multiplies), one dot2 per pair
  lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, (bf16x2_t){(__bf16)1.f, (__bf16)1.f}, lsum, false);
  pb[r / 8][r % 8] = pr[0];
  pb[r / 8][r % 8 + 1] = pr[1];
}

// The same for scores that already are log2-scaled and relative to the running
// reference (the streaming kernel folds both into the QK accumulator).
__device__ __forceinline__ void exp_pair_shifted(const f32x16_t &s, int r, float &lsum, bf16x8_t (&pb)[2]) {
  const float e0 = __builtin_amdgcn_exp2f(s[r]);
  const float e1 = __builtin_amdgcn_exp2f(s[r + 1]);
  const bf16x2_t pr = __builtin_convertvector((f32x2_t){e0, e1}, bf16x2_t);   // v_cvt_pk_bf16_f32
  lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, (bf16x2_t){(__bf16)1.f, (__bf16)1.f}, lsum, false);
  pb[r / 8][r % 8] = pr[0];
  pb[r / 8][r % 8 + 1] = pr[1];
}

// Per-lane LDS byte offsets of the streaming tile's fragment reads, relative
// to the tile buffer: computed once per kernel, so that each read is one
// ds_read with the buffer (and row-block) base in its immediate offset. The
// XOR swizzle of row r depends only on r mod 16, so value rows
// 32kb + 16h + tr_key (+8) share the offsets of rows tr_key (+8).
template <int D>
struct LaneOffsets {
  uint32_t k[TileGeo<D>::DK];        // key row col, chunk (D/16) half + j
  uint32_t ya[TileGeo<D>::DB];       // value row tr_key, head_dim column 32b + tr_col
  uint32_t yb[TileGeo<D>::DB];       // value row tr_key + 8, same column
};

template <int D>
__device__ __forceinline__ LaneOffsets<D> lane_offsets(int col, int half, int tr_key, int tr_col) {
  using G = TileGeo<D>;
  LaneOffsets<D> o;
#pragma unroll
  for (int j = 0; j < G::DK; ++j)
    o.k[j] = (uint32_t)(col * G::ROWB + 16 * swizzle_chunk<G::CPR>(col, G::DK * half + j));
#pragma unroll
  for (int b = 0; b < G::DB; ++b) {
    // head_dim column of this lane's source run; past head_dim (D = 16 only)
    // the whole 16-lane group reads column 0 (and the tile feeds zero rows).
    const int cidx = 32 * b + tr_col;
    const int cc = (G::DB * 32 == D) || cidx < D ? cidx : 0;
    const int ra = tr_key, rb = tr_key + 8;
    o.ya[b] = (uint32_t)(ra * G::ROWB + 16 * swizzle_chunk<G::CPR>(ra, cc >> 3) + 2 * (cc & 7));
    o.yb[b] = (uint32_t)(rb * G::ROWB + 16 * swizzle_chunk<G::CPR>(rb, cc >> 3) + 2 * (cc & 7));
  }
  return o;
}

// One 64-key tile in a fixed instruction order. Scheduling barriers split the
// tile into slots of one or two MFMAs each, so the compiler keeps the LDS
// reads two MFMA slots ahead of their use (it would otherwise sink every read
// next to its MFMA and wait for it there) and places the work listed per slot:
//   QK slots j = 0..DK-1:    S^T of both 32-key blocks at k-step j, key
//                            fragments of k-step j+2, on_qk(j)
//   softmax:                 mask, tile max, one lazy-rescale decision for
//                            the whole tile, weights of block 0
//   PV slots i = 0..4DB-1:   one O^T += Y^T P^T step, value fragments of step
//                            i+2, on_pv(i); during block 0's steps also the
//                            weights of block 1, two scores per slot (DB = 4)
// One rescale decision per tile (instead of per 32-key block) keeps block 1's
// weights free of any write to the accumulators that block 0's MFMAs update.
// kHalf: the tile's second 32-key block lies wholly past the keys (a group's
// ragged last tile), so only block 0's products and weights are formed, in the
// same order as in a full tile (the results are the full tile's, bit for bit).
template <int D, bool kHalf = false, typename FQ, typename FP>
__device__ __forceinline__ void stream_tile(const unsigned char *ks, const unsigned char *vs,
                                            const bf16x8_t *qb, int32_t k0, int32_t len, bool first,
                                            f32x16_t &negm, float &m_run, float &l_run, f32x16_t *oacc,
                                            int half, int tr_col, const LaneOffsets<D> &lo, FQ &&on_qk,
                                            FP &&on_pv) {
  using G = TileGeo<D>;
  constexpr int DK = G::DK, DB = G::DB;
  constexpr int AK = DK < 2 ? DK : 2;   // k-steps of key fragments in flight
  bf16x8_t kf0[DK], kf1[DK];
  auto read_k = [&](int j) __attribute__((always_inline)) {
    // rows col and 32 + col share the swizzle (it depends on the row mod 16)
    kf0[j] = *reinterpret_cast<const bf16x8_t *>(ks + lo.k[j]);
    if constexpr (!kHalf) kf1[j] = *reinterpret_cast<const bf16x8_t *>(ks + 32 * G::ROWB + lo.k[j]);
  };
#pragma unroll
  for (int j = 0; j < AK; ++j) read_k(j);
  // the accumulators start at -m_run: the MFMAs deliver s*log2(e)*q.k - m_run
  // (the queries were scaled by s*log2(e) when loaded)
  f32x16_t s0 = negm, s1;
  if constexpr (!kHalf) s1 = negm;
#pragma unroll
  for (int j = 0; j < DK; ++j) {
    __builtin_amdgcn_sched_barrier(0);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf0[j], qb[j], s0, 0, 0, 0);
    if constexpr (!kHalf) s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf1[j], qb[j], s1, 0, 0, 0);
    if (j + AK < DK) read_k(j + AK);
    on_qk(j);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- softmax of the tile: scores r of this lane are keys k0 + 8(r/4) + 4half + r%4 (+32 in s1)
  if (k0 + 64 > len) {   // ragged tile: keys past the group get -inf
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int32_t key = k0 + 8 * (r / 4) + 4 * half + (r % 4);
      if (key >= len) s0[r] = -INFINITY;
      if (!kHalf && key + 32 >= len) s1[r] = -INFINITY;
    }
  }
  // tile max of the shifted scores: two chains of three-input maxima
  float mx;
  if constexpr (kHalf) {
    float m0 = fmaxf(fmaxf(s0[0], s0[1]), s0[2]), m1 = fmaxf(fmaxf(s0[3], s0[4]), s0[5]);
#pragma unroll
    for (int r = 6; r < 14; r += 4) {
      m0 = fmaxf(fmaxf(m0, s0[r]), s0[r + 1]);
      m1 = fmaxf(fmaxf(m1, s0[r + 2]), s0[r + 3]);
    }
    mx = fmaxf(fmaxf(m0, s0[14]), fmaxf(m1, s0[15]));
  } else {
    float mx0 = fmaxf(fmaxf(s0[0], s0[1]), s0[2]), mx1 = fmaxf(fmaxf(s1[0], s1[1]), s1[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) {
      mx0 = fmaxf(fmaxf(mx0, s0[r]), s0[r + 1]);
      mx1 = fmaxf(fmaxf(mx1, s1[r]), s1[r + 1]);
    }
    mx = fmaxf(fmaxf(mx0, s0[15]), fmaxf(mx1, s1[15]));
  }
  mx = fmaxf(mx, swap_halves(mx));   // the other 16 keys of each block for this query
  // The reference m_run only moves when a score exceeds it by more than
  // kLazyRescale, and at the first tile (which sets it from that tile's max).
  if (__any(first || mx > kLazyRescale)) {
    const float delta = first ? mx : fmaxf(mx, 0.f);
    if (!first) {
      const float alpha = __builtin_amdgcn_exp2f(-delta);
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] -= delta;
      if constexpr (!kHalf) s1[r] -= delta;
    }
    m_run += delta;
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[r] = -m_run;
  }
  float lsum = 0.f;
  bf16x8_t p0[2], p1[2];
#pragma unroll
  for (int r = 0; r < 16; r += 2) exp_pair_shifted(s0, r, lsum, p0);

  // ---- O^T += Y^T P^T: step i covers block kb = i / 2DB, keys +16h (h = i / DB % 2), d-block b = i % DB
  constexpr int NPV = (kHalf ? 2 : 4) * DB;
  constexpr int AV = 2;                            // steps of value fragments in flight
  constexpr int EPS = 16 / (2 * DB);               // block-1 scores converted per block-0 step
  bf16x8_t yf[NPV];
  auto read_y = [&](int i) __attribute__((always_inline)) {
    const int kb = i / (2 * DB), h = (i / DB) & 1, b = i % DB;
    const unsigned char *rows = vs + (32 * kb + 16 * h) * G::ROWB;
    const bf16x4_t ylo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MA_LDS bf16x4_t *)(rows + lo.ya[b]));
    const bf16x4_t yhi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MA_LDS bf16x4_t *)(rows + lo.yb[b]));
    yf[i] = __builtin_shufflevector(ylo, yhi, 0, 1, 2, 3, 4, 5, 6, 7);
    // past head_dim (D = 16 only) this d-block feeds zero rows
    if (!((G::DB * 32 == D) || 32 * b + tr_col < D)) yf[i] = bf16x8_t{};
  };
#pragma unroll
  for (int i = 0; i < AV; ++i) read_y(i);
#pragma unroll
  for (int i = 0; i < NPV; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    const int kb = i / (2 * DB), h = (i / DB) & 1, b = i % DB;
    oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(yf[i], kb ? p1[h] : p0[h], oacc[b], 0, 0, 0);
    if (i + AV < NPV) read_y(i + AV);
    if (!kHalf && i < 2 * DB) {
#pragma unroll
      for (int e = 0; e < EPS; e += 2) exp_pair_shifted(s1, EPS * i + e, lsum, p1);
    }
    on_pv(i);
  }
  __builtin_amdgcn_sched_barrier(0);
  l_run += lsum;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One work item of the streaming kernel: logical workgroup `bid` (query tile,
// span, group and (batch, head) slice decoded from it). `lds` is the caller's
// LDS array of five tile buffers, value ring first: inlined into a kernel
// whose __shared__ array it is, each buffer sits at a constant offset, which
// the fragment reads carry in their immediate offsets. Ends with every DMA
// landed; the caller separates consecutive items by a barrier.
template <int D, int NW, bool kTwoLevel>
__device__ __forceinline__ void stream_item(const AttnLaunch &p, uint32_t bid, unsigned char *lds) {
  using G = TileGeo<D>;
  static_assert(G::NINST % NW == 0, "every wave must issue the same number of DMA instructions");
  constexpr int WPT = G::NINST / NW;         // DMA windows per tile, tensor and wave
  unsigned char *const yt0 = lds, *const yt1 = lds + G::TILEB;
  unsigned char *const kt0 = lds + 2 * G::TILEB, *const kt1 = lds + 3 * G::TILEB, *const kt2 = lds + 4 * G::TILEB;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool packed = p.span_waves > 0;
  const int32_t qt = (int32_t)(bid % (uint32_t)p.n_qtiles);
  const uint32_t rest0 = bid / (uint32_t)p.n_qtiles;
  const int32_t span = packed ? 0 : (int32_t)(rest0 % (uint32_t)p.n_spans);
  const uint32_t rest = packed ? rest0 : rest0 / (uint32_t)p.n_spans;
  const int32_t g = (int32_t)(rest % (uint32_t)p.ga.n_groups);
  const int64_t bh = (int64_t)(rest / (uint32_t)p.ga.n_groups);
  const GroupGeom geo = group_geom(p.ga, g);
  // This wave's queries [q0, min(q0 + 32, qhi)) attend to keys [0, qhi)
  // (qhi = 0: no queries); the workgroup streams keys [0, klen).
  int32_t q0, qhi, klen;
  if (packed) {
    // wave item i (of the group's items, in span order from the last span
    // down): span s, wave j of that span
    auto item_range = [&](int32_t i, int32_t &lo, int32_t &hi) __attribute__((always_inline)) {
      int32_t s, j;
      if (i < p.last_waves) {
        s = p.n_spans - 1;
        j = i;
      } else {
        const int32_t i2 = i - p.last_waves;
        s = p.n_spans - 2 - i2 / p.span_waves;
        j = i2 % p.span_waves;
      }
      const int32_t base = p.q_first + s * p.q_span;
      lo = s >= 0 ? base + kQueriesPerWave * j : p.q_first;
      hi = s >= 0 ? min(geo.len, base + p.q_span) : 0;
    };
    int32_t lo0;
    item_range(qt * NW, lo0, klen);   // the workgroup's first item has the longest span
    item_range(qt * NW + wave, q0, qhi);
  } else {
    // queries [span_lo, span_hi) of the group, this workgroup's q_tile of them
    const int32_t span_lo = p.q_first + span * p.q_span;
    const int32_t span_hi = p.q_span > 0 ? min(geo.len, span_lo + p.q_span) : geo.len;
    const int32_t qbase = span_lo + qt * p.q_tile;
    const int32_t qend = min(span_hi, qbase + p.q_tile);
    q0 = qbase + kQueriesPerWave * wave;
    qhi = q0 < qend ? span_hi : 0;
    klen = qbase < span_hi ? span_hi : 0;
  }
  if (klen == 0) return;   // uniform over the workgroup
  const RowMap rm = row_map(geo);

  const unsigned char *qbytes = uniform_ptr(
      reinterpret_cast<const unsigned char *>(static_cast<const u16 *>(p.q) + bh * p.head_elems));
  const unsigned char *kbytes = uniform_ptr(
      reinterpret_cast<const unsigned char *>(static_cast<const u16 *>(p.k) + bh * p.head_elems));
  const unsigned char *vbytes = uniform_ptr(
      reinterpret_cast<const unsigned char *>(static_cast<const u16 *>(p.vals) + bh * p.head_elems));

  const int col = lane & 31, half = lane >> 5;
  const int tr_key = 4 * half + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // DMA window w (of this wave's WPT per tile and tensor) of the tile holding
  // group rows [k0, k0 + 64). One-level groups (a member's token is
  // base + m * stride_in) take the offset with one 24-bit multiply-add; the
  // host picks this form only when members and the member stride in bytes fit
  // in 24 bits. Two-level groups (tiled boxes) go through row_token.
  using G0 = TileGeo<D>;
  constexpr int WPT0 = G0::NINST / NW;
  const int lane_row = lane / G0::CPR;
  const uint32_t mstride = (uint32_t)rm.stride_in * (2u * D);   // bytes between consecutive members
  uint32_t csb[WPT0];   // byte offset of member 0's row plus this lane's swizzled chunk, per window
#pragma unroll
  for (int w = 0; w < WPT0; ++w) {
    const int ii = wave + NW * w;
    const int slot = ii * 64 + lane;
    const int r = slot / G0::CPR, pos = slot % G0::CPR;
    csb[w] = (uint32_t)rm.base * (2u * D) + 16u * (uint32_t)swizzle_chunk<G0::CPR>(r, pos);
  }
  auto window = [&](const unsigned char *src, unsigned char *dst, int32_t k0, int w)
                    __attribute__((always_inline)) {
    const int ii = wave + NW * w;
    if constexpr (kTwoLevel) {
      dma_row_window<D>(src, dst, rm, k0, ii, lane);
    } else {
      const int32_t km = min(lane_row + (k0 + ii * G0::ROWS_PER_INST), rm.last);
      dma16(src, __umul24((uint32_t)km, mstride) + csb[w], dst + ii * 1024);
    }
  };

  const LaneOffsets<D> lo = lane_offsets<D>(col, half, tr_key, tr_col);

  const int32_t n = (klen + kKeyTile - 1) / kKeyTile;
  const int32_t wave_n = q0 < qhi ? (qhi + kKeyTile - 1) / kKeyTile : 0;   // tiles this wave computes
  // Prologue. The workgroup's 32*NW query rows come in like key tiles (whole
  // rows per DMA window, rather than 16 bytes of 64 rows per load) into the
  // buffers of value tile 1 and key tile 2, which stay free until step 0
  // refills them; then K(0), Y(0), K(1). Each wave loads its own 32 rows
  // (queries need not be contiguous across waves): the windows of buffer
  // rows 32*(wave % 2) .. +31, as many windows as WPT per tile of NW waves.
  {
    constexpr int QW = kQueriesPerWave / G0::ROWS_PER_INST;
    static_assert(QW == (NW > 2 ? 2 : 1) * WPT, "query windows: the count the vmcnt waits assume");
    unsigned char *qdst = wave < 2 ? yt1 : kt2;
    const int32_t qk0 = q0 - kQueriesPerWave * (wave & 1);
#pragma unroll
    for (int i = 0; i < QW; ++i) {
      const int ii = (wave & 1) * QW + i;
      if constexpr (kTwoLevel) {
        dma_row_window<D>(qbytes, qdst, rm, qk0, ii, lane);
      } else {
        const int r = ii * G0::ROWS_PER_INST + lane_row;
        const int32_t km = min(qk0 + r, rm.last);
        dma16(qbytes,
              __umul24((uint32_t)km, mstride) + (uint32_t)rm.base * (2u * D) +
                  16u * (uint32_t)swizzle_chunk<G0::CPR>(r, lane % G0::CPR),
              qdst + ii * 1024);
      }
    }
  }
#pragma unroll
  for (int w = 0; w < WPT; ++w) window(kbytes, kt0, 0, w);
#pragma unroll
  for (int w = 0; w < WPT; ++w) window(vbytes, yt0, 0, w);
#pragma unroll
  for (int w = 0; w < WPT; ++w) window(kbytes, kt1, kKeyTile, w);
  wait_vmcnt<WPT>();   // everything but K(1), as at every later step
  __syncthreads();
  // This lane's query (row 32*wave + col of the query tile) as the B operand
  // of S^T = K Q^T: the same fragments a key read of that row takes. Rows
  // past the group or this workgroup's share hold other members' data; their
  // results are never stored.
  bf16x8_t qb[G::DK];
  {
    const unsigned char *qtile = (wave < 2 ? yt1 : kt2) + (wave & 1) * 32 * G::ROWB;
#pragma unroll
    for (int j = 0; j < G::DK; ++j) {
      // scaled by s*log2(e) and rounded back to bf16, so that the QK MFMAs
      // deliver softmax exponents in log2 units
      const bf16x8_t x = *reinterpret_cast<const bf16x8_t *>(qtile + lo.k[j]);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2_t pr = __builtin_convertvector(
            (f32x2_t){(float)x[e] * p.scale_log2, (float)x[e + 1] * p.scale_log2}, bf16x2_t);
        qb[j][e] = pr[0];
        qb[j][e + 1] = pr[1];
      }
    }
  }

  f32x16_t oacc[G::DB];
#pragma unroll
  for (int b = 0; b < G::DB; ++b) oacc[b] = f32x16_t{};
  // m_run: the reference subtracted from every log2-scaled score (set from the
  // first tile's max); negm holds -m_run as the QK accumulators' initial value
  float m_run = 0.f, l_run = 0.f;
  f32x16_t negm = {};

  constexpr int NQ = G::DK;        // QK hook points per tile
  constexpr int NP = 4 * G::DB;    // PV hook points per tile
  constexpr int SQ = NQ >= WPT ? NQ / WPT : 1, SP = NP >= WPT ? NP / WPT : 1;
  constexpr int XQ = NQ / SQ < WPT ? NQ / SQ : WPT, XP = NP / SP < WPT ? NP / SP : WPT;   // windows in hooks

  // One tile: computes from (kc, yc) and fills (yn, kn).
  // One tile: computes from (kc, yc) and, with DMA, fills (yn, kn). The last
  // tile runs without DMA: tiles n and n+1 would lie past the group.
  auto step = [&](auto dma, int32_t t, const unsigned char *kc, const unsigned char *yc, unsigned char *yn,
                  unsigned char *kn) __attribute__((always_inline)) {
    constexpr bool kDma = decltype(dma)::value;
    // Outstanding: ... Y(t), K(t+1); tile t needs everything but K(t+1).
    wait_vmcnt<WPT>();
    __syncthreads();   // tile t visible; buffers of tiles t-1 (values) and t-1 (keys) free
    const int32_t yk0 = (t + 1) * kKeyTile, kk0 = (t + 2) * kKeyTile;
    if (t < wave_n) {
      // value windows of tile t+1 precede the key windows of tile t+2 in issue order
      if constexpr (kDma) {
#pragma unroll
        for (int w = XQ; w < WPT; ++w) window(vbytes, yn, yk0, w);
      }
      auto on_qk = [&](int i) __attribute__((always_inline)) {
        if (kDma && i % SQ == 0 && i / SQ < XQ) window(vbytes, yn, yk0, (i / SQ));
      };
      auto on_pv = [&](int i) __attribute__((always_inline)) {
        if (kDma && i % SP == 0 && i / SP < XP) window(kbytes, kn, kk0, (i / SP));
      };
      if (!kDma && t * kKeyTile + 32 >= qhi && t > 0) {
        // this wave's last tile holds at most 32 of its keys: block 0 only
        stream_tile<D, true>(kc, yc, qb, t * kKeyTile, qhi, false, negm, m_run, l_run, oacc, half, tr_col, lo,
                             on_qk, on_pv);
      } else {
        stream_tile<D>(kc, yc, qb, t * kKeyTile, qhi, t == 0, negm, m_run, l_run, oacc, half, tr_col, lo,
                       on_qk, on_pv);
      }
      if constexpr (kDma) {
#pragma unroll
        for (int w = XP; w < WPT; ++w) window(kbytes, kn, kk0, w);
      }
    } else if constexpr (kDma) {
#pragma unroll
      for (int w = 0; w < WPT; ++w) window(vbytes, yn, yk0, w);
#pragma unroll
      for (int w = 0; w < WPT; ++w) window(kbytes, kn, kk0, w);
    }
  };
  const std::true_type with_dma{};
  // tile t: keys in kt[t % 3], values in yt[t % 2]; fills yt[(t+1) % 2], kt[(t+2) % 3]
  const int32_t nd = n - 1;   // tiles run with DMA
  for (int32_t t = 0; t < nd; t += 6) {
    step(with_dma, t, kt0, yt0, yt1, kt2);
    if (t + 1 >= nd) break;
    step(with_dma, t + 1, kt1, yt1, yt0, kt0);
    if (t + 2 >= nd) break;
    step(with_dma, t + 2, kt2, yt0, yt1, kt1);
    if (t + 3 >= nd) break;
    step(with_dma, t + 3, kt0, yt1, yt0, kt2);
    if (t + 4 >= nd) break;
    step(with_dma, t + 4, kt1, yt0, yt1, kt0);
    if (t + 5 >= nd) break;
    step(with_dma, t + 5, kt2, yt1, yt0, kt1);
  }
  {
    const int r3 = nd % 3;
    step(std::false_type{}, nd, r3 == 0 ? kt0 : r3 == 1 ? kt1 : kt2, (nd & 1) ? yt1 : yt0, nullptr, nullptr);
  }
  // DMAs into buffers past the last tile may still be in flight; they must
  // land before the buffers are reused below (and before the workgroup's LDS
  // is handed to another workgroup).
  wait_vmcnt<0>();
  __syncthreads();
  // Output through LDS: each wave writes its normalised 32 x D tile row-major
  // (16-byte chunks XOR-swizzled by row) into its own 32*2D bytes, then
  // stores whole rows, D/8 lanes per row.
  unsigned char *ot = lds + wave * 32 * G::ROWB;
  {
    const float inv = 1.f / (l_run + swap_halves(l_run));
#pragma unroll
    for (int b = 0; b < G::DB; ++b)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * b + 8 * rq + 4 * half;   // O^T element 4rq..4rq+3 of d-block b
        if (d0 < D) {
          bf16x4_t v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (__bf16)(oacc[b][4 * rq + e] * inv);
          const int chunk = (d0 >> 3) ^ (col & (G::CPR - 1));
          *reinterpret_cast<bf16x4_t *>(ot + col * G::ROWB + 16 * chunk + 8 * half) = v;
        }
      }
  }
  u16 *oh = static_cast<u16 *>(p.out) + bh * p.head_elems;
  constexpr int RPI = 64 / G::CPR;   // rows per store instruction
#pragma unroll
  for (int r0 = 0; r0 < 32; r0 += RPI) {
    const int r = r0 + lane / G::CPR, c = lane % G::CPR;
    const uint4 v = *reinterpret_cast<const uint4 *>(ot + r * G::ROWB + 16 * (c ^ (r & (G::CPR - 1))));
    const int32_t m = q0 + r;
    if (m < qhi) *reinterpret_cast<uint4 *>(oh + (uint32_t)member_token(geo, m) * D + 8 * c) = v;
  }
}

template <int D, int NW, bool kTwoLevel>
__global__ __launch_bounds__(NW * 64, 2) void group_attn_bf16(AttnLaunch p) {
  __shared__ __align__(1024) unsigned char lds[5 * TileGeo<D>::TILEB];
  stream_item<D, NW, kTwoLevel>(p, xcd_remap(blockIdx.x, gridDim.x), lds);
}

// ---------------------------------------------------------------------------
// Persistent kernel for groups of at most 64 tokens (stage R at W <= 64, short
// stage-L groups). Workgroup w handles items w, w + G, w + 2G, ... (item =
// group + n_groups * (batch*head)), one at a time: K and V tiles by DMA, the
// queries into registers, the softmax attention of the group, the output
// staged row-major in the key buffer and stored as whole rows. There is no
// prefetch: four resident workgroups per CU (32 KB of LDS and two waves each)
// keep more loads in flight than two double-buffered ones did, and the stage
// runs at about the rate of a device-to-device copy.
template <int D>
__global__ __launch_bounds__(kBlockWaves * 64, 2) void block_attn_bf16(AttnLaunch p, int32_t n_items) {
  using G = TileGeo<D>;
  constexpr int NW = kBlockWaves;
  __shared__ __align__(1024) unsigned char kt[G::TILEB];
  __shared__ __align__(1024) unsigned char yt[G::TILEB];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int tr_key = 4 * half + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // Rows past a group are never loaded; start from finite (zero) tiles.
  for (int i = threadIdx.x; i < G::TILEB / 16; i += NW * 64) {
    reinterpret_cast<uint4 *>(kt)[i] = make_uint4(0, 0, 0, 0);
    reinterpret_cast<uint4 *>(yt)[i] = make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  for (int32_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const GroupGeom geo = group_geom(p.ga, item % p.ga.n_groups);
    const int64_t bh = item / p.ga.n_groups;
    const unsigned char *kb =
        reinterpret_cast<const unsigned char *>(static_cast<const u16 *>(p.k) + bh * p.head_elems);
    const unsigned char *vb =
        reinterpret_cast<const unsigned char *>(static_cast<const u16 *>(p.vals) + bh * p.head_elems);
    {
      // windows wholly past the group are skipped (their rows keep finite
      // data from earlier items or the zero fill; they are masked)
      const unsigned char *ku = uniform_ptr(kb), *vu = uniform_ptr(vb);
      for (int ii = wave; ii < G::NINST; ii += NW) {
        if (ii * G::ROWS_PER_INST >= geo.len) break;   // wave-uniform
        const int slot = ii * 64 + lane;
        const int r = slot / G::CPR, pos = slot % G::CPR;
        const int c = swizzle_chunk<G::CPR>(r, pos);
        const uint32_t off = ((uint32_t)member_token(geo, min(r, geo.len - 1)) * D + c * 8) * 2u;
        dma16(ku, off, kt + ii * 1024);
        dma16(vu, off, yt + ii * 1024);
      }
    }
    bf16x8_t qb[G::DK];
    load_query<D>(static_cast<const u16 *>(p.q) + bh * p.head_elems, geo, wave * kQueriesPerWave + col, half, qb);
    wait_dma();
    __syncthreads();   // the tiles are visible to both waves
    f32x16_t oacc[G::DB];
#pragma unroll
    for (int b = 0; b < G::DB; ++b) oacc[b] = f32x16_t{};
    float m_run = -INFINITY, l_run = 0.f;
    attend_tile<D>(kt, yt, qb, 0, geo.len, p.scale_log2, m_run, l_run, oacc, col, half, tr_key, tr_col);
    __syncthreads();   // both waves are done with kt: it stages the output
    unsigned char *ot = kt + wave * 32 * G::ROWB;
    const float inv = 1.f / (l_run + swap_halves(l_run));
#pragma unroll
    for (int b = 0; b < G::DB; ++b)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * b + 8 * rq + 4 * half;
        if (d0 < D) {
          bf16x4_t v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (__bf16)(oacc[b][4 * rq + e] * inv);
          const int chunk = (d0 >> 3) ^ (col & (G::CPR - 1));
          *reinterpret_cast<bf16x4_t *>(ot + col * G::ROWB + 16 * chunk + 8 * half) = v;
        }
      }
    u16 *oh = static_cast<u16 *>(p.out) + bh * p.head_elems;
    constexpr int RPI = 64 / G::CPR;
#pragma unroll
    for (int r0 = 0; r0 < 32; r0 += RPI) {
      const int r = r0 + lane / G::CPR, c = lane % G::CPR;
      const uint4 v = *reinterpret_cast<const uint4 *>(ot + r * G::ROWB + 16 * (c ^ (r & (G::CPR - 1))));
      const int32_t m = wave * kQueriesPerWave + r;
      if (m < geo.len) *reinterpret_cast<uint4 *>(oh + (uint32_t)member_token(geo, m) * D + 8 * c) = v;
    }
    __syncthreads();   // the staged rows are read before the next item's keys land in kt
  }
}

}  // namespace ma
