// attn_bwd_bf16.h -- backward of bf16 group softmax attention, used by both
// Monarch stages (the pages say the method's kernels run the forward and the
// backward pass with FlashAttention-like tiling, keeping the score matrix on
// chip: it "Finetuning e Implementazione Efficiente"; fr 2.C; zh 微调与高效实现).
//
// For one token set G (s = 1/sqrt(D)), with P = softmax_rows(s Q_G K_G^T):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = dO_i . O_i,
//   dQ = s dS K,  dK = s dS^T Q.
// Two passes per stage, each streaming one operand through LDS like the
// forward kernel (same DMA windows, swizzle and MFMA layouts):
//   bwd_dq_bf16    a workgroup owns 32*NW queries of a group and streams its
//                  key and value tiles: S^T = K Q^T and dP^T = V dO^T on the
//                  matrix cores, the online softmax of S gives e = exp2(.-m),
//                  and dQ^T += K^T (e*(dP-D))^T, rescaled like O in the
//                  forward; at the end dQ = s dQacc / l. It also writes each
//                  query's log2-sum-exp (m + log2 l) and D, in group order.
//   bwd_dkdv_bf16  a workgroup owns 32*NW keys and streams the group's query
//                  and dO tiles with their (lse, D): S = Q K^T, dP = dO V^T,
//                  P = exp2(s log2e S - lse), dS = P*(dP-D);
//                  dV^T += dO^T P and dK^T += Q^T dS; dK = s dKacc.
// Groups of at most 64 members instead take bwd_small_bf16: one workgroup per
// group does both passes' work from one LDS copy of the group.
// Rows outside the group are clamped duplicates (finite) and get zero weight.
#pragma once
#include <type_traits>

#include "attn_bf16.h"

namespace ma {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct BwdLaunch {
  const void *q, *k, *v;   // this stage's forward inputs (v: V for stage R, Y for stage L)
  const void *o;           // this stage's forward output (Y or O); dq pass only
  const void *dout;        // gradient of that output (dY or dO)
  void *dq;                // dq pass
  void *dk, *dv;           // dkdv pass (dv: dV for stage R, dY for stage L)
  float *stats;            // per query (log2-sum-exp, D), group order
  int64_t head_elems;      // N * D
  GroupAddr ga;
  int32_t n_tiles;         // row tiles of 32*NW per group (queries or keys)
  int32_t stats_stride;    // members per group in `stats`: >= 64 * ceil(max_len / 64) + 128
  int32_t accumulate;      // add to dq (dq pass) / dk (dkdv pass) instead of overwriting
  float scale;             // 1/sqrt(D)
  float scale_log2;        // scale * log2(e)
};

// The 1 KB DMA windows one wave issues per tile (window ii = wave + NW w,
// w < NINST / NW), rows past the group repeating its last member. One-level
// groups (member m at token base + m * stride_in) take a per-window offset
// computed once and one 24-bit multiply-add per window; two-level groups
// (tiled boxes spanning several outer rows, or offsets of 2^24 bytes or more)
// take the general row map.
template <int D, int NW, bool kTwoLevel>
struct RowWindows {
  using G = TileGeo<D>;
  static constexpr int WPT = G::NINST / NW;
  RowMap rm;
  uint32_t mstride;    // bytes between consecutive members
  uint32_t csb[WPT];   // member 0's row offset plus this lane's swizzled chunk, per window
  int32_t lane_row;
  int wave, lane;

  __device__ __forceinline__ RowWindows(const GroupGeom &geo, int wave_, int lane_) : wave(wave_), lane(lane_) {
    rm = row_map(geo);
    mstride = (uint32_t)rm.stride_in * (2u * D);
    lane_row = lane / G::CPR;
#pragma unroll
    for (int w = 0; w < WPT; ++w) {
      const int slot = (wave + NW * w) * 64 + lane;
      csb[w] = (uint32_t)rm.base * (2u * D) + 16u * (uint32_t)swizzle_chunk<G::CPR>(slot / G::CPR, slot % G::CPR);
    }
  }
  // window w of the tile holding group rows [k0, k0 + 64)
  __device__ __forceinline__ void issue(const unsigned char *src, unsigned char *tile, int32_t k0, int w) const {
    const int ii = wave + NW * w;
    if constexpr (kTwoLevel) {
      dma_row_window<D>(src, tile, rm, k0, ii, lane);
    } else {
      const int32_t km = min(lane_row + (k0 + ii * G::ROWS_PER_INST), rm.last);
      dma16(src, __umul24((uint32_t)km, mstride) + csb[w], tile + ii * 1024);
    }
  }
  __device__ __forceinline__ void tile(const unsigned char *src, unsigned char *dst, int32_t k0) const {
#pragma unroll
    for (int w = 0; w < WPT; ++w) issue(src, dst, k0, w);
  }
};

// c0 / c1 (rows 0..31 / 32..63 of a 64-row LDS tile, 32 columns of this
// wave) = tile rows x b, with b the B operand (k-step j: head_dim slots
// [D/2 half + 8j, +8) of this lane's column). Fragments are read two k-steps
// ahead, in fixed slots as in stream_tile.
template <int D>
__device__ __forceinline__ void tile_times(const unsigned char *ts, const bf16x8_t *b, const LaneOffsets<D> &lo,
                                           f32x16_t &c0, f32x16_t &c1) {
  using G = TileGeo<D>;
  constexpr int DK = G::DK;
  constexpr int AK = DK < 2 ? DK : 2;
  bf16x8_t a0[DK], a1[DK];
  auto rd = [&](int j) __attribute__((always_inline)) {
    a0[j] = *reinterpret_cast<const bf16x8_t *>(ts + lo.k[j]);
    a1[j] = *reinterpret_cast<const bf16x8_t *>(ts + 32 * G::ROWB + lo.k[j]);
  };
#pragma unroll
  for (int j = 0; j < AK; ++j) rd(j);
  f32x16_t x0 = {}, x1 = {};
#pragma unroll
  for (int j = 0; j < DK; ++j) {
    __builtin_amdgcn_sched_barrier(0);
    x0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[j], b[j], x0, 0, 0, 0);
    x1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[j], b[j], x1, 0, 0, 0);
    if (j + AK < DK) rd(j + AK);
  }
  __builtin_amdgcn_sched_barrier(0);
  c0 = x0;
  c1 = x1;
}

// acc[b] += T^T W over the 64 rows of an LDS tile: T^T (head_dim x rows) read
// transposed, W (rows x 32 columns) from registers in the layout of a C
// block's elements (w0: rows 0..31, w1: rows 32..63; pair h holds elements
// 8h..8h+7 of that block), as the forward's O^T += Y^T P^T.
template <int D>
__device__ __forceinline__ void tile_t_times(const unsigned char *ts, const bf16x8_t (&w0)[2],
                                             const bf16x8_t (&w1)[2], const LaneOffsets<D> &lo, int tr_col,
                                             f32x16_t *acc) {
  using G = TileGeo<D>;
  constexpr int DB = G::DB;
  constexpr int NPV = 4 * DB;
  constexpr int AV = 2;
  bf16x8_t yf[NPV];
  auto rd = [&](int i) __attribute__((always_inline)) {
    const int kb = i / (2 * DB), h = (i / DB) & 1, b = i % DB;
    const unsigned char *rows = ts + (32 * kb + 16 * h) * G::ROWB;
    const bf16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MA_LDS bf16x4_t *)(rows + lo.ya[b]));
    const bf16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MA_LDS bf16x4_t *)(rows + lo.yb[b]));
    yf[i] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
    if (!((G::DB * 32 == D) || 32 * b + tr_col < D)) yf[i] = bf16x8_t{};
  };
#pragma unroll
  for (int i = 0; i < AV; ++i) rd(i);
#pragma unroll
  for (int i = 0; i < NPV; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    const int kb = i / (2 * DB), h = (i / DB) & 1, b = i % DB;
    acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(yf[i], kb ? w1[h] : w0[h], acc[b], 0, 0, 0);
    if (i + AV < NPV) rd(i + AV);
  }
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void pack_pair(float a, float b, int r, bf16x8_t (&pb)[2]) {
  const bf16x2_t pr = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
  pb[r / 8][r % 8] = pr[0];
  pb[r / 8][r % 8 + 1] = pr[1];
}

// This lane's row m (clamped into the group) of one tensor, half `half`, as
// the B operand fragments used by tile_times.
template <int D>
__device__ __forceinline__ void load_row_frags(const u16 *base, const GroupGeom &geo, int32_t m, int half,
                                               bf16x8_t *frag) {
  const int32_t mm = m < geo.len ? m : geo.len - 1;
  const u16 *row = base + (uint32_t)member_token(geo, mm) * D + (D / 2) * half;
#pragma unroll
  for (int j = 0; j < D / 16; ++j)
    frag[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(row + 8 * j));
}

// Writes this wave's 32 x D result through LDS as whole rows: acc holds it
// transposed (acc[b] element r of lane (col, half) is head_dim 32b + 8(r/4) +
// 4 half + r%4 of row col), scaled per column by `colscale`. Rows m0 + r with
// m0 + r < mend go to base + token * D; with `add`, onto the values there, or
// onto `old_rows` (those values, loaded earlier by load_old_rows).
template <int D>
__device__ __forceinline__ void store_rows_lds(unsigned char *ot, const f32x16_t *acc, float colscale, int col,
                                               int half, int lane, u16 *base, const GroupGeom &geo, int32_t m0,
                                               int32_t mend, bool add, const uint4 *old_rows = nullptr) {
  using G = TileGeo<D>;
#pragma unroll
  for (int b = 0; b < G::DB; ++b)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = 32 * b + 8 * rq + 4 * half;
      if (d0 < D) {
        f32x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[b][4 * rq + e] * colscale;
        const int chunk = (d0 >> 3) ^ (col & (G::CPR - 1));
        *reinterpret_cast<f32x4_t *>(ot + col * (4 * D) + 16 * (2 * chunk + half)) = v;
      }
    }
  // read back 8 values (two 16-byte fp32 chunks) per lane: D/8 lanes per row
  constexpr int RPI = 64 / G::CPR;
#pragma unroll
  for (int r0 = 0; r0 < 32; r0 += RPI) {
    const int r = r0 + lane / G::CPR, c = lane % G::CPR;
    const int sc = c ^ (r & (G::CPR - 1));
    const f32x4_t lo4 = *reinterpret_cast<const f32x4_t *>(ot + r * (4 * D) + 16 * (2 * sc));
    const f32x4_t hi4 = *reinterpret_cast<const f32x4_t *>(ot + r * (4 * D) + 16 * (2 * sc + 1));
    const int32_t m = m0 + r;
    if (m < mend) {
      u16 *dst = base + (uint32_t)member_token(geo, m) * D + 8 * c;
      float x[8] = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      if (add) {
        const bf16x8_t old =
            __builtin_bit_cast(bf16x8_t, old_rows ? old_rows[r0 / RPI] : *reinterpret_cast<const uint4 *>(dst));
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] += (float)old[e];
      }
      bf16x8_t outv;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2_t pr = __builtin_convertvector((f32x2_t){x[e], x[e + 1]}, bf16x2_t);
        outv[e] = pr[0];
        outv[e + 1] = pr[1];
      }
      *reinterpret_cast<uint4 *>(dst) = __builtin_bit_cast(uint4, outv);
    }
  }
}

// The values store_rows_lds(..., add) would read back, in its order: rows
// m0 + r (r = r0 + lane / (D/8), r0 = 0, 64/(D/8), ...; m0 + r < mend), 16 bytes
// each at chunk lane % (D/8); zero for rows past mend.
template <int D>
__device__ __forceinline__ void load_old_rows(const u16 *base, const GroupGeom &geo, int32_t m0, int32_t mend,
                                              int lane, uint4 *old_rows) {
  using G = TileGeo<D>;
  constexpr int RPI = 64 / G::CPR;
#pragma unroll
  for (int r0 = 0; r0 < 32; r0 += RPI) {
    const int r = r0 + lane / G::CPR, c = lane % G::CPR;
    const int32_t m = m0 + r;
    old_rows[r0 / RPI] = m < mend ? *reinterpret_cast<const uint4 *>(base + (uint32_t)member_token(geo, m) * D + 8 * c)
                                  : make_uint4(0, 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// dQ pass (two workgroups per CU: 80 KB of LDS and at most 256 registers).
// Ring: keys in LDS tiles 0..2 (tile t in t % 3), values in 3..4.
// Step t issues the value windows of tile t+1, then the key windows of tile
// t+2 (rows past the group clamped), so the wait opening step t+1 may leave
// the newest WPT windows in flight.
template <int D, int NW, bool kTwoLevel>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq_bf16(BwdLaunch p) {
  using G = TileGeo<D>;
  static_assert(G::NINST % NW == 0, "every wave must issue the same number of DMA instructions");
  constexpr int WPT = G::NINST / NW;
  constexpr int DK = G::DK, DB = G::DB;
  __shared__ __align__(1024) unsigned char lds[5 * G::TILEB];

  const uint32_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int32_t qt = (int32_t)(bid % (uint32_t)p.n_tiles);
  const uint32_t rest = bid / (uint32_t)p.n_tiles;
  const int32_t g = (int32_t)(rest % (uint32_t)p.ga.n_groups);
  const int64_t bh = (int64_t)(rest / (uint32_t)p.ga.n_groups);
  const GroupGeom geo = group_geom(p.ga, g);
  const int32_t qbase = qt * 32 * NW;
  if (qbase >= geo.len) return;   // uniform
  const int32_t qend = min(geo.len, qbase + 32 * NW);
  const int64_t slice = bh * p.head_elems;
  const unsigned char *kbytes = uniform_ptr(reinterpret_cast<const unsigned char *>(static_cast<const u16 *>(p.k) + slice));
  const unsigned char *vbytes = uniform_ptr(reinterpret_cast<const unsigned char *>(static_cast<const u16 *>(p.v) + slice));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int tr_key = 4 * half + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const LaneOffsets<D> lo = lane_offsets<D>(col, half, tr_key, tr_col);
  const int32_t q0 = qbase + wave * 32, qm = q0 + col;
  const bool wave_active = q0 < qend;

  const RowWindows<D, NW, kTwoLevel> win(geo, wave, lane);
  const int32_t n = (geo.len + kKeyTile - 1) / kKeyTile;
  // prologue: K(0), V(0), K(1), then this lane's query, dO and O rows
  win.tile(kbytes, lds, 0);
  win.tile(vbytes, lds + 3 * G::TILEB, 0);
  win.tile(kbytes, lds + G::TILEB, kKeyTile);
  bf16x8_t qb[DK], db[DK], ob[DK];
  load_row_frags<D>(static_cast<const u16 *>(p.q) + slice, geo, qm, half, qb);
  load_row_frags<D>(static_cast<const u16 *>(p.dout) + slice, geo, qm, half, db);
  load_row_frags<D>(static_cast<const u16 *>(p.o) + slice, geo, qm, half, ob);
  float dsum = 0.f;   // D = dO . O over this lane's half of head_dim
#pragma unroll
  for (int j = 0; j < DK; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) dsum = fmaf((float)db[j][e], (float)ob[j][e], dsum);
  const float Dq = dsum + swap_halves(dsum);
  wait_vmcnt<0>();
  __syncthreads();

  f32x16_t acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;
  // Tile t: keys in buffer t % 3, values in 3 + t % 2; unrolled by six so that
  // every buffer is a constant offset of the fragment reads.
  auto step = [&](int32_t t, auto ks_c, auto ys_c) __attribute__((always_inline)) {
    constexpr int ks = decltype(ks_c)::value, ys = decltype(ys_c)::value;
    if (t > 0) wait_vmcnt<WPT>();   // leave the key windows of tile t+1 in flight
    __syncthreads();
    const unsigned char *kc = lds + ks * G::TILEB;
    const unsigned char *vc = lds + (3 + ys) * G::TILEB;
    unsigned char *vn = lds + (3 + (ys ^ 1)) * G::TILEB;
    unsigned char *kn = lds + (ks == 0 ? 2 : ks - 1) * G::TILEB;
    win.tile(vbytes, vn, (t + 1) * kKeyTile);
    win.tile(kbytes, kn, (t + 2) * kKeyTile);
    if (wave_active) {
      f32x16_t s0, s1, t0, t1;
      tile_times<D>(kc, qb, lo, s0, s1);   // S^T: rows = keys
      tile_times<D>(vc, db, lo, t0, t1);   // dP^T
      const int32_t k0 = t * kKeyTile;
      if (k0 + kKeyTile > geo.len) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int32_t key = k0 + 8 * (r / 4) + 4 * half + (r % 4);
          if (key >= geo.len) s0[r] = -INFINITY;
          if (key + 32 >= geo.len) s1[r] = -INFINITY;
        }
      }
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
      mx = fmaxf(mx, swap_halves(mx));
      const float tmax = mx * p.scale_log2;
      if (__any(tmax > m_run + kLazyRescale)) {
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[b][r] *= alpha;
        m_run = m_new;
      }
      bf16x8_t w0[2], w1[2];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float e0 = __builtin_amdgcn_exp2f(fmaf(s0[r], p.scale_log2, -m_run));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(s0[r + 1], p.scale_log2, -m_run));
        const float f0 = __builtin_amdgcn_exp2f(fmaf(s1[r], p.scale_log2, -m_run));
        const float f1 = __builtin_amdgcn_exp2f(fmaf(s1[r + 1], p.scale_log2, -m_run));
        l_run += (e0 + e1) + (f0 + f1);
        pack_pair(e0 * (t0[r] - Dq), e1 * (t0[r + 1] - Dq), r, w0);
        pack_pair(f0 * (t1[r] - Dq), f1 * (t1[r + 1] - Dq), r, w1);
      }
      tile_t_times<D>(kc, w0, w1, lo, tr_col, acc);   // dQ^T += K^T w^T
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  for (int32_t t = 0; t < n; t += 6) {
    step(t, I0{}, I0{});
    if (t + 1 >= n) break;
    step(t + 1, I1{}, I1{});
    if (t + 2 >= n) break;
    step(t + 2, I2{}, I0{});
    if (t + 3 >= n) break;
    step(t + 3, I0{}, I1{});
    if (t + 4 >= n) break;
    step(t + 4, I1{}, I0{});
    if (t + 5 >= n) break;
    step(t + 5, I2{}, I1{});
  }
  wait_vmcnt<0>();   // DMAs into buffers past the last tile
  __syncthreads();
  const float l_tot = l_run + swap_halves(l_run);
  // outputs: dQ = s * acc / l through LDS (each wave 32 rows x 4D bytes, fp32)
  unsigned char *ot = lds + wave * 32 * (4 * D);
  store_rows_lds<D>(ot, acc, p.scale / l_tot, col, half, lane, static_cast<u16 *>(p.dq) + slice, geo, q0, qend,
                    p.accumulate != 0);
  if (half == 0 && qm < qend) {
    float2 *st = reinterpret_cast<float2 *>(p.stats) + ((int64_t)bh * p.ga.n_groups + g) * p.stats_stride + qm;
    *st = make_float2(m_run + __builtin_log2f(l_tot), Dq);
  }
}

// ---------------------------------------------------------------------------
// dK/dV pass. Double buffers: query tiles in LDS tiles 0..1, dO tiles in
// 2..3, and the (lse, D) window of each dO tile (128 members x 8 bytes, of
// which the tile uses 64) in two 1 KB slots; step t issues dO, stats and Q of
// tile t+1. kPart selects the outputs: 0 both, 1 dK only, 2 dV only. With
// both, the live registers at head_dim 128 (dK^T and dV^T accumulators, this
// wave's key and value rows, S and dP of a tile) exceed the 256 that two
// waves per SIMD allow; each single-output part fits them, at the price of a
// second S (the dV part needs neither V rows nor dP).
template <int D, int NW, bool kTwoLevel, int kPart>
__global__ __launch_bounds__(NW * 64, (D >= 128 && kPart == 0) ? 1 : 2) void bwd_dkdv_bf16(BwdLaunch p) {
  constexpr bool kDK = kPart != 2, kDV = kPart != 1;
  using G = TileGeo<D>;
  static_assert(G::NINST % NW == 0, "every wave must issue the same number of DMA instructions");
  constexpr int DK = G::DK, DB = G::DB;
  __shared__ __align__(1024) unsigned char lds[4 * G::TILEB + 2048];
  unsigned char *const st_lds = lds + 4 * G::TILEB;

  const uint32_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int32_t kt = (int32_t)(bid % (uint32_t)p.n_tiles);
  const uint32_t rest = bid / (uint32_t)p.n_tiles;
  const int32_t g = (int32_t)(rest % (uint32_t)p.ga.n_groups);
  const int64_t bh = (int64_t)(rest / (uint32_t)p.ga.n_groups);
  const GroupGeom geo = group_geom(p.ga, g);
  const int32_t kbase = kt * 32 * NW;
  if (kbase >= geo.len) return;   // uniform
  const int32_t kend = min(geo.len, kbase + 32 * NW);
  const int64_t slice = bh * p.head_elems;
  const unsigned char *qbytes = uniform_ptr(reinterpret_cast<const unsigned char *>(static_cast<const u16 *>(p.q) + slice));
  const unsigned char *dbytes = uniform_ptr(reinterpret_cast<const unsigned char *>(static_cast<const u16 *>(p.dout) + slice));
  const unsigned char *sbytes = uniform_ptr(reinterpret_cast<const unsigned char *>(
      reinterpret_cast<const float2 *>(p.stats) + ((int64_t)bh * p.ga.n_groups + g) * p.stats_stride));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int tr_key = 4 * half + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const LaneOffsets<D> lo = lane_offsets<D>(col, half, tr_key, tr_col);
  const int32_t k0w = kbase + wave * 32, km = k0w + col;
  const bool wave_active = k0w < kend;

  const RowWindows<D, NW, kTwoLevel> win(geo, wave, lane);
  const int32_t n = (geo.len + kKeyTile - 1) / kKeyTile;
  auto stats_window = [&](int32_t t, int slot) __attribute__((always_inline)) {
    // members [64t, 64t + 128): 1 KB, 16 bytes per lane; every wave issues the same window
    dma16(sbytes, (uint32_t)(t * kKeyTile * 8 + 16 * lane), st_lds + slot * 1024);
  };
  win.tile(qbytes, lds, 0);
  win.tile(dbytes, lds + 2 * G::TILEB, 0);
  stats_window(0, 0);
  bf16x8_t kb[DK], vb[DK];
  load_row_frags<D>(static_cast<const u16 *>(p.k) + slice, geo, km, half, kb);
  if constexpr (kDK) load_row_frags<D>(static_cast<const u16 *>(p.v) + slice, geo, km, half, vb);
  wait_vmcnt<0>();
#pragma unroll
  for (int j = 0; j < DK; ++j) {
    asm volatile("" ::"v"(kb[j]));
    if constexpr (kDK) asm volatile("" ::"v"(vb[j]));
  }
  __syncthreads();

  f32x16_t dka[DB], dva[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    if constexpr (kDK) dka[b] = f32x16_t{};
    if constexpr (kDV) dva[b] = f32x16_t{};
  }
  // Tile t in buffers t % 2. Only the group's last query tile can hold rows
  // past the group: the tiles before it take a form without the per-row
  // validity selects, unrolled by two so that every buffer is a constant
  // offset of the fragment reads.
  auto step = [&](int32_t t, auto cur_c, auto ragged_c) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr bool kRagged = decltype(ragged_c)::value;
    if (t > 0) wait_vmcnt<0>();   // tile t: the only DMAs in flight
    __syncthreads();              // ... landed for every wave, and tile t-1's buffers are free
    const unsigned char *qc = lds + cur * G::TILEB;
    const unsigned char *dc = lds + (2 + cur) * G::TILEB;
    const unsigned char *sc = st_lds + cur * 1024;
    win.tile(dbytes, lds + (3 - cur) * G::TILEB, (t + 1) * kKeyTile);
    stats_window(t + 1, cur ^ 1);
    win.tile(qbytes, lds + (1 - cur) * G::TILEB, (t + 1) * kKeyTile);
    if (wave_active) {
      f32x16_t s0, s1, t0, t1;
      tile_times<D>(qc, kb, lo, s0, s1);   // S: rows = queries of the tile, columns = this wave's keys
      if constexpr (kDK) tile_times<D>(dc, vb, lo, t0, t1);   // dP
      bf16x8_t p0[2], p1[2], g0[2], g1[2];
      const int32_t q0t = t * kKeyTile;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int row = 32 * blk + 8 * r4 + 4 * half;   // rows row .. row+3 of the tile
          const f32x4_t st01 = *reinterpret_cast<const f32x4_t *>(sc + row * 8);
          const f32x4_t st23 = *reinterpret_cast<const f32x4_t *>(sc + row * 8 + 16);
          const float lse[4] = {st01[0], st01[2], st23[0], st23[2]};
          const float dd[4] = {st01[1], st01[3], st23[1], st23[3]};
          float pv[4], gv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * r4 + e;
            const float sv = blk ? s1[r] : s0[r];
            // (lse, D) of members past the group are never written: select them away
            // before any arithmetic so that whatever bytes they hold cannot propagate
            const bool valid = !kRagged || q0t + row + e < geo.len;
            const float lv = valid ? lse[e] : 0.f;
            const float pr = valid ? __builtin_amdgcn_exp2f(fmaf(sv, p.scale_log2, -lv)) : 0.f;
            pv[e] = pr;
            if constexpr (kDK) {
              const float tv = blk ? t1[r] : t0[r];
              gv[e] = pr * (tv - (valid ? dd[e] : 0.f));
            }
          }
          bf16x8_t(&pp)[2] = blk ? p1 : p0;
          bf16x8_t(&gg)[2] = blk ? g1 : g0;
          if constexpr (kDV) {
            pack_pair(pv[0], pv[1], 4 * r4, pp);
            pack_pair(pv[2], pv[3], 4 * r4 + 2, pp);
          }
          if constexpr (kDK) {
            pack_pair(gv[0], gv[1], 4 * r4, gg);
            pack_pair(gv[2], gv[3], 4 * r4 + 2, gg);
          }
        }
      }
      if constexpr (kDV) tile_t_times<D>(dc, p0, p1, lo, tr_col, dva);   // dV^T += dO^T P
      if constexpr (kDK) tile_t_times<D>(qc, g0, g1, lo, tr_col, dka);   // dK^T += Q^T dS
    }
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  const int32_t n_full = geo.len / kKeyTile;   // query tiles with every row inside the group
  int32_t t = 0;
  for (; t + 2 <= n_full; t += 2) {
    step(t, C0{}, std::false_type{});
    step(t + 1, C1{}, std::false_type{});
  }
  for (; t < n; ++t) {   // at most one full tile and the ragged one
    if (t & 1)
      step(t, C1{}, std::true_type{});
    else
      step(t, C0{}, std::true_type{});
  }
  wait_vmcnt<0>();
  __syncthreads();
  // dK = s * dKacc, dV = dVacc, each through LDS (waves use separate 32-row fp32 areas)
  unsigned char *ot = lds + wave * 32 * (4 * D);
  if constexpr (kDK)
    store_rows_lds<D>(ot, dka, p.scale, col, half, lane, static_cast<u16 *>(p.dk) + slice, geo, k0w, kend,
                      p.accumulate != 0);
  if constexpr (kDK && kDV) __syncthreads();
  if constexpr (kDV)
    store_rows_lds<D>(ot, dva, 1.f, col, half, lane, static_cast<u16 *>(p.dv) + slice, geo, k0w, kend, false);
}

// ---------------------------------------------------------------------------
// Groups of at most 64 members: the whole backward of one group in one
// workgroup, from one LDS copy of its Q, K, V and dO tiles (rows past the
// group repeat its last member). Waves 0-1 own queries 32w..32w+31: S^T and
// dP^T against the key and value tiles, the row softmax, D = sum_k P dP (the
// whole row is on chip, so dO . O is not needed), (lse, D) into LDS, then
// dQ^T = K^T dS^T. Waves 2-3 own keys 32w..32w+31: S and dP against the
// query and dO tiles while the query waves finish the softmax, then, with
// (lse, D) from LDS, P, dS, dV^T = dO^T P and dK^T = Q^T dS.
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_small_bf16(BwdLaunch p) {
  using G = TileGeo<D>;
  constexpr int DK = G::DK, DB = G::DB;
  __shared__ __align__(1024) unsigned char lds[4 * G::TILEB + 64 * 8];
  unsigned char *const qt = lds, *const kt = lds + G::TILEB, *const vt = lds + 2 * G::TILEB,
                       *const dt = lds + 3 * G::TILEB;
  unsigned char *const stl = lds + 4 * G::TILEB;   // (lse, D) per member, float2

  const uint32_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int32_t g = (int32_t)(bid % (uint32_t)p.ga.n_groups);
  const int64_t bh = (int64_t)(bid / (uint32_t)p.ga.n_groups);
  const GroupGeom geo = group_geom(p.ga, g);
  if (geo.len <= 0) return;   // uniform
  const RowMap rm = row_map(geo);
  const int64_t slice = bh * p.head_elems;
  const void *const srcs[4] = {p.q, p.k, p.v, p.dout};

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int tr_key = 4 * half + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const LaneOffsets<D> lo = lane_offsets<D>(col, half, tr_key, tr_col);

#pragma unroll
  for (int tile = 0; tile < 4; ++tile) {
    const unsigned char *src =
        uniform_ptr(reinterpret_cast<const unsigned char *>(static_cast<const u16 *>(srcs[tile]) + slice));
    for (int ii = wave; ii < G::NINST; ii += 4) dma_row_window<D>(src, lds + tile * G::TILEB, rm, 0, ii, lane);
  }
  wait_vmcnt<0>();
  __syncthreads();

  const bool qrole = wave < 2;
  const int w2 = wave & 1;
  // The rows this wave adds its dQ (query waves) or dK (key waves) onto, loaded
  // now so that the load overlaps the whole computation instead of the store.
  constexpr int kOldRows = 32 * G::CPR / 64;
  uint4 old_rows[kOldRows];
  if (p.accumulate != 0)
    load_old_rows<D>(static_cast<const u16 *>(qrole ? p.dq : p.dk) + slice, geo, 32 * w2, geo.len, lane, old_rows);
  // this lane's own row (a query or a key) of the two register operands, read from its tile
  const unsigned char *own_a = (qrole ? qt : kt) + 32 * w2 * G::ROWB;
  const unsigned char *own_b = (qrole ? dt : vt) + 32 * w2 * G::ROWB;
  bf16x8_t fa[DK], fb[DK];
#pragma unroll
  for (int j = 0; j < DK; ++j) {
    fa[j] = *reinterpret_cast<const bf16x8_t *>(own_a + lo.k[j]);
    fb[j] = *reinterpret_cast<const bf16x8_t *>(own_b + lo.k[j]);
  }
  // query waves: S^T = K Q^T, dP^T = V dO^T; key waves: S = Q K^T, dP = dO V^T
  f32x16_t s0, s1, t0, t1;
  tile_times<D>(qrole ? kt : qt, fa, lo, s0, s1);
  tile_times<D>(qrole ? vt : dt, fb, lo, t0, t1);

  bf16x8_t w0[2], w1[2];   // query waves: dS^T (rows = keys)
  if (qrole) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int32_t key = 8 * (r / 4) + 4 * half + (r % 4);
      if (key >= geo.len) s0[r] = -INFINITY;
      if (key + 32 >= geo.len) s1[r] = -INFINITY;
    }
    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    mx = fmaxf(mx, swap_halves(mx));
    const float m = mx * p.scale_log2;
    float l = 0.f, u = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], p.scale_log2, -m));
      s1[r] = __builtin_amdgcn_exp2f(fmaf(s1[r], p.scale_log2, -m));
      l += s0[r] + s1[r];
      u = fmaf(s0[r], t0[r], fmaf(s1[r], t1[r], u));
    }
    l += swap_halves(l);
    u += swap_halves(u);
    const float inv_l = 1.f / l;
    const float dq_row = u * inv_l;   // D = sum_k P dP of this query
    if (half == 0) {
      float2 *st = reinterpret_cast<float2 *>(stl) + 32 * w2 + col;
      *st = make_float2(m + __builtin_log2f(l), dq_row);
    }
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      pack_pair(s0[r] * inv_l * (t0[r] - dq_row), s0[r + 1] * inv_l * (t0[r + 1] - dq_row), r, w0);
      pack_pair(s1[r] * inv_l * (t1[r] - dq_row), s1[r + 1] * inv_l * (t1[r + 1] - dq_row), r, w1);
    }
  }
  __syncthreads();   // (lse, D) of every query in LDS

  f32x16_t acc_a[DB], acc_b[DB];   // query waves: dQ^T in acc_a; key waves: dK^T in acc_a, dV^T in acc_b
#pragma unroll
  for (int b = 0; b < DB; ++b) acc_a[b] = acc_b[b] = f32x16_t{};
  if (qrole) {
    tile_t_times<D>(kt, w0, w1, lo, tr_col, acc_a);
  } else {
    bf16x8_t p0[2], p1[2], g0[2], g1[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int row = 32 * blk + 8 * r4 + 4 * half;   // queries row .. row+3
        const f32x4_t st01 = *reinterpret_cast<const f32x4_t *>(stl + row * 8);
        const f32x4_t st23 = *reinterpret_cast<const f32x4_t *>(stl + row * 8 + 16);
        const float lse[4] = {st01[0], st01[2], st23[0], st23[2]};
        const float dd[4] = {st01[1], st01[3], st23[1], st23[3]};
        float pv[4], gv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          const float sv = blk ? s1[r] : s0[r];
          const float tv = blk ? t1[r] : t0[r];
          const bool valid = row + e < geo.len;   // repeated rows past the group get zero weight
          const float pr = valid ? __builtin_amdgcn_exp2f(fmaf(sv, p.scale_log2, -lse[e])) : 0.f;
          pv[e] = pr;
          gv[e] = pr * (tv - dd[e]);
        }
        bf16x8_t(&pp)[2] = blk ? p1 : p0;
        bf16x8_t(&gg)[2] = blk ? g1 : g0;
        pack_pair(pv[0], pv[1], 4 * r4, pp);
        pack_pair(pv[2], pv[3], 4 * r4 + 2, pp);
        pack_pair(gv[0], gv[1], 4 * r4, gg);
        pack_pair(gv[2], gv[3], 4 * r4 + 2, gg);
      }
    }
    tile_t_times<D>(dt, p0, p1, lo, tr_col, acc_b);   // dV^T += dO^T P
    tile_t_times<D>(qt, g0, g1, lo, tr_col, acc_a);   // dK^T += Q^T dS
  }
  __syncthreads();   // every tile read: the waves' 32-row fp32 staging areas may reuse them
  unsigned char *ot = lds + wave * 32 * (4 * D);
  const int32_t r0 = 32 * w2;
  store_rows_lds<D>(ot, acc_a, p.scale, col, half, lane,
                    static_cast<u16 *>(qrole ? p.dq : p.dk) + slice, geo, r0, geo.len, p.accumulate != 0, old_rows);
  __syncthreads();
  if (!qrole)
    store_rows_lds<D>(ot, acc_b, 1.f, col, half, lane, static_cast<u16 *>(p.dv) + slice, geo, r0, geo.len, false);
}

}  // namespace ma
