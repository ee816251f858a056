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
// Rows outside the group are clamped duplicates (finite) and get zero weight.
#pragma once
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
// m0 + r < mend go to base + token * D; with `add`, onto the values there.
template <int D>
__device__ __forceinline__ void store_rows_lds(unsigned char *ot, const f32x16_t *acc, float colscale, int col,
                                               int half, int lane, u16 *base, const GroupGeom &geo, int32_t m0,
                                               int32_t mend, bool add) {
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
        const bf16x8_t old = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(dst));
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

// ---------------------------------------------------------------------------
// dQ pass. Ring: keys in LDS tiles 0..2 (tile t in t % 3), values in 3..4.
// Step t issues the value windows of tile t+1, then the key windows of tile
// t+2 (rows past the group clamped), so the wait opening step t+1 may leave
// the newest WPT windows in flight.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dq_bf16(BwdLaunch p) {
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
  const RowMap rm = row_map(geo);
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

  const int32_t n = (geo.len + kKeyTile - 1) / kKeyTile;
  // prologue: K(0), V(0), K(1), then this lane's query, dO and O rows
#pragma unroll
  for (int w = 0; w < WPT; ++w) dma_row_window<D>(kbytes, lds, rm, 0, wave + NW * w, lane);
#pragma unroll
  for (int w = 0; w < WPT; ++w) dma_row_window<D>(vbytes, lds + 3 * G::TILEB, rm, 0, wave + NW * w, lane);
#pragma unroll
  for (int w = 0; w < WPT; ++w) dma_row_window<D>(kbytes, lds + G::TILEB, rm, kKeyTile, wave + NW * w, lane);
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
  int ks = 0, ys = 0;
  for (int32_t t = 0; t < n; ++t) {
    if (t > 0) wait_vmcnt<WPT>();   // leave the key windows of tile t+1 in flight
    __syncthreads();
    const unsigned char *kc = lds + ks * G::TILEB;
    const unsigned char *vc = lds + (3 + ys) * G::TILEB;
    unsigned char *vn = lds + (3 + (ys ^ 1)) * G::TILEB;
    unsigned char *kn = lds + (ks == 0 ? 2 : ks - 1) * G::TILEB;
#pragma unroll
    for (int w = 0; w < WPT; ++w) dma_row_window<D>(vbytes, vn, rm, (t + 1) * kKeyTile, wave + NW * w, lane);
#pragma unroll
    for (int w = 0; w < WPT; ++w) dma_row_window<D>(kbytes, kn, rm, (t + 2) * kKeyTile, wave + NW * w, lane);
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
    ks = ks == 2 ? 0 : ks + 1;
    ys ^= 1;
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
// dK/dV pass. Ring: query tiles in LDS tiles 0..2, dO tiles in 3..4, and the
// (lse, D) window of each dO tile (128 members x 8 bytes, of which the tile
// uses 64) in two 1 KB slots. Step t issues dO(t+1), stats(t+1), then Q(t+2).
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dkdv_bf16(BwdLaunch p) {
  using G = TileGeo<D>;
  static_assert(G::NINST % NW == 0, "every wave must issue the same number of DMA instructions");
  constexpr int WPT = G::NINST / NW;
  constexpr int DK = G::DK, DB = G::DB;
  __shared__ __align__(1024) unsigned char lds[5 * G::TILEB + 2048];
  unsigned char *const st_lds = lds + 5 * G::TILEB;

  const uint32_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int32_t kt = (int32_t)(bid % (uint32_t)p.n_tiles);
  const uint32_t rest = bid / (uint32_t)p.n_tiles;
  const int32_t g = (int32_t)(rest % (uint32_t)p.ga.n_groups);
  const int64_t bh = (int64_t)(rest / (uint32_t)p.ga.n_groups);
  const GroupGeom geo = group_geom(p.ga, g);
  const int32_t kbase = kt * 32 * NW;
  if (kbase >= geo.len) return;   // uniform
  const int32_t kend = min(geo.len, kbase + 32 * NW);
  const RowMap rm = row_map(geo);
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

  const int32_t n = (geo.len + kKeyTile - 1) / kKeyTile;
  auto stats_window = [&](int32_t t, int slot) __attribute__((always_inline)) {
    // members [64t, 64t + 128): 1 KB, 16 bytes per lane; every wave issues the same window
    dma16(sbytes, (uint32_t)(t * kKeyTile * 8 + 16 * lane), st_lds + slot * 1024);
  };
#pragma unroll
  for (int w = 0; w < WPT; ++w) dma_row_window<D>(qbytes, lds, rm, 0, wave + NW * w, lane);
#pragma unroll
  for (int w = 0; w < WPT; ++w) dma_row_window<D>(dbytes, lds + 3 * G::TILEB, rm, 0, wave + NW * w, lane);
  stats_window(0, 0);
#pragma unroll
  for (int w = 0; w < WPT; ++w) dma_row_window<D>(qbytes, lds + G::TILEB, rm, kKeyTile, wave + NW * w, lane);
  bf16x8_t kb[DK], vb[DK];
  load_row_frags<D>(static_cast<const u16 *>(p.k) + slice, geo, km, half, kb);
  load_row_frags<D>(static_cast<const u16 *>(p.v) + slice, geo, km, half, vb);
  wait_vmcnt<0>();
#pragma unroll
  for (int j = 0; j < DK; ++j) asm volatile("" ::"v"(kb[j]), "v"(vb[j]));
  __syncthreads();

  f32x16_t dka[DB], dva[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) dka[b] = dva[b] = f32x16_t{};
  int qs = 0, ds = 0;
  for (int32_t t = 0; t < n; ++t) {
    if (t > 0) wait_vmcnt<WPT>();   // leave the query windows of tile t+1 in flight
    __syncthreads();
    const unsigned char *qc = lds + qs * G::TILEB;
    const unsigned char *dc = lds + (3 + ds) * G::TILEB;
    const unsigned char *sc = st_lds + ds * 1024;
    unsigned char *dn = lds + (3 + (ds ^ 1)) * G::TILEB;
    unsigned char *qn = lds + (qs == 0 ? 2 : qs - 1) * G::TILEB;
#pragma unroll
    for (int w = 0; w < WPT; ++w) dma_row_window<D>(dbytes, dn, rm, (t + 1) * kKeyTile, wave + NW * w, lane);
    stats_window(t + 1, ds ^ 1);
#pragma unroll
    for (int w = 0; w < WPT; ++w) dma_row_window<D>(qbytes, qn, rm, (t + 2) * kKeyTile, wave + NW * w, lane);
    if (wave_active) {
      f32x16_t s0, s1, t0, t1;
      tile_times<D>(qc, kb, lo, s0, s1);   // S: rows = queries of the tile, columns = this wave's keys
      tile_times<D>(dc, vb, lo, t0, t1);   // dP
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
            const float tv = blk ? t1[r] : t0[r];
            // (lse, D) of members past the group are never written: select them away
            // before any arithmetic so that whatever bytes they hold cannot propagate
            const bool valid = q0t + row + e < geo.len;
            const float lv = valid ? lse[e] : 0.f, dv_ = valid ? dd[e] : 0.f;
            const float pr = valid ? __builtin_amdgcn_exp2f(fmaf(sv, p.scale_log2, -lv)) : 0.f;
            pv[e] = pr;
            gv[e] = pr * (tv - dv_);
          }
          if (blk) {
            pack_pair(pv[0], pv[1], 4 * r4, p1);
            pack_pair(pv[2], pv[3], 4 * r4 + 2, p1);
            pack_pair(gv[0], gv[1], 4 * r4, g1);
            pack_pair(gv[2], gv[3], 4 * r4 + 2, g1);
          } else {
            pack_pair(pv[0], pv[1], 4 * r4, p0);
            pack_pair(pv[2], pv[3], 4 * r4 + 2, p0);
            pack_pair(gv[0], gv[1], 4 * r4, g0);
            pack_pair(gv[2], gv[3], 4 * r4 + 2, g0);
          }
        }
      }
      tile_t_times<D>(dc, p0, p1, lo, tr_col, dva);   // dV^T += dO^T P
      tile_t_times<D>(qc, g0, g1, lo, tr_col, dka);   // dK^T += Q^T dS
    }
    qs = qs == 2 ? 0 : qs + 1;
    ds ^= 1;
  }
  wait_vmcnt<0>();
  __syncthreads();
  // dK = s * dKacc, dV = dVacc, each through LDS (waves use separate 32-row fp32 areas)
  unsigned char *ot = lds + wave * 32 * (4 * D);
  store_rows_lds<D>(ot, dka, p.scale, col, half, lane, static_cast<u16 *>(p.dk) + slice, geo, k0w, kend,
                    p.accumulate != 0);
  __syncthreads();
  store_rows_lds<D>(ot, dva, 1.f, col, half, lane, static_cast<u16 *>(p.dv) + slice, geo, k0w, kend, false);
}

}  // namespace ma
