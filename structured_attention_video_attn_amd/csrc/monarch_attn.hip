// monarch_attn.hip -- C ABI entry points: argument checks, stage planning, launches.
//
// Monarch attention (MonarchRT summaries: nl "Methodologie", zh 2.1-2.2) runs
// as two launches on the caller's stream: stage R (softmax attention inside
// each aligned block) writes Y into the caller's workspace, stage L (softmax
// attention across blocks, among tokens with the same intra-block index, or
// inside a frame x row tile of them) reads Y and writes the output. Stream
// order is the only synchronisation between them. A stage whose groups all
// have a single member is the identity and is not launched.
#include <hip/hip_runtime.h>

#include <math.h>

#include <atomic>
#include <mutex>

#include "../../include/monarch_attn.h"
#include "attn_bf16.h"
#include "attn_bwd_bf16.h"
#include "attn_f32.h"
#include "attn_f32_mfma.h"
#include "validate.h"

namespace ma {
namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MA_OK;
  g_last_hip_error = (int)e;
  return MA_ERR_HIP;
}

// ------------------------------------------------- fixed buffer of the no-allocation entry point
// monarch_attn_fwd_noalloc keeps the stage-R output Y in this array instead of a
// caller's workspace. Each GPU the library runs on holds its own copy (allocated
// when the code object is loaded, kept until the process ends). In host code the
// name is only a stand-in: the device address comes from hipGetSymbolAddress,
// once per device, and only that address is ever handed to a kernel.
constexpr size_t kScratchBytes = size_t(128) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on the current device (looked up once per device).
int scratch_address(void **out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= 0 && dev < kMaxDevices && addr[dev] != nullptr) {
    *out = addr[dev];
    return MA_OK;
  }
  void *p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return hip_status(e);
  if (p == nullptr) return MA_ERR_HIP;
  if (dev >= 0 && dev < kMaxDevices) addr[dev] = p;
  *out = p;
  return MA_OK;
}

enum class Kernel { kF32, kF32Mfma, kBlock, kStream };

// Host-side plan of one group-attention launch.
struct Plan {
  AttnLaunch a;
  uint32_t blocks;    // workgroups (the persistent kernel: an upper bound, see run_plan)
  int32_t n_items;    // groups * batch * heads (persistent kernel only)
  int32_t waves;      // waves per workgroup (streaming kernel only)
  bool two_level;     // streaming kernel: some group spans several outer rows (tiled boxes), or
                      // member offsets do not fit the 24-bit one-level DMA addressing
  Kernel kernel;
};

// Compute units of the current device, cached per device (the persistent
// kernel launches kBlockResident workgroups per CU).
int device_cus(int *cus) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return MA_OK;
    }
  }
  int c = 0;
  e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_status(e);
  if (c <= 0) c = 1;
  if (dev >= 0 && dev < 64) cache[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return MA_OK;
}

template <int D>
int launch_d(const Plan &pl, hipStream_t s) {
  switch (pl.kernel) {
    case Kernel::kF32:
      // the vector-ALU fp32 kernel serves head_dim 16 only (plan_launch sends
      // 32..128 to the matrix-core kernel), so it is instantiated for 16 only
      if constexpr (D == 16) {
        hipLaunchKernelGGL(group_attn_f32<D>, dim3(pl.blocks), dim3(kF32Threads), 0, s, pl.a);
      } else {
        return MA_ERR_UNSUPPORTED;
      }
      break;
    case Kernel::kF32Mfma:
      if constexpr (D >= 32) {
        if (pl.waves >= 4)
          hipLaunchKernelGGL((group_attn_f32_mfma<D, 4>), dim3(pl.blocks), dim3(4 * 64), 0, s, pl.a);
        else
          hipLaunchKernelGGL((group_attn_f32_mfma<D, 2>), dim3(pl.blocks), dim3(2 * 64), 0, s, pl.a);
      } else {
        return MA_ERR_UNSUPPORTED;
      }
      break;
    case Kernel::kBlock: {
      int cus = 0;
      const int st = device_cus(&cus);
      if (st != MA_OK) return st;
      const uint32_t resident = kBlockResident * (uint32_t)cus;
      const uint32_t blocks = pl.blocks < resident ? pl.blocks : resident;
      hipLaunchKernelGGL(block_attn_bf16<D>, dim3(blocks), dim3(kBlockWaves * 64), 0, s, pl.a, pl.n_items);
      break;
    }
    default:
      // waves per workgroup; every wave must issue whole DMA instructions
      if constexpr (TileGeo<D>::NINST % 4 == 0) {
        if (pl.waves >= 4) {
          if (pl.two_level)
            hipLaunchKernelGGL((group_attn_bf16<D, 4, true>), dim3(pl.blocks), dim3(4 * 64), 0, s, pl.a);
          else
            hipLaunchKernelGGL((group_attn_bf16<D, 4, false>), dim3(pl.blocks), dim3(4 * 64), 0, s, pl.a);
          break;
        }
      }
      if (pl.two_level)
        hipLaunchKernelGGL((group_attn_bf16<D, 2, true>), dim3(pl.blocks), dim3(2 * 64), 0, s, pl.a);
      else
        hipLaunchKernelGGL((group_attn_bf16<D, 2, false>), dim3(pl.blocks), dim3(2 * 64), 0, s, pl.a);
      break;
  }
  return hip_status(hipGetLastError());
}

// The streaming kernels' DMA addressing: two-level when some group spans
// several outer rows (tiled boxes), or when member offsets do not fit the
// 24-bit multiply of the one-level form.
bool two_level(const Problem &p, const GroupAddr &ga) {
  // A box whose inner extent is whole (tile_i >= len_i) and whose outer stride
  // continues the inner one is a single run: member m at base + m * stride_in.
  const bool whole_rows = ga.tile_i >= ga.len_i && (int64_t)ga.stride_out == (int64_t)ga.len_i * ga.stride_in;
  const bool outer = ga.len_o > 1 && ga.tile_o > 1 && !whole_rows;
  const int64_t mstride = (int64_t)ga.stride_in * 2 * p.D;
  return outer || ga.max_len >= (1 << 24) || mstride >= (1 << 24);
}

// Query ranges (streaming bf16 kernel only): queries from member q_first on,
// cut into spans of q_span members (0: one span) whose keys end with the span.
struct QueryRange {
  int32_t q_first = 0;
  int32_t q_span = 0;
  bool stream = false;   // take the streaming kernel even for short groups
};

int plan_launch(const Problem &p, const GroupAddr &ga, const void *q, const void *k,
                const void *vals, void *out, Plan *pl, QueryRange qr = QueryRange{}) {
  AttnLaunch a{};
  a.q = q;
  a.k = k;
  a.vals = vals;
  a.out = out;
  a.head_elems = p.slice_elems;
  a.ga = ga;
  const bool ranged = qr.q_first > 0 || qr.q_span > 0 || qr.stream;
  if (ranged && p.dtype != MA_BF16) return MA_ERR_UNSUPPORTED;
  const int32_t queries = ga.max_len - qr.q_first;   // per group, from q_first on
  const int32_t qlen = qr.q_span > 0 && qr.q_span < queries ? qr.q_span : queries;
  a.q_first = qr.q_first;
  a.q_span = qr.q_span > 0 && qr.q_span < queries ? qr.q_span : 0;
  a.n_spans = a.q_span > 0 ? (queries + a.q_span - 1) / a.q_span : 1;
  a.n_bh = (int32_t)(p.batch * p.heads);
  a.scale = (float)(1.0 / sqrt((double)p.D));
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)p.D));
  int q_per_block;
  if (p.dtype == MA_F32 && p.D >= 32) {
    // matrix-core fp32 kernel: waves of 32 queries, two or four per workgroup
    const int64_t need = (qlen + kQueriesPerWave - 1) / kQueriesPerWave;
    pl->waves = need > 2 ? 4 : 2;
    q_per_block = kQueriesPerWave * pl->waves;
    pl->kernel = Kernel::kF32Mfma;
  } else if (p.dtype == MA_F32) {
    q_per_block = kF32Threads;
    pl->kernel = Kernel::kF32;
  } else if (ga.max_len <= kKeyTile && !ranged) {
    q_per_block = kKeyTile;   // one group per work item
    pl->kernel = Kernel::kBlock;
  } else {
    // Workgroups of up to 4 waves (128 queries), two resident per CU, each with
    // a ring of three key and two value tiles: measured faster on MI355X than
    // 8-wave workgroups (a 4-deep ring shared by 256 queries, or two items whose
    // halves alternate matrix and vector sections), whose waves all meet at
    // every barrier together.
    // The group's queries are spread evenly over its workgroups; the wave
    // count is the power of two that covers a share and that the DMA split
    // allows (D/8 16-byte chunks per row).
    const int max_waves = p.D >= 32 ? 4 : 2;
    const int64_t cap = (int64_t)kQueriesPerWave * max_waves;
    const int64_t per_group = (qlen + cap - 1) / cap;
    const int64_t share = (qlen + per_group - 1) / per_group;
    const int64_t need = (share + kQueriesPerWave - 1) / kQueriesPerWave;
    int w = 2;
    while (w < need && w < max_waves) w *= 2;
    pl->waves = w;
    q_per_block = (int)(kQueriesPerWave * need);
    pl->kernel = Kernel::kStream;
    pl->two_level = two_level(p, ga);
  }
  a.n_qtiles = (qlen + q_per_block - 1) / q_per_block;
  a.q_tile = q_per_block;
  uint64_t per_group = (uint64_t)a.n_qtiles * (uint64_t)a.n_spans;
  if (pl->kernel == Kernel::kStream && a.n_spans > 1) {
    // Several spans: workgroups of full width take wave items (32 queries of
    // one span) from the longest span down, so a workgroup's waves stream
    // about as many keys as each other and no wave slot idles for want of
    // queries (a span rarely fills a whole workgroup).
    pl->waves = p.D >= 32 ? 4 : 2;
    a.span_waves = (a.q_span + kQueriesPerWave - 1) / kQueriesPerWave;
    const int32_t last = queries - (a.n_spans - 1) * a.q_span;
    a.last_waves = (last + kQueriesPerWave - 1) / kQueriesPerWave;
    const int64_t items = (int64_t)a.last_waves + (int64_t)(a.n_spans - 1) * a.span_waves;
    a.n_qtiles = (int32_t)((items + pl->waves - 1) / pl->waves);
    a.q_tile = kQueriesPerWave * pl->waves;
    per_group = (uint64_t)a.n_qtiles;
  }
  const uint64_t blocks = per_group * (uint64_t)ga.n_groups * (uint64_t)a.n_bh;
  if (blocks > (uint64_t)INT32_MAX) return MA_ERR_UNSUPPORTED;
  pl->blocks = (uint32_t)blocks;
  pl->n_items = (int32_t)blocks;
  pl->a = a;
  return MA_OK;
}

int run_plan(const Problem &p, const Plan &pl, hipStream_t s) {
  if (pl.blocks == 0) return MA_OK;
  switch (p.D) {
    case 16: return launch_d<16>(pl, s);
    case 32: return launch_d<32>(pl, s);
    case 64: return launch_d<64>(pl, s);
    default: return launch_d<128>(pl, s);
  }
}

int copy_async(void *dst, const void *src, size_t bytes, hipStream_t s) {
  if (bytes == 0) return MA_OK;
  return hip_status(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s));
}

// Stage-L members per frame (b1 / T): a group holds one member per (frame, row)
// at r_axes = 1, one per frame at 2, one per token at 0.
int64_t members_per_frame(const Problem &p) { return p.T > 0 ? p.b1 / p.T : 0; }

// chunk_t > 0: chunk-causal stage L (bf16, r_axes 0..2): a query in chunk c
// attends to the members of its group in chunks 0..c.
int monarch_common(const void *q, const void *k, const void *v, void *out, void *ws, size_t ws_bytes,
                   int32_t batch, int32_t heads, int32_t T, int32_t H, int32_t W, int32_t r_axes,
                   int32_t tile_t, int32_t tile_h, bool tiled, int32_t head_dim, int32_t dtype,
                   hipStream_t stream, int32_t chunk_t = 0) {
  Problem p;
  int st = resolve_grid(batch, heads, T, H, W, r_axes, tile_t, tile_h, tiled, head_dim, dtype, &p);
  if (st != MA_OK) return st;
  QueryRange lr;
  if (chunk_t != 0) {
    if (chunk_t < 0 || r_axes > 2 || tiled) return MA_ERR_INVALID_ARG;
    if (dtype != MA_BF16) return MA_ERR_UNSUPPORTED;
    const int64_t span = (int64_t)chunk_t * members_per_frame(p);
    lr.q_span = span < p.b1 ? (int32_t)span : 0;
    lr.stream = true;
  }
  if (p.empty) return MA_OK;
  st = check_tensor_ptrs(q, k, v, out, p.tensor_bytes);
  if (st != MA_OK) return st;
  const size_t need = workspace_needed(p);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need) return MA_ERR_WORKSPACE;
    if (!aligned16(ws)) return MA_ERR_ALIGNMENT;
    if (overlaps(ws, q, need) || overlaps(ws, k, need) || overlaps(ws, v, need) ||
        overlaps(ws, out, need))
      return MA_ERR_INVALID_ARG;
  }
  Plan pr{}, pl{};
  const bool run_r = !p.r_trivial, run_l = !p.l_trivial;
  void *y = run_l ? ws : out;   // stage R output
  const void *y_in = run_r ? (const void *)ws : v;
  if (run_r) {
    st = plan_launch(p, stage_r_groups(p), q, k, v, y, &pr);
    if (st != MA_OK) return st;
  }
  if (run_l) {
    st = plan_launch(p, stage_l_groups(p), q, k, y_in, out, &pl, lr);
    if (st != MA_OK) return st;
  }
  if (!run_r && !run_l) return copy_async(out, v, p.tensor_bytes, stream);
  if (run_r) {
    st = run_plan(p, pr, stream);
    if (st != MA_OK) return st;
  }
  if (run_l) st = run_plan(p, pl, stream);
  return st;
}

// ---------------------------------------------------------------- backward
// Rows per backward workgroup tile and waves (every wave issues whole DMA windows).
template <int D>
constexpr int bwd_waves() {
  return TileGeo<D>::NINST % 4 == 0 ? 4 : 2;
}

int bwd_waves_for(int64_t d) {
  switch (d) {
    case 16: return bwd_waves<16>();
    case 32: return bwd_waves<32>();
    case 64: return bwd_waves<64>();
    default: return bwd_waves<128>();
  }
}

// Members per group in the (lse, D) rows: the dK/dV pass reads 128-member
// windows starting at 64t for t up to ceil(len / 64) (the last one is a
// prefetch past the group), so every window stays inside its group's rows.
int64_t stats_stride(const GroupAddr &ga) { return ((int64_t)ga.max_len + 63) / 64 * 64 + 128; }

size_t stats_bytes(const Problem &p, const GroupAddr &ga) {
  return (size_t)(p.batch * p.heads) * (size_t)ga.n_groups * (size_t)stats_stride(ga) * 8u;
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of the backward: Y and dY (one tensor each), then the (lse, D)
// rows of stage L and of stage R.
size_t bwd_workspace_needed(const Problem &p) {
  if (p.empty) return 0;
  return 2 * round256(p.tensor_bytes) + round256(stats_bytes(p, stage_l_groups(p))) +
         round256(stats_bytes(p, stage_r_groups(p)));
}

template <int D>
int launch_bwd_d(bool dq_pass, bool two_level, const BwdLaunch &a, uint32_t blocks, hipStream_t s) {
  constexpr int NW = bwd_waves<D>();
  const dim3 grid(blocks), block(NW * 64);
  if (dq_pass) {
    if (two_level)
      hipLaunchKernelGGL((bwd_dq_bf16<D, NW, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dq_bf16<D, NW, false>), grid, block, 0, s, a);
  } else if constexpr (D >= 128) {
    // dV, then dK: each pass fits two waves per SIMD, where both together do not
    if (two_level) {
      hipLaunchKernelGGL((bwd_dkdv_bf16<D, NW, true, 2>), grid, block, 0, s, a);
      hipLaunchKernelGGL((bwd_dkdv_bf16<D, NW, true, 1>), grid, block, 0, s, a);
    } else {
      hipLaunchKernelGGL((bwd_dkdv_bf16<D, NW, false, 2>), grid, block, 0, s, a);
      hipLaunchKernelGGL((bwd_dkdv_bf16<D, NW, false, 1>), grid, block, 0, s, a);
    }
  } else {
    if (two_level)
      hipLaunchKernelGGL((bwd_dkdv_bf16<D, NW, true, 0>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dkdv_bf16<D, NW, false, 0>), grid, block, 0, s, a);
  }
  return hip_status(hipGetLastError());
}

// Whole backward of one stage whose groups have at most 64 members.
int run_bwd_small(const Problem &p, const GroupAddr &ga, BwdLaunch a, hipStream_t s) {
  a.head_elems = p.N * p.D;
  a.ga = ga;
  a.scale = (float)(1.0 / sqrt((double)p.D));
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)p.D));
  const uint64_t blocks = (uint64_t)ga.n_groups * (uint64_t)(p.batch * p.heads);
  if (blocks == 0) return MA_OK;
  if (blocks > (uint64_t)INT32_MAX) return MA_ERR_UNSUPPORTED;
  const dim3 grid((uint32_t)blocks), block(256);
  switch (p.D) {
    case 16: hipLaunchKernelGGL((bwd_small_bf16<16>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((bwd_small_bf16<32>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((bwd_small_bf16<64>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((bwd_small_bf16<128>), grid, block, 0, s, a); break;
  }
  return hip_status(hipGetLastError());
}

// One backward pass of one stage over the groups `ga`.
int run_bwd(const Problem &p, const GroupAddr &ga, bool dq_pass, BwdLaunch a, hipStream_t s) {
  const int nw = bwd_waves_for(p.D);
  a.head_elems = p.N * p.D;
  a.ga = ga;
  a.n_tiles = (ga.max_len + 32 * nw - 1) / (32 * nw);
  a.stats_stride = (int32_t)stats_stride(ga);
  a.scale = (float)(1.0 / sqrt((double)p.D));
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)p.D));
  const uint64_t blocks = (uint64_t)a.n_tiles * (uint64_t)ga.n_groups * (uint64_t)(p.batch * p.heads);
  if (blocks == 0) return MA_OK;
  if (blocks > (uint64_t)INT32_MAX) return MA_ERR_UNSUPPORTED;
  const bool tl = two_level(p, ga);
  switch (p.D) {
    case 16: return launch_bwd_d<16>(dq_pass, tl, a, (uint32_t)blocks, s);
    case 32: return launch_bwd_d<32>(dq_pass, tl, a, (uint32_t)blocks, s);
    case 64: return launch_bwd_d<64>(dq_pass, tl, a, (uint32_t)blocks, s);
    default: return launch_bwd_d<128>(dq_pass, tl, a, (uint32_t)blocks, s);
  }
}

// Backward of one stage: dq (+)= dQ, dk (+)= dK (accumulate), dv = dV, for the
// stage O_s = softmax-attention(q, k, v) over the groups `ga`, given the
// stage's output `o` and its gradient `dout`; `stats` holds the (lse, D) rows
// of the two-pass form.
int run_stage_bwd(const Problem &p, const GroupAddr &ga, const void *q, const void *k, const void *v,
                  const void *o, const void *dout, void *dq, void *dk, void *dv, float *stats, bool accumulate,
                  hipStream_t s) {
  BwdLaunch a{};
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.dq = dq; a.dk = dk; a.dv = dv;
  a.accumulate = accumulate ? 1 : 0;
  if (ga.max_len <= kKeyTile) return run_bwd_small(p, ga, a, s);
  a.o = o; a.stats = stats;
  int st = run_bwd(p, ga, true, a, s);
  if (st != MA_OK) return st;
  return run_bwd(p, ga, false, a, s);
}

}  // namespace
}  // namespace ma

using namespace ma;

extern "C" {

size_t ma_workspace_bytes(int32_t batch, int32_t heads, int32_t T, int32_t H, int32_t W,
                          int32_t r_axes, int32_t tile_t, int32_t tile_h, int32_t head_dim,
                          int32_t dtype) {
  Problem p;
  const bool tiled = tile_t != 0 || tile_h != 0;
  if (resolve_grid(batch, heads, T, H, W, r_axes, tile_t, tile_h, tiled, head_dim, dtype, &p) != MA_OK)
    return 0;
  return workspace_needed(p);
}

int monarch_attn_fwd(const void *q, const void *k, const void *v, void *out, void *workspace,
                     size_t workspace_bytes, int32_t batch, int32_t heads, int32_t T, int32_t H,
                     int32_t W, int32_t r_axes, int32_t head_dim, int32_t dtype,
                     struct ihipStream_t *stream) {
  return monarch_common(q, k, v, out, workspace, workspace_bytes, batch, heads, T, H, W, r_axes, 0,
                        0, false, head_dim, dtype, stream);
}

int monarch_attn_fwd_noalloc(const void *q, const void *k, const void *v, void *out, int32_t batch,
                             int32_t heads, int32_t T, int32_t H, int32_t W, int32_t r_axes, int32_t head_dim,
                             int32_t dtype, struct ihipStream_t *stream) {
  // every host-side check first, as in monarch_attn_fwd, then the buffer's address
  Problem p;
  int st = resolve_grid(batch, heads, T, H, W, r_axes, 0, 0, false, head_dim, dtype, &p);
  if (st != MA_OK || p.empty) return st;
  st = check_tensor_ptrs(q, k, v, out, p.tensor_bytes);
  if (st != MA_OK) return st;
  const size_t need = workspace_needed(p);
  if (need > kScratchBytes) return MA_ERR_SCRATCH;
  void *ws = nullptr;
  if (need > 0) {
    st = scratch_address(&ws);
    if (st != MA_OK) return st;
  }
  return monarch_common(q, k, v, out, ws, need > 0 ? kScratchBytes : 0, batch, heads, T, H, W, r_axes, 0, 0,
                        false, head_dim, dtype, stream);
}

size_t ma_noalloc_scratch_bytes(void) { return kScratchBytes; }

int monarch_attn_tiled_fwd(const void *q, const void *k, const void *v, void *out, void *workspace,
                           size_t workspace_bytes, int32_t batch, int32_t heads, int32_t T,
                           int32_t H, int32_t W, int32_t tile_t, int32_t tile_h, int32_t head_dim,
                           int32_t dtype, struct ihipStream_t *stream) {
  return monarch_common(q, k, v, out, workspace, workspace_bytes, batch, heads, T, H, W, 1, tile_t,
                        tile_h, true, head_dim, dtype, stream);
}

int monarch_attn_causal_fwd(const void *q, const void *k, const void *v, void *out, void *workspace,
                            size_t workspace_bytes, int32_t batch, int32_t heads, int32_t T, int32_t H,
                            int32_t W, int32_t r_axes, int32_t chunk_t, int32_t head_dim, int32_t dtype,
                            struct ihipStream_t *stream) {
  if (chunk_t < 1) return MA_ERR_INVALID_ARG;
  return monarch_common(q, k, v, out, workspace, workspace_bytes, batch, heads, T, H, W, r_axes, 0, 0,
                        false, head_dim, dtype, stream, chunk_t);
}

int monarch_attn_chunk_fwd(const void *q, const void *k, const void *v, void *y, void *out, int32_t batch,
                           int32_t heads, int32_t T, int32_t H, int32_t W, int32_t r_axes, int32_t t0,
                           int32_t chunk_t, int32_t head_dim, int32_t dtype, struct ihipStream_t *stream) {
  Problem p;
  int st = resolve_grid(batch, heads, T, H, W, r_axes, 0, 0, false, head_dim, dtype, &p);
  if (st != MA_OK) return st;
  if (r_axes > 2 || chunk_t < 1 || t0 < 0 || (int64_t)t0 + chunk_t > T) return MA_ERR_INVALID_ARG;
  if (dtype != MA_BF16) return MA_ERR_UNSUPPORTED;
  if (p.empty) return MA_OK;
  st = check_tensor_ptrs(q, k, v, out, p.tensor_bytes);
  if (st != MA_OK) return st;
  const bool use_y = !p.r_trivial;   // at r_axes = 0, Y is V and y is not used
  if (use_y) {
    if (y == nullptr) return MA_ERR_INVALID_ARG;
    if (!aligned16(y)) return MA_ERR_ALIGNMENT;
    if (overlaps(y, q, p.tensor_bytes) || overlaps(y, k, p.tensor_bytes) || overlaps(y, v, p.tensor_bytes) ||
        overlaps(y, out, p.tensor_bytes))
      return MA_ERR_INVALID_ARG;
  }
  // stage R over the chunk's frames: the same buffers seen from frame t0, with
  // the full buffers' distance between (batch, head) slices
  Problem pc;
  st = resolve_grid(batch, heads, chunk_t, H, W, r_axes, 0, 0, false, head_dim, dtype, &pc);
  if (st != MA_OK) return st;
  pc.slice_elems = p.slice_elems;
  // stage L over the frames [0, t0 + chunk_t), queries from the chunk's first member on
  Problem pl;
  st = resolve_grid(batch, heads, t0 + chunk_t, H, W, r_axes, 0, 0, false, head_dim, dtype, &pl);
  if (st != MA_OK) return st;
  pl.slice_elems = p.slice_elems;
  QueryRange lr;
  lr.q_first = (int32_t)((int64_t)t0 * members_per_frame(pl));
  lr.stream = true;
  const size_t off = (size_t)t0 * (size_t)(H * W) * (size_t)head_dim * p.elem_bytes;
  auto at = [off](const void *x) { return static_cast<const unsigned char *>(x) + off; };
  Plan pr{}, pll{};
  if (use_y) {
    st = plan_launch(pc, stage_r_groups(pc), at(q), at(k), at(v), static_cast<unsigned char *>(y) + off, &pr);
    if (st != MA_OK) return st;
  }
  st = plan_launch(pl, stage_l_groups(pl), q, k, use_y ? (const void *)y : v, out, &pll, lr);
  if (st != MA_OK) return st;
  if (use_y) {
    st = run_plan(pc, pr, stream);
    if (st != MA_OK) return st;
  }
  return run_plan(pl, pll, stream);
}

int dense_attn_fwd(const void *q, const void *k, const void *v, void *out, int32_t batch,
                   int32_t heads, int32_t n_tokens, int32_t head_dim, int32_t dtype,
                   struct ihipStream_t *stream) {
  Problem p;
  // dense attention is the single-block spec over a 1 x 1 x n_tokens grid
  int st = resolve_grid(batch, heads, 1, 1, n_tokens, 3, 0, 0, false, head_dim, dtype, &p);
  if (st != MA_OK || p.empty) return st;
  st = check_tensor_ptrs(q, k, v, out, p.tensor_bytes);
  if (st != MA_OK) return st;
  Plan pl{};
  st = plan_launch(p, dense_groups((int32_t)p.N), q, k, v, out, &pl);
  if (st != MA_OK) return st;
  return run_plan(p, pl, stream);
}

int ma_stage_r_fwd(const void *q, const void *k, const void *v, void *y, int32_t batch,
                   int32_t heads, int32_t T, int32_t H, int32_t W, int32_t r_axes,
                   int32_t head_dim, int32_t dtype, struct ihipStream_t *stream) {
  Problem p;
  int st = resolve_grid(batch, heads, T, H, W, r_axes, 0, 0, false, head_dim, dtype, &p);
  if (st != MA_OK || p.empty) return st;
  st = check_tensor_ptrs(q, k, v, y, p.tensor_bytes);
  if (st != MA_OK) return st;
  if (p.r_trivial) return copy_async(y, v, p.tensor_bytes, stream);
  Plan pl{};
  st = plan_launch(p, stage_r_groups(p), q, k, v, y, &pl);
  if (st != MA_OK) return st;
  return run_plan(p, pl, stream);
}

int ma_stage_l_fwd(const void *q, const void *k, const void *y, void *out, int32_t batch,
                   int32_t heads, int32_t T, int32_t H, int32_t W, int32_t r_axes, int32_t tile_t,
                   int32_t tile_h, int32_t head_dim, int32_t dtype, struct ihipStream_t *stream) {
  Problem p;
  const bool tiled = tile_t != 0 || tile_h != 0;
  int st = resolve_grid(batch, heads, T, H, W, r_axes, tile_t, tile_h, tiled, head_dim, dtype, &p);
  if (st != MA_OK || p.empty) return st;
  st = check_tensor_ptrs(q, k, y, out, p.tensor_bytes);
  if (st != MA_OK) return st;
  if (p.l_trivial) return copy_async(out, y, p.tensor_bytes, stream);
  Plan pl{};
  st = plan_launch(p, stage_l_groups(p), q, k, y, out, &pl);
  if (st != MA_OK) return st;
  return run_plan(p, pl, stream);
}

size_t ma_bwd_workspace_bytes(int32_t batch, int32_t heads, int32_t T, int32_t H, int32_t W,
                              int32_t r_axes, int32_t tile_t, int32_t tile_h, int32_t head_dim,
                              int32_t dtype) {
  Problem p;
  const bool tiled = tile_t != 0 || tile_h != 0;
  if (resolve_grid(batch, heads, T, H, W, r_axes, tile_t, tile_h, tiled, head_dim, dtype, &p) != MA_OK)
    return 0;
  if (dtype != MA_BF16) return 0;
  return bwd_workspace_needed(p);
}

int monarch_attn_bwd(const void *q, const void *k, const void *v, const void *out, const void *dout,
                     const void *y_fwd, void *dq, void *dk, void *dv, void *workspace, size_t workspace_bytes,
                     int32_t batch, int32_t heads, int32_t T, int32_t H, int32_t W, int32_t r_axes,
                     int32_t tile_t, int32_t tile_h, int32_t head_dim, int32_t dtype,
                     struct ihipStream_t *stream) {
  Problem p;
  const bool tiled = tile_t != 0 || tile_h != 0;
  int st = resolve_grid(batch, heads, T, H, W, r_axes, tile_t, tile_h, tiled, head_dim, dtype, &p);
  if (st != MA_OK) return st;
  if (dtype != MA_BF16) return MA_ERR_UNSUPPORTED;
  if (p.empty) return MA_OK;
  const void *ins[5] = {q, k, v, out, dout};
  void *outs[3] = {dq, dk, dv};
  for (const void *x : ins)
    if (x == nullptr) return MA_ERR_INVALID_ARG;
  for (const void *x : outs)
    if (x == nullptr) return MA_ERR_INVALID_ARG;
  for (const void *x : ins)
    if (!aligned16(x)) return MA_ERR_ALIGNMENT;
  for (const void *x : outs)
    if (!aligned16(x)) return MA_ERR_ALIGNMENT;
  const size_t tb = p.tensor_bytes;
  for (int i = 0; i < 3; ++i) {
    for (const void *x : ins)
      if (overlaps(outs[i], x, tb)) return MA_ERR_INVALID_ARG;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], outs[j], tb)) return MA_ERR_INVALID_ARG;
  }
  const size_t need = bwd_workspace_needed(p);
  if (workspace == nullptr || workspace_bytes < need) return MA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MA_ERR_ALIGNMENT;
  for (const void *x : ins)
    if (ranges_overlap(workspace, need, x, tb)) return MA_ERR_INVALID_ARG;
  for (const void *x : outs)
    if (ranges_overlap(workspace, need, x, tb)) return MA_ERR_INVALID_ARG;
  // the forward's Y, when the caller kept it (read only): used only when both stages run
  const bool have_y = y_fwd != nullptr && !p.r_trivial && !p.l_trivial;
  if (have_y) {
    if (!aligned16(y_fwd)) return MA_ERR_ALIGNMENT;
    if (ranges_overlap(workspace, need, y_fwd, tb)) return MA_ERR_INVALID_ARG;
    for (const void *x : outs)
      if (overlaps(x, y_fwd, tb)) return MA_ERR_INVALID_ARG;
  }

  unsigned char *ws = static_cast<unsigned char *>(workspace);
  void *y = ws;
  void *dy = ws + round256(tb);
  const GroupAddr gl = stage_l_groups(p), gr = stage_r_groups(p);
  float *st_l = reinterpret_cast<float *>(ws + 2 * round256(tb));
  float *st_r = reinterpret_cast<float *>(ws + 2 * round256(tb) + round256(stats_bytes(p, gl)));
  if (p.l_trivial && !p.r_trivial) {
    // stage L is the identity: O = Y and dY = dO, and stage R alone writes dq and dk
    return run_stage_bwd(p, gr, q, k, v, out, dout, dq, dk, dv, st_r, false, stream);
  }
  // Y = stage R of the forward: the caller's copy, or recomputed into the
  // workspace (V itself when stage R is the identity)
  const void *yv = v;
  if (have_y) {
    yv = y_fwd;
  } else if (!p.r_trivial) {
    Plan pr{};
    st = plan_launch(p, gr, q, k, v, y, &pr);
    if (st == MA_OK) st = run_plan(p, pr, stream);
    if (st != MA_OK) return st;
    yv = y;
  }
  // stage L: dQ_L into dq, dK_L into dk, and dY (which is dV itself when stage R
  // is the identity: its single-member groups add nothing to dq and dk)
  st = run_stage_bwd(p, gl, q, k, yv, out, dout, dq, dk, p.r_trivial ? dv : dy, st_l, false, stream);
  if (st != MA_OK || p.r_trivial) return st;
  // stage R, fed dY: dQ_R and dK_R added to dq and dk; dV
  return run_stage_bwd(p, gr, q, k, v, yv, dy, dq, dk, dv, st_r, true, stream);
}

const char *ma_status_string(int status) {
  switch (status) {
    case MA_OK: return "MA_OK";
    case MA_ERR_INVALID_ARG: return "MA_ERR_INVALID_ARG: null pointer, negative size, bad r_axes or tile, or overlapping buffers";
    case MA_ERR_UNSUPPORTED: return "MA_ERR_UNSUPPORTED: head_dim/dtype not supported or problem too large";
    case MA_ERR_ALIGNMENT: return "MA_ERR_ALIGNMENT: a pointer is not 16-byte aligned";
    case MA_ERR_WORKSPACE: return "MA_ERR_WORKSPACE: workspace missing or too small";
    case MA_ERR_HIP: return "MA_ERR_HIP: the HIP runtime rejected a launch";
    case MA_ERR_SCRATCH: return "MA_ERR_SCRATCH: the problem needs more than the library's fixed buffer (ma_noalloc_scratch_bytes)";
    default: return "unknown ma_status";
  }
}

int ma_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
