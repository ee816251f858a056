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

#include "../../include/monarch_attn.h"
#include "attn_bf16.h"
#include "attn_f32.h"
#include "validate.h"

namespace ma {
namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MA_OK;
  g_last_hip_error = (int)e;
  return MA_ERR_HIP;
}

template <int D>
int launch_d(const AttnLaunch &a, int nw, uint32_t blocks, hipStream_t s) {
  if (nw == 0) {
    hipLaunchKernelGGL(group_attn_f32<D>, dim3(blocks), dim3(kF32Threads), 0, s, a);
  } else if (nw == 2) {   // groups of at most 64 tokens: one key tile
    hipLaunchKernelGGL((group_attn_bf16<D, 2, 1>), dim3(blocks), dim3(128), 0, s, a);
  } else {                 // longer groups: double-buffered key/value tiles
    hipLaunchKernelGGL((group_attn_bf16<D, 4, 2>), dim3(blocks), dim3(256), 0, s, a);
  }
  return hip_status(hipGetLastError());
}

// Host-side plan of one group-attention launch; fails before any HIP call.
struct Plan {
  AttnLaunch a;
  uint32_t blocks;
  int nw;   // waves per workgroup of the chosen kernel (0: fp32 kernel)
};

int plan_launch(const Problem &p, const GroupAddr &ga, const void *q, const void *k,
                const void *vals, void *out, Plan *pl) {
  AttnLaunch a{};
  a.q = q;
  a.k = k;
  a.vals = vals;
  a.out = out;
  a.head_elems = p.N * p.D;
  a.ga = ga;
  a.n_bh = (int32_t)(p.batch * p.heads);
  a.scale = (float)(1.0 / sqrt((double)p.D));
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)p.D));
  int q_per_block;
  if (p.dtype == MA_F32) {
    q_per_block = kF32Threads;
    pl->nw = 0;
  } else {
    pl->nw = ga.max_len <= kQueriesPerWave * 2 ? 2 : 4;
    q_per_block = kQueriesPerWave * pl->nw;
  }
  a.n_qtiles = (ga.max_len + q_per_block - 1) / q_per_block;
  const uint64_t blocks = (uint64_t)a.n_qtiles * (uint64_t)ga.n_groups * (uint64_t)a.n_bh;
  if (blocks > (uint64_t)INT32_MAX) return MA_ERR_UNSUPPORTED;
  pl->blocks = (uint32_t)blocks;
  pl->a = a;
  return MA_OK;
}

int run_plan(const Problem &p, const Plan &pl, hipStream_t s) {
  if (pl.blocks == 0) return MA_OK;
  switch (p.D) {
    case 16: return launch_d<16>(pl.a, pl.nw, pl.blocks, s);
    case 32: return launch_d<32>(pl.a, pl.nw, pl.blocks, s);
    case 64: return launch_d<64>(pl.a, pl.nw, pl.blocks, s);
    default: return launch_d<128>(pl.a, pl.nw, pl.blocks, s);
  }
}

int copy_async(void *dst, const void *src, size_t bytes, hipStream_t s) {
  if (bytes == 0) return MA_OK;
  return hip_status(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s));
}

int monarch_common(const void *q, const void *k, const void *v, void *out, void *ws, size_t ws_bytes,
                   int32_t batch, int32_t heads, int32_t T, int32_t H, int32_t W, int32_t r_axes,
                   int32_t tile_t, int32_t tile_h, bool tiled, int32_t head_dim, int32_t dtype,
                   hipStream_t stream) {
  Problem p;
  int st = resolve_grid(batch, heads, T, H, W, r_axes, tile_t, tile_h, tiled, head_dim, dtype, &p);
  if (st != MA_OK || p.empty) return st;
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
    st = plan_launch(p, stage_l_groups(p), q, k, y_in, out, &pl);
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

int monarch_attn_tiled_fwd(const void *q, const void *k, const void *v, void *out, void *workspace,
                           size_t workspace_bytes, int32_t batch, int32_t heads, int32_t T,
                           int32_t H, int32_t W, int32_t tile_t, int32_t tile_h, int32_t head_dim,
                           int32_t dtype, struct ihipStream_t *stream) {
  return monarch_common(q, k, v, out, workspace, workspace_bytes, batch, heads, T, H, W, 1, tile_t,
                        tile_h, true, head_dim, dtype, stream);
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

const char *ma_status_string(int status) {
  switch (status) {
    case MA_OK: return "MA_OK";
    case MA_ERR_INVALID_ARG: return "MA_ERR_INVALID_ARG: null pointer, negative size, bad r_axes or tile, or overlapping buffers";
    case MA_ERR_UNSUPPORTED: return "MA_ERR_UNSUPPORTED: head_dim/dtype not supported or problem too large";
    case MA_ERR_ALIGNMENT: return "MA_ERR_ALIGNMENT: a pointer is not 16-byte aligned";
    case MA_ERR_WORKSPACE: return "MA_ERR_WORKSPACE: workspace missing or too small";
    case MA_ERR_HIP: return "MA_ERR_HIP: the HIP runtime rejected a launch";
    default: return "unknown ma_status";
  }
}

int ma_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
