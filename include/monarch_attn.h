/*
 * monarch_attn.h -- C ABI of the MI355X (gfx950) Monarch-factored video attention library.
 *
 * Operation. For a video token grid (T, H, W) flattened as n = (t*H + h)*W + w,
 * the attention matrix is taken as a product of permutation and block-diagonal
 * factors, M = P . blockdiag(L_0..L_{b2-1}) . P^T . blockdiag(R_0..R_{b1-1})
 * (MonarchRT summaries, nl page "Methodologie"; P a permutation: zh page 2.1),
 * with blocks aligned to whole grid axes, (b1, b2) = (T*H, W) and b1*b2 = N
 * (zh page 2.2, "block alignment"). The library computes O = M V with
 *   stage R: Y[a*b2+i] = sum_j softmax_j(s q_{a*b2+i} . k_{a*b2+j}) v_{a*b2+j}
 *            (softmax attention inside each block of b2 contiguous tokens),
 *   stage L: O[a*b2+i] = sum_c softmax_c(s q_{a*b2+i} . k_{c*b2+i}) Y[c*b2+i]
 *            (softmax attention among the b1 tokens that share intra-block
 *            index i; the stride permutation P is applied by addressing only),
 * s = 1/sqrt(head_dim), the original Q and K in both stages, R applied first.
 * Tiled Monarch (zh page 2.2 "Tiled Monarch"; fr page 2.B; nl "Methodologie")
 * restricts each stage-L softmax to a box of tile_t frames x tile_h rows at a
 * fixed w; the last box on an axis may be shorter.
 *
 * Tensors. q, k, v, out (and the workspace) are dense row-major
 * [batch, heads, N, head_dim] arrays of one dtype (MA_BF16 or MA_F32), head_dim
 * fastest, N = T*H*W. All pointers are caller-owned DEVICE pointers, 16-byte
 * aligned. The library allocates nothing, keeps no state between calls, and is
 * reentrant; work is enqueued on `stream` (NULL = the default stream) and every
 * call returns without synchronizing. bf16 inputs are accumulated in fp32; the
 * stage-R intermediate Y is stored in the input dtype. MA_F32 evaluates every
 * product as fp32 x fp32 with fp32 accumulation (fp32 matrix-core instructions
 * at head_dim 32 to 128, the vector ALUs at 16; no reduced-precision mode).
 *
 * Errors. Every argument is checked on the host before any HIP call; a failed
 * check returns a negative ma_status and enqueues nothing. A zero-sized problem
 * (batch, heads or a grid axis equal to 0) is a no-op returning MA_OK. A HIP
 * launch failure returns MA_ERR_HIP (details: ma_last_hip_error()).
 */
#ifndef MONARCH_ATTN_H_
#define MONARCH_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t; /* hipStream_t is `struct ihipStream_t *` */

typedef enum {
  MA_OK = 0,
  MA_ERR_INVALID_ARG = -1,  /* null pointer, negative size, bad r_axes or tile, aliasing */
  MA_ERR_UNSUPPORTED = -2,  /* head_dim not in {16,32,64,128}, dtype unknown, size limits */
  MA_ERR_ALIGNMENT = -3,    /* a pointer is not 16-byte aligned */
  MA_ERR_WORKSPACE = -4,    /* workspace missing or smaller than ma_workspace_bytes() */
  MA_ERR_HIP = -5,          /* the HIP runtime rejected a launch */
  MA_ERR_SCRATCH = -6       /* monarch_attn_fwd_noalloc: Y larger than the fixed buffer */
} ma_status;

typedef enum { MA_BF16 = 0, MA_F32 = 1 } ma_dtype;

/* Block spec `r_axes`: how many trailing grid axes form one stage-R block.
 *   1: b2 = W,     b1 = T*H  (the aligned (f*h, w) split; the default)
 *   2: b2 = H*W,   b1 = T    (the aligned (f, h*w) split)
 *   3: b2 = N,     b1 = 1    (one block: plain dense attention, stage L skipped)
 *   0: b2 = 1,     b1 = N    (stage R skipped: plain dense attention through stage L) */

/* Bytes of workspace (the stage-R output Y) that monarch_attn_fwd /
 * monarch_attn_tiled_fwd need for this problem; 0 when one stage is trivial and
 * Y is written straight to `out` or read straight from `v`. Returns 0 for
 * invalid arguments too (the entry points then report the error). */
size_t ma_workspace_bytes(int32_t batch, int32_t heads, int32_t T, int32_t H, int32_t W,
                          int32_t r_axes, int32_t tile_t, int32_t tile_h,
                          int32_t head_dim, int32_t dtype);

/* Monarch attention, untiled: O = P L P^T R V as defined above.
 * workspace: device buffer of at least ma_workspace_bytes(...) bytes (may be
 * NULL when that is 0); it must not overlap q, k, v or out. out must not
 * overlap q, k, v. */
int monarch_attn_fwd(const void *q, const void *k, const void *v, void *out,
                     void *workspace, size_t workspace_bytes,
                     int32_t batch, int32_t heads, int32_t T, int32_t H, int32_t W,
                     int32_t r_axes, int32_t head_dim, int32_t dtype,
                     struct ihipStream_t *stream);

/* monarch_attn_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same operation, arguments, checks and
 * kernels as monarch_attn_fwd; the stage-R output Y goes to a buffer the
 * library holds per GPU (ma_noalloc_scratch_bytes() = 128 MiB, reserved on
 * each GPU the library is loaded on until the process ends). The call
 * allocates nothing. MA_ERR_SCRATCH when Y (ma_workspace_bytes(...) bytes)
 * is larger than that buffer. Every call on one GPU uses the same buffer:
 * calls on one GPU must not overlap in time (issue them on one stream, or
 * order streams with events); overlapping calls race on it. The buffer keeps
 * the last call's Y; nothing in it needs to start at any value. */
int monarch_attn_fwd_noalloc(const void *q, const void *k, const void *v, void *out,
                             int32_t batch, int32_t heads, int32_t T, int32_t H, int32_t W,
                             int32_t r_axes, int32_t head_dim, int32_t dtype,
                             struct ihipStream_t *stream);

/* Size in bytes of the per-GPU buffer behind monarch_attn_fwd_noalloc. */
size_t ma_noalloc_scratch_bytes(void);

/* Tiled Monarch attention: as monarch_attn_fwd with r_axes = 1, but each
 * stage-L softmax runs only over the box {(t', h') : t'/tile_t = t/tile_t,
 * h'/tile_h = h/tile_h} at the same w. tile_t, tile_h >= 1; tiles larger than
 * the grid clamp to it (tile (T, H) equals the untiled operator; tile (1, 1)
 * makes stage L the identity, so O = Y). */
int monarch_attn_tiled_fwd(const void *q, const void *k, const void *v, void *out,
                           void *workspace, size_t workspace_bytes,
                           int32_t batch, int32_t heads, int32_t T, int32_t H, int32_t W,
                           int32_t tile_t, int32_t tile_h, int32_t head_dim, int32_t dtype,
                           struct ihipStream_t *stream);

/* Chunk-causal Monarch attention over the whole sequence (bf16 only).
 * The pages' real-time target is autoregressive generation a few frames at a
 * time (it 1 and 3; fr 1 and 4; zh 1); they do not define Monarch over a causal
 * sequence. Reading: frames form chunks of chunk_t (chunk(t) = t div chunk_t);
 * stage R is as in monarch_attn_fwd (its blocks never cross a frame); in
 * stage L a query of chunk c uses only the members of its group in chunks
 * 0..c (bidirectional inside a chunk). The rows of chunk c therefore equal
 * monarch_attn_fwd over frames [0, (c+1) chunk_t). r_axes must be 0, 1 or 2
 * (at 3 the single stage-R block would cross frames): MA_ERR_INVALID_ARG
 * otherwise, or for chunk_t < 1. chunk_t >= T is the bidirectional operator.
 * Workspace, layout and overlap rules as monarch_attn_fwd; MA_ERR_UNSUPPORTED
 * for MA_F32. */
int monarch_attn_causal_fwd(const void *q, const void *k, const void *v, void *out,
                            void *workspace, size_t workspace_bytes,
                            int32_t batch, int32_t heads, int32_t T, int32_t H, int32_t W,
                            int32_t r_axes, int32_t chunk_t, int32_t head_dim, int32_t dtype,
                            struct ihipStream_t *stream);

/* One autoregressive step with a cache (bf16 only), under the reading above:
 * the chunk of frames [t0, t0 + chunk_t) attends to every frame up to its own
 * end. q, k, v, y and out are whole buffers [batch, heads, T*H*W, head_dim]
 * for T allocated frames (t0 + chunk_t <= T); only frames below t0 + chunk_t
 * are read.
 *   y   in:  frames [0, t0) hold the stage-R output Y of earlier steps (the
 *            cache); out: frames [t0, t0 + chunk_t) receive this chunk's Y.
 *            Not used (may be NULL) at r_axes = 0, where Y is V.
 *   out frames [t0, t0 + chunk_t) receive O; other frames are not written.
 * Stage R runs over the chunk's frames only; stage L over the members of each
 * group in frames [0, t0 + chunk_t), with queries in the chunk. Calling it
 * for t0 = 0, chunk_t, 2 chunk_t, ... reproduces monarch_attn_causal_fwd.
 * y and out must not overlap each other or q, k, v. MA_ERR_INVALID_ARG for
 * r_axes = 3, chunk_t < 1, t0 < 0 or t0 + chunk_t > T; MA_ERR_UNSUPPORTED for
 * MA_F32. No workspace. */
int monarch_attn_chunk_fwd(const void *q, const void *k, const void *v, void *y, void *out,
                           int32_t batch, int32_t heads, int32_t T, int32_t H, int32_t W,
                           int32_t r_axes, int32_t t0, int32_t chunk_t, int32_t head_dim,
                           int32_t dtype, struct ihipStream_t *stream);

/* Dense comparator: O = softmax(s Q K^T) V over all n_tokens, per (batch, head)
 * (the quadratic 3D self-attention the method replaces: it page 1, zh overview).
 * out must not overlap q, k, v. */
int dense_attn_fwd(const void *q, const void *k, const void *v, void *out,
                   int32_t batch, int32_t heads, int32_t n_tokens, int32_t head_dim,
                   int32_t dtype, struct ihipStream_t *stream);

/* The two stages as separate calls (same definitions; used to time and test
 * each kernel on its own).
 * ma_stage_r_fwd writes Y = blockdiag(R) V into y (same shape as v).
 * ma_stage_l_fwd reads Y from y and writes O = P L P^T Y into out; tile_t =
 * tile_h = 0 selects the untiled stage L, otherwise tiles need r_axes = 1.
 * y must not overlap q, k, v (stage R) or q, k, out (stage L). */
int ma_stage_r_fwd(const void *q, const void *k, const void *v, void *y,
                   int32_t batch, int32_t heads, int32_t T, int32_t H, int32_t W,
                   int32_t r_axes, int32_t head_dim, int32_t dtype,
                   struct ihipStream_t *stream);
int ma_stage_l_fwd(const void *q, const void *k, const void *y, void *out,
                   int32_t batch, int32_t heads, int32_t T, int32_t H, int32_t W,
                   int32_t r_axes, int32_t tile_t, int32_t tile_h,
                   int32_t head_dim, int32_t dtype, struct ihipStream_t *stream);

/* Backward pass (bf16 only). The pages state that the method's kernels run
 * the forward and the backward pass with FlashAttention-like tiling (it page
 * "Finetuning e Implementazione Efficiente"; fr page 2.C; zh page on
 * finetuning and efficient implementation); the gradient itself is the chain
 * rule of the forward above. Given dO = dL/dout for out = the forward of
 * (q, k, v) with the same r_axes and tile (tile_t = tile_h = 0: untiled;
 * otherwise r_axes = 1), writes dq = dL/dq, dk = dL/dk, dv = dL/dv:
 *   per token set G of a stage, with P = softmax_rows(s Q_G K_G^T):
 *     dV_G = P^T dO_G,  dS = P * (dO_G V_G^T - D),  D_i = dO_i . O_i,
 *     dQ_G = s dS K_G,  dK_G = s dS^T Q_G;
 *   stage L (V := Y, O := out) gives dQ_L, dK_L and dY; stage R (O := Y,
 *   dO := dY) gives dQ_R, dK_R and dV; dq = dQ_L + dQ_R, dk = dK_L + dK_R.
 * out must be the forward output (it enters D). y_fwd may be NULL, or the
 * forward's Y (the contents of monarch_attn_fwd's / monarch_attn_tiled_fwd's
 * workspace after that call, same shape and dtype as q; read only, 16-byte
 * aligned, not overlapping the workspace or dq, dk, dv): given, the backward
 * takes it instead of recomputing stage R (ignored when a stage is the
 * identity); the gradients are the same bits either way. The workspace (at
 * least ma_bwd_workspace_bytes(...) bytes) holds the recomputed Y, dY and
 * per-query softmax statistics; it must not overlap any tensor argument, and
 * dq, dk, dv must not overlap each other or the inputs. dtype MA_F32 returns
 * MA_ERR_UNSUPPORTED; ma_bwd_workspace_bytes then returns 0. */
size_t ma_bwd_workspace_bytes(int32_t batch, int32_t heads, int32_t T, int32_t H, int32_t W,
                              int32_t r_axes, int32_t tile_t, int32_t tile_h,
                              int32_t head_dim, int32_t dtype);
int monarch_attn_bwd(const void *q, const void *k, const void *v, const void *out,
                     const void *dout, const void *y_fwd, void *dq, void *dk, void *dv,
                     void *workspace, size_t workspace_bytes,
                     int32_t batch, int32_t heads, int32_t T, int32_t H, int32_t W,
                     int32_t r_axes, int32_t tile_t, int32_t tile_h,
                     int32_t head_dim, int32_t dtype, struct ihipStream_t *stream);

/* Static text for a status code (never NULL). */
const char *ma_status_string(int status);

/* The hipError_t value behind the last MA_ERR_HIP returned on this thread
 * (0 if none). */
int ma_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MONARCH_ATTN_H_ */
