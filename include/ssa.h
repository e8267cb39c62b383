/*
 * ssa.h - C ABI of a HIP (gfx950) library for Spatial Sparse Attention (SSA).
 *
 * SSA, as described for Direct3D-S2 (nav.superapi.store page "Direct3D-S2",
 * section "Technical principles of Direct3D-S2", first bullet; pixal-3d.com page
 * "Direct3D-S2", sections "What is Direct3D-S2?" and FAQ "What is SSA?"):
 * tokens carrying 3D voxel coordinates are partitioned into blocks by
 * coordinate; a compression branch attends to one pooled token per block; the
 * compression branch's attention scores select the most important blocks, whose
 * tokens are attended at full resolution; a window branch attends to the tokens
 * of the query's local window cell; and predicted per-token, per-head gates sum
 * the three branch outputs.
 *
 * Definitions used by every entry point (N tokens, H heads, head dim d):
 *   block of token i  = floor(c_i / B) per axis; block key
 *                       kappa = (b_x * n_y + b_y) * n_z + b_z, n_a = ceil(G_a / B);
 *                       blocks are the occupied keys in ascending order (ids 0..M-1)
 *   compressed keys   = ktil[h,b] = mean_{i in b} K[i,h,:] @ W_k   (likewise vtil, W_v)
 *   compressed branch = softmax_b(scale * q . ktil[h,b]) @ vtil[h]     over all M blocks
 *   importance        = sigma[h,Bq,b] = sum over tokens i of block Bq of the compressed
 *                       softmax probability of block b
 *   selection         = the min(topk, M) blocks of largest sigma (ties: lower id),
 *                       ascending ids, -1 padded
 *   selected branch   = one softmax over all tokens of the selected blocks
 *   window branch     = one softmax over the tokens of the query's window cell
 *                       floor(c / w) (non-overlapping w^3 cells at the origin)
 *   out[i,h]          = g[i,h,0]*o_cmp + g[i,h,1]*o_sel + g[i,h,2]*o_win
 *
 * Memory: every pointer is device memory unless marked (host).  The caller owns
 * every buffer; the library never allocates device memory.  Tensors are dense,
 * row-major, in the caller's token order: coords int32 [N,3]; q, k, v, out
 * [N,H,d]; gates [N,H,3]; W_k, W_v [d,d] (row-vector convention, k~ = kbar @ W).
 * Floating-point tensors share one dtype (ssa_dtype).
 *
 * Errors: calls return ssa_status and never throw.  Argument checks run on the
 * host before any launch.  Only ssa_plan_create synchronises its stream; the
 * forward is stream-ordered and asynchronous.
 */
#ifndef SSA_H
#define SSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSA_OK = 0,
  SSA_ERR_INVALID_ARG = 1,   /* null pointer, negative size, bad enum, zero edge ... */
  SSA_ERR_UNSUPPORTED = 2,   /* valid but outside what the kernels implement (d, dtype, window) */
  SSA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the *_workspace_size query */
  SSA_ERR_COORD_RANGE = 4,   /* a coordinate outside [0, grid) (detected on the device) */
  SSA_ERR_HIP = 5,           /* a HIP runtime call or kernel launch failed */
  SSA_ERR_BAD_PLAN = 6       /* null or destroyed plan handle */
} ssa_status;

typedef enum { SSA_F32 = 0, SSA_F16 = 1, SSA_BF16 = 2 } ssa_dtype;

typedef struct ssa_plan_s* ssa_plan;

/* Views of a plan's device arrays (owned by the plan's workspace), for tests. */
typedef struct {
  int64_t n;               /* tokens */
  int64_t num_blocks;      /* M: occupied blocks */
  int64_t num_cells;       /* occupied window cells */
  int32_t block, window;   /* B, w */
  int32_t max_block_rows;  /* largest block occupancy */
  const int32_t* perm;     /* [N]   token index at block-sorted position r */
  const int32_t* blk_off;  /* [M+1] first sorted position of each block; blk_off[M] = N */
  const int32_t* blk_key;  /* [M]   block key kappa, ascending */
  const int32_t* tok2blk;  /* [N]   block id of each token (caller order) */
  const int32_t* blk_cell; /* [M]   window cell of each block */
  const int32_t* cell_off; /* [C+1] offsets into cell_blk */
  const int32_t* cell_blk; /* [M]   block ids grouped by cell, ascending within a cell */
  const int32_t* lpt;      /* [M]   block ids by descending occupancy (ties: lower id) */
} ssa_plan_info_t;

/*
 * Block partition of a coordinate set (the pages' "partitions input tokens by 3D
 * coordinates").  Computed on the device: block keys, a stable LSD radix sort of
 * the keys (token index order inside a block), segment offsets, the window-cell
 * grouping of blocks and a longest-first block order.
 *
 * grid (host, [3]): grid extent per axis, each >= 1.  block B >= 1.  window w >= 1;
 * the window cells must be unions of blocks: w % B == 0, or w >= every grid extent
 * (one cell), else SSA_ERR_UNSUPPORTED.  n = 0 is allowed (an empty plan).
 * ws: caller-owned device workspace of at least ssa_plan_workspace_size(...) bytes;
 * it holds the plan's arrays and must outlive the plan.  The call synchronises
 * `stream` once (to read M back).  Coordinates outside [0, grid) give
 * SSA_ERR_COORD_RANGE.  *out (host) receives the plan handle.
 */
size_t ssa_plan_workspace_size(int64_t n, const int32_t grid[3], int32_t block, int32_t window);
ssa_status ssa_plan_create(const int32_t* coords, int64_t n, const int32_t grid[3], int32_t block,
                           int32_t window, void* ws, size_t ws_bytes, hipStream_t stream,
                           ssa_plan* out);
ssa_status ssa_plan_get_info(ssa_plan plan, ssa_plan_info_t* info /* host */);
/* Frees the host-side handle only (the workspace stays the caller's). */
void ssa_plan_destroy(ssa_plan plan);

/*
 * SSA forward.  dtype in {F32, F16, BF16}; head dim d in {32, 64, 96, 128};
 * heads >= 1; topk >= 1 (topk >= M selects every block, remaining slots -1).
 * scale = 0 means 1/sqrt(d).  wk and wv may alias.  out [N,H,d] (dtype) is
 * written completely.  sel_out, if not NULL, receives the selection int32
 * [H,M,topk] (ascending block ids, -1 padded).  ws: device workspace of at
 * least ssa_forward_workspace_size(...) bytes, queried with the same
 * save_for_bwd; distinct concurrent calls need distinct workspaces.  With
 * save_for_bwd != 0 the workspace also keeps what ssa_backward needs (per-branch
 * log-sum-exp and branch outputs).  Asynchronous on `stream`; returns SSA_ERR_HIP
 * if a launch fails.  Accumulation is fp32 (the compressed scores that decide the
 * selection are computed from a split of the fp32 pooled keys into two (f16) or
 * three (bf16) dtype terms, so they carry fp32-level accuracy).  The selection
 * keeps each work item's importance vector in on-chip memory, which bounds the
 * number of occupied blocks M: at most 6144, and at most 5760 (f32) or 4480
 * (bf16) for d = 128; a larger plan returns SSA_ERR_UNSUPPORTED.
 */
size_t ssa_forward_workspace_size(ssa_plan plan, ssa_dtype dtype, int32_t heads, int32_t dim,
                                  int32_t topk, int save_for_bwd);
ssa_status ssa_forward(ssa_plan plan, ssa_dtype dtype, int32_t heads, int32_t dim,
                       const void* q, const void* k, const void* v, const void* wk,
                       const void* wv, const void* gates, int32_t topk, float scale,
                       void* out, int32_t* sel_out, void* ws, size_t ws_bytes,
                       int save_for_bwd, hipStream_t stream);

/*
 * The forward's three stages, for per-stage timing: bit 0 = pooled keys and
 * values; bit 1 = compressed branch and block selection; bit 2 = selected and
 * window branches and the gated combine.  ssa_forward is stages 7.  A stage reads
 * what the earlier stages left in the same workspace, so stages must run in
 * order on the same stream with identical arguments.
 */
enum { SSA_STAGE_POOL = 1, SSA_STAGE_SELECT = 2, SSA_STAGE_ATTEND = 4, SSA_STAGE_ALL = 7 };
ssa_status ssa_forward_stages(ssa_plan plan, ssa_dtype dtype, int32_t heads, int32_t dim,
                              const void* q, const void* k, const void* v, const void* wk,
                              const void* wv, const void* gates, int32_t topk, float scale,
                              void* out, int32_t* sel_out, void* ws, size_t ws_bytes,
                              int save_for_bwd, hipStream_t stream, uint32_t stages);

/*
 * SSA backward (the gradients that a training step at the 80k-voxel shape needs):
 * given dout = dL/dout [N,H,d] (dtype) and the selection sel [H,M,topk] that the
 * forward used (held fixed: no gradient flows through the importance scores or the
 * top-k, and none into W_k, W_v), writes fp32 dq, dk, dv [N,H,d] and dgates
 * [N,H,3] (order: compressed, selected, window).  fwd_ws is the workspace of an
 * ssa_forward call with save_for_bwd != 0 on the same plan and inputs (read only).
 * ws: device workspace of at least ssa_backward_workspace_size(...) bytes.  Every
 * sum runs in a fixed order (no atomics), so results are bitwise reproducible.
 * The plan must be within the forward's block limit (else SSA_ERR_UNSUPPORTED).
 * Asynchronous on `stream`.
 */
size_t ssa_backward_workspace_size(ssa_plan plan, ssa_dtype dtype, int32_t heads, int32_t dim,
                                   int32_t topk);
ssa_status ssa_backward(ssa_plan plan, ssa_dtype dtype, int32_t heads, int32_t dim,
                        const void* q, const void* k, const void* v, const void* wk,
                        const void* wv, const void* gates, int32_t topk, float scale,
                        const int32_t* sel, const void* dout, float* dq, float* dk, float* dv,
                        float* dgates, const void* fwd_ws, size_t fwd_ws_bytes, void* ws,
                        size_t ws_bytes, hipStream_t stream);

const char* ssa_status_string(ssa_status status);

#ifdef __cplusplus
}
#endif
#endif /* SSA_H */
