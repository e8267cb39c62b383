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
  SSA_ERR_BAD_PLAN = 6,      /* null or destroyed plan handle */
  SSA_ERR_TOO_LARGE = 7      /* ssa_forward_noalloc: the problem needs more than its scratch area */
} ssa_status;

typedef enum { SSA_F32 = 0, SSA_F16 = 1, SSA_BF16 = 2 } ssa_dtype;

typedef struct ssa_plan_s* ssa_plan;

/* Views of a plan's device arrays (owned by the plan's workspace), for tests.  They
 * come back in one struct, filled by ssa_plan_get_info, rather than as a list of
 * out-parameters, so that views can be added without changing the call. */
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
  /* window partition (see ssa_window_t) */
  int32_t window_kind;     /* SSA_WINDOW_CUBE or SSA_WINDOW_SFC */
  int32_t window_shift[3]; /* CUBE: cell origin shift */
  int32_t window_tokens;   /* SFC: tokens per window */
  int32_t cells_are_block_unions; /* 1: cells are blk_cell/cell_off/cell_blk above; 0: the w* views */
  int64_t num_wcells;      /* C': cells of the token-level window partition (0 if unions of blocks) */
  int32_t max_wcell_rows;  /* tokens of its largest cell */
  const int32_t* wperm;    /* [N]    token index at window-sorted position r */
  const int32_t* wcell_off;/* [C'+1] first window-sorted position of each cell */
  const int32_t* wlpt;     /* [C']   cell ids by descending size (ties: lower id) */
} ssa_plan_info_t;

/*
 * The window branch's cells (pixal-3d.com "Direct3D-S2", "What is Direct3D-S2?": local
 * windows; Hi3D pipeline page, "Stage 4": fixed-size windows along a space-filling curve).
 *   SSA_WINDOW_CUBE: a token attends to every token of its cubic cell floor((c + shift) / edge)
 *                    (per axis; edge >= 1, 0 <= shift < edge).  Shifting alternate layers by
 *                    edge / 2 gives shifted windows.
 *   SSA_WINDOW_SFC:  tokens sorted by the Morton code of their voxel (bits interleaved x, y, z,
 *                    x most significant; equal codes in token order) are cut into consecutive
 *                    windows of `tokens` tokens (the last one shorter); a token attends to its
 *                    window.  Grid extents up to 1024.
 * Cells that are unions of blocks (CUBE with no shift and edge a multiple of the block edge, or
 * one cell covering the grid) run inside the selected branch's kernel; any other partition gets
 * a token-level sort of its own and a separate window pass, and is forward-only (the backward
 * and save_for_bwd return SSA_ERR_UNSUPPORTED).
 */
typedef enum { SSA_WINDOW_CUBE = 0, SSA_WINDOW_SFC = 1 } ssa_window_kind;
typedef struct {
  int32_t kind;      /* ssa_window_kind */
  int32_t edge;      /* CUBE: cell edge */
  int32_t shift[3];  /* CUBE: cell origin shift per axis */
  int32_t tokens;    /* SFC: tokens per window */
} ssa_window_t;

/*
 * Block partition of a coordinate set (the partition step of nav.superapi.store,
 * "Technical principles of Direct3D-S2": tokens grouped by 3D coordinates).  Computed on the device: block keys, a stable LSD radix sort of
 * the keys (token index order inside a block), segment offsets, the window-cell
 * grouping of blocks and a longest-first block order.
 *
 * grid (host, [3]): grid extent per axis, each >= 1.  block B >= 1.  window w >= 1: cubic
 * window cells of edge w (see ssa_window_t).  n = 0 is allowed (an empty plan).
 * ws: caller-owned device workspace of at least ssa_plan_workspace_size(...) bytes;
 * it holds the plan's arrays and must outlive the plan.  The call synchronises
 * `stream` once (to read M back).  Coordinates outside [0, grid) give
 * SSA_ERR_COORD_RANGE.  *out (host) receives the plan handle.
 */
size_t ssa_plan_workspace_size(int64_t n, const int32_t grid[3], int32_t block, int32_t window);
ssa_status ssa_plan_create(const int32_t* coords, int64_t n, const int32_t grid[3], int32_t block,
                           int32_t window, void* ws, size_t ws_bytes, hipStream_t stream,
                           ssa_plan* out);
/* The same with any window partition (ssa_window_t, host).  ssa_plan_create(..., window, ...)
 * is ssa_plan_create_ex with {SSA_WINDOW_CUBE, window, {0, 0, 0}, 0}.  Window cells that are
 * not unions of blocks synchronise the stream once or twice more. */
size_t ssa_plan_workspace_size_ex(int64_t n, const int32_t grid[3], int32_t block,
                                  const ssa_window_t* win);
ssa_status ssa_plan_create_ex(const int32_t* coords, int64_t n, const int32_t grid[3], int32_t block,
                              const ssa_window_t* win, void* ws, size_t ws_bytes, hipStream_t stream,
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
 * number of occupied blocks M (ssa_forward_max_blocks; from 7296 for f32 at d = 128
 * to 34944 for 16-bit types at d = 32); a larger plan returns SSA_ERR_UNSUPPORTED.
 */
size_t ssa_forward_workspace_size(ssa_plan plan, ssa_dtype dtype, int32_t heads, int32_t dim,
                                  int32_t topk, int save_for_bwd);
/* The largest number of occupied blocks M the forward (and backward) accepts for this dtype
 * and head dimension on the current device (the importance vectors' share of the selection
 * kernel's on-chip memory); 0 for an invalid dtype or dim or when the device cannot be
 * queried. */
int64_t ssa_forward_max_blocks(ssa_dtype dtype, int32_t dim);
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
 * SSA forward and backward with the sparse-convolution compressor (nav.superapi.store
 * "Direct3D-S2", "Technical principles of Direct3D-S2": block-level information by sparse 3D
 * convolution and pooling).  A convolution with kernel size and stride B over the occupied
 * voxels -- every block one output site, every voxel weighted by its position inside the
 * block -- then the mean over the block's occupied voxels:
 *   ktil[h,b] = (1/n_b) sum_{i in b} k[i,h] Wc_k[o(i)]^T,   vtil likewise with Wc_v,
 * o(i) = ((c_x mod B) * B + (c_y mod B)) * B + (c_z mod B).  wk_conv, wv_conv: [B^3][d][d],
 * each position's matrix in linear-layer layout [d_out][d_in].  Every other argument and
 * result as ssa_forward / ssa_backward (the workspace sizes are the same queries); with
 * uniform position weights Wc[o] = W^T the results equal those of ssa_forward.  The backward
 * must be ssa_backward_conv on a workspace saved by ssa_forward_conv (and ssa_backward on one
 * saved by ssa_forward), else SSA_ERR_INVALID_ARG for the plan's 16 most recent forwards.
 */
ssa_status ssa_forward_conv(ssa_plan plan, ssa_dtype dtype, int32_t heads, int32_t dim,
                            const void* q, const void* k, const void* v, const void* wk_conv,
                            const void* wv_conv, const void* gates, int32_t topk, float scale,
                            void* out, int32_t* sel_out, void* ws, size_t ws_bytes,
                            int save_for_bwd, hipStream_t stream);
ssa_status ssa_backward_conv(ssa_plan plan, ssa_dtype dtype, int32_t heads, int32_t dim,
                             const void* q, const void* k, const void* v, const void* wk_conv,
                             const void* wv_conv, const void* gates, int32_t topk, float scale,
                             const int32_t* sel, const void* dout, float* dq, float* dk, float* dv,
                             float* dgates, const void* fwd_ws, size_t fwd_ws_bytes, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): ssa_forward without a workspace
 * argument.  The workspace is a fixed array of SSA_NOALLOC_SCRATCH_BYTES (64 MiB) in
 * the library's device code, one copy per GPU, held from the library's first use on
 * that GPU until the process ends; the call itself allocates nothing.  A problem whose
 * forward workspace (ssa_forward_workspace_size with save_for_bwd = 0, less its 256
 * bytes of alignment slack) exceeds it returns SSA_ERR_TOO_LARGE before any launch.
 * Arguments and results as ssa_forward with ws = NULL and save_for_bwd = 0.  Every call
 * on one GPU uses that GPU's one array: calls that overlap on a GPU (concurrent streams
 * or threads) race and give undefined results; calls ordered on one stream are safe.
 * Nothing in the array needs to start zeroed.
 */
#define SSA_NOALLOC_SCRATCH_BYTES (64u << 20)
ssa_status ssa_forward_noalloc(ssa_plan plan, ssa_dtype dtype, int32_t heads, int32_t dim,
                               const void* q, const void* k, const void* v, const void* wk,
                               const void* wv, const void* gates, int32_t topk, float scale,
                               void* out, int32_t* sel_out, hipStream_t stream);

/*
 * Several samples in one call (a varlen batch; SSA never mixes tokens of different
 * samples: each sample has its own plan, blocks, selection and windows).  Sample i owns
 * tokens [tok_off[i], tok_off[i+1]) of the concatenated q, k, v, gates and out tensors
 * ([N_total,H,d] / [N_total,H,3]); plans[i] (host array) is its plan, with
 * plans[i]->n == tok_off[i+1] - tok_off[i]; tok_off (host, [nsamples+1]) starts at 0.
 * W_k, W_v, dtype, heads, dim, topk and scale are shared.  The samples run one after
 * another on `stream` through one workspace of ssa_forward_batch_workspace_size bytes
 * (the largest sample's forward workspace).  Every argument check runs before the first
 * launch.  The selection is not returned.
 */
size_t ssa_forward_batch_workspace_size(const ssa_plan* plans, int32_t nsamples, ssa_dtype dtype,
                                        int32_t heads, int32_t dim, int32_t topk);
ssa_status ssa_forward_batch(const ssa_plan* plans, int32_t nsamples, const int64_t* tok_off,
                             ssa_dtype dtype, int32_t heads, int32_t dim, const void* q, const void* k,
                             const void* v, const void* wk, const void* wv, const void* gates,
                             int32_t topk, float scale, void* out, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/*
 * SSA backward: the gradient of the forward defined above (the pages report SSA's
 * backward pass alongside its forward: pixal-3d.com "Direct3D-S2", sections "What
 * is Direct3D-S2?" and "Technical snapshot", where training at 1024^3 resolution
 * relies on it).  Given dout = dL/dout [N,H,d] (dtype) and the selection sel [H,M,topk] that the
 * forward used (held fixed: no gradient flows through the importance scores or the
 * top-k, and none into W_k, W_v), writes fp32 dq, dk, dv [N,H,d] and dgates
 * [N,H,3] (order: compressed, selected, window).  fwd_ws is the workspace of an
 * ssa_forward call with save_for_bwd != 0 on the same plan and inputs (read only).
 * ws: device workspace of at least ssa_backward_workspace_size(...) bytes.  Every
 * sum runs in a fixed order (no atomics), so results are bitwise reproducible.
 * The plan must be within the forward's block limit (else SSA_ERR_UNSUPPORTED).
 * scale must be the value the forward used (0 = 1/sqrt(d)): the saved log-sum-exp
 * values hold it, and a backward on a workspace whose saving forward (one of the
 * plan's 16 most recent) ran with another scale returns SSA_ERR_INVALID_ARG.
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

/*
 * The step before SSA: each token's queries, keys, values and gates from its features
 * (Hi3D pipeline page, "Stage 3": RMS normalisation of the self-attention queries and keys,
 * rotary position embeddings; nav.superapi.store "Direct3D-S2", "Technical principles of
 * Direct3D-S2": the model predicts the per-branch gates), in one kernel:
 *   y = x W_qkv^T, W_qkv [3*H*d, C] (linear-layer layout; output features q | k | v, each
 *       head-major), x [N, C];
 *   q = rope(rmsnorm(y_q) * gamma_q), k = rope(rmsnorm(y_k) * gamma_k), v = y_v   [N,H,d];
 *       rmsnorm over each head's d features with eps (0 means 1e-6); rope rotates features
 *       (2Pa + 2i, 2Pa + 2i + 1), P = floor(d / 6), of axis a by coords[n][a] * base^(-i / P)
 *       (rope_base 0 means 10000); features past 6P are not rotated;
 *   gates = sigmoid(x W_gate^T + b_gate), W_gate [3*H, C], b_gate [3*H] or NULL;
 *       layout [N, H, 3] (feature h * 3 + branch: compressed, selected, window).
 * dtype F16 or BF16 (F32 returns SSA_ERR_UNSUPPORTED); d in {32, 64, 96, 128}; C a multiple
 * of 8.  gamma_q, gamma_k [d]; coords int32 [N,3].  All device pointers; fp32 accumulation;
 * outputs in the dtype.  Asynchronous on `stream`; allocates nothing.
 */
ssa_status ssa_qkv_gates(ssa_dtype dtype, int64_t n, int32_t channels, int32_t heads, int32_t dim,
                         const void* x, const void* w_qkv, const void* w_gate, const void* b_gate,
                         const void* gamma_q, const void* gamma_k, const int32_t* coords,
                         float rope_base, float eps, void* q, void* k, void* v, void* gates,
                         hipStream_t stream);

const char* ssa_status_string(ssa_status status);

#ifdef __cplusplus
}
#endif
#endif /* SSA_H */
