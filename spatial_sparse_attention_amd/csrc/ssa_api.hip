// Host side of the C ABI: argument validation, workspace carving and stage launches.
#include <hip/hip_runtime.h>
#include <math.h>
#include "ssa_internal.h"

namespace {
constexpr int KT = 32;
constexpr int64_t MAX_BLOCKS = 6144;  // importance vector of one work item lives in LDS (24 KB)
constexpr int MAX_TOPK = 256;

bool dim_ok(int d) { return d == 32 || d == 64 || d == 96 || d == 128; }

ssa_status check_common(ssa_plan p, ssa_dtype dt, int32_t H, int32_t d, int32_t topk) {
  if (!p || p->magic != SSA_PLAN_MAGIC) return SSA_ERR_BAD_PLAN;
  if ((int)dt < 0 || (int)dt > 2) return SSA_ERR_INVALID_ARG;
  if (H < 1 || d < 1 || topk < 1) return SSA_ERR_INVALID_ARG;
  if (!dim_ok(d) || topk > MAX_TOPK) return SSA_ERR_UNSUPPORTED;
  if (p->M > MAX_BLOCKS) return SSA_ERR_UNSUPPORTED;
  if (p->n * (int64_t)H >= ((int64_t)1 << 31)) return SSA_ERR_UNSUPPORTED;
  return SSA_OK;
}
}  // namespace

size_t fwd_carve(Carver& c, const ssa_plan_s* p, ssa_dtype dt, int H, int d, int topk, int save,
                 FwdWs* w) {
  const int64_t Mp = pooled_rows(p->M);
  const int64_t n1 = p->n > 0 ? p->n : 1;
  const size_t es = esize_of(dt);
  FwdWs t;
  t.pooled = c.take<char>((size_t)H * (Mp / POOL_TILE) * stage_elems(dt, d) * es);
  t.pooled_v = c.take<char>((size_t)H * Mp * vrow_of(dt, d) * es);
  t.oc = c.take<char>((size_t)H * n1 * d * es);
  t.sel = c.take<int32_t>((size_t)H * (p->M > 0 ? p->M : 1) * topk);
  t.sigma = split_topk(p->M, H) ? c.take<float>((size_t)H * (p->M > 0 ? p->M : 1) * Mp) : nullptr;
  t.lse = nullptr;
  t.obr = nullptr;
  if (save) {
    t.lse = c.take<float>((size_t)3 * H * n1);
    t.obr = c.take<float>((size_t)3 * H * n1 * d);
  }
  t.lsec = save ? t.lse : c.take<float>((size_t)H * n1);
  if (w) *w = t;
  return c.off;
}

extern "C" size_t ssa_forward_workspace_size(ssa_plan p, ssa_dtype dt, int32_t H, int32_t d,
                                             int32_t topk, int save_for_bwd) {
  if (check_common(p, dt, H, d, topk) != SSA_OK) return 0;
  Carver c(nullptr);
  return fwd_carve(c, p, dt, H, d, topk, save_for_bwd ? 1 : 0, nullptr) + 256;
}

extern "C" ssa_status ssa_forward_stages(ssa_plan p, ssa_dtype dt, int32_t H, int32_t d,
                                         const void* q, const void* k, const void* v,
                                         const void* wk, const void* wv, const void* gates,
                                         int32_t topk, float scale, void* out, int32_t* sel_out,
                                         void* ws, size_t ws_bytes, int save_for_bwd,
                                         hipStream_t stream, uint32_t stages) {
  ssa_status st = check_common(p, dt, H, d, topk);
  if (st != SSA_OK) return st;
  if (stages == 0 || (stages & ~7u)) return SSA_ERR_INVALID_ARG;
  if (!(scale >= 0.f) || isinf(scale)) return SSA_ERR_INVALID_ARG;
  if (scale == 0.f) scale = 1.f / sqrtf((float)d);
  if (p->n == 0) return SSA_OK;
  if (!q || !k || !v || !wk || !wv || !gates || !out) return SSA_ERR_INVALID_ARG;
  if (!ws) return SSA_ERR_WORKSPACE;
  const int save = save_for_bwd ? 1 : 0;
  if (ws_bytes < ssa_forward_workspace_size(p, dt, H, d, topk, save)) return SSA_ERR_WORKSPACE;
  Carver c(ws);
  c.off = (256 - (reinterpret_cast<uintptr_t>(ws) & 255)) & 255;
  FwdWs w;
  fwd_carve(c, p, dt, H, d, topk, save, &w);
  int32_t* sel = sel_out ? sel_out : w.sel;
  if (stages & SSA_STAGE_POOL)
    if (launch_pool(dt, p, H, d, k, v, wk, wv, w, stream) != hipSuccess) return SSA_ERR_HIP;
  if (stages & SSA_STAGE_SELECT) {
    if (p->M > select_block_limit(dt, d)) return SSA_ERR_UNSUPPORTED;
    if (launch_select(dt, p, H, d, topk, scale, q, w, sel, stream) != hipSuccess) return SSA_ERR_HIP;
  }
  if (stages & SSA_STAGE_ATTEND)
    if (launch_attend(dt, p, H, d, topk, scale, q, k, v, gates, w, sel, out, stream) != hipSuccess)
      return SSA_ERR_HIP;
  return SSA_OK;
}

extern "C" ssa_status ssa_forward(ssa_plan p, ssa_dtype dt, int32_t H, int32_t d, const void* q,
                                  const void* k, const void* v, const void* wk, const void* wv,
                                  const void* gates, int32_t topk, float scale, void* out,
                                  int32_t* sel_out, void* ws, size_t ws_bytes, int save_for_bwd,
                                  hipStream_t stream) {
  return ssa_forward_stages(p, dt, H, d, q, k, v, wk, wv, gates, topk, scale, out, sel_out, ws,
                            ws_bytes, save_for_bwd, stream, SSA_STAGE_ALL);
}

extern "C" size_t ssa_backward_workspace_size(ssa_plan p, ssa_dtype dt, int32_t H, int32_t d,
                                              int32_t topk) {
  if (check_common(p, dt, H, d, topk) != SSA_OK) return 0;
  Carver c(nullptr);
  return bwd_carve(c, p, H, d, topk, nullptr) + 256;
}

extern "C" ssa_status ssa_backward(ssa_plan p, ssa_dtype dt, int32_t H, int32_t d, const void* q,
                                   const void* k, const void* v, const void* wk, const void* wv,
                                   const void* gates, int32_t topk, float scale,
                                   const int32_t* sel, const void* dout, float* dq, float* dk,
                                   float* dv, float* dgates, const void* fwd_ws,
                                   size_t fwd_ws_bytes, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  ssa_status st = check_common(p, dt, H, d, topk);
  if (st != SSA_OK) return st;
  if (!(scale >= 0.f) || isinf(scale)) return SSA_ERR_INVALID_ARG;
  if (scale == 0.f) scale = 1.f / sqrtf((float)d);
  if (p->n == 0) return SSA_OK;
  if (!q || !k || !v || !wk || !wv || !gates || !sel || !dout || !dq || !dk || !dv || !dgates)
    return SSA_ERR_INVALID_ARG;
  if (p->M > select_block_limit(dt, d)) return SSA_ERR_UNSUPPORTED;  // the forward's limit
  if (!fwd_ws || fwd_ws_bytes < ssa_forward_workspace_size(p, dt, H, d, topk, 1)) return SSA_ERR_WORKSPACE;
  if (!ws || ws_bytes < ssa_backward_workspace_size(p, dt, H, d, topk)) return SSA_ERR_WORKSPACE;
  Carver c(const_cast<void*>(fwd_ws));
  c.off = (256 - (reinterpret_cast<uintptr_t>(fwd_ws) & 255)) & 255;
  FwdWs fw;
  fwd_carve(c, p, dt, H, d, topk, 1, &fw);
  if (launch_backward(dt, p, H, d, topk, scale, q, k, v, wk, wv, gates, sel, dout, dq, dk, dv,
                      dgates, fw, ws, stream) != hipSuccess)
    return SSA_ERR_HIP;
  return SSA_OK;
}

extern "C" const char* ssa_status_string(ssa_status s) {
  switch (s) {
    case SSA_OK: return "ok";
    case SSA_ERR_INVALID_ARG: return "invalid argument";
    case SSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SSA_ERR_WORKSPACE: return "workspace missing or too small";
    case SSA_ERR_COORD_RANGE: return "coordinate outside the grid";
    case SSA_ERR_HIP: return "HIP runtime error";
    case SSA_ERR_BAD_PLAN: return "invalid plan handle";
  }
  return "unknown status";
}
