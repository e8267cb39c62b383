// Host side of the C ABI: argument validation, workspace carving and stage launches.
#include <hip/hip_runtime.h>
#include <math.h>
#include <algorithm>
#include "ssa_internal.h"

namespace {
constexpr int KT = 32;
constexpr int MAX_TOPK = 256;

bool dim_ok(int d) { return d == 32 || d == 64 || d == 96 || d == 128; }

ssa_status check_common(ssa_plan p, ssa_dtype dt, int32_t H, int32_t d, int32_t topk) {
  if (!p || p->magic != SSA_PLAN_MAGIC) return SSA_ERR_BAD_PLAN;
  if ((int)dt < 0 || (int)dt > 2) return SSA_ERR_INVALID_ARG;
  if (H < 1 || d < 1 || topk < 1) return SSA_ERR_INVALID_ARG;
  if (!dim_ok(d) || topk > MAX_TOPK) return SSA_ERR_UNSUPPORTED;
  if (p->n * (int64_t)H >= ((int64_t)1 << 31)) return SSA_ERR_UNSUPPORTED;
  return SSA_OK;
}
// The saved log-sum-exp values of a forward hold its scale: remember it per workspace so
// that a backward with another scale is refused instead of returning wrong gradients.
void record_forward(ssa_plan_s* p, const void* ws, float scale, int conv) {
  std::lock_guard<std::mutex> lk(p->rec_mu);
  for (auto& r : p->rec)
    if (r.ws == ws) { r.scale = scale; r.conv = conv; return; }
  p->rec[p->rec_next] = {ws, scale, conv};
  p->rec_next = (p->rec_next + 1) % ssa_plan_s::NREC;
}

// True unless this plan's record of a saving forward on fwd_ws holds a different scale or
// compressor (a workspace the record no longer holds, after NREC later ones, is not checked).
bool recorded_forward_matches(ssa_plan_s* p, const void* fwd_ws, float scale, int conv) {
  std::lock_guard<std::mutex> lk(p->rec_mu);
  for (const auto& r : p->rec)
    if (r.ws == fwd_ws) return r.scale == scale && r.conv == conv;
  return true;
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
  t.sdesc = c.take<int2>((size_t)H * (p->M > 0 ? p->M : 1) * topk);
  t.utab = c.take<int4>((size_t)std::max<int64_t>(std::max<int64_t>(p->M, p->wC), 1));
  t.sigma = split_topk(p->M, H) ? c.take<float>((size_t)H * (p->M > 0 ? p->M : 1) * Mp) : nullptr;
  t.lse = nullptr;
  t.obr = nullptr;
  if (save) {
    t.lse = c.take<float>((size_t)3 * H * n1);
    t.obr = save_f16(dt) ? (void*)c.take<uint16_t>((size_t)2 * H * n1 * d) : (void*)c.take<float>((size_t)3 * H * n1 * d);
  }
  t.lsec = save ? t.lse : c.take<float>((size_t)H * n1);
  t.ow = p->wkind != 0 ? c.take<char>((size_t)n1 * H * d * es) : nullptr;
  if (w) *w = t;
  return c.off;
}

extern "C" int64_t ssa_forward_max_blocks(ssa_dtype dt, int32_t d) {
  if (!abi_enum_in(&dt, 0, 2) || !dim_ok(d)) return 0;
  return select_block_limit(dt, d);
}

extern "C" size_t ssa_forward_workspace_size(ssa_plan p, ssa_dtype dt, int32_t H, int32_t d,
                                             int32_t topk, int save_for_bwd) {
  if (!abi_enum_in(&dt, 0, 2)) return 0;
  if (check_common(p, dt, H, d, topk) != SSA_OK) return 0;
  Carver c(nullptr);
  return fwd_carve(c, p, dt, H, d, topk, save_for_bwd ? 1 : 0, nullptr) + 256;
}

static ssa_status forward_impl(ssa_plan p, ssa_dtype dt, int32_t H, int32_t d, const void* q, const void* k,
                               const void* v, const void* wk, const void* wv, const void* gates, int32_t topk,
                               float scale, void* out, int32_t* sel_out, void* ws, size_t ws_bytes,
                               int save_for_bwd, hipStream_t stream, uint32_t stages, int conv) {
  ssa_status st = check_common(p, dt, H, d, topk);
  if (st != SSA_OK) return st;
  if (stages == 0 || (stages & ~7u)) return SSA_ERR_INVALID_ARG;
  if (!(scale >= 0.f) || isinf(scale)) return SSA_ERR_INVALID_ARG;
  if (scale == 0.f) scale = 1.f / sqrtf((float)d);
  if (p->n == 0) return SSA_OK;
  if (!q || !k || !v || !wk || !wv || !gates || !out) return SSA_ERR_INVALID_ARG;
  if (!ws) return SSA_ERR_WORKSPACE;
  const int save = save_for_bwd ? 1 : 0;
  if (p->M > select_block_limit(dt, d)) return SSA_ERR_UNSUPPORTED;  // before any launch
  if (save && p->wkind != 0) return SSA_ERR_UNSUPPORTED;  // the backward needs cells of blocks
  // the size query adds 256 bytes of alignment slack; what counts is the carve from the
  // workspace's actual alignment
  Carver c(ws);
  c.off = (256 - (reinterpret_cast<uintptr_t>(ws) & 255)) & 255;
  FwdWs w;
  if (ws_bytes < fwd_carve(c, p, dt, H, d, topk, save, &w)) return SSA_ERR_WORKSPACE;
  int32_t* sel = sel_out ? sel_out : w.sel;
  if (save && (stages & SSA_STAGE_SELECT)) record_forward(p, ws, scale, conv);
  if (stages & SSA_STAGE_POOL) {
    RoctxRange r(conv ? "ssa_forward/pool_conv" : "ssa_forward/pool");
    const hipError_t e = conv ? launch_pool_conv(dt, p, H, d, k, v, wk, wv, w, stream)
                              : launch_pool(dt, p, H, d, k, v, wk, wv, w, stream);
    if (e != hipSuccess) return SSA_ERR_HIP;
  }
  if (stages & SSA_STAGE_SELECT) {
    RoctxRange r("ssa_forward/select");
    if (launch_select(dt, p, H, d, topk, scale, q, w, sel, stream) != hipSuccess) return SSA_ERR_HIP;
  }
  if (stages & SSA_STAGE_ATTEND) {
    RoctxRange r("ssa_forward/attend");
    if (launch_attend(dt, p, H, d, topk, scale, q, k, v, gates, w, sel, out, stream) != hipSuccess)
      return SSA_ERR_HIP;
  }
  return SSA_OK;
}

extern "C" ssa_status ssa_forward_stages(ssa_plan p, ssa_dtype dt, int32_t H, int32_t d,
                                         const void* q, const void* k, const void* v,
                                         const void* wk, const void* wv, const void* gates,
                                         int32_t topk, float scale, void* out, int32_t* sel_out,
                                         void* ws, size_t ws_bytes, int save_for_bwd,
                                         hipStream_t stream, uint32_t stages) {
  if (!abi_enum_in(&dt, 0, 2)) return SSA_ERR_INVALID_ARG;
  return forward_impl(p, dt, H, d, q, k, v, wk, wv, gates, topk, scale, out, sel_out, ws, ws_bytes, save_for_bwd,
                      stream, stages, 0);
}

extern "C" ssa_status ssa_forward_conv(ssa_plan p, ssa_dtype dt, int32_t H, int32_t d, const void* q,
                                       const void* k, const void* v, const void* wk_conv, const void* wv_conv,
                                       const void* gates, int32_t topk, float scale, void* out,
                                       int32_t* sel_out, void* ws, size_t ws_bytes, int save_for_bwd,
                                       hipStream_t stream) {
  if (!abi_enum_in(&dt, 0, 2)) return SSA_ERR_INVALID_ARG;
  return forward_impl(p, dt, H, d, q, k, v, wk_conv, wv_conv, gates, topk, scale, out, sel_out, ws, ws_bytes,
                      save_for_bwd, stream, SSA_STAGE_ALL, 1);
}

extern "C" ssa_status ssa_forward(ssa_plan p, ssa_dtype dt, int32_t H, int32_t d, const void* q,
                                  const void* k, const void* v, const void* wk, const void* wv,
                                  const void* gates, int32_t topk, float scale, void* out,
                                  int32_t* sel_out, void* ws, size_t ws_bytes, int save_for_bwd,
                                  hipStream_t stream) {
  if (!abi_enum_in(&dt, 0, 2)) return SSA_ERR_INVALID_ARG;
  return ssa_forward_stages(p, dt, H, d, q, k, v, wk, wv, gates, topk, scale, out, sel_out, ws,
                            ws_bytes, save_for_bwd, stream, SSA_STAGE_ALL);
}

// ------------------------------------------------------------------ no-allocation forward
// The forward's workspace in a fixed device array instead of a caller's buffer.  Host code
// never uses the array's name as an address: the name is a host-side stand-in, and the
// device address of each GPU's copy comes from hipGetSymbolAddress, fetched once per device
// with that device current.
static __device__ __align__(256) char scratch[SSA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES] = {};

// The current device's copy of the scratch array, or nullptr on a HIP error.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lk(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    scratch_ptr[dev] = ptr;
  }
  return scratch_ptr[dev];
}
}  // namespace

extern "C" ssa_status ssa_forward_noalloc(ssa_plan p, ssa_dtype dt, int32_t H, int32_t d,
                                          const void* q, const void* k, const void* v,
                                          const void* wk, const void* wv, const void* gates,
                                          int32_t topk, float scale, void* out, int32_t* sel_out,
                                          hipStream_t stream) {
  if (!abi_enum_in(&dt, 0, 2)) return SSA_ERR_INVALID_ARG;
  ssa_status st = check_common(p, dt, H, d, topk);
  if (st != SSA_OK) return st;
  if (p->n == 0) return ssa_forward_stages(p, dt, H, d, q, k, v, wk, wv, gates, topk, scale, out,
                                           sel_out, nullptr, 0, 0, stream, SSA_STAGE_ALL);
  Carver c(nullptr);  // the array is 256-byte aligned: the carve starts at offset 0
  if (fwd_carve(c, p, dt, H, d, topk, 0, nullptr) > (size_t)SSA_NOALLOC_SCRATCH_BYTES)
    return SSA_ERR_TOO_LARGE;
  void* ws = scratch_address();
  if (!ws) return SSA_ERR_HIP;
  return ssa_forward_stages(p, dt, H, d, q, k, v, wk, wv, gates, topk, scale, out, sel_out, ws,
                            (size_t)SSA_NOALLOC_SCRATCH_BYTES, 0, stream, SSA_STAGE_ALL);
}

// ------------------------------------------------------------------ several samples
extern "C" size_t ssa_forward_batch_workspace_size(const ssa_plan* plans, int32_t nsamples, ssa_dtype dt,
                                                   int32_t H, int32_t d, int32_t topk) {
  if (!abi_enum_in(&dt, 0, 2)) return 0;
  if (!plans || nsamples < 1) return 0;
  size_t mx = 0;
  for (int i = 0; i < nsamples; ++i) {
    const size_t sz = ssa_forward_workspace_size(plans[i], dt, H, d, topk, 0);
    if (sz == 0) return 0;
    mx = sz > mx ? sz : mx;
  }
  return mx;
}

extern "C" ssa_status ssa_forward_batch(const ssa_plan* plans, int32_t nsamples, const int64_t* tok_off,
                                        ssa_dtype dt, int32_t H, int32_t d, const void* q, const void* k,
                                        const void* v, const void* wk, const void* wv, const void* gates,
                                        int32_t topk, float scale, void* out, void* ws, size_t ws_bytes,
                                        hipStream_t stream) {
  if (!abi_enum_in(&dt, 0, 2)) return SSA_ERR_INVALID_ARG;
  if (!plans || !tok_off || nsamples < 1) return SSA_ERR_INVALID_ARG;
  if (tok_off[0] != 0) return SSA_ERR_INVALID_ARG;
  for (int i = 0; i < nsamples; ++i) {  // every check before any launch
    const ssa_status st = check_common(plans[i], dt, H, d, topk);
    if (st != SSA_OK) return st;
    if (tok_off[i + 1] - tok_off[i] != plans[i]->n) return SSA_ERR_INVALID_ARG;
    if (plans[i]->M > select_block_limit(dt, d)) return SSA_ERR_UNSUPPORTED;
  }
  if (ws_bytes < ssa_forward_batch_workspace_size(plans, nsamples, dt, H, d, topk)) return SSA_ERR_WORKSPACE;
  const size_t es = esize_of(dt);
  auto at = [&](const void* base, int64_t tok, int64_t per) -> const void* {
    return base ? static_cast<const char*>(base) + (size_t)tok * per * es : nullptr;
  };
  for (int i = 0; i < nsamples; ++i) {
    const int64_t t0 = tok_off[i];
    const ssa_status st = ssa_forward_stages(
        plans[i], dt, H, d, at(q, t0, (int64_t)H * d), at(k, t0, (int64_t)H * d), at(v, t0, (int64_t)H * d), wk, wv,
        at(gates, t0, (int64_t)H * 3), topk, scale, const_cast<void*>(at(out, t0, (int64_t)H * d)), nullptr, ws,
        ws_bytes, 0, stream, SSA_STAGE_ALL);
    if (st != SSA_OK) return st;
  }
  return SSA_OK;
}

extern "C" size_t ssa_backward_workspace_size(ssa_plan p, ssa_dtype dt, int32_t H, int32_t d,
                                              int32_t topk) {
  if (!abi_enum_in(&dt, 0, 2)) return 0;
  if (check_common(p, dt, H, d, topk) != SSA_OK || p->wkind != 0) return 0;
  Carver c(nullptr);
  return bwd_carve(c, p, H, d, topk, nullptr) + 256;
}

static ssa_status backward_impl(ssa_plan p, ssa_dtype dt, int32_t H, int32_t d, const void* q, const void* k,
                                const void* v, const void* wk, const void* wv, const void* gates, int32_t topk,
                                float scale, const int32_t* sel, const void* dout, float* dq, float* dk,
                                float* dv, float* dgates, const void* fwd_ws, size_t fwd_ws_bytes, void* ws,
                                size_t ws_bytes, hipStream_t stream, int conv) {
  ssa_status st = check_common(p, dt, H, d, topk);
  if (st != SSA_OK) return st;
  if (!(scale >= 0.f) || isinf(scale)) return SSA_ERR_INVALID_ARG;
  if (scale == 0.f) scale = 1.f / sqrtf((float)d);
  if (p->n == 0) return SSA_OK;
  if (!q || !k || !v || !wk || !wv || !gates || !sel || !dout || !dq || !dk || !dv || !dgates)
    return SSA_ERR_INVALID_ARG;
  if (p->M > select_block_limit(dt, d)) return SSA_ERR_UNSUPPORTED;  // the forward's limit
  if (p->wkind != 0) return SSA_ERR_UNSUPPORTED;  // window cells must be unions of blocks
  if (!fwd_ws || fwd_ws_bytes < ssa_forward_workspace_size(p, dt, H, d, topk, 1)) return SSA_ERR_WORKSPACE;
  if (!ws || ws_bytes < ssa_backward_workspace_size(p, dt, H, d, topk)) return SSA_ERR_WORKSPACE;
  if (!recorded_forward_matches(p, fwd_ws, scale, conv)) return SSA_ERR_INVALID_ARG;
  Carver c(const_cast<void*>(fwd_ws));
  c.off = (256 - (reinterpret_cast<uintptr_t>(fwd_ws) & 255)) & 255;
  FwdWs fw;
  fwd_carve(c, p, dt, H, d, topk, 1, &fw);
  RoctxRange r(conv ? "ssa_backward_conv" : "ssa_backward");
  if (launch_backward(dt, p, H, d, topk, scale, q, k, v, wk, wv, gates, sel, dout, dq, dk, dv,
                      dgates, fw, ws, stream, conv) != hipSuccess)
    return SSA_ERR_HIP;
  return SSA_OK;
}

extern "C" ssa_status ssa_backward(ssa_plan p, ssa_dtype dt, int32_t H, int32_t d, const void* q,
                                   const void* k, const void* v, const void* wk, const void* wv,
                                   const void* gates, int32_t topk, float scale,
                                   const int32_t* sel, const void* dout, float* dq, float* dk,
                                   float* dv, float* dgates, const void* fwd_ws,
                                   size_t fwd_ws_bytes, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  if (!abi_enum_in(&dt, 0, 2)) return SSA_ERR_INVALID_ARG;
  return backward_impl(p, dt, H, d, q, k, v, wk, wv, gates, topk, scale, sel, dout, dq, dk, dv, dgates, fwd_ws,
                       fwd_ws_bytes, ws, ws_bytes, stream, 0);
}

extern "C" ssa_status ssa_backward_conv(ssa_plan p, ssa_dtype dt, int32_t H, int32_t d, const void* q,
                                        const void* k, const void* v, const void* wk_conv, const void* wv_conv,
                                        const void* gates, int32_t topk, float scale, const int32_t* sel,
                                        const void* dout, float* dq, float* dk, float* dv, float* dgates,
                                        const void* fwd_ws, size_t fwd_ws_bytes, void* ws, size_t ws_bytes,
                                        hipStream_t stream) {
  if (!abi_enum_in(&dt, 0, 2)) return SSA_ERR_INVALID_ARG;
  return backward_impl(p, dt, H, d, q, k, v, wk_conv, wv_conv, gates, topk, scale, sel, dout, dq, dk, dv, dgates,
                       fwd_ws, fwd_ws_bytes, ws, ws_bytes, stream, 1);
}

extern "C" const char* ssa_status_string(ssa_status s) {
  if (!abi_enum_in(&s, SSA_OK, SSA_ERR_TOO_LARGE)) return "unknown status";
  switch (s) {
    case SSA_OK: return "ok";
    case SSA_ERR_INVALID_ARG: return "invalid argument";
    case SSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SSA_ERR_WORKSPACE: return "workspace missing or too small";
    case SSA_ERR_COORD_RANGE: return "coordinate outside the grid";
    case SSA_ERR_HIP: return "HIP runtime error";
    case SSA_ERR_BAD_PLAN: return "invalid plan handle";
    case SSA_ERR_TOO_LARGE:
      return "the forward's workspace exceeds the fixed scratch area of ssa_forward_noalloc";
  }
  return "unknown status";
}
