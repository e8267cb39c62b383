// Internal declarations shared by the library's translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include "ssa.h"

#define SSA_PLAN_MAGIC 0x53534150u  // "SSAP"

// Host-side plan handle.  Device arrays live in the caller's plan workspace.
struct ssa_plan_s {
  uint32_t magic;
  int64_t n;
  int32_t grid[3];
  int32_t block, window;
  int32_t dims[3];          // blocks per axis
  int64_t M, ncells;
  int32_t max_rows;
  bool window_is_block;     // w == B: cells alias blocks
  int32_t *perm, *blk_off, *blk_key, *tok2blk, *blk_cell, *cell_off, *cell_blk, *lpt;
};

// Bump allocator over a caller workspace.  With base == nullptr it only measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T> T* take(size_t count) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

// Plan workspace layout (sizes depend on n only).
struct PlanWs {
  int32_t *perm, *blk_off, *blk_key, *tok2blk, *blk_cell, *cell_off, *cell_blk, *lpt;
  uint32_t *key_a, *key_b;
  int32_t *val_a, *val_b, *rank, *hist, *tile_cnt, *counters, *scan_part;
  int32_t* cell_key;
};
size_t plan_carve(Carver& c, int64_t n, PlanWs* w);

static inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
static inline int nsplit_of(ssa_dtype dt) { return dt == SSA_F32 ? 1 : (dt == SSA_F16 ? 2 : 3); }
static inline size_t esize_of(ssa_dtype dt) { return dt == SSA_F32 ? 4 : 2; }

// Row strides (elements) of the padded 32-row tiles staged in LDS.  The pooled keys and
// values are stored in HBM as one "stage" per (head, 32-block tile): the NSPLIT key planes
// ([32][krow] each) followed by the value tile ([32][vrow]), exactly the LDS layout, so a
// tile is one contiguous copy.
static inline int krow_of(ssa_dtype dt, int d) { return d + (dt == SSA_F32 ? 4 : 8); }
static inline int vrow_of(ssa_dtype dt, int d) { return d + (dt == SSA_F32 ? 8 : 16); }
static inline int64_t stage_elems(ssa_dtype dt, int d) {
  return (int64_t)32 * (nsplit_of(dt) * krow_of(dt, d) + vrow_of(dt, d));
}

// Forward workspace layout.
struct FwdWs {
  void* pooled;      // [H][Mp/32][stage] dtype: pooled key planes + pooled values, padding zero
  void* oc;          // [H][N][d] compressed-branch output, block-sorted rows (dtype)
  int32_t* sel;      // [H][M][topk]
};
size_t fwd_carve(Carver& c, const ssa_plan_s* p, ssa_dtype dt, int H, int d, int topk, FwdWs* w);


#define SSA_HIP_CHECK(expr)                          \
  do {                                               \
    if ((expr) != hipSuccess) return SSA_ERR_HIP;    \
  } while (0)

// Kernel-launch entry points implemented in the .hip files.
hipError_t launch_pool(ssa_dtype dt, const ssa_plan_s* p, int H, int d, const void* k,
                       const void* v, const void* wk, const void* wv, const FwdWs& w,
                       hipStream_t s);
hipError_t launch_select(ssa_dtype dt, const ssa_plan_s* p, int H, int d, int topk, float scale,
                         const void* q, const FwdWs& w, int32_t* sel, hipStream_t s);
hipError_t launch_attend(ssa_dtype dt, const ssa_plan_s* p, int H, int d, int topk, float scale,
                         const void* q, const void* k, const void* v, const void* gates,
                         const FwdWs& w, const int32_t* sel, void* out, hipStream_t s);
