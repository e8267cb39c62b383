// Internal declarations shared by the library's translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <cstring>
#include <mutex>
#include <rocprofiler-sdk-roctx/roctx.h>
#include "ssa.h"

#define SSA_PLAN_MAGIC 0x53534150u  // "SSAP"

// A roctx range around one host call's launches (rocprofv3 --marker-trace shows them per
// phase; without a profiler attached a push or pop is a call into an empty table).
struct RoctxRange {
  explicit RoctxRange(const char* name) { roctxRangePushA(name); }
  ~RoctxRange() { roctxRangePop(); }
  RoctxRange(const RoctxRange&) = delete;
  RoctxRange& operator=(const RoctxRange&) = delete;
};

// Enum arguments of the C ABI may carry any int (C allows that); C++ forbids reading an
// enum object whose value lies outside its enumerators' range, so entry points test the raw
// bits before the first read of such an argument.
template <class E>
inline bool abi_enum_in(const E* e, int lo, int hi) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized on this ABI");
  int v;
  std::memcpy(&v, e, sizeof v);
  return v >= lo && v <= hi;
}

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
  // Window cells that are not unions of blocks get a token-level partition of their own:
  // wkind 0 = cells are unions of blocks (blk_cell, cell_off, cell_blk above); 1 = cubic
  // cells floor((c + wshift) / window); 2 = runs of sfc_tokens tokens along the Morton order.
  int32_t wkind = 0;
  int32_t wshift[3] = {0, 0, 0};
  int32_t sfc_tokens = 0;
  int64_t wC = 0;           // cells of the token-level partition
  int32_t wmax_rows = 0;    // tokens of its largest cell
  int32_t *wperm = nullptr, *wcell_off = nullptr, *wlpt = nullptr;
  int32_t* pos = nullptr;   // [N] position of each token inside its block, x-major, in [0, B^3)
  // Softmax scale of the most recent forwards that saved state for the backward, by
  // workspace address: the saved log-sum-exp values hold that scale, so a backward on
  // the same workspace must use it.  Guarded by rec_mu (a plan may serve several threads).
  struct FwdRecord { const void* ws; float scale; int conv; };
  static constexpr int NREC = 16;
  FwdRecord rec[NREC] = {};
  int rec_next = 0;
  std::mutex rec_mu;
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
  int32_t *wperm, *wcell_off, *wlpt;  // token-level window partition (when cells are not unions of blocks)
  int32_t* pos;                       // position of each token inside its block
};
size_t plan_carve(Carver& c, int64_t n, PlanWs* w);

static inline int nsplit_of(ssa_dtype dt) { return dt == SSA_F32 ? 1 : (dt == SSA_F16 ? 2 : 3); }
static inline size_t esize_of(ssa_dtype dt) { return dt == SSA_F32 ? 4 : 2; }

// Row strides (elements) of the padded tiles staged in LDS.  The pooled keys and values
// are stored in HBM as one "stage" per (head, 64-block tile): the NSPLIT key planes
// ([64][krow] each) followed by the values transposed ([d][vtrow]), exactly the LDS
// layout, so a tile is one contiguous copy.  A row-major copy of the pooled values
// ([H][Mp][vrow]) serves the backward.
constexpr int POOL_TILE = 64;
// Workgroups for nunits units of `per` members each, dealt to the 8 XCDs round-robin.
static inline unsigned xcd_grid(int64_t nunits, int64_t per) { return (unsigned)((nunits + 7) / 8 * 8 * per); }
// Gathers from a token tensor use 32-bit byte offsets (buffer loads) when it is below 4 GiB.
static inline bool buffer_addressable(int64_t bytes) { return bytes <= (int64_t)0xFFFFFFF0; }
// Pooled blocks per head as stored: a whole, even number of 64-block stages, so that every
// pass of the selection starts on the same stage buffer.
static inline int64_t pooled_rows(int64_t M) { return ((M > 0 ? M : 1) + 127) / 128 * 128; }
// The top-k runs as its own kernel (one wave per (head, query block) row) when the importance
// rows are short and their buffer small; else at the end of the selection kernel.
constexpr int TOPK_SPLIT_MAX_M = 1024;
static inline bool split_topk(int64_t M, int64_t H) {
  return M <= TOPK_SPLIT_MAX_M && H * M * pooled_rows(M) * 4 <= ((int64_t)256 << 20);
}
static inline int krow_of(ssa_dtype dt, int d) { return d + (dt == SSA_F32 ? 4 : 8); }
static inline int vrow_of(ssa_dtype dt, int d) { return d + (dt == SSA_F32 ? 8 : 16); }
static inline int vtrow_of(ssa_dtype dt) { return dt == SSA_F32 ? POOL_TILE + 1 : POOL_TILE + 4; }
static inline int64_t stage_elems(ssa_dtype dt, int d) {
  return (int64_t)POOL_TILE * nsplit_of(dt) * krow_of(dt, d) + (int64_t)d * vtrow_of(dt);
}

// Forward workspace layout.  Rows r are block-sorted token positions.
struct FwdWs {
  void* pooled;      // [H][Mp/64][stage] dtype: pooled key planes + pooled values^T, padding zero
  void* pooled_v;    // [H][Mp][vrow] dtype: pooled values, row-major
  void* oc;          // [N][H][d] compressed-branch output (dtype)
  int32_t* sel;      // [H][M][topk]
  int2* sdesc;       // [H][M][topk] first sorted row and size of each selected block ((0, 0) for -1)
  int4* utab;        // [max(M, window cells)] per longest-first unit: (block, first row, rows, 0)
  float* sigma;      // [H][M][Mp] importance scores when the top-k runs as its own kernel, else null
  float* lsec;       // [H][N] log2-sum-exp2 of the compressed branch's scaled scores (= lse plane 0)
  void* ow;          // [N][H][d] dtype, caller order: the window branch's output when window cells
                     // have a token-level partition of their own (else null)
  // saved for the backward (save_for_bwd only; else null)
  float* lse;        // [3][H][N] per-branch log2-sum-exp2 of the scaled scores
  void* obr;         // the branch outputs, sorted rows: fp32 [3][N][H][d] (compressed, selected,
                     // window); f16 inputs: f16 [2][N][H][d] (selected, window; the compressed
                     // output is oc itself)
};
// Saved branch outputs: f16 inputs keep them in f16 (the backward's dgates and D read them
// once; f16 rounding is below the gradients' own), other types in fp32.
static inline bool save_f16(ssa_dtype dt) { return dt == SSA_F16; }
size_t fwd_carve(Carver& c, const ssa_plan_s* p, ssa_dtype dt, int H, int d, int topk, int save,
                 FwdWs* w);


#define SSA_HIP_CHECK(expr)                          \
  do {                                               \
    if ((expr) != hipSuccess) return SSA_ERR_HIP;    \
  } while (0)

// Device sorting helpers of the plan (stable LSD radix sort on 8-bit digits).
namespace ssa_sort {
int bits_for(uint64_t maxval);
void device_scan(int32_t* a, int len, int32_t* total, int32_t* part, hipStream_t s);
hipError_t radix_sort(uint32_t*& ka, int32_t*& va, uint32_t*& kb, int32_t*& vb, int n, int nbits,
                      int32_t* rank, int32_t* hist, int32_t* part, hipStream_t s);
}  // namespace ssa_sort
// Scratch sizes of radix_sort over n elements.
static inline int64_t radix_hist_len(int64_t n) { return (n + 255) / 256 * 256; }
static inline int64_t scan_part_len(int64_t len) { return len / 4096 + 2; }

// Kernel-launch entry points implemented in the .hip files.
hipError_t launch_pool(ssa_dtype dt, const ssa_plan_s* p, int H, int d, const void* k,
                       const void* v, const void* wk, const void* wv, const FwdWs& w,
                       hipStream_t s);
constexpr int LDS_BYTES = 160 * 1024;  // LDS of one workgroup on gfx950
int64_t select_block_limit(ssa_dtype dt, int d);
hipError_t launch_select(ssa_dtype dt, const ssa_plan_s* p, int H, int d, int topk, float scale,
                         const void* q, const FwdWs& w, int32_t* sel, hipStream_t s);
hipError_t launch_backward(ssa_dtype dt, const ssa_plan_s* p, int H, int d, int topk, float scale,
                           const void* q, const void* k, const void* v, const void* wk,
                           const void* wv, const void* gates, const int32_t* sel, const void* dout,
                           float* dq, float* dk, float* dv, float* dgates, const FwdWs& fw,
                           void* ws, hipStream_t s, int conv);
// The sparse-convolution compressor (wk, wv are [B^3][d][d] position weights).
hipError_t launch_pool_conv(ssa_dtype dt, const ssa_plan_s* p, int H, int d, const void* k, const void* v,
                            const void* wck, const void* wcv, const FwdWs& w, hipStream_t s);
hipError_t launch_conv_term(ssa_dtype dt, const ssa_plan_s* p, int H, int d, const void* wck, const void* wcv,
                            const float* gk, const float* gv, float* dk, float* dv, hipStream_t s);
size_t bwd_carve(Carver& c, const ssa_plan_s* p, int H, int d, int topk, void* w);
hipError_t launch_attend(ssa_dtype dt, const ssa_plan_s* p, int H, int d, int topk, float scale,
                         const void* q, const void* k, const void* v, const void* gates,
                         const FwdWs& w, const int32_t* sel, void* out, hipStream_t s);
