// Block partition of a voxel coordinate set on the GPU.
//
// The pages state that SSA partitions its input tokens by their 3D coordinates
// (nav.superapi.store "Direct3D-S2", section "Technical principles of
// Direct3D-S2").  Here a block is the B^3 cube floor(c / B); tokens are sorted by
// the x-major block key with a stable LSD radix sort (8-bit digits, one tile of
// 256 keys per workgroup, in-tile ranks from wave ballots), then run boundaries
// give the segment offsets.  The same kernels group blocks into window cells and
// order blocks longest-first for load balance.
#include <hip/hip_runtime.h>
#include <string.h>
#include <algorithm>
#include "ssa_internal.h"

namespace {

constexpr int RTILE = 256;   // radix tile: one key per thread
constexpr int STILE = 1024;  // segment-scan tile: 4 elements per thread

__global__ void k_block_keys(const int32_t* __restrict__ coords, int64_t n, int3 grid, int B,
                             int3 dims, uint32_t* __restrict__ keys, int32_t* __restrict__ vals,
                             int32_t* __restrict__ err, int32_t* __restrict__ pos) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  int x = coords[3 * i], y = coords[3 * i + 1], z = coords[3 * i + 2];
  bool ok = x >= 0 && y >= 0 && z >= 0 && x < grid.x && y < grid.y && z < grid.z;
  if (!ok) {
    atomicOr(err, 1);
    x = y = z = 0;
  }
  uint32_t bx = x / B, by = y / B, bz = z / B;
  keys[i] = (bx * (uint32_t)dims.y + by) * (uint32_t)dims.z + bz;
  vals[i] = (int32_t)i;
  // position inside the block, x-major (the sparse-convolution compressor's weight index)
  pos[i] = (int32_t)(((x - bx * B) * (uint32_t)B + (y - by * B)) * (uint32_t)B + (z - bz * B));
}

// Per tile: stable rank of every key among equal digits, and the tile's digit histogram
// stored digit-major (hist[digit * tiles + tile]).
__global__ __launch_bounds__(RTILE) void k_radix_hist(const uint32_t* __restrict__ keys, int n,
                                                      int shift, int32_t* __restrict__ rank,
                                                      int32_t* __restrict__ hist, int tiles) {
  __shared__ int32_t wcount[RTILE / 64][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int j = tid; j < (RTILE / 64) * 256; j += RTILE) (&wcount[0][0])[j] = 0;
  __syncthreads();
  const int i = blockIdx.x * RTILE + tid;
  const bool valid = i < n;
  const uint32_t digit = valid ? ((keys[i] >> shift) & 255u) : 0u;
  // lanes holding the same digit: AND of per-bit agreement masks
  uint64_t same = __ballot(valid);
  for (int b = 0; b < 8; ++b) {
    uint64_t m = __ballot(valid && ((digit >> b) & 1u));
    same &= ((digit >> b) & 1u) ? m : ~m;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rw = __popcll(same & below);
  if (valid && rw == 0) wcount[wave][digit] = __popcll(same);
  __syncthreads();
  if (valid) {
    int r = rw;
    for (int w = 0; w < wave; ++w) r += wcount[w][digit];
    rank[i] = r;
  }
  {
    const int d = tid;  // RTILE == 256 digits
    int tot = 0;
    for (int w = 0; w < RTILE / 64; ++w) tot += wcount[w][d];
    hist[(int64_t)d * tiles + blockIdx.x] = tot;
  }
}

// Exclusive scan of `len` ints in place, one workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void k_scan_single(int32_t* __restrict__ a, int len,
                                                      int32_t* __restrict__ total) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int per = (len + 1023) / 1024;
  const int lo = min(len, tid * per), hi = min(len, lo + per);
  int s = 0;
  for (int j = lo; j < hi; ++j) s += a[j];
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int t = (tid >= off) ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += t;
    __syncthreads();
  }
  int run = part[tid] - s;
  for (int j = lo; j < hi; ++j) {
    int x = a[j];
    a[j] = run;
    run += x;
  }
  if (tid == 1023 && total) *total = part[1023];
}

// Multi-workgroup exclusive scan for long arrays: per-chunk sums, a scan of the chunk
// sums, then a scan of each chunk plus its offset.
constexpr int SCHUNK = 4096;  // 256 threads x 16 elements

__global__ __launch_bounds__(256) void k_scan_reduce(const int32_t* __restrict__ a, int len,
                                                     int32_t* __restrict__ part) {
  __shared__ int32_t red[256];
  const int base = blockIdx.x * SCHUNK + threadIdx.x * 16;
  int s = 0;
  for (int j = 0; j < 16; ++j) s += base + j < len ? a[base + j] : 0;
  red[threadIdx.x] = s;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void k_scan_apply(int32_t* __restrict__ a, int len,
                                                    const int32_t* __restrict__ part) {
  __shared__ int32_t pre[256];
  const int tid = threadIdx.x;
  const int base = blockIdx.x * SCHUNK + tid * 16;
  int v[16], s = 0;
  for (int j = 0; j < 16; ++j) {
    v[j] = base + j < len ? a[base + j] : 0;
    s += v[j];
  }
  pre[tid] = s;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int t = tid >= off ? pre[tid - off] : 0;
    __syncthreads();
    pre[tid] += t;
    __syncthreads();
  }
  int run = part[blockIdx.x] + pre[tid] - s;
  for (int j = 0; j < 16; ++j) {
    if (base + j < len) a[base + j] = run;
    run += v[j];
  }
}

__global__ __launch_bounds__(RTILE) void k_radix_scatter(
    const uint32_t* __restrict__ kin, const int32_t* __restrict__ vin, int n, int shift,
    const int32_t* __restrict__ rank, const int32_t* __restrict__ hist, int tiles,
    uint32_t* __restrict__ kout, int32_t* __restrict__ vout) {
  const int i = blockIdx.x * RTILE + threadIdx.x;
  if (i >= n) return;
  const uint32_t key = kin[i];
  const uint32_t digit = (key >> shift) & 255u;
  const int dst = hist[(int64_t)digit * tiles + blockIdx.x] + rank[i];
  kout[dst] = key;
  vout[dst] = vin[i];
}

// Segment boundaries of a sorted key array: count run starts per tile.
__global__ __launch_bounds__(256) void k_seg_count(const uint32_t* __restrict__ keys, int n,
                                                   int32_t* __restrict__ tile_cnt) {
  __shared__ int32_t red[256];
  const int base = blockIdx.x * STILE + threadIdx.x * 4;
  int c = 0;
  for (int j = 0; j < 4; ++j) {
    int r = base + j;
    if (r < n) c += (r == 0 || keys[r] != keys[r - 1]);
  }
  red[threadIdx.x] = c;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) tile_cnt[blockIdx.x] = red[0];
}

// Emit segment ids: seg_off[id] = start, seg_key[id] = key, elem_seg[vals[r]] = id.
__global__ __launch_bounds__(256) void k_seg_emit(const uint32_t* __restrict__ keys,
                                                  const int32_t* __restrict__ vals, int n,
                                                  const int32_t* __restrict__ tile_base,
                                                  int32_t* __restrict__ seg_off,
                                                  int32_t* __restrict__ seg_key,
                                                  int32_t* __restrict__ elem_seg) {
  __shared__ int32_t part[256];
  const int tid = threadIdx.x;
  const int base = blockIdx.x * STILE + tid * 4;
  int f[4], c = 0;
  for (int j = 0; j < 4; ++j) {
    int r = base + j;
    f[j] = (r < n) && (r == 0 || keys[r] != keys[r - 1]);
    c += f[j];
  }
  part[tid] = c;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    int t = (tid >= off) ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += t;
    __syncthreads();
  }
  int id = tile_base[blockIdx.x] + part[tid] - c - 1;  // id of the run before this thread's first
  for (int j = 0; j < 4; ++j) {
    int r = base + j;
    if (r >= n) break;
    id += f[j];
    if (f[j]) {
      seg_off[id] = r;
      if (seg_key) seg_key[id] = (int32_t)keys[r];
    }
    if (elem_seg) elem_seg[vals[r]] = id;
    if (r == n - 1) seg_off[id + 1] = n;
  }
}

__global__ void k_block_stats(const int32_t* __restrict__ blk_off, int M, int n,
                              uint32_t* __restrict__ lpt_key, int32_t* __restrict__ ids,
                              int32_t* __restrict__ max_rows) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= M) return;
  int rows = blk_off[b + 1] - blk_off[b];
  atomicMax(max_rows, rows);
  lpt_key[b] = (uint32_t)(n - rows);
  ids[b] = b;
}

// Longest-first block order for up to LPT_RANK_MAX blocks: block i goes to position
// #{j : size_j > size_i} + #{j < i : size_j == size_i}, which is the stable order by descending
// size, i.e. the number of keys (size_j, -j) above (size_i, -i) taken as one 64-bit integer;
// also the largest block size.  Every workgroup holds all keys in LDS (padded with -1, which
// never counts) and ranks LPT_NT blocks, two keys per LDS access.  M^2 comparisons spread over
// M / LPT_NT workgroups: about 10 us at M = 2048, where a radix sort of the keys takes about 30.
constexpr int LPT_RANK_MAX = 2048, LPT_NT = 256;
// M is read from device memory (launched before the host learns it, LPT_RANK_MAX / LPT_NT
// workgroups); with more than LPT_RANK_MAX blocks the kernel does nothing and the host sorts
// instead.
__global__ __launch_bounds__(LPT_NT) void k_lpt_rank(const int32_t* __restrict__ blk_off, const int32_t* __restrict__ Mdev,
                                                     int32_t* __restrict__ lpt, int32_t* __restrict__ max_rows) {
  __shared__ longlong2 key2[LPT_RANK_MAX / 2];
  long long* key = reinterpret_cast<long long*>(key2);
  const int M = *Mdev;
  if (M > LPT_RANK_MAX || (int)blockIdx.x * LPT_NT >= M) return;  // the whole workgroup
  const int tid = threadIdx.x;
  const int M2 = (M + 1) / 2;
  for (int j = tid; j < 2 * M2; j += LPT_NT)
    key[j] = j < M ? ((long long)(blk_off[j + 1] - blk_off[j]) << 32) | (long long)(0x7FFFFFFF - j) : -1ll;
  __syncthreads();
  const int i = blockIdx.x * LPT_NT + tid;
  if (i < M) {
    const long long ki = key[i];
    int r = 0;
    for (int j2 = 0; j2 < M2; ++j2) {
      const longlong2 v = key2[j2];
      r += v.x > ki ? 1 : 0;
      r += v.y > ki ? 1 : 0;
    }
    lpt[r] = i;
    if (r == 0) *max_rows = (int32_t)(ki >> 32);  // the longest block
  }
}

__global__ void k_cell_keys(const int32_t* __restrict__ blk_key, int M, int3 dims, int ratio,
                            bool single, int3 cdims, uint32_t* __restrict__ ckey,
                            int32_t* __restrict__ ids) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= M) return;
  uint32_t key = (uint32_t)blk_key[b];
  uint32_t bz = key % dims.z, t = key / dims.z;
  uint32_t by = t % dims.y, bx = t / dims.y;
  uint32_t c = 0;
  if (!single) {
    uint32_t cx = bx / ratio, cy = by / ratio, cz = bz / ratio;
    c = (cx * cdims.y + cy) * cdims.z + cz;
  }
  ckey[b] = c;
  ids[b] = b;
}

// Window cells equal to blocks; the block count M is read from device memory (the plan
// launches this before the host learns M), grid-stride.
__global__ void k_identity_cells(const int32_t* __restrict__ Mdev, int32_t* blk_cell, int32_t* cell_off,
                                 int32_t* cell_blk) {
  const int M = *Mdev;
  for (int b = blockIdx.x * blockDim.x + threadIdx.x; b <= M; b += gridDim.x * blockDim.x) {
    cell_off[b] = b;
    if (b < M) {
      blk_cell[b] = b;
      cell_blk[b] = b;
    }
  }
}

// Keys of the token-level window partition: kind 1 = cubic cells floor((c + shift) / w)
// (x-major cell key over cdims), kind 2 = Morton code of the voxel (bit b of x, y, z at
// bits 3b+2, 3b+1, 3b: x most significant in each triple).  Coordinates were range-checked
// by k_block_keys.
__global__ void k_window_keys(const int32_t* __restrict__ coords, int64_t n, int kind, int w, int3 shift,
                              int3 cdims, int sfc_bits, uint32_t* __restrict__ keys, int32_t* __restrict__ vals) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t x = (uint32_t)coords[3 * i], y = (uint32_t)coords[3 * i + 1], z = (uint32_t)coords[3 * i + 2];
  uint32_t key = 0;
  if (kind == 1) {
    const uint32_t cx = (x + shift.x) / w, cy = (y + shift.y) / w, cz = (z + shift.z) / w;
    key = (cx * (uint32_t)cdims.y + cy) * (uint32_t)cdims.z + cz;
  } else {
    for (int b = sfc_bits - 1; b >= 0; --b)
      key = (key << 3) | (((x >> b) & 1u) << 2) | (((y >> b) & 1u) << 1) | ((z >> b) & 1u);
  }
  keys[i] = key;
  vals[i] = (int32_t)i;
}

// Cells of a space-filling-curve window partition: runs of `per` consecutive tokens of the
// Morton order, the last one shorter; *count = number of cells.
__global__ void k_sfc_cells(int32_t* __restrict__ cell_off, int n, int per, int ncell, int32_t* __restrict__ count) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j <= ncell) cell_off[j] = (int32_t)min((int64_t)j * per, (int64_t)n);
  if (j == 0) *count = ncell;
}

}  // namespace

namespace ssa_sort {

int bits_for(uint64_t maxval) {
  int b = 0;
  while (b < 32 && (maxval >> b) != 0) ++b;
  return b;
}

// Exclusive scan of a[0..len) in place; `total` (device, may be null) receives the sum.
// `part` needs len / SCHUNK + 2 ints.
void device_scan(int32_t* a, int len, int32_t* total, int32_t* part, hipStream_t s) {
  if (len <= SCHUNK) {
    hipLaunchKernelGGL(k_scan_single, dim3(1), dim3(1024), 0, s, a, len, total);
    return;
  }
  const int chunks = (len + SCHUNK - 1) / SCHUNK;
  hipLaunchKernelGGL(k_scan_reduce, dim3(chunks), dim3(256), 0, s, a, len, part);
  hipLaunchKernelGGL(k_scan_single, dim3(1), dim3(1024), 0, s, part, chunks, total);
  hipLaunchKernelGGL(k_scan_apply, dim3(chunks), dim3(256), 0, s, a, len, part);
}

// Stable LSD radix sort of (key, val) pairs; returns which buffers hold the result.
hipError_t radix_sort(uint32_t*& ka, int32_t*& va, uint32_t*& kb, int32_t*& vb, int n, int nbits,
                      int32_t* rank, int32_t* hist, int32_t* part, hipStream_t s) {
  const int tiles = (n + RTILE - 1) / RTILE;
  for (int shift = 0; shift < nbits; shift += 8) {
    hipLaunchKernelGGL(k_radix_hist, dim3(tiles), dim3(RTILE), 0, s, ka, n, shift, rank, hist, tiles);
    device_scan(hist, tiles * 256, nullptr, part, s);
    hipLaunchKernelGGL(k_radix_scatter, dim3(tiles), dim3(RTILE), 0, s, ka, va, n, shift, rank, hist,
                       tiles, kb, vb);
    std::swap(ka, kb);
    std::swap(va, vb);
  }
  return hipGetLastError();
}

hipError_t segments(const uint32_t* keys, const int32_t* vals, int n, int32_t* tile_cnt,
                    int32_t* total, int32_t* seg_off, int32_t* seg_key, int32_t* elem_seg,
                    int32_t* part, hipStream_t s) {
  const int tiles = (n + STILE - 1) / STILE;
  hipLaunchKernelGGL(k_seg_count, dim3(tiles), dim3(256), 0, s, keys, n, tile_cnt);
  device_scan(tile_cnt, tiles, total, part, s);
  hipLaunchKernelGGL(k_seg_emit, dim3(tiles), dim3(256), 0, s, keys, vals, n, tile_cnt, seg_off,
                     seg_key, elem_seg);
  return hipGetLastError();
}

}  // namespace ssa_sort

namespace {
using namespace ssa_sort;

// Window cells that are unions of blocks: one cell covering the grid, or an edge that is a
// multiple of the block edge with no shift.
bool window_is_union(const int32_t grid[3], int B, const ssa_window_t& win, bool* single) {
  *single = false;
  if (win.kind != SSA_WINDOW_CUBE) return false;
  const int w = win.edge;
  const bool noshift = win.shift[0] == 0 && win.shift[1] == 0 && win.shift[2] == 0;
  *single = noshift && w >= grid[0] && w >= grid[1] && w >= grid[2];
  return *single || (noshift && w % B == 0);
}

// The token-level window partition: keys, a stable radix sort, cells (key runs, or runs of
// sfc_tokens tokens) and their longest-first order.  Synchronises the stream once or twice.
ssa_status build_window_partition(ssa_plan_s* p, const int32_t* coords, PlanWs& w, hipStream_t stream) {
  const int ni = (int)p->n;
  int3 cd = make_int3(1, 1, 1);
  int nbits = 0;
  uint64_t maxkey = 1;
  if (p->wkind == 1) {
    cd = make_int3((p->grid[0] + p->wshift[0] + p->window - 1) / p->window,
                   (p->grid[1] + p->wshift[1] + p->window - 1) / p->window,
                   (p->grid[2] + p->wshift[2] + p->window - 1) / p->window);
    maxkey = (uint64_t)cd.x * cd.y * cd.z;
  } else {
    const int g = std::max(p->grid[0], std::max(p->grid[1], p->grid[2]));
    nbits = bits_for((uint64_t)(g - 1));
    maxkey = (uint64_t)1 << (3 * nbits);
  }
  hipLaunchKernelGGL(k_window_keys, dim3((ni + 255) / 256), dim3(256), 0, stream, coords, p->n, p->wkind,
                     p->window, make_int3(p->wshift[0], p->wshift[1], p->wshift[2]), cd, nbits, w.key_a, w.val_a);
  uint32_t *ka = w.key_a, *kb = w.key_b;
  int32_t *va = w.val_a, *vb = w.val_b;
  if (radix_sort(ka, va, kb, vb, ni, bits_for(maxkey - 1), w.rank, w.hist, w.scan_part, stream) != hipSuccess)
    return SSA_ERR_HIP;
  if (hipMemcpyAsync(w.wperm, va, p->n * sizeof(int32_t), hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return SSA_ERR_HIP;
  if (p->wkind == 1) {
    if (segments(ka, va, ni, w.tile_cnt, w.counters + 3, w.wcell_off, nullptr, nullptr, w.scan_part, stream) !=
        hipSuccess)
      return SSA_ERR_HIP;
  } else {
    const int nc = (int)((p->n + p->sfc_tokens - 1) / p->sfc_tokens);
    hipLaunchKernelGGL(k_sfc_cells, dim3((nc + 256) / 256), dim3(256), 0, stream, w.wcell_off, ni, p->sfc_tokens,
                       nc, w.counters + 3);
  }
  hipLaunchKernelGGL(k_lpt_rank, dim3(LPT_RANK_MAX / LPT_NT), dim3(LPT_NT), 0, stream, w.wcell_off, w.counters + 3,
                     w.wlpt, w.counters + 4);
  int32_t host_cnt[8];
  if (hipMemcpyAsync(host_cnt, w.counters, sizeof(host_cnt), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return SSA_ERR_HIP;
  const int C = host_cnt[3];
  if (C > LPT_RANK_MAX) {  // longest-first cell order by a radix sort of (n - size)
    hipLaunchKernelGGL(k_block_stats, dim3((C + 255) / 256), dim3(256), 0, stream, w.wcell_off, C, ni, w.key_a,
                       w.val_a, w.counters + 4);
    ka = w.key_a; kb = w.key_b; va = w.val_a; vb = w.val_b;
    if (radix_sort(ka, va, kb, vb, C, bits_for((uint64_t)p->n), w.rank, w.hist, w.scan_part, stream) != hipSuccess)
      return SSA_ERR_HIP;
    if (hipMemcpyAsync(w.wlpt, va, C * sizeof(int32_t), hipMemcpyDeviceToDevice, stream) != hipSuccess ||
        hipMemcpyAsync(host_cnt, w.counters, sizeof(host_cnt), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      return SSA_ERR_HIP;
  }
  p->wC = C;
  p->wmax_rows = host_cnt[4];
  return SSA_OK;
}

}  // namespace

size_t plan_carve(Carver& c, int64_t n, PlanWs* w) {
  const int64_t n1 = n > 0 ? n : 1;
  const int64_t tiles = (n1 + RTILE - 1) / RTILE;
  PlanWs t;
  t.perm = c.take<int32_t>(n1);
  t.blk_off = c.take<int32_t>(n1 + 1);
  t.blk_key = c.take<int32_t>(n1);
  t.tok2blk = c.take<int32_t>(n1);
  t.blk_cell = c.take<int32_t>(n1);
  t.cell_off = c.take<int32_t>(n1 + 1);
  t.cell_blk = c.take<int32_t>(n1);
  t.lpt = c.take<int32_t>(n1);
  t.key_a = c.take<uint32_t>(n1);
  t.key_b = c.take<uint32_t>(n1);
  t.val_a = c.take<int32_t>(n1);
  t.val_b = c.take<int32_t>(n1);
  t.rank = c.take<int32_t>(n1);
  t.hist = c.take<int32_t>(tiles * 256);
  t.tile_cnt = c.take<int32_t>((n1 + STILE - 1) / STILE + 1);
  t.counters = c.take<int32_t>(8);
  t.scan_part = c.take<int32_t>(tiles * 256 / 4096 + 2);
  t.cell_key = c.take<int32_t>(n1);
  t.wperm = c.take<int32_t>(n1);
  t.wcell_off = c.take<int32_t>(n1 + 1);
  t.wlpt = c.take<int32_t>(n1);
  t.pos = c.take<int32_t>(n1);
  if (w) *w = t;
  return c.off;
}

extern "C" size_t ssa_plan_workspace_size(int64_t n, const int32_t grid[3], int32_t block,
                                          int32_t window) {
  (void)grid; (void)block; (void)window;
  if (n < 0 || n >= (int64_t)1 << 31) return 0;  // ssa_plan_create refuses n >= 2^31
  Carver c(nullptr);
  return plan_carve(c, n, nullptr) + 256;
}

extern "C" size_t ssa_plan_workspace_size_ex(int64_t n, const int32_t grid[3], int32_t block,
                                             const ssa_window_t* win) {
  (void)win;
  return ssa_plan_workspace_size(n, grid, block, 1);
}

extern "C" ssa_status ssa_plan_create(const int32_t* coords, int64_t n, const int32_t grid[3],
                                      int32_t block, int32_t window, void* ws, size_t ws_bytes,
                                      hipStream_t stream, ssa_plan* out) {
  ssa_window_t win = {SSA_WINDOW_CUBE, window, {0, 0, 0}, 0};
  return ssa_plan_create_ex(coords, n, grid, block, &win, ws, ws_bytes, stream, out);
}

extern "C" ssa_status ssa_plan_create_ex(const int32_t* coords, int64_t n, const int32_t grid[3],
                                         int32_t block, const ssa_window_t* winp, void* ws, size_t ws_bytes,
                                         hipStream_t stream, ssa_plan* out) {
  if (!out || !grid || !winp) return SSA_ERR_INVALID_ARG;
  *out = nullptr;
  const ssa_window_t win = *winp;
  if (n < 0 || block < 1) return SSA_ERR_INVALID_ARG;
  if (grid[0] < 1 || grid[1] < 1 || grid[2] < 1) return SSA_ERR_INVALID_ARG;
  if (n > 0 && !coords) return SSA_ERR_INVALID_ARG;
  if (win.kind == SSA_WINDOW_CUBE) {
    if (win.edge < 1) return SSA_ERR_INVALID_ARG;
    for (int a = 0; a < 3; ++a)
      if (win.shift[a] < 0 || win.shift[a] >= win.edge) return SSA_ERR_INVALID_ARG;
    uint64_t ncell = 1;
    for (int a = 0; a < 3; ++a) ncell *= (uint64_t)((grid[a] + win.shift[a] + win.edge - 1) / win.edge);
    if (ncell > (1ull << 31)) return SSA_ERR_UNSUPPORTED;
  } else if (win.kind == SSA_WINDOW_SFC) {
    if (win.tokens < 1) return SSA_ERR_INVALID_ARG;
    if (grid[0] > 1024 || grid[1] > 1024 || grid[2] > 1024) return SSA_ERR_UNSUPPORTED;  // 30-bit codes
  } else {
    return SSA_ERR_INVALID_ARG;
  }
  if (n >= (int64_t)1 << 31) return SSA_ERR_UNSUPPORTED;
  int32_t dims[3];
  uint64_t nblocks = 1;
  for (int a = 0; a < 3; ++a) {
    dims[a] = (grid[a] + block - 1) / block;
    nblocks *= (uint64_t)dims[a];
  }
  if (nblocks > (1ull << 31)) return SSA_ERR_UNSUPPORTED;
  bool single = false;
  const bool uni = window_is_union(grid, block, win, &single);
  const int32_t window = win.kind == SSA_WINDOW_CUBE ? win.edge : 0;
  if (!ws) return SSA_ERR_WORKSPACE;
  if (ws_bytes < ssa_plan_workspace_size(n, grid, block, 1)) return SSA_ERR_WORKSPACE;
  RoctxRange range("ssa_plan_create");

  Carver c(ws);
  c.off = (256 - (reinterpret_cast<uintptr_t>(ws) & 255)) & 255;
  PlanWs w;
  plan_carve(c, n, &w);

  ssa_plan_s* p = new ssa_plan_s();
  p->magic = SSA_PLAN_MAGIC;
  p->n = n;
  memcpy(p->grid, grid, sizeof(p->grid));
  memcpy(p->dims, dims, sizeof(p->dims));
  p->block = block;
  p->window = window;
  p->window_is_block = uni && ((window == block) || (single && nblocks == 1));
  p->wkind = uni ? 0 : (win.kind == SSA_WINDOW_CUBE ? 1 : 2);
  for (int a = 0; a < 3; ++a) p->wshift[a] = win.kind == SSA_WINDOW_CUBE ? win.shift[a] : 0;
  p->sfc_tokens = win.kind == SSA_WINDOW_SFC ? win.tokens : 0;
  p->wperm = w.wperm; p->wcell_off = w.wcell_off; p->wlpt = w.wlpt;
  p->pos = w.pos;
  p->perm = w.perm; p->blk_off = w.blk_off; p->blk_key = w.blk_key; p->tok2blk = w.tok2blk;
  p->blk_cell = w.blk_cell; p->cell_off = w.cell_off; p->cell_blk = w.cell_blk; p->lpt = w.lpt;
  p->M = 0; p->ncells = 0; p->max_rows = 0;
  if (n == 0) {
    *out = p;
    return SSA_OK;
  }
  const int ni = (int)n;
  int32_t host_cnt[8];
  auto fail = [&](ssa_status st) { delete p; return st; };
  if (hipMemsetAsync(w.counters, 0, 8 * sizeof(int32_t), stream) != hipSuccess) return fail(SSA_ERR_HIP);
  hipLaunchKernelGGL(k_block_keys, dim3((ni + 255) / 256), dim3(256), 0, stream, coords, n,
                     make_int3(grid[0], grid[1], grid[2]), block, make_int3(dims[0], dims[1], dims[2]),
                     w.key_a, w.val_a, w.counters + 7, w.pos);
  uint32_t *ka = w.key_a, *kb = w.key_b;
  int32_t *va = w.val_a, *vb = w.val_b;
  if (radix_sort(ka, va, kb, vb, ni, bits_for(nblocks - 1), w.rank, w.hist, w.scan_part, stream) != hipSuccess)
    return fail(SSA_ERR_HIP);
  if (hipMemcpyAsync(w.perm, va, n * sizeof(int32_t), hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return fail(SSA_ERR_HIP);
  if (segments(ka, va, ni, w.tile_cnt, w.counters + 0, w.blk_off, w.blk_key, w.tok2blk, w.scan_part, stream) !=
      hipSuccess)
    return fail(SSA_ERR_HIP);
  // Before the host learns M: the longest-first order by ranking (up to LPT_RANK_MAX blocks)
  // and, when cells are blocks, the identity cells, so that the usual plan needs one host
  // synchronisation.
  hipLaunchKernelGGL(k_lpt_rank, dim3(LPT_RANK_MAX / LPT_NT), dim3(LPT_NT), 0, stream, w.blk_off, w.counters + 0,
                     w.lpt, w.counters + 1);
  if (p->window_is_block)
    hipLaunchKernelGGL(k_identity_cells, dim3((unsigned)std::min<int64_t>((n + 256) / 256, 1024)), dim3(256), 0,
                       stream, w.counters + 0, w.blk_cell, w.cell_off, w.cell_blk);
  if (hipMemcpyAsync(host_cnt, w.counters, sizeof(host_cnt), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return fail(SSA_ERR_HIP);
  if (host_cnt[7]) return fail(SSA_ERR_COORD_RANGE);
  const int M = host_cnt[0];
  p->M = M;
  if (p->window_is_block && M <= LPT_RANK_MAX) {  // everything is in place
    p->max_rows = host_cnt[1];
    p->ncells = M;
    *out = p;
    return SSA_OK;
  }

  // longest-first block order (stable: ties keep ascending block id)
  if (M > LPT_RANK_MAX) {
    hipLaunchKernelGGL(k_block_stats, dim3((M + 255) / 256), dim3(256), 0, stream, w.blk_off, M, ni,
                       w.key_a, w.val_a, w.counters + 1);
    ka = w.key_a; kb = w.key_b; va = w.val_a; vb = w.val_b;
    if (radix_sort(ka, va, kb, vb, M, bits_for((uint64_t)n), w.rank, w.hist, w.scan_part, stream) != hipSuccess)
      return fail(SSA_ERR_HIP);
    if (hipMemcpyAsync(w.lpt, va, M * sizeof(int32_t), hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return fail(SSA_ERR_HIP);
  }

  // window cells as groups of blocks (identity cells were written above)
  if (!p->window_is_block && p->wkind == 0) {
    const int ratio = single ? 1 : window / block;
    int3 cd = make_int3(1, 1, 1);
    if (!single)
      cd = make_int3((dims[0] + ratio - 1) / ratio, (dims[1] + ratio - 1) / ratio,
                     (dims[2] + ratio - 1) / ratio);
    uint64_t ncmax = (uint64_t)cd.x * cd.y * cd.z;
    hipLaunchKernelGGL(k_cell_keys, dim3((M + 255) / 256), dim3(256), 0, stream, w.blk_key, M,
                       make_int3(dims[0], dims[1], dims[2]), ratio, single, cd, w.key_a, w.val_a);
    ka = w.key_a; kb = w.key_b; va = w.val_a; vb = w.val_b;
    if (radix_sort(ka, va, kb, vb, M, bits_for(ncmax - 1), w.rank, w.hist, w.scan_part, stream) != hipSuccess)
      return fail(SSA_ERR_HIP);
    if (hipMemcpyAsync(w.cell_blk, va, M * sizeof(int32_t), hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return fail(SSA_ERR_HIP);
    if (segments(ka, va, M, w.tile_cnt, w.counters + 2, w.cell_off, nullptr, w.blk_cell, w.scan_part, stream) !=
        hipSuccess)
      return fail(SSA_ERR_HIP);
  }
  if (hipMemcpyAsync(host_cnt, w.counters, sizeof(host_cnt), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return fail(SSA_ERR_HIP);
  p->max_rows = host_cnt[1];
  p->ncells = p->wkind != 0 ? 0 : (p->window_is_block ? M : host_cnt[2]);
  if (p->wkind != 0) {
    const ssa_status st = build_window_partition(p, coords, w, stream);
    if (st != SSA_OK) return fail(st);
  }
  *out = p;
  return SSA_OK;
}

extern "C" ssa_status ssa_plan_get_info(ssa_plan p, ssa_plan_info_t* info) {
  if (!p || p->magic != SSA_PLAN_MAGIC) return SSA_ERR_BAD_PLAN;
  if (!info) return SSA_ERR_INVALID_ARG;
  info->n = p->n;
  info->num_blocks = p->M;
  info->num_cells = p->ncells;
  info->block = p->block;
  info->window = p->window;
  info->max_block_rows = p->max_rows;
  info->perm = p->perm;
  info->blk_off = p->blk_off;
  info->blk_key = p->blk_key;
  info->tok2blk = p->tok2blk;
  info->blk_cell = p->blk_cell;
  info->cell_off = p->cell_off;
  info->cell_blk = p->cell_blk;
  info->lpt = p->lpt;
  info->window_kind = p->wkind == 2 ? SSA_WINDOW_SFC : SSA_WINDOW_CUBE;
  for (int a = 0; a < 3; ++a) info->window_shift[a] = p->wshift[a];
  info->window_tokens = p->sfc_tokens;
  info->cells_are_block_unions = p->wkind == 0;
  info->num_wcells = p->wkind != 0 ? p->wC : 0;
  info->max_wcell_rows = p->wkind != 0 ? p->wmax_rows : 0;
  info->wperm = p->wkind != 0 ? p->wperm : nullptr;
  info->wcell_off = p->wkind != 0 ? p->wcell_off : nullptr;
  info->wlpt = p->wkind != 0 ? p->wlpt : nullptr;
  return SSA_OK;
}

extern "C" void ssa_plan_destroy(ssa_plan p) {
  if (p && p->magic == SSA_PLAN_MAGIC) {
    p->magic = 0;
    delete p;
  }
}
