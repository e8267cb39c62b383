// SSA forward kernels for gfx950: pooled keys/values, the compressed branch with
// block selection, and the selected + window branches with the gated combine.
//
// Method (Direct3D-S2 pages: nav.superapi.store "Technical principles of
// Direct3D-S2"; pixal-3d.com "What is Direct3D-S2?"): a compression module pools
// each block to one token and attends to all of them; its attention scores pick
// the important blocks for fine attention; a local window module attends to the
// query's neighbourhood; predicted gates aggregate the three outputs.
//
// Scores come from 32x32 MFMA tiles; each wave owns 32 query rows.  Key and value
// tiles (32 keys) are copied straight from HBM into LDS (global_load_lds), double
// buffered: the next tile's copy is issued before the current tile's math.  The PV
// product is O^T += V^T P^T: P^T comes straight from the score registers and V^T from
// LDS transpose reads of the row-major value tile.
//
// The compressed branch runs twice over the pooled keys:
//   pass 1 (k_compress, over fixed chunks of the token order) computes
//          S^T = Ktil Q^T (a lane holds one query, 16 keys), keeps an online
//          softmax, accumulates O^T, and yields o_c and the exact log-sum-exp;
//   pass 2 (k_select, per query block) computes S = Q Ktil^T (a lane holds one
//          key, 16 queries), so the importance column sums over the block's
//          queries are register sums.
// The pooled keys are fp32; they enter the MFMA as two (f16) or three (bf16) dtype
// planes whose sum reproduces the fp32 value, so the scores that decide the top-k
// carry fp32-level error.
#include <hip/hip_runtime.h>
#include <algorithm>
#include <type_traits>
#include "ssa_internal.h"
#include "ssa_mfma.h"
#include "ssa_tiles.h"

namespace {

using namespace ssa_dev;
constexpr int CMP_WAVES = 8;      // compressed pass 1: waves per workgroup, 32 query rows each
constexpr int SEL_WAVES = 8;      // importance pass: waves per workgroup (256 rows per sweep)
constexpr int ATT_WAVES = 4;      // selected/window: waves per workgroup, 32 query rows each
constexpr int ATT_ROWS = 32 * ATT_WAVES;
// k_attend modes: both branches of the block partition (window cells are unions of blocks);
// the window branch alone over a token-level window partition (its output to a buffer);
// the selected branch alone, combined with that buffer.
enum { ATT_BOTH = 0, ATT_WINDOW = 1, ATT_SELECTED = 2 };

// ------------------------------------------------------------------ pooling
// One workgroup per (block, group of hg heads), blocks longest first: ktil[h,b] =
// mean_{i in b} K[i,h] @ Wk, vtil likewise.  Each token row of the block is read whole for the
// group's heads (hg * D contiguous elements of K and of V): thread t owns the 16-byte columns
// t, t + POOL_NT, ... of the [K | V] row pair, so a column sum needs no exchange, and POOL_U
// rows are in flight per thread.  The means go to LDS and are projected by Wk, Wv with fp32
// dot products.  Writes the fp32 pooled key split into NSPLIT dtype planes and the pooled
// value (transposed) in the per-(head, 64-block tile) stage layout, plus the row-major pooled
// value; padding blocks (b >= M) and row padding are zero.
constexpr int POOL_NT = 512, POOL_CPT = 2, POOL_U = 16;

template <int DT, int D>
__global__ __launch_bounds__(POOL_NT) void k_pool(
    const typename Tr<DT>::T* __restrict__ kin, const typename Tr<DT>::T* __restrict__ vin,
    const typename Tr<DT>::T* __restrict__ wk, const typename Tr<DT>::T* __restrict__ wv,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ blk_off,
    const int32_t* __restrict__ lpt, int M, int Mp, int H, int hg,
    typename Tr<DT>::T* __restrict__ pooled, typename Tr<DT>::T* __restrict__ pooled_v) {
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  constexpr int NS = C::NS, EPC = C::EPC;
  extern __shared__ float bar[];  // [2][hg * D]: K means, then V means
  const int nhg = (H + hg - 1) / hg;
  const int unit = blockIdx.x / nhg, h0 = (blockIdx.x % nhg) * hg;
  const int hn = min(hg, H - h0);
  const int tid = threadIdx.x;
  const int b = unit < M ? lpt[unit] : unit;  // padding blocks M..Mp-1 follow the real ones
  auto stage_of = [&](int h) { return pooled + ((int64_t)h * (Mp / C::PT) + b / C::PT) * C::STAGE; };
  if (b >= M) {  // zero padding block
    for (int j = tid; j < hn * D; j += POOL_NT) {
      const int h = h0 + j / D, c = j % D;
      T* stg = stage_of(h);
      for (int s = 0; s < NS; ++s) stg[s * C::KPLANE + (b % C::PT) * C::KROW + c] = (T)0.f;
      stg[NS * C::KPLANE + c * C::VTROW + (b % C::PT)] = (T)0.f;
      pooled_v[((int64_t)h * Mp + b) * C::VROW + c] = (T)0.f;
    }
    for (int j = tid; j < hn * (C::KROW - D); j += POOL_NT) {
      const int h = h0 + j / (C::KROW - D), c = D + j % (C::KROW - D);
      for (int s = 0; s < NS; ++s) stage_of(h)[s * C::KPLANE + (b % C::PT) * C::KROW + c] = (T)0.f;
    }
    return;
  }
  const int r0 = blk_off[b], r1 = blk_off[b + 1];
  const int cols = hn * D / EPC;  // 16-byte columns per tensor
  float acc[POOL_CPT][EPC];
  int col[POOL_CPT];
#pragma unroll
  for (int m = 0; m < POOL_CPT; ++m) {
    col[m] = tid + m * POOL_NT;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[m][e] = 0.f;
  }
  const int64_t rowlen = (int64_t)H * D;
  for (int r = r0; r < r1; r += POOL_U) {
    uint4 buf[POOL_U][POOL_CPT];
#pragma unroll
    for (int u = 0; u < POOL_U; ++u) {
      const int rr = r + u < r1 ? r + u : r;  // past the block: reload row r, not summed
      const int64_t base = (int64_t)perm[rr] * rowlen + (int64_t)h0 * D;
#pragma unroll
      for (int m = 0; m < POOL_CPT; ++m) {
        const bool on = col[m] < 2 * cols;
        const int cc = col[m] < cols ? col[m] : (on ? col[m] - cols : 0);  // K columns, then V
        const T* src = (col[m] < cols ? kin : vin) + base + (int64_t)cc * EPC;
        buf[u][m] = on ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < POOL_U; ++u) {
      if (r + u < r1) {
#pragma unroll
        for (int m = 0; m < POOL_CPT; ++m) {
          const T* x = reinterpret_cast<const T*>(&buf[u][m]);
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[m][e] += Tr<DT>::up(x[e]);
        }
      }
    }
  }
  const float inv = 1.f / (float)(r1 - r0);
#pragma unroll
  for (int m = 0; m < POOL_CPT; ++m)
    if (col[m] < 2 * cols) {
      const int kv = col[m] < cols ? 0 : 1, cc = kv ? col[m] - cols : col[m];
#pragma unroll
      for (int e = 0; e < EPC; ++e) bar[kv * hn * D + cc * EPC + e] = acc[m][e] * inv;
    }
  __syncthreads();
  for (int j = tid; j < 2 * hn * D; j += POOL_NT) {
    const int kv = j / (hn * D), hh = (j % (hn * D)) / D, c = j % D;
    const T* W = kv ? wv : wk;
    const float* xb = bar + kv * hn * D + hh * D;
    float s0 = 0.f, s1 = 0.f;
#pragma unroll 8
    for (int i = 0; i < D; i += 2) {
      s0 += xb[i] * Tr<DT>::up(W[i * D + c]);
      s1 += xb[i + 1] * Tr<DT>::up(W[(i + 1) * D + c]);
    }
    const float val = s0 + s1;
    const int h = h0 + hh;
    T* stg = stage_of(h);
    if (kv == 0) {
      float rem = val;
      for (int s = 0; s < NS; ++s) {
        const T part = Tr<DT>::cvt(rem);
        stg[s * C::KPLANE + (b % C::PT) * C::KROW + c] = part;
        rem -= Tr<DT>::up(part);
      }
      if (c < C::KROW - D)
        for (int s = 0; s < NS; ++s) stg[s * C::KPLANE + (b % C::PT) * C::KROW + D + c] = (T)0.f;
    } else {
      const T v = Tr<DT>::cvt(val);
      stg[NS * C::KPLANE + c * C::VTROW + (b % C::PT)] = v;
      pooled_v[((int64_t)h * Mp + b) * C::VROW + c] = v;
    }
  }
}

// ------------------------------------------------------------------ compressed + select
// Scores of one wave's 32 query rows against the 64 pooled keys of a stage, as two 32-key
// halves a0 (keys 0..31) and a1 (keys 32..63), summed over the NSPLIT key planes.
// KQ: S^T layout (lane = query; pooled keys are the A operand), else S layout (lane = key).
// krow: this lane's row of key plane 0 (row lane%32, column offset (lane/32)*KPL).
// The fragment reads run PF steps ahead of the MFMAs that use them.  With vtt != nullptr the
// transposed value fragments of both halves (for O^T += V^T P^T) are read into vt behind the
// key fragments, so that they arrive while the softmax runs.
template <int DT, int D, bool KQ, bool VPRE>
__device__ inline void stage_scores(const typename Tr<DT>::T* krow, const typename Tr<DT>::frag* qf,
                                    ssa_f16v& a0, ssa_f16v& a1, const typename Tr<DT>::T* vtt,
                                    typename Tr<DT>::frag (*vt)[Cfg<DT, D>::PK][Cfg<DT, D>::NDV],
                                    int lane) {
  using C = Cfg<DT, D>;
  using F = typename Tr<DT>::frag;
  constexpr int NST = C::NS * C::NKS, PF = 3;
  F f0[NST], f1[NST];
#pragma unroll
  for (int i = 0; i < NST; ++i) {
    const int s = i / C::NKS, ks = i % C::NKS;
    f0[i] = load_frag<DT>(krow + s * C::KPLANE + ks * C::KS);
    f1[i] = load_frag<DT>(krow + s * C::KPLANE + 32 * C::KROW + ks * C::KS);
  }
  a0 = zero16();
  a1 = zero16();
#pragma unroll
  for (int i = 0; i < NST; ++i) {
    const int ks = i % C::NKS;
    if constexpr (KQ) {
      a0 = Tr<DT>::mma(f0[i], qf[ks], a0);
      a1 = Tr<DT>::mma(f1[i], qf[ks], a1);
    } else {
      a0 = Tr<DT>::mma(qf[ks], f0[i], a0);
      a1 = Tr<DT>::mma(qf[ks], f1[i], a1);
    }
  }
  if constexpr (VPRE) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ks = 0; ks < C::PK; ++ks)
#pragma unroll
        for (int j = 0; j < C::NDV; ++j) vt[h][ks][j] = vtt_frag<DT, D>(vtt, 32 * h, ks, j, lane);
  }
  // schedule (16-bit types): PF steps of key reads, then per step two MFMAs and the reads PF
  // steps ahead.  fp32 (one register per fragment, 2x the steps) is left to the compiler.
  if constexpr (sizeof(typename Tr<DT>::T) == 2) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (i + PF < NST) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  }
}

// Stores 4 consecutive floats as the element type (one 8- or 16-byte store).
template <typename T>
__device__ inline void store4(T* p, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  } else {
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    const T v[4] = {(T)a, (T)b, (T)c, (T)d};
    *reinterpret_cast<u2*>(p) = __builtin_bit_cast(u2, v);
  }
}

// Loads 4 consecutive elements as floats (one 8- or 16-byte load).
template <typename T>
__device__ inline void load4(const T* p, float* v) {
  if constexpr (sizeof(T) == 4) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else {
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    struct V4 { T e[4]; };
    const V4 x = __builtin_bit_cast(V4, *reinterpret_cast<const u2*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (float)x.e[i];
  }
}

// Top keff = min(topk, M) entries of sig[0..M) (in LDS, zero from M up to the next multiple of
// four; ties to the lower id) by one wave, written in ascending id order to out[0..keff),
// out[keff..topk) = -1.  sig >= 0, so the fp32 bit patterns order like the values.
// Usual case (keff <= 64): the keff-th largest of the 64 lane maxima is a lower bound lb of the
// keff-th largest entry (keff lanes hold an entry at or above it), so every entry that can be
// chosen is at least lb; those entries are compacted in id order into the wave's candidate
// buffer cbuf (64 patterns, then 64 ids) and, when there are at most 64, the exact threshold
// and the placement are found among them, one candidate per lane: two passes over the row in
// all.  Otherwise (more candidates, keff > 64, lb = 0) the keff-th largest pattern T is found
// bit by bit from the top over the whole row, each step counting the entries at or above the
// candidate (four 16-byte LDS reads in flight per lane, then across the wave; the zeros never
// count), and a scan in id order places every entry above T and the first entries equal to T.
// The rows of a workgroup's blocks are taken one per wave.
__device__ void topk_wave(const float* sig, int M, int topk, int32_t* __restrict__ out, int lane,
                          uint32_t* cbuf) {
  const int keff = min(topk, M);
  const bool all = keff == M;
  const uint32_t* u32 = reinterpret_cast<const uint32_t*>(sig);
  const uint4* u4 = reinterpret_cast<const uint4*>(sig);  // rows start 16-byte aligned
  const int NQ = (M + 3) / 4;
  auto wave_rank = [&](uint64_t m) {  // set bits of m below this lane
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  };
  if (!all && keff <= 64) {
    uint32_t lmax = 0;
    for (int q = lane; q < NQ; q += 256) {
      uint4 v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = q + 64 * t < NQ ? u4[q + 64 * t] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int t = 0; t < 4; ++t) lmax = max(lmax, max(max(v[t].x, v[t].y), max(v[t].z, v[t].w)));
    }
    uint32_t lb = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = lb | (1u << bit);
      if (__builtin_popcountll(__builtin_amdgcn_ballot_w64(lmax >= cand)) >= keff) lb = cand;
    }
    if (lb > 0) {
      int nc = 0;
      for (int base = 0; base < M; base += 256) {
        uint32_t v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = base + 64 * t + lane < M ? u32[base + 64 * t + lane] : 0u;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bool in = v[t] >= lb;  // the zeros past M never reach lb >= 1
          const uint64_t bm = __builtin_amdgcn_ballot_w64(in);
          const int pos = nc + wave_rank(bm);
          if (in && pos < 64) {
            cbuf[pos] = v[t];
            cbuf[64 + pos] = (uint32_t)(base + 64 * t + lane);
          }
          nc += __builtin_popcountll(bm);
        }
      }
      if (nc <= 64) {
        // LDS operations of a wave complete in order: the candidates are in place once the
        // writes above have been issued and the compiler keeps the reads behind them
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const uint32_t cu = lane < nc ? cbuf[lane] : 0u;  // ids ascend with the lane
        const int cj = lane < nc ? (int)cbuf[64 + lane] : 0;
        // the search over the candidates alone finds the row's threshold: every entry at or
        // above a trial value that does not exceed it is a candidate
        uint32_t T = 0;
        for (int bit = 31; bit >= 0; --bit) {
          const uint32_t cand = T | (1u << bit);
          if (__builtin_popcountll(__builtin_amdgcn_ballot_w64(cu >= cand)) >= keff) T = cand;
        }
        const uint64_t bg = __builtin_amdgcn_ballot_w64(cu > T), be = __builtin_amdgcn_ballot_w64(lane < nc && cu == T);
        const int need = keff - __builtin_popcountll(bg);
        const int lg = wave_rank(bg), le = wave_rank(be);
        if (cu > T || (lane < nc && cu == T && le < need)) out[lg + min(le, need)] = cj;
        for (int t = keff + lane; t < topk; t += 64) out[t] = -1;
        return;
      }
    }
  }
  auto count_ge = [&](uint32_t cand) {  // entries with pattern >= cand (cand >= 1), wave total
    int cnt = 0;
    for (int q = lane; q < NQ; q += 256) {
      uint4 v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = q + 64 * t < NQ ? u4[q + 64 * t] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        cnt += (v[t].x >= cand ? 1 : 0) + (v[t].y >= cand ? 1 : 0) + (v[t].z >= cand ? 1 : 0) + (v[t].w >= cand ? 1 : 0);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    return cnt;
  };
  uint32_t T = 0;
  int need = keff;
  if (!all) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      if (count_ge(cand) >= keff) T = cand;
    }
    need = keff - count_ge(T + 1u);  // ties at T to take, lowest ids first
  }
  int run_gt = 0, run_eq = 0;
  for (int base = 0; base < M; base += 64) {
    const int j = base + lane;
    const uint32_t u = j < M ? u32[j] : 0u;
    const bool gt = j < M && (all || u > T);
    const bool eq = j < M && !all && u == T;
    const uint64_t bg = __builtin_amdgcn_ballot_w64(gt), be = __builtin_amdgcn_ballot_w64(eq);
    const int lg = run_gt + wave_rank(bg), le = run_eq + wave_rank(be);
    if (gt || (eq && le < need)) out[lg + min(le, need)] = j;
    run_gt += __builtin_popcountll(bg);
    run_eq += __builtin_popcountll(be);
  }
  for (int t = keff + lane; t < topk; t += 64) out[t] = -1;
}

// Compressed branch, pass 1 (query-stationary).  Every query attends to all pooled blocks of
// its head, so this pass needs no block structure: the block-sorted token order is cut into
// chunks of 32 * CMP_WAVES rows (units (head, chunk), head-major), and every wave but the
// last of a head owns a full tile of 32 query rows.  The grid is resident: the units of XCD x
// are the contiguous range [x per, (x + 1) per), so an XCD's L2 holds the pooled stages of the
// few heads it works on, and its wpx workgroups take them in turn.  A workgroup's units form
// one stream of pooled stages (ntv per unit) through a ring of NB LDS buffers, copies issued
// NB - 1 steps ahead across unit bounds; the queries of the next unit are loaded during the
// last step of the current one.  Each wave keeps an online softmax and writes its rows' o_c
// and exact lse.
template <int DT, int D>
constexpr int cmp_depth() {
  constexpr int bytes = (Cfg<DT, D>::STAGE * (int)sizeof(typename Tr<DT>::T) + 1023) / 1024 * 1024;
  return LDS_BYTES / bytes >= 4 ? 4 : LDS_BYTES / bytes;
}

template <int DT, int D>
__global__ __launch_bounds__(64 * CMP_WAVES) void k_compress(
    const typename Tr<DT>::T* __restrict__ q, const typename Tr<DT>::T* __restrict__ pooled,
    const int32_t* __restrict__ perm, int M, int Mp, int H, int64_t N, int nch, int per, int wpx,
    float sl2, typename Tr<DT>::T* __restrict__ oc, float* __restrict__ lsec,
    float* __restrict__ oc_save) {
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  using F = typename Tr<DT>::frag;
  constexpr int NS = C::NS;
  constexpr int ROWS = 32 * CMP_WAVES;
  constexpr int NB = cmp_depth<DT, D>();
  static_assert(NB >= 2, "two pooled stages fit LDS");
  constexpr int NCH1 = C::STAGE * sizeof(T) / 16;                // 16-byte chunks of a stage
  constexpr int NI = ((NCH1 + 63) / 64 + CMP_WAVES - 1) / CMP_WAVES;  // copy instructions per wave
  SSA_STAGE_BUFFERS(T, C::STAGE, NB);

  const int x = blockIdx.x % 8, j = blockIdx.x / 8;
  const int U = H * nch;
  const int cx = max(0, min(U, (x + 1) * per) - x * per);  // units of this XCD
  const int nmine = j < cx ? (cx - j + wpx - 1) / wpx : 0;
  const int ntv = (M + C::PT - 1) / C::PT;  // stages holding real blocks
  const int nsteps = nmine * ntv;
  if (nsteps == 0) return;  // the whole workgroup
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntile = Mp / C::PT;
  auto unit_of = [&](int m) __attribute__((always_inline)) { return x * per + j + m * wpx; };
  auto tile_row = [&](int m) __attribute__((always_inline)) {  // first row of this wave's tile
    return (int64_t)(unit_of(m) % nch) * ROWS + wave * 32;
  };
  auto perm_of = [&](int m) __attribute__((always_inline)) {  // token of this lane's row, or -1
    const int64_t r = tile_row(m) + c;
    return r < N ? perm[r] : -1;
  };
  auto load_unit_q = [&](F* dst, int m, int tok) __attribute__((always_inline)) {
    load_q<DT, D>(dst, q + ((int64_t)(tok >= 0 ? tok : 0) * H + unit_of(m) / nch) * D, tok >= 0, lane);
  };

  // the next unit's queries are prefetched where the registers allow it
  constexpr bool QPRE = D <= 96;
  F qf[C::NKS], qn[QPRE ? C::NKS : 1];
  bool qn_ok = false;
  // prefetch: the loads always run (row 0 for a missing row) and the mask applies at the copy,
  // so that nothing writes the registers while their loads are in flight
  auto prefetch_q = [&](int m, int tok) __attribute__((always_inline)) {
    qn_ok = tok >= 0;
    const T* qrow = q + ((int64_t)(tok >= 0 ? tok : 0) * H + unit_of(m) / nch) * D + (lane >> 5) * C::KPL;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) qn[ks] = load_frag<DT>(qrow + ks * C::KS);
  };
  if constexpr (QPRE) prefetch_q(0, perm_of(0));
  // the next unit's tokens come by a copy into LDS (lanes 0-7 of a wave, 16 bytes each), so
  // that no register load has to be waited for inside the stream; rows past N read padding
  // inside the token array's 256-byte slot and are not used
  __shared__ int32_t ptok[CMP_WAVES][32];
  const __amdgpu_buffer_rsrc_t rperm =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(perm), 0, (int)((N + 3) / 4 * 16), 0x00020000);
  Online<C::NDV> st;
  const T* src = nullptr;
  auto fetch = [&](int s) __attribute__((always_inline)) {
    src = pooled + ((int64_t)(unit_of(s / ntv) / nch) * ntile + s % ntv) * C::STAGE;
  };
  auto issue = [&](T* dst) __attribute__((always_inline)) { dma_stage<CMP_WAVES, NI>(dst, src, NCH1, wave, lane); };
  // unit mu's compressed output and lse (the online state still holds it)
  auto flush = [&](int mu) __attribute__((always_inline)) {
    const int64_t row0 = tile_row(mu);
    if (row0 < N) {
      const float ltot = xor32_sum(st.l);
      const int64_t my_row = row0 + c;
      if (my_row < N) {
        const int h = unit_of(mu) / nch;
        const float inv = 1.f / ltot;
        T* orow = oc + (my_row * H + h) * D;
        float* srow = oc_save ? oc_save + (my_row * H + h) * D : nullptr;
        if (g == 0) lsec[(int64_t)h * N + my_row] = st.m + fast_log2(ltot);
#pragma unroll
        for (int jj = 0; jj < C::NDV; ++jj)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const int col = 32 * jj + 8 * rq + 4 * g;
            const float v0 = st.o[jj][4 * rq] * inv, v1 = st.o[jj][4 * rq + 1] * inv;
            const float v2 = st.o[jj][4 * rq + 2] * inv, v3 = st.o[jj][4 * rq + 3] * inv;
            store4(orow + col, v0, v1, v2, v3);
            if (srow) store4(srow + col, v0, v1, v2, v3);
          }
      }
    }
  };
  // The stream of steps: stage s lands in buffer s % NB; its copy is issued NB - 1 steps
  // ahead.  Vector memory operations complete in issue order, so before step s a wave waits
  // until only what it issued after stage s's copy is outstanding: the later stages' copies
  // and, from the steps in between that began a unit, that unit's predecessor's output
  // stores (E of them at least).  The stores thus never hold up a step; the copies issued
  // after them land NB - 1 steps later, when the stores are long done.  A step stores the
  // previous unit's outputs at a unit's first step, runs the scores' MFMAs, then issues its
  // copy (which overlaps the MFMAs), the softmax and P.V.
  constexpr int E = C::NDV * 4;  // output stores of a flush
  auto flushed_at = [&](int s2) __attribute__((always_inline)) {
    if (s2 < 0) return false;
    const int m2 = s2 / ntv;
    return s2 == m2 * ntv && m2 > 0 && tile_row(m2 - 1) < N;
  };
#pragma unroll
  for (int u = 0; u < NB - 1; ++u)
    if (u < nsteps) {
      fetch(u);
      issue(bufs[u]);
    }
  if (NB - 1 < nsteps) fetch(NB - 1);
  for (int s0 = 0; s0 < nsteps; s0 += NB) {
    static_for<0, NB>([&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      const int s = s0 + u;
      if (s >= nsteps) return;
      int nf = 0;
#pragma unroll
      for (int j = 1; j <= NB - 2; ++j) nf += flushed_at(s - j) ? 1 : 0;
      vm_wait_kn<NI, E, (NB > 2 ? NB - 2 : 0)>(min(NB - 2, nsteps - 1 - s), nf);
      lds_barrier();
      T* cur = bufs[u];
      auto next = [&]() __attribute__((always_inline)) {
        if (s + NB - 1 < nsteps) issue(bufs[(u + NB - 1) % NB]);
        if (s + NB < nsteps) fetch(s + NB);
      };
      const int m = s / ntv, t = s - m * ntv;
      // next unit's queries: its tokens at step 0, its rows two steps before the end, so that
      // the copies in flight need not drain to use them
      if (t == 0) {
        if constexpr (QPRE) {
#pragma unroll
          for (int ks = 0; ks < C::NKS; ++ks) qf[ks] = qn_ok ? qn[ks] : zero_frag<DT>();
        } else {
          load_unit_q(qf, m, perm_of(m));
        }
        if constexpr (QPRE)
          if (m + 1 < nmine && lane < 8)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rperm, (lds_void_t*)&ptok[wave][0], 16,
                                                     (uint32_t)((tile_row(m + 1) + 4 * lane) * 4), 0, 0, 0);
        if (m > 0) flush(m - 1);
        st.init();
      }
      // the next unit's rows, once the token copy is covered by the stage waits (NB - 1 steps
      // on; a unit shorter than that waits for it)
      if constexpr (QPRE) {
        const int tq = min(NB - 1, ntv - 1);
        if (t == tq && m + 1 < nmine) {
          if (tq < NB - 1) vm_wait<0>();
          const int64_t r = tile_row(m + 1) + c;
          prefetch_q(m + 1, r < N ? ptok[wave][c] : -1);
        }
      }
      if (tile_row(m) < N) {
        ssa_f16v a0, a1;
        // value fragments read ahead for 16-bit types (fp32 ones would take 2*D registers)
        constexpr bool VPRE = sizeof(T) == 2;
        const T* vtt = cur + NS * C::KPLANE;
        F vt[2][C::PK][C::NDV];
        stage_scores<DT, D, true, VPRE>(cur + (lane & 31) * C::KROW + (lane >> 5) * C::KPL, qf, a0, a1,
                                        vtt, vt, lane);
        next();
        if ((t + 1) * C::PT > M) {  // padding blocks
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if (t * C::PT + res_row(r, g) >= M) a0[r] = -INFINITY;
            if (t * C::PT + 32 + res_row(r, g) >= M) a1[r] = -INFINITY;
          }
        }
        st.update2(a0, a1, sl2);
#pragma unroll
        for (int ks = 0; ks < C::PK; ++ks) {
          const F p0 = p_frag<DT>(a0, ks), p1f = p_frag<DT>(a1, ks);
#pragma unroll
          for (int jj = 0; jj < C::NDV; ++jj) {
            if constexpr (VPRE) {
              st.o[jj] = Tr<DT>::mma(vt[0][ks][jj], p0, st.o[jj]);
              st.o[jj] = Tr<DT>::mma(vt[1][ks][jj], p1f, st.o[jj]);
            } else {
              st.o[jj] = Tr<DT>::mma(vtt_frag<DT, D>(vtt, 0, ks, jj, lane), p0, st.o[jj]);
              st.o[jj] = Tr<DT>::mma(vtt_frag<DT, D>(vtt, 32, ks, jj, lane), p1f, st.o[jj]);
            }
          }
        }
      } else {
        next();
      }
    });
  }
  flush(nmine - 1);
}

// Compressed branch, pass 2 (key-stationary) and the top-k.  One workgroup per (group of G
// consecutive query blocks in longest-first order, head): with small blocks several blocks
// share each pooled key tile the workgroup loads (G = 1 for blocks of a few hundred rows).
// The group's 32-row query tiles (a tile never mixes blocks) are taken SEL_WAVES at a time
// (a sweep): their queries and pass-1 lse go to LDS; the (32-key tile, query tile) pairs,
// key-tile major, are split into equal contiguous ranges, one per wave, so a wave keeps a key
// tile's fragments in registers while it walks query tiles, and column-sums the
// probabilities into the importance row of the tile's block (one row per member in LDS).  A
// (key tile, block) segment that lies in one wave's range goes straight into the row; the
// pieces of segments cut by range ends are added in wave order, so every sum is in a fixed
// order.
constexpr int SEL_GMAX = 8;  // blocks per workgroup at most
template <int DT, int D, bool GRP>
__global__ __launch_bounds__(64 * SEL_WAVES) void k_select(
    const typename Tr<DT>::T* __restrict__ q, const typename Tr<DT>::T* __restrict__ pooled,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ blk_off,
    const int32_t* __restrict__ lpt, int M, int Mp, int H, int64_t N, float sl2, int topk, int G,
    const float* __restrict__ lsec, int32_t* __restrict__ sel, float* __restrict__ sigma_out) {
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  using F = typename Tr<DT>::frag;
  // the sweep's queries, one 32-row tile per wave: row stride QROW
  constexpr int QROW = sizeof(T) == 2 ? D + 8 : D;
  __shared__ __attribute__((aligned(1024))) T qlds[SEL_WAVES * 32 * QROW];
  __shared__ float lse_lds[SEL_WAVES * 32];
  __shared__ float bpart[SEL_WAVES][2][32];  // column sums of a range's first / last segment
  __shared__ int32_t bkt[SEL_WAVES][2];      // their key tile * SEL_GMAX + member, -1 none
  __shared__ int32_t mb[SEL_GMAX], mr0[SEL_GMAX], mrows[SEL_GMAX], mtp[SEL_GMAX + 1];
  extern __shared__ __attribute__((aligned(16))) float sig[];  // [G][Mp]

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // items (head, group) head-major, in one contiguous range per XCD (workgroup i runs on XCD
  // i % 8): the workgroups on an XCD at any time mostly share a head, whose pooled keys every
  // one of them streams, so those stay in that XCD's L2
  const int ngrp = (M + G - 1) / G;
  const int per = (ngrp * H + NXCD - 1) / NXCD;
  const int item = (int)(blockIdx.x % NXCD) * per + (int)(blockIdx.x / NXCD);
  if (item >= ngrp * H) return;  // the whole workgroup
  const int h = item / ngrp;
  const int gi = item % ngrp;
  const int G0 = gi * G, Gk = min(G, M - G0);  // members
  if (tid < 64) {  // member k in lane k (loads side by side), first tiles by a scan over the lanes
    int bb = 0, r0m = 0, rows = 0;
    if (tid < Gk) {
      bb = lpt[G0 + tid];
      r0m = blk_off[bb];
      rows = blk_off[bb + 1] - r0m;
    }
    const int nt = (rows + 31) / 32;
    int incl = nt;
#pragma unroll
    for (int off = 1; off < SEL_GMAX; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (tid >= off) incl += o;
    }
    if (tid < Gk) {
      mb[tid] = bb;
      mr0[tid] = r0m;
      mrows[tid] = rows;
      mtp[tid] = incl - nt;
    }
    if (tid == Gk - 1) mtp[Gk] = incl;
  }
  const int ntile = Mp / C::PT;
  const int nkt = (M + KT - 1) / KT;  // 32-key tiles holding real blocks
  const T* pstage = pooled + (int64_t)h * ntile * C::STAGE;
  for (int j = tid; j < Gk * Mp; j += 64 * SEL_WAVES) sig[j] = 0.f;
  __syncthreads();
  const int T_all = mtp[Gk];
  auto member_of = [&](int ti) __attribute__((always_inline)) {  // block of group tile ti
    int k = 0;
    if constexpr (GRP)
      while (k + 1 < Gk && mtp[k + 1] <= ti) ++k;
    return k;
  };

  for (int ts = 0; ts < T_all; ts += SEL_WAVES) {
    const int nq = min(SEL_WAVES, T_all - ts);  // query tiles of this sweep
    {  // this wave's query tile to LDS (zero past its block), lse beside it
      const int ti = ts + wave;
      int tok = -1;
      float lse = INFINITY;  // rows past a block get +inf: their probabilities are exactly zero
      if (ti < T_all) {
        const int k = member_of(ti);
        const int row = (ti - mtp[k]) * 32 + c;
        if (row < mrows[k]) {
          tok = perm[mr0[k] + row];
          lse = lsec[(int64_t)h * N + mr0[k] + row];
        }
      }
      F qf[C::NKS];
      load_q<DT, D>(qf, q + ((int64_t)(tok >= 0 ? tok : 0) * H + h) * D, tok >= 0, lane);
      T* qrow = qlds + (wave * 32 + c) * QROW + g * C::KPL;
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) *reinterpret_cast<F*>(qrow + ks * C::KS) = qf[ks];
      if (g == 0) lse_lds[wave * 32 + c] = lse;
    }
    if (tid < SEL_WAVES * 2) bkt[tid / 2][tid % 2] = -1;
    __syncthreads();

    const int npair = nkt * nq;
    const int pa = (int)((int64_t)npair * wave / SEL_WAVES), pb = (int)((int64_t)npair * (wave + 1) / SEL_WAVES);
    F kf[C::NS][C::NKS];
    float cs = 0.f;
    int kt_cur = -1, k_cur = -1;
    auto flush = [&]() __attribute__((always_inline)) {  // column sums of segment (kt_cur, k_cur)
      const float tot = xor32_sum(cs);
      const int ulo = GRP ? max(mtp[k_cur] - ts, 0) : 0, uhi = GRP ? min(mtp[k_cur + 1] - ts, nq) : nq;
      const bool first = kt_cur * nq + ulo < pa, last = kt_cur * nq + uhi > pb;
      const int key = kt_cur * KT + c;
      if (!first && !last) {  // the whole segment in this range
        if (g == 0 && key < M) sig[k_cur * Mp + key] += tot;
      } else {
        const int slot = first ? 0 : 1;  // a range within one segment uses slot 0
        if (g == 0) bpart[wave][slot][c] = tot;
        if (lane == 0) bkt[wave][slot] = kt_cur * SEL_GMAX + k_cur;
      }
      cs = 0.f;
    };
#pragma unroll 1
    for (int p = pa; p < pb; ++p) {
      const int kt = p / nq, u = p % nq;
      const int k = member_of(ts + u);
      if (kt != kt_cur || k != k_cur) {
        if (kt_cur >= 0) flush();
        if (kt != kt_cur) {
          const T* krow = pstage + (int64_t)(kt / 2) * C::STAGE + ((kt % 2) * KT + (lane & 31)) * C::KROW +
                          (lane >> 5) * C::KPL;
#pragma unroll
          for (int s2 = 0; s2 < C::NS; ++s2)
#pragma unroll
            for (int ks = 0; ks < C::NKS; ++ks) kf[s2][ks] = load_frag<DT>(krow + s2 * C::KPLANE + ks * C::KS);
        }
        kt_cur = kt;
        k_cur = k;
      }
      const T* qrow = qlds + (u * 32 + (lane & 31)) * QROW + (lane >> 5) * C::KPL;
      ssa_f16v acc = zero16();
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) {
        const F qq = load_frag<DT>(qrow + ks * C::KS);
#pragma unroll
        for (int s2 = 0; s2 < C::NS; ++s2) acc = Tr<DT>::mma(qq, kf[s2][ks], acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r)
        cs += fast_exp2(__builtin_fmaf(acc[r], sl2, -lse_lds[u * 32 + res_row(r, g)]));
    }
    if (kt_cur >= 0) flush();
    __syncthreads();
    if (tid < KT) {  // cut segments, in wave order
      for (int w = 0; w < SEL_WAVES; ++w)
        for (int sl = 0; sl < 2; ++sl) {
          const int tag = bkt[w][sl];
          if (tag >= 0) {
            const int kt = tag / SEL_GMAX, k = tag % SEL_GMAX;
            if (kt * KT + tid < M) sig[k * Mp + kt * KT + tid] += bpart[w][sl][tid];
          }
        }
    }
    __syncthreads();  // the rows are complete for this sweep; the query tiles are free again
  }
  if (sigma_out) {  // the top-k kernel takes it from here
    for (int k = 0; k < Gk; ++k) {
      float* dst = sigma_out + ((int64_t)h * M + mb[k]) * Mp;
      for (int j = tid; j < M; j += 64 * SEL_WAVES) dst[j] = sig[k * Mp + j];
    }
  } else {
    for (int k = wave; k < Gk; k += SEL_WAVES)
      topk_wave(sig + k * Mp, M, topk, sel + ((int64_t)h * M + mb[k]) * topk, lane,
                reinterpret_cast<uint32_t*>(qlds) + wave * 128);  // the query tiles are free now
  }
}

// Top-k of one importance row per wave (rows of at most TOPK_SPLIT_MAX_M entries, held in
// registers): the keff-th largest fp32 bit pattern T is found bit by bit from the top with
// ballot counts, then the entries above T and the first ties at T are placed in id order.
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ sigma, int M, int Mp,
                                              int nrows, int topk, int32_t* __restrict__ sel) {
  constexpr int MAXV = TOPK_SPLIT_MAX_M / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= nrows) return;  // uniform per wave
  const float* src = sigma + (int64_t)row * Mp;
  int32_t* out = sel + (int64_t)row * topk;
  const int nv = (M + 63) / 64;
  uint32_t u[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) u[i] = (i < nv && lane + 64 * i < M) ? __float_as_uint(src[lane + 64 * i]) : 0u;
  auto ok = [&](int i) { return i < nv && lane + 64 * i < M; };
  const int keff = min(topk, M);
  const bool all = keff == M;
  uint32_t T = 0;
  if (!all) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < MAXV; ++i)
        if (i < nv) cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(ok(i) && u[i] >= cand));
      if (cnt >= keff) T = cand;
    }
  }
  int ngt = 0;
  if (!all) {
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
      if (i < nv) ngt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(ok(i) && u[i] > T));
  }
  const int need = keff - ngt;  // ties at T to take, lowest ids first
  int run_gt = 0, run_eq = 0;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    if (i >= nv) break;
    const bool gt = ok(i) && (all || u[i] > T);
    const bool eq = ok(i) && !all && u[i] == T;
    const uint64_t bg = __builtin_amdgcn_ballot_w64(gt), be = __builtin_amdgcn_ballot_w64(eq);
    const int lg = run_gt + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bg >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bg, 0u));
    const int le = run_eq + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(be >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)be, 0u));
    if (gt || (eq && le < need)) out[lg + min(le, need)] = lane + 64 * i;
    run_gt += __builtin_popcountll(bg);
    run_eq += __builtin_popcountll(be);
  }
  for (int t = keff + lane; t < topk; t += 64) out[t] = -1;
}

// ------------------------------------------------------------------ selected + window + combine
// A key set is a list of blocks (the selected blocks, or the blocks of the query's window
// cell), concatenated in sorted token order and cut into 32-key tiles.  The set is staged in
// segments of up to KSEG keys: first the token of every key of the segment goes to LDS
// (keytok), then the segment's tiles stream through NB stage buffers, the copy of tile
// t + NB - 1 being issued while tile t is in use.  Keys past the end of a segment reuse its first
// key (finite values; their scores are masked).
constexpr int KSEG = 2048;

// S^T = K Q^T of a 32-key tile (K rows at the stage start), every fragment read issued
// before the first MFMA (16-bit types: in one asm statement, see lds_frags_b128).
template <int DT, int D>
__device__ inline ssa_f16v s_chain(const typename Tr<DT>::T* cur, const typename Tr<DT>::frag* qf, int lane) {
  using C = Cfg<DT, D>;
  const typename Tr<DT>::T* krow = cur + (lane & 31) * C::KROW + (lane >> 5) * C::KPL;
  typename Tr<DT>::frag ka[C::NKS];
  if constexpr (C::KPL != 1) {
    lds_frags_b128<C::NKS, C::KS * (int)sizeof(typename Tr<DT>::T)>(krow, ka);  // one asm statement
  } else {
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) ka[ks] = load_frag<DT>(krow + ks * C::KS);
  }
  ssa_f16v acc = zero16();
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) acc = Tr<DT>::mma(ka[ks], qf[ks], acc);
  return acc;
}

template <int DT, int D, bool BUF, int NB>
__device__ inline void gathered_branch(
    Online<D / 32>& st, const TileCopy<DT, D, ATT_WAVES>& tc0, const int32_t* blist, int nlist,
    const typename Tr<DT>::frag* qf, const typename Tr<DT>::T* __restrict__ kin,
    const typename Tr<DT>::T* __restrict__ vin, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ blk_off, int H, int h, float sl2, bool wave_active,
    typename Tr<DT>::T* const* bufs, int32_t* pre, int32_t* lst_off, int32_t* keytok) {
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  using F = typename Tr<DT>::frag;
  using TC = TileCopy<DT, D, ATT_WAVES>;
  constexpr int NTH = 64 * ATT_WAVES;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  st.init();
  TC tc = tc0;
  for (int l0 = 0; l0 < nlist; l0 += NTH) {
    const int L = min(NTH, nlist - l0);
    __syncthreads();
    int sz = 0;
    if (tid < L) {
      const int bb = blist[l0 + tid];
      lst_off[tid] = blk_off[bb];
      sz = blk_off[bb + 1] - blk_off[bb];
    }
    pre[tid + 1] = sz;
    if (tid == 0) pre[0] = 0;
    __syncthreads();
    if (L > 1) {
      for (int off = 1; off < NTH; off <<= 1) {
        const int t = (tid + 1 > off) ? pre[tid + 1 - off] : 0;
        __syncthreads();
        pre[tid + 1] += t;
        __syncthreads();
      }
    }
    const int total = pre[L];
    for (int ks0 = 0; ks0 < total; ks0 += KSEG) {
      const int n = min(KSEG, total - ks0);
      __syncthreads();  // the previous segment's tiles have been read
      fill_tokens<KSEG / NTH, NTH>(keytok, n, [&](int j) {
        const int key = ks0 + j;
        int lo = 0, hi = L - 1;  // last list entry starting at or before the key
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (pre[mid] <= key) lo = mid; else hi = mid - 1;
        }
        return lst_off[lo] + (key - pre[lo]);
      }, perm);
      __syncthreads();
      tile_pipeline<NB, TC::NI>(
          (n + KT - 1) / KT, bufs,
          [&](int t) __attribute__((always_inline)) { tc.fetch(keytok, t * KT, n); },
          [&](T* dst) __attribute__((always_inline)) { tc.template issue<BUF>(dst, kin, vin, H, h, wave); },
          [&](int t, const T* cur, auto&& next) __attribute__((always_inline)) {
            ssa_f16v acc = zero16();
            if (wave_active) {
              acc = s_chain<DT, D>(cur, qf, lane);
              if ((t + 1) * KT > n) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                  if (t * KT + res_row(r, g) >= n) acc[r] = -INFINITY;
              }
              st.update(acc, sl2);
            }
            // the value fragments are read before the next copy is issued: the transpose
            // reads carry no alias information, so reading after it would wait for that copy
            VFrags<DT, D> vf;
            if (wave_active) vf.read(cur + TC::VOFF, lane);
            next();
            if (wave_active) {
#pragma unroll
              for (int ks = 0; ks < C::PK; ++ks) {
                const F pf = p_frag<DT>(acc, ks);
#pragma unroll
                for (int j = 0; j < C::NDV; ++j) st.o[j] = Tr<DT>::mma(vf.f[ks][j], pf, st.o[j]);
              }
            }
          });
    }
  }
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ inline int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// One workgroup per (ATT_ROWS-row chunk of a query block, head); a block's chunks and heads
// form one XCD unit (they gather the same key rows), blocks in longest-first order.
//
// Usual case (at most 64 selected and 64 window blocks, at most KSEG keys in all): both key
// sets form one stream -- the selected blocks' keys, padding to a whole tile, then the window
// cell's keys -- whose token table is built once, and whose tiles flow through the stage
// buffers without a break; at the boundary tile the selected branch is closed (its gated
// output kept in registers) and the window branch starts.  Otherwise each set is streamed on
// its own (gathered_branch).
template <int DT, int D, bool BUF, int MODE>
__global__ __launch_bounds__(64 * ATT_WAVES) __attribute__((amdgpu_waves_per_eu(D <= 96 ? 2 : 1))) void k_attend(
    const typename Tr<DT>::T* __restrict__ q, const typename Tr<DT>::T* __restrict__ kin,
    const typename Tr<DT>::T* __restrict__ vin, const typename Tr<DT>::T* __restrict__ gates,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ blk_off,
    const int32_t* __restrict__ blk_cell, const int32_t* __restrict__ cell_off,
    const int32_t* __restrict__ cell_blk, const int32_t* __restrict__ lpt,
    const int32_t* __restrict__ sel, const typename Tr<DT>::T* __restrict__ oc, int M, int H,
    int nchunk, int64_t N, int topk, float sl2, int window_is_block, typename Tr<DT>::T* __restrict__ out,
    float* __restrict__ lse_save, typename SaveT<DT>::type* __restrict__ os_save,
    typename SaveT<DT>::type* __restrict__ ow_save, const typename Tr<DT>::T* __restrict__ ow_in,
    const int4* __restrict__ utab,
    const int2* __restrict__ sdesc) {
  constexpr int mode = MODE;
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  using F = typename Tr<DT>::frag;
  using TC = TileCopy<DT, D, ATT_WAVES>;
  constexpr int NTH = 64 * ATT_WAVES;
  static_assert(NTH >= 256, "one thread per top-k slot");
  // two workgroups per CU
  constexpr int NB = stage_depth<DT, D, ATT_WAVES>(LDS_BYTES / 2 - 2048,
                                                   KSEG * 4 + (2 * NTH + 257) * 4 + 4 * 129 * 4);
  SSA_STAGE_BUFFERS(T, TC::ELEMS, NB);
  __shared__ int32_t pre[NTH + 1];
  __shared__ int32_t lst_off[NTH];
  __shared__ int32_t sel_lds[256];
  __shared__ int32_t keytok[KSEG];
  __shared__ int32_t e_pre[2][65];  // stream offsets of the usual case's entries (per set)
  __shared__ int32_t e_off[2][64];  // their first sorted position

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int unit, member;
  xcd_split(blockIdx.x, nchunk * H, unit, member);
  if (unit >= M) return;
  const int h = member % H, chunk = member / H;
  const int4 ut = utab[unit];  // (block, first row, rows)
  const int b = ut.x;
  const int r0 = ut.y, rows = ut.z;
  if (chunk * ATT_ROWS >= rows) return;  // uniform across the workgroup

  // ---- metadata, loads issued side by side: selection row and its blocks' extents, window
  // cell, queries, gates
  const int64_t srow = ((int64_t)h * M + b) * topk + tid;
  const int sb = mode != ATT_WINDOW && tid < topk ? sel[srow] : -1;  // ascending, -1 padded
  const int2 sd = mode != ATT_WINDOW && tid < 64 && tid < topk ? sdesc[srow] : make_int2(0, 0);
  int c0 = b, c1 = b + 1;                       // window cell as a range of cell_blk
  if (!window_is_block) {
    const int cell = blk_cell[b];
    c0 = cell_off[cell];
    c1 = cell_off[cell + 1];
  }
  const int wbase = chunk * ATT_ROWS + wave * 32;
  const bool wave_active = wbase < rows;
  const int my_row = wbase + c;
  const bool valid = my_row < rows;
  const int64_t tok_q = valid ? perm[r0 + my_row] : 0;
  F qf[C::NKS];
  load_q<DT, D>(qf, q + (tok_q * H + h) * D, valid, lane);
  float gt[3] = {0.f, 0.f, 0.f};
  if (valid && mode != ATT_WINDOW) {
#pragma unroll
    for (int x = 0; x < 3; ++x) gt[x] = Tr<DT>::up(gates[(tok_q * H + h) * 3 + x]);
  }
  // 16-bit types: this lane's part of the compressed branch's output row, read now so that
  // the combine at the end need not wait for it (rows past the block read row 0, unused)
  typedef unsigned ocv_t __attribute__((ext_vector_type(2)));
  constexpr bool OCPRE = sizeof(T) == 2 && (BUF || D <= 64);  // register budget
  ocv_t ocv[OCPRE ? C::NDV * 4 : 1];
  if constexpr (OCPRE && MODE != ATT_WINDOW) {
    const T* orow0 = oc + ((int64_t)(r0 + (valid ? my_row : 0)) * H + h) * D + 4 * g;
#pragma unroll
    for (int j = 0; j < C::NDV; ++j)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) ocv[j * 4 + rq] = *reinterpret_cast<const ocv_t*>(orow0 + 32 * j + 8 * rq);
  }
  if (sb >= 0) sel_lds[tid] = sb;
  const int nsel = __syncthreads_count(sb >= 0);
  const int nwin = mode == ATT_SELECTED ? 0 : c1 - c0;
  TC tc;
  tc.init(wave, lane);
  Online<C::NDV> st;
  ssa_f16v res[C::NDV];  // the selected branch's gated output

  auto close_selected = [&]() __attribute__((always_inline)) {
    const float ls = xor32_sum(st.l);
    const float f = gt[1] / ls;
    if (lse_save && wave_active && valid) {
      const int64_t row = r0 + my_row;
      if (g == 0) lse_save[(int64_t)(H + h) * N + row] = st.m + fast_log2(ls);
      typename SaveT<DT>::type* srow2 = os_save + (row * H + h) * D;
      const float inv = 1.f / ls;
#pragma unroll
      for (int j = 0; j < C::NDV; ++j)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          store4(srow2 + 32 * j + 8 * rq + 4 * g, st.o[j][4 * rq] * inv, st.o[j][4 * rq + 1] * inv,
                 st.o[j][4 * rq + 2] * inv, st.o[j][4 * rq + 3] * inv);
    }
#pragma unroll
    for (int j = 0; j < C::NDV; ++j) res[j] = st.o[j] * f;
  };

  bool fast = nsel <= 64 && nwin <= 64;
  if (fast) {
    // entries: wave 0 the selected blocks, wave 1 the window cell's blocks
    if (wave < 2) {
      const int ne = wave == 0 ? nsel : nwin;
      int off = 0, sz = 0;
      if (lane < ne) {
        if (wave == 0) {  // selected block `lane` is this thread's entry
          off = sd.x;
          sz = sd.y;
        } else if (window_is_block) {
          off = r0;
          sz = rows;
        } else {
          const int blk = cell_blk[c0 + lane];
          off = blk_off[blk];
          sz = blk_off[blk + 1] - off;
        }
      }
      const int incl = wave_incl_scan(sz, lane);
      if (lane < ne) {
        e_off[wave][lane] = off;
        e_pre[wave][lane + 1] = incl;
      }
      if (lane == 0) e_pre[wave][0] = 0;
    }
    __syncthreads();
    const int S = e_pre[0][nsel], W = e_pre[1][nwin];
    fast = (S + KT - 1) / KT * KT + W <= KSEG;
  }
  if (fast) {
    const int S = e_pre[0][nsel], W = e_pre[1][nwin];
    const int P1 = (S + KT - 1) / KT * KT;  // the window keys start on a tile
    const int tot = P1 + W;
    fill_tokens<KSEG / NTH, NTH>(keytok, tot, [&](int j) {
      const int part = j < P1 ? 0 : 1;
      const int key = part ? j - P1 : (j < S ? j : 0);  // padding keys reuse key 0
      const int ne = part ? nwin : nsel;
      int lo = 0, hi = ne - 1;  // last entry starting at or before the key
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (e_pre[part][mid] <= key) lo = mid; else hi = mid - 1;
      }
      return e_off[part][lo] + (key - e_pre[part][lo]);
    }, perm);
    __syncthreads();
    const int tb = P1 / KT;
    st.init();
    tile_pipeline<NB, TC::NI>(
        (tot + KT - 1) / KT, bufs,
        [&](int t) __attribute__((always_inline)) { tc.fetch(keytok, t * KT, tot); },
        [&](T* dst) __attribute__((always_inline)) { tc.template issue<BUF>(dst, kin, vin, H, h, wave); },
        [&](int t, const T* cur, auto&& next) __attribute__((always_inline)) {
          if (t == tb && tb > 0) {  // first window tile: close the selected branch
            close_selected();
            st.init();
          }
          const int lim = t < tb ? S : tot;  // keys at or past lim are masked
          ssa_f16v acc = zero16();
          if (wave_active) {
            acc = s_chain<DT, D>(cur, qf, lane);
            if ((t + 1) * KT > lim) {
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (t * KT + res_row(r, g) >= lim) acc[r] = -INFINITY;
            }
            st.update(acc, sl2);
          }
          // the value fragments are read before the next copy is issued: the transpose reads
          // carry no alias information, so reading after it would wait for that copy
          VFrags<DT, D> vf;
          if (wave_active) vf.read(cur + TC::VOFF, lane);
          next();
          if (wave_active) {
#pragma unroll
            for (int ks = 0; ks < C::PK; ++ks) {
              const F pf = p_frag<DT>(acc, ks);
#pragma unroll
              for (int j = 0; j < C::NDV; ++j) st.o[j] = Tr<DT>::mma(vf.f[ks][j], pf, st.o[j]);
            }
          }
        });
    if (mode == ATT_SELECTED) close_selected();
  } else {
    if (mode != ATT_WINDOW) {
      gathered_branch<DT, D, BUF, NB>(st, tc, sel_lds, nsel, qf, kin, vin, perm, blk_off, H, h, sl2,
                                      wave_active, bufs, pre, lst_off, keytok);
      close_selected();
    }
    if (mode != ATT_SELECTED) {
      const int32_t* wlist = window_is_block ? lpt + unit : cell_blk + c0;  // lpt[unit] == b
      gathered_branch<DT, D, BUF, NB>(st, tc, wlist, nwin, qf, kin, vin, perm, blk_off, H, h, sl2,
                                      wave_active, bufs, pre, lst_off, keytok);
    }
  }
  if (wave_active && valid && mode == ATT_WINDOW) {  // the window branch's output, caller order
    const float inv = 1.f / xor32_sum(st.l);
    T* dst = out + (tok_q * H + h) * D;
#pragma unroll
    for (int j = 0; j < C::NDV; ++j)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        store4(dst + 32 * j + 8 * rq + 4 * g, st.o[j][4 * rq] * inv, st.o[j][4 * rq + 1] * inv,
               st.o[j][4 * rq + 2] * inv, st.o[j][4 * rq + 3] * inv);
  }
  if (wave_active && valid && mode != ATT_WINDOW) {
    const float ltot = mode == ATT_SELECTED ? 1.f : xor32_sum(st.l);
    const float f = gt[2] / ltot;
    const T* orow = oc + ((int64_t)(r0 + my_row) * H + h) * D;
    T* dst = out + (tok_q * H + h) * D;
    if (lse_save) {
      if (g == 0) lse_save[(int64_t)(2 * H + h) * N + r0 + my_row] = st.m + fast_log2(ltot);
      typename SaveT<DT>::type* wrow = ow_save + ((int64_t)(r0 + my_row) * H + h) * D;
      const float inv = 1.f / ltot;
#pragma unroll
      for (int j = 0; j < C::NDV; ++j)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          store4(wrow + 32 * j + 8 * rq + 4 * g, st.o[j][4 * rq] * inv, st.o[j][4 * rq + 1] * inv,
                 st.o[j][4 * rq + 2] * inv, st.o[j][4 * rq + 3] * inv);
    }
#pragma unroll
    for (int j = 0; j < C::NDV; ++j)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int col = 32 * j + 8 * rq + 4 * g;
        float v[4];
        if constexpr (OCPRE) {
          struct V4 { T e[4]; };
          const V4 x = __builtin_bit_cast(V4, ocv[j * 4 + rq]);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (float)x.e[e];
        } else {
          load4(orow + col, v);
        }
        if (mode == ATT_SELECTED) {  // the window branch came from its own pass
          float w4[4];
          load4(ow_in + (tok_q * H + h) * D + col, w4);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = res[j][4 * rq + e] + gt[2] * w4[e] + gt[0] * v[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = res[j][4 * rq + e] + f * st.o[j][4 * rq + e] + gt[0] * v[e];
        }
        store4(dst + col, v[0], v[1], v[2], v[3]);
      }
  }
}

// ------------------------------------------------------------------ launchers
template <int DT, int D>
hipError_t run_pool(const ssa_plan_s* p, int H, const void* k, const void* v, const void* wk,
                    const void* wv, const FwdWs& w, hipStream_t s) {
  using T = typename Tr<DT>::T;
  const int Mp = (int)pooled_rows(p->M);
  // heads per workgroup: the group's columns fit POOL_CPT per thread, its means the LDS
  const int hg = std::max(1, std::min(H, POOL_NT * POOL_CPT * Cfg<DT, D>::EPC / (2 * D)));
  const int nhg = (H + hg - 1) / hg;
  const size_t shm = (size_t)2 * hg * D * sizeof(float);
  hipLaunchKernelGGL((k_pool<DT, D>), dim3((unsigned)(Mp * nhg)), dim3(POOL_NT), shm, s, (const T*)k,
                     (const T*)v, (const T*)wk, (const T*)wv, p->perm, p->blk_off, p->lpt, (int)p->M,
                     Mp, H, hg, (T*)w.pooled, (T*)w.pooled_v);
  return hipGetLastError();
}

template <int DT, int D>
int64_t select_static_lds();

template <int DT, int D>
hipError_t run_select(const ssa_plan_s* p, int H, int topk, float sl2, const void* q,
                      const FwdWs& w, int32_t* sel, hipStream_t s) {
  using T = typename Tr<DT>::T;
  const int Mp = (int)pooled_rows(p->M);
  const size_t shm = (size_t)Mp * sizeof(float);
  const int nch = (int)((p->n + 32 * CMP_WAVES - 1) / (32 * CMP_WAVES));
  const int per = (int)(((int64_t)H * nch + 7) / 8);
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_compress<DT, D>, 64 * CMP_WAVES, 0)) !=
      hipSuccess)
    return e;
  const int wpx = std::max(1, std::min(per, cus * std::max(per_cu, 1) / 8));  // workgroups per XCD
  hipLaunchKernelGGL((k_compress<DT, D>), dim3((unsigned)(8 * wpx)), dim3(64 * CMP_WAVES), 0, s,
                     (const T*)q, (const T*)w.pooled, p->perm, (int)p->M, Mp, H, p->n, nch, per, wpx, sl2,
                     (T*)w.oc, w.lsec, DT == DT_F16 ? nullptr : (float*)w.obr);  // f16: oc is the saved plane
  // blocks per importance workgroup: one for blocks of 64 rows and more on average, else
  // enough for about 256 rows, as far as their importance rows fit the LDS
  int G = 1;
  const int64_t avg = p->n / p->M;
  if (avg < 64) {
    const int64_t room = (int64_t)LDS_BYTES - select_static_lds<DT, D>();
    const int64_t fit = room / ((int64_t)Mp * (int64_t)sizeof(float));
    const int64_t want = 256 / ((avg + 31) / 32 * 32);
    G = (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)SEL_GMAX, fit, want}));
  }
  const int ngrp = (int)((p->M + G - 1) / G);
  const unsigned sel_grid = (unsigned)((ngrp * H + NXCD - 1) / NXCD * NXCD);
  if (G > 1)
    hipLaunchKernelGGL((k_select<DT, D, true>), dim3(sel_grid), dim3(64 * SEL_WAVES), shm * G, s,
                       (const T*)q, (const T*)w.pooled, p->perm, p->blk_off, p->lpt, (int)p->M, Mp, H,
                       p->n, sl2, topk, G, w.lsec, sel, w.sigma);
  else
    hipLaunchKernelGGL((k_select<DT, D, false>), dim3(sel_grid), dim3(64 * SEL_WAVES), shm, s,
                       (const T*)q, (const T*)w.pooled, p->perm, p->blk_off, p->lpt, (int)p->M, Mp, H,
                       p->n, sl2, topk, 1, w.lsec, sel, w.sigma);
  if (w.sigma) {
    const int nrows = (int)(p->M * H);
    hipLaunchKernelGGL(k_topk, dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, s, w.sigma, (int)p->M,
                       Mp, nrows, topk, sel);
  }
  return hipGetLastError();
}

// Per launch of k_attend: its units' (block, first row, rows) and, with a selection, each
// selected block's first sorted row and size, so that a work item reads them in one step.
__global__ __launch_bounds__(256) void k_att_prep(const int32_t* __restrict__ lpt, const int32_t* __restrict__ off,
                                                  int units, int4* __restrict__ utab,
                                                  const int32_t* __restrict__ sel,
                                                  const int32_t* __restrict__ blk_off, int64_t nsel,
                                                  int2* __restrict__ sdesc) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < units) {
    const int b = lpt[i], r0 = off[b];
    utab[i] = make_int4(b, r0, off[b + 1] - r0, 0);
  }
  if (i < nsel) {
    const int s = sel[i];
    sdesc[i] = s >= 0 ? make_int2(blk_off[s], blk_off[s + 1] - blk_off[s]) : make_int2(0, 0);
  }
}

template <int DT, int D>
hipError_t run_attend(const ssa_plan_s* p, int H, int topk, float sl2, const void* q,
                      const void* k, const void* v, const void* gates, const FwdWs& w,
                      const int32_t* sel, void* out, hipStream_t s) {
  using T = typename Tr<DT>::T;
  const bool buf = buffer_addressable(p->n * H * D * (int64_t)sizeof(T));
  auto launch = [&](int mode, int64_t units, const int32_t* perm, const int32_t* off, const int32_t* lpt,
                    int max_rows, int wib, T* dst) {
    const int nchunk = (max_rows + ATT_ROWS - 1) / ATT_ROWS;
    float* lse = mode == ATT_BOTH ? w.lse : nullptr;
    using ST = typename SaveT<DT>::type;
    const int64_t plane = p->n * H * D;  // f16 keeps no compressed plane (oc is it)
    ST* os = mode == ATT_BOTH && w.obr ? (ST*)w.obr + (DT == DT_F16 ? 0 : plane) : nullptr;
    ST* ows = mode == ATT_BOTH && w.obr ? (ST*)w.obr + (DT == DT_F16 ? 1 : 2) * plane : nullptr;
    const int64_t nsel = mode == ATT_WINDOW ? 0 : (int64_t)H * p->M * topk;
    const int64_t nprep = std::max<int64_t>(units, nsel);
    hipLaunchKernelGGL(k_att_prep, dim3((unsigned)((nprep + 255) / 256)), dim3(256), 0, s, lpt, off, (int)units,
                       w.utab, sel, p->blk_off, nsel, w.sdesc);
    auto kern = mode == ATT_BOTH ? (buf ? k_attend<DT, D, true, ATT_BOTH> : k_attend<DT, D, false, ATT_BOTH>)
              : mode == ATT_WINDOW ? (buf ? k_attend<DT, D, true, ATT_WINDOW> : k_attend<DT, D, false, ATT_WINDOW>)
                                   : (buf ? k_attend<DT, D, true, ATT_SELECTED> : k_attend<DT, D, false, ATT_SELECTED>);
    hipLaunchKernelGGL(kern, dim3(xcd_grid(units, (int64_t)H * nchunk)), dim3(64 * ATT_WAVES), 0, s,
                       (const T*)q, (const T*)k, (const T*)v, (const T*)gates, perm, off, p->blk_cell,
                       p->cell_off, p->cell_blk, lpt, sel, (const T*)w.oc, (int)units, H, nchunk, p->n,
                       topk, sl2, wib, dst, lse, os, ows, (const T*)w.ow, w.utab, w.sdesc);
  };
  if (p->wkind == 0) {
    launch(ATT_BOTH, p->M, p->perm, p->blk_off, p->lpt, p->max_rows, (int)p->window_is_block, (T*)out);
  } else {
    // window cells that are not unions of blocks: the window branch over its own partition
    // (each cell's tokens attend to each other), then the selected branch and the combine
    launch(ATT_WINDOW, p->wC, p->wperm, p->wcell_off, p->wlpt, p->wmax_rows, 1, (T*)w.ow);
    launch(ATT_SELECTED, p->M, p->perm, p->blk_off, p->lpt, p->max_rows, 1, (T*)out);
  }
  return hipGetLastError();
}

template <int DT>
hipError_t pool_d(int d, const ssa_plan_s* p, int H, const void* k, const void* v, const void* wk,
                  const void* wv, const FwdWs& w, hipStream_t s) {
  switch (d) {
    case 32: return run_pool<DT, 32>(p, H, k, v, wk, wv, w, s);
    case 64: return run_pool<DT, 64>(p, H, k, v, wk, wv, w, s);
    case 96: return run_pool<DT, 96>(p, H, k, v, wk, wv, w, s);
    case 128: return run_pool<DT, 128>(p, H, k, v, wk, wv, w, s);
  }
  return hipErrorInvalidValue;
}

// Most pooled blocks the selection kernel takes: its importance vector [pooled_rows(M)]
// fp32 lives in LDS beside the kernel's static arrays, within the 160 KB of a workgroup.
// Static LDS of the importance kernel (its importance rows come on top).
template <int DT, int D>
int64_t select_static_lds() {
  static int64_t bytes = -1;
  if (bytes < 0) {
    hipFuncAttributes a;
    if (hipFuncGetAttributes(&a, reinterpret_cast<const void*>(&k_select<DT, D, false>)) != hipSuccess) return LDS_BYTES;
    bytes = (int64_t)a.sharedSizeBytes;
  }
  return bytes;
}

template <int DT, int D>
int64_t select_limit() {
  static int64_t lim = -1;
  if (lim < 0) {
    hipFuncAttributes a;
    if (hipFuncGetAttributes(&a, reinterpret_cast<const void*>(&k_select<DT, D, false>)) != hipSuccess) return 0;
    const int64_t room = (int64_t)LDS_BYTES - (int64_t)a.sharedSizeBytes;
    lim = room <= 0 ? 0 : room / (int64_t)sizeof(float) / 128 * 128;  // pooled_rows(M) fits
  }
  return lim;
}

template <int DT>
int64_t select_limit_d(int d) {
  switch (d) {
    case 32: return select_limit<DT, 32>();
    case 64: return select_limit<DT, 64>();
    case 96: return select_limit<DT, 96>();
    case 128: return select_limit<DT, 128>();
  }
  return 0;
}

template <int DT>
hipError_t select_d(int d, const ssa_plan_s* p, int H, int topk, float sl2, const void* q,
                    const FwdWs& w, int32_t* sel, hipStream_t s) {
  switch (d) {
    case 32: return run_select<DT, 32>(p, H, topk, sl2, q, w, sel, s);
    case 64: return run_select<DT, 64>(p, H, topk, sl2, q, w, sel, s);
    case 96: return run_select<DT, 96>(p, H, topk, sl2, q, w, sel, s);
    case 128: return run_select<DT, 128>(p, H, topk, sl2, q, w, sel, s);
  }
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t attend_d(int d, const ssa_plan_s* p, int H, int topk, float sl2, const void* q,
                    const void* k, const void* v, const void* gates, const FwdWs& w,
                    const int32_t* sel, void* out, hipStream_t s) {
  switch (d) {
    case 32: return run_attend<DT, 32>(p, H, topk, sl2, q, k, v, gates, w, sel, out, s);
    case 64: return run_attend<DT, 64>(p, H, topk, sl2, q, k, v, gates, w, sel, out, s);
    case 96: return run_attend<DT, 96>(p, H, topk, sl2, q, k, v, gates, w, sel, out, s);
    case 128: return run_attend<DT, 128>(p, H, topk, sl2, q, k, v, gates, w, sel, out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_pool(ssa_dtype dt, const ssa_plan_s* p, int H, int d, const void* k,
                       const void* v, const void* wk, const void* wv, const FwdWs& w,
                       hipStream_t s) {
  switch (dt) {
    case SSA_F32: return pool_d<DT_F32>(d, p, H, k, v, wk, wv, w, s);
    case SSA_F16: return pool_d<DT_F16>(d, p, H, k, v, wk, wv, w, s);
    case SSA_BF16: return pool_d<DT_BF16>(d, p, H, k, v, wk, wv, w, s);
  }
  return hipErrorInvalidValue;
}

int64_t select_block_limit(ssa_dtype dt, int d) {
  switch (dt) {
    case SSA_F32: return select_limit_d<DT_F32>(d);
    case SSA_F16: return select_limit_d<DT_F16>(d);
    case SSA_BF16: return select_limit_d<DT_BF16>(d);
  }
  return 0;
}

hipError_t launch_select(ssa_dtype dt, const ssa_plan_s* p, int H, int d, int topk, float scale,
                         const void* q, const FwdWs& w, int32_t* sel, hipStream_t s) {
  const float sl2 = scale * 1.4426950408889634f;
  switch (dt) {
    case SSA_F32: return select_d<DT_F32>(d, p, H, topk, sl2, q, w, sel, s);
    case SSA_F16: return select_d<DT_F16>(d, p, H, topk, sl2, q, w, sel, s);
    case SSA_BF16: return select_d<DT_BF16>(d, p, H, topk, sl2, q, w, sel, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attend(ssa_dtype dt, const ssa_plan_s* p, int H, int d, int topk, float scale,
                         const void* q, const void* k, const void* v, const void* gates,
                         const FwdWs& w, const int32_t* sel, void* out, hipStream_t s) {
  const float sl2 = scale * 1.4426950408889634f;
  switch (dt) {
    case SSA_F32: return attend_d<DT_F32>(d, p, H, topk, sl2, q, k, v, gates, w, sel, out, s);
    case SSA_F16: return attend_d<DT_F16>(d, p, H, topk, sl2, q, k, v, gates, w, sel, out, s);
    case SSA_BF16: return attend_d<DT_BF16>(d, p, H, topk, sl2, q, k, v, gates, w, sel, out, s);
  }
  return hipErrorInvalidValue;
}
