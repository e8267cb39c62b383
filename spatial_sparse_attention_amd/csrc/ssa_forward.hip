// SSA forward kernels for gfx950: pooled keys/values, the compressed branch with
// block selection, and the selected + window branches with the gated combine.
//
// Method (Direct3D-S2 pages: nav.superapi.store "Technical principles of
// Direct3D-S2"; pixal-3d.com "What is Direct3D-S2?"): a compression module pools
// each block to one token and attends to all of them; its attention scores pick
// the important blocks for fine attention; a local window module attends to the
// query's neighbourhood; predicted gates aggregate the three outputs.
//
// Work item of the attention kernels: one (query block, head), taken in
// longest-block-first order.  Four waves each own 32 query rows per sweep.
// Scores come from 32x32 MFMA tiles.  The compressed branch runs twice over the
// pooled keys:
//   pass 1 computes S^T = Ktil Q^T (a lane holds one query, 16 keys), keeps an
//          online softmax and accumulates O^T += Vtil^T P^T with P^T straight
//          from registers; it yields o_c and the exact log-sum-exp;
//   pass 2 computes S = Q Ktil^T (a lane holds one key, 16 queries), so the
//          importance column sums over the block's queries are register sums.
// The pooled keys are fp32; they enter the MFMA as two (f16) or three (bf16)
// dtype planes whose sum reproduces the fp32 value, so the scores that decide the
// top-k carry fp32-level error.
#include <hip/hip_runtime.h>
#include "ssa_internal.h"
#include "ssa_mfma.h"

namespace {

constexpr int NWAVE = 4;
constexpr int NT = 64 * NWAVE;
constexpr int ROWS_PER_SWEEP = 32 * NWAVE;
constexpr int KT = 32;  // keys per tile

template <class T> struct Pad { static constexpr int v = 16 / sizeof(T); };

// ------------------------------------------------------------------ pooling
// grid (Mp, H).  ktil[h,b] = mean_{i in b} K[i,h] @ Wk ; same for V.  Writes the fp32
// value split into NSPLIT dtype planes ksplit[s][h][b][:], and vtil_t[h][:][b].
template <int DT>
__global__ __launch_bounds__(256) void k_pool(
    const typename Tr<DT>::T* __restrict__ kin, const typename Tr<DT>::T* __restrict__ vin,
    const typename Tr<DT>::T* __restrict__ wk, const typename Tr<DT>::T* __restrict__ wv,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ blk_off, int M, int Mp, int H,
    int d, typename Tr<DT>::T* __restrict__ ksplit, typename Tr<DT>::T* __restrict__ vtil_t) {
  using T = typename Tr<DT>::T;
  constexpr int NS = Tr<DT>::NSPLIT;
  constexpr int VEC = 16 / sizeof(T);
  extern __shared__ float smem[];
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  if (b >= M) {  // padding keys: zeros
    for (int j = tid; j < d; j += 256) {
      for (int s = 0; s < NS; ++s) ksplit[(((int64_t)s * H + h) * Mp + b) * d + j] = (T)0.f;
      vtil_t[((int64_t)h * d + j) * Mp + b] = (T)0.f;
    }
    return;
  }
  const int CH = d / VEC, RSUB = 256 / CH;
  float* redk = smem;               // [RSUB][d]
  float* redv = smem + RSUB * d;    // [RSUB][d]
  float* kbar = redv + RSUB * d;    // [d]
  float* vbar = kbar + d;           // [d]
  const int r0 = blk_off[b], r1 = blk_off[b + 1];
  const int sub = tid / CH, ch = tid % CH;
  if (sub < RSUB) {
    float ak[VEC], av[VEC];
    for (int e = 0; e < VEC; ++e) ak[e] = av[e] = 0.f;
    for (int r = r0 + sub; r < r1; r += RSUB) {
      const int64_t base = ((int64_t)perm[r] * H + h) * d + ch * VEC;
      const T* kp = kin + base;
      const T* vp = vin + base;
      for (int e = 0; e < VEC; ++e) {
        ak[e] += Tr<DT>::up(kp[e]);
        av[e] += Tr<DT>::up(vp[e]);
      }
    }
    for (int e = 0; e < VEC; ++e) {
      redk[sub * d + ch * VEC + e] = ak[e];
      redv[sub * d + ch * VEC + e] = av[e];
    }
  }
  __syncthreads();
  const float inv = 1.f / (float)(r1 - r0);
  for (int j = tid; j < 2 * d; j += 256) {
    const float* red = j < d ? redk : redv;
    const int c = j < d ? j : j - d;
    float s = 0.f;
    for (int u = 0; u < RSUB; ++u) s += red[u * d + c];
    (j < d ? kbar : vbar)[c] = s * inv;
  }
  __syncthreads();
  for (int j = tid; j < 2 * d; j += 256) {
    const bool isk = j < d;
    const int c = isk ? j : j - d;
    const T* W = isk ? wk : wv;
    const float* xb = isk ? kbar : vbar;
    float acc = 0.f;
    for (int i = 0; i < d; ++i) acc += xb[i] * Tr<DT>::up(W[(int64_t)i * d + c]);
    if (isk) {
      float rem = acc;
      for (int s = 0; s < NS; ++s) {
        T part = Tr<DT>::cvt(rem);
        ksplit[(((int64_t)s * H + h) * Mp + b) * d + c] = part;
        rem -= Tr<DT>::up(part);
      }
    } else {
      vtil_t[((int64_t)h * d + c) * Mp + b] = Tr<DT>::cvt(acc);
    }
  }
}

// ------------------------------------------------------------------ shared pieces
template <int DT, int D>
struct Frags {
  using T = typename Tr<DT>::T;
  using F = typename Tr<DT>::frag;
  static constexpr int KS = Tr<DT>::KS, KPL = Tr<DT>::KPL;
  static constexpr int NKS = D / KS;   // K steps over the head dim
  static constexpr int NDV = D / 32;   // 32-wide output column tiles
  static constexpr int KROW = D + Pad<T>::v;
  static constexpr int VROW = KT + Pad<T>::v;
  static constexpr int PK = KT / KS;   // K steps over a 32-key tile (PV product)
};

// A operand of O^T += V^T P^T for K step `ks` of a 32-key tile: lane (dv = row, g)
// supplies V^T[dv][key] for the keys held by P^T registers ks*KPL .. ks*KPL+KPL-1.
template <int DT, int D>
__device__ inline typename Tr<DT>::frag vt_frag(const typename Tr<DT>::T* vrow, int ks, int g) {
  using Fr = Frags<DT, D>;
  typename Tr<DT>::frag f;
  if constexpr (Fr::KPL == 1) {
    f = vrow[res_row(ks, g)];
  } else {
    // registers ks*8 .. ks*8+7 hold keys 16ks + {4g..4g+3, 8+4g..8+4g+3}
    typedef typename Tr<DT>::T T;
    typedef T T4 __attribute__((ext_vector_type(4)));
    const T4 lo = *reinterpret_cast<const T4*>(vrow + 16 * ks + 4 * g);
    const T4 hi = *reinterpret_cast<const T4*>(vrow + 16 * ks + 8 + 4 * g);
    f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
  }
  return f;
}

// B operand (P^T) for K step ks from the 16 fp32 probabilities of a lane.
template <int DT>
__device__ inline typename Tr<DT>::frag p_frag(const ssa_f16v& p, int ks) {
  typename Tr<DT>::frag f;
  if constexpr (Tr<DT>::KPL == 1) {
    f = p[ks];
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) f[t] = Tr<DT>::cvt(p[ks * 8 + t]);
  }
  return f;
}

template <int DT>
__device__ inline typename Tr<DT>::frag zero_frag() {
  typename Tr<DT>::frag f;
  if constexpr (Tr<DT>::KPL == 1) f = 0.f;
  else {
#pragma unroll
    for (int t = 0; t < 8; ++t) f[t] = (typename Tr<DT>::T)0.f;
  }
  return f;
}

// Online-softmax state of one query row (duplicated in lanes c and c+32, which hold
// different keys of the same row).  Scores are in log2 units.
template <int NDV>
struct Online {
  float m, l;
  ssa_f16v o[NDV];
  __device__ inline void init() {
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int j = 0; j < NDV; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[j][r] = 0.f;
  }
  // x: the lane's 16 scores (log2 units, -inf for masked keys); returns p in place.
  __device__ inline void update(ssa_f16v& x) {
    float mt = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, x[r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(m, mt);
    const float alpha = fast_exp2(m - mn);
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      x[r] = fast_exp2(x[r] - mn);
      s += x[r];
    }
    l = l * alpha + s;
#pragma unroll
    for (int j = 0; j < NDV; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[j][r] *= alpha;
    m = mn;
  }
};

// O^T += V^T P^T for one 32-key tile.
template <int DT, int D>
__device__ inline void pv_tile(Online<D / 32>& st, const ssa_f16v& p,
                               const typename Tr<DT>::T* v_lds, int c, int g) {
  using Fr = Frags<DT, D>;
#pragma unroll
  for (int ks = 0; ks < Fr::PK; ++ks) {
    const typename Tr<DT>::frag pf = p_frag<DT>(p, ks);
#pragma unroll
    for (int j = 0; j < Fr::NDV; ++j) {
      const typename Tr<DT>::frag vf = vt_frag<DT, D>(v_lds + (32 * j + c) * Fr::VROW, ks, g);
      st.o[j] = Tr<DT>::mma(vf, pf, st.o[j]);
    }
  }
}

// ------------------------------------------------------------------ compressed + select
template <int DT, int D>
__global__ __launch_bounds__(NT) void k_select(
    const typename Tr<DT>::T* __restrict__ q, const typename Tr<DT>::T* __restrict__ ksplit,
    const typename Tr<DT>::T* __restrict__ vtil_t, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ blk_off, const int32_t* __restrict__ lpt, int M, int Mp, int H,
    int64_t N, float sl2, int topk, typename Tr<DT>::T* __restrict__ oc,
    int32_t* __restrict__ sel) {
  using Fr = Frags<DT, D>;
  using T = typename Tr<DT>::T;
  using F = typename Tr<DT>::frag;
  constexpr int NS = Tr<DT>::NSPLIT;
  __shared__ __attribute__((aligned(16))) T k_lds[NS][KT][Fr::KROW];
  __shared__ __attribute__((aligned(16))) T v_lds[D][Fr::VROW];
  __shared__ float stage[NWAVE][32];
  __shared__ float lse_lds[ROWS_PER_SWEEP];
  __shared__ int32_t pick[256];
  extern __shared__ float sig[];  // [Mp]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, c = lane & 31;
  const int h = blockIdx.x % H;
  const int b = lpt[blockIdx.x / H];
  const int r0 = blk_off[b], rows = blk_off[b + 1] - r0;
  for (int j = tid; j < Mp; j += NT) sig[j] = 0.f;
  const int ntile = Mp / KT;
  constexpr int KCH = D * sizeof(T) / 16;  // 16-byte chunks per key row
  constexpr int VCH = KT * sizeof(T) / 16;  // 16-byte chunks per V^T row
  constexpr int EPC = 16 / sizeof(T);

  for (int sw = 0; sw * ROWS_PER_SWEEP < rows; ++sw) {
    const int row_base = sw * ROWS_PER_SWEEP + wave * 32;
    const bool wave_active = row_base < rows;
    const int my_row = row_base + c;
    const bool valid = my_row < rows;
    F qf[Fr::NKS];
    {
      const int64_t tok = valid ? perm[r0 + my_row] : 0;
      const T* qrow = q + (tok * H + h) * D;
#pragma unroll
      for (int s = 0; s < Fr::NKS; ++s)
        qf[s] = valid ? load_frag<DT>(qrow + s * Fr::KS + g * Fr::KPL) : zero_frag<DT>();
    }
    // ---------------- pass 1: online softmax, o_c, lse
    Online<Fr::NDV> st;
    st.init();
    for (int kt = 0; kt < ntile; ++kt) {
      __syncthreads();
      for (int idx = tid; idx < NS * KT * KCH; idx += NT) {
        const int s = idx / (KT * KCH), rem = idx % (KT * KCH), key = rem / KCH, ch = rem % KCH;
        *reinterpret_cast<uint4*>(&k_lds[s][key][ch * EPC]) = *reinterpret_cast<const uint4*>(
            ksplit + (((int64_t)s * H + h) * Mp + kt * KT + key) * D + ch * EPC);
      }
      for (int idx = tid; idx < D * VCH; idx += NT) {
        const int dv = idx / VCH, ch = idx % VCH;
        *reinterpret_cast<uint4*>(&v_lds[dv][ch * EPC]) = *reinterpret_cast<const uint4*>(
            vtil_t + ((int64_t)h * D + dv) * Mp + kt * KT + ch * EPC);
      }
      __syncthreads();
      if (!wave_active) continue;
      ssa_f16v acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int ks = 0; ks < Fr::NKS; ++ks)
          acc = Tr<DT>::mma(load_frag<DT>(&k_lds[s][c][ks * Fr::KS + g * Fr::KPL]), qf[ks], acc);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt * KT + res_row(r, g);
        acc[r] = key < M ? acc[r] * sl2 : -INFINITY;
      }
      st.update(acc);
      pv_tile<DT, D>(st, acc, &v_lds[0][0], c, g);
    }
    const float ltot = st.l + __shfl_xor(st.l, 32);
    const float inv = 1.f / ltot;
    if (wave_active && valid) {
      T* orow = oc + ((int64_t)h * N + r0 + my_row) * D;
#pragma unroll
      for (int j = 0; j < Fr::NDV; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) orow[32 * j + res_row(r, g)] = Tr<DT>::cvt(st.o[j][r] * inv);
    }
    if (g == 0) lse_lds[wave * 32 + c] = st.m + fast_log2(ltot);
    __syncthreads();
    // ---------------- pass 2: importance column sums
    float lrow[16];
    bool vrow[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rr = res_row(r, g);
      vrow[r] = row_base + rr < rows;
      lrow[r] = lse_lds[wave * 32 + rr];
    }
    for (int kt = 0; kt < ntile; ++kt) {
      __syncthreads();
      for (int idx = tid; idx < NS * KT * KCH; idx += NT) {
        const int s = idx / (KT * KCH), rem = idx % (KT * KCH), key = rem / KCH, ch = rem % KCH;
        *reinterpret_cast<uint4*>(&k_lds[s][key][ch * EPC]) = *reinterpret_cast<const uint4*>(
            ksplit + (((int64_t)s * H + h) * Mp + kt * KT + key) * D + ch * EPC);
      }
      __syncthreads();
      float colsum = 0.f;
      if (wave_active) {
        ssa_f16v acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int ks = 0; ks < Fr::NKS; ++ks)
            acc = Tr<DT>::mma(qf[ks], load_frag<DT>(&k_lds[s][c][ks * Fr::KS + g * Fr::KPL]), acc);
#pragma unroll
        for (int r = 0; r < 16; ++r) colsum += vrow[r] ? fast_exp2(acc[r] * sl2 - lrow[r]) : 0.f;
        colsum += __shfl_xor(colsum, 32);
      }
      if (g == 0) stage[wave][c] = colsum;
      __syncthreads();
      if (tid < 32) {
        const int key = kt * KT + tid;
        float s = stage[0][tid];
#pragma unroll
        for (int w = 1; w < NWAVE; ++w) s += stage[w][tid];
        if (key < M) sig[key] += s;
      }
    }
  }
  __syncthreads();
  // ---------------- top-k (wave 0): repeated arg-max of (sigma bits, ~id) below the last pick
  if (wave == 0) {
    const int keff = min(topk, M);
    uint64_t prev = ~0ull;
    for (int it = 0; it < keff; ++it) {
      uint64_t best = 0;
      for (int j = lane; j < M; j += 64) {
        const uint64_t key = ((uint64_t)__float_as_uint(sig[j]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
        if (key < prev && key > best) best = key;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)best, off), hi = __shfl_xor((uint32_t)(best >> 32), off);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        best = o > best ? o : best;
      }
      prev = best;
      if (lane == 0) pick[it] = (int32_t)(0xFFFFFFFFu - (uint32_t)best);
    }
    if (lane == 0) {
      for (int i = 1; i < keff; ++i) {  // ascending ids
        int x = pick[i], j = i - 1;
        while (j >= 0 && pick[j] > x) { pick[j + 1] = pick[j]; --j; }
        pick[j + 1] = x;
      }
    }
    for (int t = lane; t < topk; t += 64) sel[((int64_t)h * M + b) * topk + t] = t < keff ? pick[t] : -1;
  }
}

// ------------------------------------------------------------------ selected + window + combine
// Key sets are lists of blocks (the selected blocks; the blocks of the query's window
// cell), concatenated in sorted token order and cut into 32-key tiles.
template <int DT, int D>
__device__ inline void gathered_branch(
    Online<D / 32>& st, const int32_t* blist, int nlist, const typename Tr<DT>::frag* qf,
    const typename Tr<DT>::T* __restrict__ kin, const typename Tr<DT>::T* __restrict__ vin,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ blk_off, int H, int h,
    float sl2, bool wave_active, typename Tr<DT>::T (*k_lds)[Frags<DT, D>::KROW],
    typename Tr<DT>::T (*v_lds)[Frags<DT, D>::VROW], int32_t* pre, int32_t* lst, int32_t* tok) {
  using Fr = Frags<DT, D>;
  using T = typename Tr<DT>::T;
  constexpr int KCH = D * sizeof(T) / 16;
  constexpr int EPC = 16 / sizeof(T);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c = lane & 31;
  st.init();
  for (int l0 = 0; l0 < nlist; l0 += NT) {
    const int L = min(NT, nlist - l0);
    __syncthreads();
    // exclusive prefix of the chunk's block sizes
    int sz = 0;
    if (tid < L) {
      const int bb = blist[l0 + tid];
      lst[tid] = bb;
      sz = blk_off[bb + 1] - blk_off[bb];
    }
    pre[tid + 1] = sz;
    if (tid == 0) pre[0] = 0;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
      const int t = (tid + 1 > off) ? pre[tid + 1 - off] : 0;
      __syncthreads();
      pre[tid + 1] += t;
      __syncthreads();
    }
    const int total = pre[L];
    for (int k0 = 0; k0 < total; k0 += KT) {
      __syncthreads();
      if (tid < KT) {
        const int j = k0 + tid;
        int t = -1;
        if (j < total) {
          int lo = 0, hi = L - 1;  // last block with pre[idx] <= j
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] <= j) lo = mid; else hi = mid - 1;
          }
          t = perm[blk_off[lst[lo]] + (j - pre[lo])];
        }
        tok[tid] = t;
      }
      __syncthreads();
      for (int idx = tid; idx < KT * KCH; idx += NT) {
        const int key = idx / KCH, ch = idx % KCH;
        const int t = tok[key];
        uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
        if (t >= 0) {
          const int64_t base = ((int64_t)t * H + h) * D + ch * EPC;
          kv = *reinterpret_cast<const uint4*>(kin + base);
          vv = *reinterpret_cast<const uint4*>(vin + base);
        }
        *reinterpret_cast<uint4*>(&k_lds[key][ch * EPC]) = kv;
        const T* ve = reinterpret_cast<const T*>(&vv);
#pragma unroll
        for (int e = 0; e < EPC; ++e) v_lds[ch * EPC + e][key] = ve[e];
      }
      __syncthreads();
      if (!wave_active) continue;
      ssa_f16v acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < Fr::NKS; ++ks)
        acc = Tr<DT>::mma(load_frag<DT>(&k_lds[c][ks * Fr::KS + g * Fr::KPL]), qf[ks], acc);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = k0 + res_row(r, g);
        acc[r] = j < total ? acc[r] * sl2 : -INFINITY;
      }
      st.update(acc);
      pv_tile<DT, D>(st, acc, &v_lds[0][0], c, g);
    }
  }
}

template <int DT, int D>
__global__ __launch_bounds__(NT) void k_attend(
    const typename Tr<DT>::T* __restrict__ q, const typename Tr<DT>::T* __restrict__ kin,
    const typename Tr<DT>::T* __restrict__ vin, const typename Tr<DT>::T* __restrict__ gates,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ blk_off,
    const int32_t* __restrict__ blk_cell, const int32_t* __restrict__ cell_off,
    const int32_t* __restrict__ cell_blk, const int32_t* __restrict__ lpt,
    const int32_t* __restrict__ sel, const typename Tr<DT>::T* __restrict__ oc, int M, int H,
    int64_t N, int topk, float sl2, typename Tr<DT>::T* __restrict__ out) {
  using Fr = Frags<DT, D>;
  using T = typename Tr<DT>::T;
  using F = typename Tr<DT>::frag;
  __shared__ __attribute__((aligned(16))) T k_lds[KT][Fr::KROW];
  __shared__ __attribute__((aligned(16))) T v_lds[D][Fr::VROW];
  __shared__ int32_t pre[NT + 1];
  __shared__ int32_t lst[NT];
  __shared__ int32_t tok[KT];
  __shared__ int32_t sel_lds[256];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, c = lane & 31;
  const int h = blockIdx.x % H;
  const int b = lpt[blockIdx.x / H];
  const int r0 = blk_off[b], rows = blk_off[b + 1] - r0;
  // selected block list (valid ids)
  int nsel = 0;
  for (int t = 0; t < topk; ++t) nsel += sel[((int64_t)h * M + b) * topk + t] >= 0;
  for (int t = tid; t < nsel; t += NT) sel_lds[t] = sel[((int64_t)h * M + b) * topk + t];
  const int cell = blk_cell[b];
  const int c0 = cell_off[cell], c1 = cell_off[cell + 1];

  for (int sw = 0; sw * ROWS_PER_SWEEP < rows; ++sw) {
    const int row_base = sw * ROWS_PER_SWEEP + wave * 32;
    const bool wave_active = row_base < rows;
    const int my_row = row_base + c;
    const bool valid = my_row < rows;
    const int64_t tok_q = valid ? perm[r0 + my_row] : 0;
    F qf[Fr::NKS];
    {
      const T* qrow = q + (tok_q * H + h) * D;
#pragma unroll
      for (int s = 0; s < Fr::NKS; ++s)
        qf[s] = valid ? load_frag<DT>(qrow + s * Fr::KS + g * Fr::KPL) : zero_frag<DT>();
    }
    float gate[3] = {0.f, 0.f, 0.f};
    if (valid)
      for (int x = 0; x < 3; ++x) gate[x] = Tr<DT>::up(gates[(tok_q * H + h) * 3 + x]);
    // result = g0 * o_c
    ssa_f16v res[Fr::NDV];
    {
      const T* orow = oc + ((int64_t)h * N + r0 + (valid ? my_row : 0)) * D;
#pragma unroll
      for (int j = 0; j < Fr::NDV; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) res[j][r] = valid ? gate[0] * Tr<DT>::up(orow[32 * j + res_row(r, g)]) : 0.f;
    }
    Online<Fr::NDV> st;
    gathered_branch<DT, D>(st, sel_lds, nsel, qf, kin, vin, perm, blk_off, H, h, sl2, wave_active,
                           k_lds, v_lds, pre, lst, tok);
    {
      const float ltot = st.l + __shfl_xor(st.l, 32);
      const float f = gate[1] / ltot;
#pragma unroll
      for (int j = 0; j < Fr::NDV; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) res[j][r] += f * st.o[j][r];
    }
    gathered_branch<DT, D>(st, cell_blk + c0, c1 - c0, qf, kin, vin, perm, blk_off, H, h, sl2,
                           wave_active, k_lds, v_lds, pre, lst, tok);
    {
      const float ltot = st.l + __shfl_xor(st.l, 32);
      const float f = gate[2] / ltot;
#pragma unroll
      for (int j = 0; j < Fr::NDV; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) res[j][r] += f * st.o[j][r];
    }
    if (wave_active && valid) {
      T* orow = out + (tok_q * H + h) * D;
#pragma unroll
      for (int j = 0; j < Fr::NDV; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) orow[32 * j + res_row(r, g)] = Tr<DT>::cvt(res[j][r]);
    }
  }
}

template <int DT, int D>
hipError_t run_select(const ssa_plan_s* p, int H, int topk, float sl2, const void* q,
                      const FwdWs& w, int32_t* sel, hipStream_t s) {
  using T = typename Tr<DT>::T;
  const int Mp = (int)round_up(p->M, KT);
  const size_t shm = (size_t)Mp * sizeof(float);
  hipLaunchKernelGGL((k_select<DT, D>), dim3((unsigned)(p->M * H)), dim3(NT), shm, s,
                     (const T*)q, (const T*)w.ksplit, (const T*)w.vtil_t, p->perm, p->blk_off,
                     p->lpt, (int)p->M, Mp, H, p->n, sl2, topk, (T*)w.oc, sel);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t run_attend(const ssa_plan_s* p, int H, int topk, float sl2, const void* q,
                      const void* k, const void* v, const void* gates, const FwdWs& w,
                      const int32_t* sel, void* out, hipStream_t s) {
  using T = typename Tr<DT>::T;
  hipLaunchKernelGGL((k_attend<DT, D>), dim3((unsigned)(p->M * H)), dim3(NT), 0, s, (const T*)q,
                     (const T*)k, (const T*)v, (const T*)gates, p->perm, p->blk_off, p->blk_cell,
                     p->cell_off, p->cell_blk, p->lpt, sel, (const T*)w.oc, (int)p->M, H, p->n,
                     topk, sl2, (T*)out);
  return hipGetLastError();
}

template <int DT>
hipError_t run_pool(const ssa_plan_s* p, int H, int d, const void* k, const void* v,
                    const void* wk, const void* wv, const FwdWs& w, hipStream_t s) {
  using T = typename Tr<DT>::T;
  const int Mp = (int)round_up(p->M, KT);
  const int VEC = 16 / sizeof(T), CH = d / VEC, RSUB = 256 / CH;
  const size_t shm = (size_t)(2 * RSUB * d + 2 * d) * sizeof(float);
  hipLaunchKernelGGL((k_pool<DT>), dim3(Mp, H), dim3(256), shm, s, (const T*)k, (const T*)v,
                     (const T*)wk, (const T*)wv, p->perm, p->blk_off, (int)p->M, Mp, H, d,
                     (T*)w.ksplit, (T*)w.vtil_t);
  return hipGetLastError();
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
    case SSA_F32: return run_pool<DT_F32>(p, H, d, k, v, wk, wv, w, s);
    case SSA_F16: return run_pool<DT_F16>(p, H, d, k, v, wk, wv, w, s);
    case SSA_BF16: return run_pool<DT_BF16>(p, H, d, k, v, wk, wv, w, s);
  }
  return hipErrorInvalidValue;
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
