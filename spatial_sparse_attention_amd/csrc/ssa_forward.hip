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
//   pass 1 computes S^T = Ktil Q^T (a lane holds one query, 16 keys), keeps an
//          online softmax, accumulates O^T, and yields o_c and the exact
//          log-sum-exp;
//   pass 2 computes S = Q Ktil^T (a lane holds one key, 16 queries), so the
//          importance column sums over the block's queries are register sums.
// The pooled keys are fp32; they enter the MFMA as two (f16) or three (bf16) dtype
// planes whose sum reproduces the fp32 value, so the scores that decide the top-k
// carry fp32-level error.
#include <hip/hip_runtime.h>
#include <type_traits>
#include "ssa_internal.h"
#include "ssa_mfma.h"

namespace {

constexpr int KT = 32;            // keys per tile
constexpr int SEL_RT = 1;         // compressed/select: 32-row query tiles per wave
constexpr int SEL_WAVES = 8;      //   and waves per workgroup (256 rows per sweep)
constexpr int ATT_RT = 2;         // selected/window: 32-row query tiles per wave
constexpr int ATT_WAVES = 4;      //   and waves per workgroup (256 rows per chunk)
constexpr int ATT_ROWS = 32 * ATT_RT * ATT_WAVES;
constexpr float RESCALE_SLACK = 8.f;  // log2 units the running max may lag the true max

// ------------------------------------------------------------------ tile geometry
template <int DT, int D>
struct Cfg {
  using T = typename Tr<DT>::T;
  using F = typename Tr<DT>::frag;
  static constexpr int NS = Tr<DT>::NSPLIT;
  static constexpr int KS = Tr<DT>::KS, KPL = Tr<DT>::KPL;
  static constexpr int NKS = D / KS;                    // K steps over the head dim
  static constexpr int NDV = D / 32;                    // 32-wide output column tiles
  static constexpr int EPC = 16 / sizeof(T);            // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;                   // data chunks per row
  static constexpr int KROW = D + 16 / sizeof(T);       // K tile row (b128 fragment reads)
  static constexpr int VROW = D + 32 / sizeof(T);       // V tile row (transpose reads)
  static constexpr int KTILE = KT * KROW, VTILE = KT * VROW;
  static constexpr int KCH = KTILE * sizeof(T) / 16;    // 16-byte chunks of a K tile
  static constexpr int VCH = VTILE * sizeof(T) / 16;
  static constexpr int STAGE = NS * KTILE + VTILE;      // pooled stage (elements)
  static constexpr int PK = KT / KS;                    // K steps over a 32-key tile (PV)
};

// ------------------------------------------------------------------ pooling
// grid (Mp, H).  ktil[h,b] = mean_{i in b} K[i,h] @ Wk ; same for V.  Writes the fp32
// pooled key split into NSPLIT dtype planes and the pooled value, in the per-(head, tile)
// stage layout; row padding and padding blocks (b >= M) are zero.
template <int DT, int D>
__global__ __launch_bounds__(256) void k_pool(
    const typename Tr<DT>::T* __restrict__ kin, const typename Tr<DT>::T* __restrict__ vin,
    const typename Tr<DT>::T* __restrict__ wk, const typename Tr<DT>::T* __restrict__ wv,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ blk_off, int M, int Mp, int H,
    typename Tr<DT>::T* __restrict__ pooled) {
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  constexpr int NS = C::NS, VEC = C::EPC, CH = C::CPR, RSUB = 256 / CH;
  constexpr int U = 4;  // rows in flight per thread
  __shared__ float redk[RSUB * D], redv[RSUB * D], kbar[D], vbar[D];
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  T* stg = pooled + ((int64_t)h * (Mp / KT) + b / KT) * C::STAGE;
  T* krow = stg + (b % KT) * C::KROW;                    // plane s at + s * KTILE
  T* vrow = stg + NS * C::KTILE + (b % KT) * C::VROW;
  for (int j = (b >= M ? 0 : D) + tid; j < C::KROW; j += 256)
    for (int s = 0; s < NS; ++s) krow[s * C::KTILE + j] = (T)0.f;
  for (int j = (b >= M ? 0 : D) + tid; j < C::VROW; j += 256) vrow[j] = (T)0.f;
  if (b >= M) return;
  const int r0 = blk_off[b], r1 = blk_off[b + 1];
  const int sub = tid / CH, ch = tid % CH;
  if (sub < RSUB) {
    float ak[VEC], av[VEC];
    for (int e = 0; e < VEC; ++e) ak[e] = av[e] = 0.f;
    for (int r = r0 + sub; r < r1; r += U * RSUB) {
      uint4 kb[U], vb[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int rr = r + u * RSUB;
        if (rr < r1) {
          const int64_t base = ((int64_t)perm[rr] * H + h) * D + ch * VEC;
          kb[u] = *reinterpret_cast<const uint4*>(kin + base);
          vb[u] = *reinterpret_cast<const uint4*>(vin + base);
        } else {
          kb[u] = vb[u] = make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const T* kp = reinterpret_cast<const T*>(&kb[u]);
        const T* vp = reinterpret_cast<const T*>(&vb[u]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          ak[e] += Tr<DT>::up(kp[e]);
          av[e] += Tr<DT>::up(vp[e]);
        }
      }
    }
    for (int e = 0; e < VEC; ++e) {
      redk[sub * D + ch * VEC + e] = ak[e];
      redv[sub * D + ch * VEC + e] = av[e];
    }
  }
  __syncthreads();
  const float inv = 1.f / (float)(r1 - r0);
  for (int j = tid; j < 2 * D; j += 256) {
    const float* red = j < D ? redk : redv;
    const int c = j < D ? j : j - D;
    float s = 0.f;
    for (int u = 0; u < RSUB; ++u) s += red[u * D + c];
    (j < D ? kbar : vbar)[c] = s * inv;
  }
  __syncthreads();
  for (int j = tid; j < 2 * D; j += 256) {
    const bool isk = j < D;
    const int c = isk ? j : j - D;
    const T* W = isk ? wk : wv;
    const float* xb = isk ? kbar : vbar;
    float acc = 0.f;
    for (int i = 0; i < D; ++i) acc += xb[i] * Tr<DT>::up(W[(int64_t)i * D + c]);
    if (isk) {
      float rem = acc;
      for (int s = 0; s < NS; ++s) {
        const T part = Tr<DT>::cvt(rem);
        krow[s * C::KTILE + c] = part;
        rem -= Tr<DT>::up(part);
      }
    } else {
      vrow[c] = Tr<DT>::cvt(acc);
    }
  }
}

// ------------------------------------------------------------------ MFMA building blocks
// Reduction with the other half of the wave (lanes l and l^32 hold the same query row):
// v_permlane32_swap returns the pair {x[l], x[l^32]} in its two results.
__device__ inline float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A operand (V^T) of O^T += V^T P^T, K step ks of a 32-key tile stored row-major in LDS
// (vt[key][dv], row stride VROW), output columns 32*j .. 32*j+31.  Lane l covers
// dv = 32j + l%32 and the keys held by P^T registers ks*KPL .. ks*KPL + KPL - 1, i.e.
// keys 16ks + 4g + {0..3} and 16ks + 8 + 4g + {0..3} (g = l/32) for 16-bit types.
template <int DT, int D>
__device__ inline typename Tr<DT>::frag vt_frag(const typename Tr<DT>::T* vt, int ks, int j, int lane) {
  using C = Cfg<DT, D>;
  if constexpr (C::KPL == 1) {
    return vt[res_row(ks, lane >> 5) * C::VROW + 32 * j + (lane & 31)];
  } else {
    const int i = lane & 15, G = lane >> 4;
    const typename Tr<DT>::T* p =
        vt + (16 * ks + 4 * (G >> 1) + (i >> 2)) * C::VROW + 32 * j + 16 * (G & 1) + 4 * (i & 3);
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    const u2 a = __builtin_bit_cast(u2, lds_read_tr16(p));
    const u2 b = __builtin_bit_cast(u2, lds_read_tr16(p + 8 * C::VROW));
    const u4 u = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(typename Tr<DT>::frag, u);
  }
}

// The V^T fragments of one 32-key tile, read before the next tile's copy is issued: the
// transpose reads carry no alias information, so reading them after the copy is issued
// would make the compiler wait for that copy.
template <int DT, int D>
struct VFrags {
  typename Tr<DT>::frag f[Cfg<DT, D>::PK][Cfg<DT, D>::NDV];
  __device__ inline void read(const typename Tr<DT>::T* vt, int lane) {
#pragma unroll
    for (int ks = 0; ks < Cfg<DT, D>::PK; ++ks)
#pragma unroll
      for (int j = 0; j < Cfg<DT, D>::NDV; ++j) f[ks][j] = vt_frag<DT, D>(vt, ks, j, lane);
  }
};

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
  if constexpr (Tr<DT>::KPL == 1) {
    f = 0.f;
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) f[t] = (typename Tr<DT>::T)0.f;
  }
  return f;
}

__device__ inline ssa_f16v zero16() {
  ssa_f16v z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// Online softmax of one query row (duplicated in lanes c and c+32, which hold different
// keys of the row), in log2 units.  The running max m may lag the true max by up to
// RESCALE_SLACK, so the accumulator is rescaled only when a tile raises the max by more
// than that (probabilities stay below 2^RESCALE_SLACK); the normalisation by l and
// lse = m + log2(l) are exact either way.
template <int NDV>
struct Online {
  float m, l;
  ssa_f16v o[NDV];
  __device__ inline void init() {
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int j = 0; j < NDV; ++j) o[j] = zero16();
  }
  // s: raw scores (-inf for masked keys); sl2 = scale * log2(e) > 0.  Returns p in s.
  __device__ inline void update(ssa_f16v& s, float sl2) {
    float mt = fmaxf(s[0], s[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) mt = fmaxf(mt, fmaxf(s[r], s[r + 1]));
    mt = xor32_max(mt) * sl2;
    if (__builtin_amdgcn_ballot_w64(mt > m + RESCALE_SLACK)) {
      const float mn = fmaxf(m, mt);
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int j = 0; j < NDV; ++j) o[j] *= alpha;
      m = mn;
    }
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = fast_exp2(__builtin_fmaf(s[r], sl2, -m));
      sum += s[r];
    }
    l += sum;
  }
};

// S^T tile (keys x queries) from a K tile in LDS ([32][KROW]).
template <int DT, int D>
__device__ inline ssa_f16v st_tile(const typename Tr<DT>::T* kt, const typename Tr<DT>::frag* qf,
                                   ssa_f16v acc, int lane) {
  using C = Cfg<DT, D>;
  const typename Tr<DT>::T* row = kt + (lane & 31) * C::KROW + (lane >> 5) * C::KPL;
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) acc = Tr<DT>::mma(load_frag<DT>(row + ks * C::KS), qf[ks], acc);
  return acc;
}

// S tile (queries x keys) from a K tile in LDS.
template <int DT, int D>
__device__ inline ssa_f16v s_tile(const typename Tr<DT>::T* kt, const typename Tr<DT>::frag* qf,
                                  ssa_f16v acc, int lane) {
  using C = Cfg<DT, D>;
  const typename Tr<DT>::T* row = kt + (lane & 31) * C::KROW + (lane >> 5) * C::KPL;
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) acc = Tr<DT>::mma(qf[ks], load_frag<DT>(row + ks * C::KS), acc);
  return acc;
}

template <int DT, int D>
__device__ inline void pv_tile(Online<D / 32>& st, const ssa_f16v& p, const VFrags<DT, D>& vf) {
  using C = Cfg<DT, D>;
#pragma unroll
  for (int ks = 0; ks < C::PK; ++ks) {
    const typename Tr<DT>::frag pf = p_frag<DT>(p, ks);
#pragma unroll
    for (int j = 0; j < C::NDV; ++j) st.o[j] = Tr<DT>::mma(vf.f[ks][j], pf, st.o[j]);
  }
}

template <int DT, int D>
__device__ inline void load_q(typename Tr<DT>::frag* qf, const typename Tr<DT>::T* qrow, bool valid,
                              int lane) {
  using C = Cfg<DT, D>;
#pragma unroll
  for (int s = 0; s < C::NKS; ++s)
    qf[s] = valid ? load_frag<DT>(qrow + s * C::KS + (lane >> 5) * C::KPL) : zero_frag<DT>();
}

// ------------------------------------------------------------------ direct global->LDS copies
// global_load_lds_dwordx4: lane l of a wave writes its 16 bytes at the (wave-uniform) LDS
// base + 16*l.  A tile is a sequence of 16-byte positions; instruction i covers positions
// 64i .. 64i+63, and the workgroup's waves take instructions round-robin.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ inline void dma16(const void* g, void* lds_instr_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds_instr_base, 16, 0, 0);
}
__device__ inline void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int NW>
__device__ inline void dma_contiguous(void* lds, const void* g, int nchunks, int wave, int lane) {
  for (int i = wave; i * 64 < nchunks; i += NW) {
    const int p = i * 64 + lane;
    if (p < nchunks) dma16((const char*)g + (int64_t)p * 16, (char*)lds + i * 1024);
  }
}

// ------------------------------------------------------------------ compressed + select
// One workgroup per (query block, head), longest blocks first.  Each wave owns RT row
// tiles of 32 queries, so every K or V fragment read from LDS feeds RT MFMAs.
template <int DT, int D>
__global__ __launch_bounds__(64 * SEL_WAVES) void k_select(
    const typename Tr<DT>::T* __restrict__ q, const typename Tr<DT>::T* __restrict__ pooled,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ blk_off,
    const int32_t* __restrict__ lpt, int M, int Mp, int H, int64_t N, float sl2, int topk,
    typename Tr<DT>::T* __restrict__ oc, int32_t* __restrict__ sel) {
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  using F = typename Tr<DT>::frag;
  constexpr int NS = C::NS;
  constexpr int RT = SEL_RT;
  constexpr int ROWS = 32 * RT * SEL_WAVES;
  __shared__ __attribute__((aligned(1024))) T stage0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) T stage1[C::STAGE];
  __shared__ float stage_sum[2][SEL_WAVES][32];
  __shared__ float lse_lds[ROWS];
  __shared__ int32_t pick[256];
  extern __shared__ float sig[];  // [Mp]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, c = lane & 31;
  const int h = blockIdx.x % H;
  const int b = lpt[blockIdx.x / H];
  const int r0 = blk_off[b], rows = blk_off[b + 1] - r0;
  for (int j = tid; j < Mp; j += 64 * SEL_WAVES) sig[j] = 0.f;
  const int ntile = Mp / KT;
  const T* pstage = pooled + (int64_t)h * ntile * C::STAGE;
  constexpr int NCH1 = C::STAGE * sizeof(T) / 16, NCH2 = NS * C::KCH;

  for (int sw = 0; sw * ROWS < rows; ++sw) {
    const int wbase = sw * ROWS + wave * 32 * RT;   // first row of this wave
    const bool wave_active = wbase < rows;
    F qf[RT][C::NKS];
    bool valid[RT];
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      const int my_row = wbase + 32 * u + c;
      valid[u] = my_row < rows;
      load_q<DT, D>(qf[u], q + ((int64_t)(valid[u] ? perm[r0 + my_row] : 0) * H + h) * D, valid[u], lane);
    }

    // ---------------- pass 1: online softmax over all pooled keys -> o_c, lse
    Online<C::NDV> st[RT];
#pragma unroll
    for (int u = 0; u < RT; ++u) st[u].init();
    {
      auto p1 = [&](int t, T* cur, T* nxt) {
        dma_wait();
        __syncthreads();
        VFrags<DT, D> vf;
        if (wave_active) vf.read(cur + NS * C::KTILE, lane);
        if (t + 1 < ntile) dma_contiguous<SEL_WAVES>(nxt, pstage + (int64_t)(t + 1) * C::STAGE, NCH1, wave, lane);
        if (wave_active) {
          ssa_f16v acc[RT];
#pragma unroll
          for (int u = 0; u < RT; ++u) acc[u] = zero16();
          const T* krow = cur + (lane & 31) * C::KROW + (lane >> 5) * C::KPL;
#pragma unroll
          for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int ks = 0; ks < C::NKS; ++ks) {
              const F kf = load_frag<DT>(krow + s * C::KTILE + ks * C::KS);
#pragma unroll
              for (int u = 0; u < RT; ++u) acc[u] = Tr<DT>::mma(kf, qf[u][ks], acc[u]);
            }
#pragma unroll
          for (int u = 0; u < RT; ++u) {
            if (t == ntile - 1) {
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (t * KT + res_row(r, g) >= M) acc[u][r] = -INFINITY;
            }
            st[u].update(acc[u], sl2);
          }
#pragma unroll
          for (int ks = 0; ks < C::PK; ++ks)
#pragma unroll
            for (int u = 0; u < RT; ++u) {
              const F pf = p_frag<DT>(acc[u], ks);
#pragma unroll
              for (int j = 0; j < C::NDV; ++j) st[u].o[j] = Tr<DT>::mma(vf.f[ks][j], pf, st[u].o[j]);
            }
        }
      };
      __syncthreads();  // the previous sweep is done with both stage buffers
      dma_contiguous<SEL_WAVES>(stage0, pstage, NCH1, wave, lane);
      for (int t = 0; t < ntile; t += 2) {
        p1(t, stage0, stage1);
        if (t + 1 < ntile) p1(t + 1, stage1, stage0);
      }
    }
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      const float ltot = xor32_sum(st[u].l);
      const int my_row = wbase + 32 * u + c;
      if (wave_active && valid[u]) {
        const float inv = 1.f / ltot;
        T* orow = oc + ((int64_t)h * N + r0 + my_row) * D;
#pragma unroll
        for (int j = 0; j < C::NDV; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) orow[32 * j + res_row(r, g)] = Tr<DT>::cvt(st[u].o[j][r] * inv);
      }
      // rows past the block get +inf, so their probabilities in pass 2 are exactly zero
      if (g == 0) lse_lds[wave * 32 * RT + 32 * u + c] = valid[u] ? st[u].m + fast_log2(ltot) : INFINITY;
    }
    __syncthreads();

    // ---------------- pass 2: importance column sums (S layout)
    float lrow[RT][16];
#pragma unroll
    for (int u = 0; u < RT; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) lrow[u][r] = lse_lds[wave * 32 * RT + 32 * u + res_row(r, g)];
    {
      auto fold = [&](int t) {  // sum the per-wave column sums of tile t into sigma (fixed order)
        if (tid < 32) {
          const int key = t * KT + tid;
          float s = stage_sum[t & 1][0][tid];
#pragma unroll
          for (int w = 1; w < SEL_WAVES; ++w) s += stage_sum[t & 1][w][tid];
          if (key < M) sig[key] += s;
        }
      };
      auto p2 = [&](int t, T* cur, T* nxt) {
        dma_wait();
        __syncthreads();
        if (t + 1 < ntile) dma_contiguous<SEL_WAVES>(nxt, pstage + (int64_t)(t + 1) * C::STAGE, NCH2, wave, lane);
        if (t > 0) fold(t - 1);
        float colsum = 0.f;
        if (wave_active) {
          ssa_f16v acc[RT];
#pragma unroll
          for (int u = 0; u < RT; ++u) acc[u] = zero16();
          const T* krow = cur + (lane & 31) * C::KROW + (lane >> 5) * C::KPL;
#pragma unroll
          for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int ks = 0; ks < C::NKS; ++ks) {
              const F kf = load_frag<DT>(krow + s * C::KTILE + ks * C::KS);
#pragma unroll
              for (int u = 0; u < RT; ++u) acc[u] = Tr<DT>::mma(qf[u][ks], kf, acc[u]);
            }
#pragma unroll
          for (int u = 0; u < RT; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) colsum += fast_exp2(__builtin_fmaf(acc[u][r], sl2, -lrow[u][r]));
          colsum = xor32_sum(colsum);
        }
        if (g == 0) stage_sum[t & 1][wave][c] = colsum;
      };
      dma_contiguous<SEL_WAVES>(stage0, pstage, NCH2, wave, lane);
      for (int t = 0; t < ntile; t += 2) {
        p2(t, stage0, stage1);
        if (t + 1 < ntile) p2(t + 1, stage1, stage0);
      }
      __syncthreads();
      fold(ntile - 1);
      __syncthreads();
    }
  }

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
      for (int i = 1; i < keff; ++i) {
        int x = pick[i], j = i - 1;
        while (j >= 0 && pick[j] > x) { pick[j + 1] = pick[j]; --j; }
        pick[j + 1] = x;
      }
    }
    for (int t = lane; t < topk; t += 64) sel[((int64_t)h * M + b) * topk + t] = t < keff ? pick[t] : -1;
  }
}

// ------------------------------------------------------------------ selected + window + combine
// A key set is a list of blocks (the selected blocks, or the blocks of the query's window
// cell), concatenated in sorted token order and cut into 32-key tiles.  A stage holds the
// tile's K rows ([32][KROW]) followed by its V rows ([32][VROW]), copied straight from the
// caller's K and V through the token permutation.  Keys past the end of the set reuse the
// set's first key (finite values; their scores are masked).
template <int DT, int D>
struct Gather {
  using C = Cfg<DT, D>;
  static constexpr int KRC = C::KCH / KT, VRC = C::VCH / KT;  // chunks per padded row
  static constexpr int NPOS = C::KCH + C::VCH;
  static constexpr int NINSTR = (NPOS + 63) / 64;
  static constexpr int NI = (NINSTR + ATT_WAVES - 1) / ATT_WAVES;  // copies per lane per tile
  int32_t row[NI];    // tile row of each copy (-1: none)
  int32_t goff[NI];   // element offset inside the token's head row, with bit 30 set for V
  int32_t tok[NI];
  __device__ inline void init(int wave, int lane) {
#pragma unroll
    for (int m = 0; m < NI; ++m) {
      const int i = wave + m * ATT_WAVES, p = i * 64 + lane;
      const bool isk = p < C::KCH;
      const int q = isk ? p : p - C::KCH;
      const int rr = isk ? q / KRC : q / VRC, ch = isk ? q % KRC : q % VRC;
      const bool ok = i < NINSTR && p < NPOS && ch < C::CPR;
      row[m] = ok ? rr : -1;
      goff[m] = ch * C::EPC + (isk ? 0 : (1 << 30));
    }
  }
  // tokens of this lane's copies for the tile starting at key k0
  __device__ inline void lookup(int k0, int total, int L, const int32_t* pre, const int32_t* lst_off,
                                const int32_t* __restrict__ perm) {
#pragma unroll
    for (int m = 0; m < NI; ++m) {
      int j = k0 + (row[m] < 0 ? 0 : row[m]);
      if (j >= total) j = 0;
      int lo = 0, hi = L - 1;  // last list entry starting at or before key j (none to search
      while (lo < hi) {        // when the list is one block)
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= j) lo = mid; else hi = mid - 1;
      }
      tok[m] = perm[lst_off[lo] + (j - pre[lo])];
    }
  }
  __device__ inline void issue(typename Tr<DT>::T* stage, const typename Tr<DT>::T* kin,
                               const typename Tr<DT>::T* vin, int H, int h, int wave) const {
#pragma unroll
    for (int m = 0; m < NI; ++m) {
      if (row[m] >= 0) {
        const bool isv = goff[m] & (1 << 30);
        const typename Tr<DT>::T* src = (isv ? vin : kin) + ((int64_t)tok[m] * H + h) * D + (goff[m] & ((1 << 30) - 1));
        dma16(src, stage + (wave + m * ATT_WAVES) * 64 * C::EPC);
      }
    }
  }
};

template <int DT, int D>
__device__ inline void gathered_branch(
    Online<D / 32>* st, const Gather<DT, D>& ga0, const int32_t* blist, int nlist,
    const typename Tr<DT>::frag (*qf)[Cfg<DT, D>::NKS], const typename Tr<DT>::T* __restrict__ kin,
    const typename Tr<DT>::T* __restrict__ vin, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ blk_off, int H, int h, float sl2, bool wave_active,
    typename Tr<DT>::T* stage0, typename Tr<DT>::T* stage1, int32_t* pre, int32_t* lst_off) {
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  using F = typename Tr<DT>::frag;
  constexpr int NTH = 64 * ATT_WAVES;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, wave = tid >> 6;
#pragma unroll
  for (int u = 0; u < ATT_RT; ++u) st[u].init();
  Gather<DT, D> ga = ga0;
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
    const int ntile = (total + KT - 1) / KT;
    auto step = [&](int t, T* cur, T* nxt) {
      dma_wait();
      __syncthreads();
      VFrags<DT, D> vf;
      if (wave_active) vf.read(cur + C::KTILE, lane);
      if (t + 1 < ntile) ga.issue(nxt, kin, vin, H, h, wave);
      if (t + 2 < ntile) ga.lookup((t + 2) * KT, total, L, pre, lst_off, perm);
      if (wave_active) {
        ssa_f16v acc[ATT_RT];
#pragma unroll
        for (int u = 0; u < ATT_RT; ++u) acc[u] = zero16();
        const T* krow = cur + (lane & 31) * C::KROW + (lane >> 5) * C::KPL;
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
          const F kf = load_frag<DT>(krow + ks * C::KS);
#pragma unroll
          for (int u = 0; u < ATT_RT; ++u) acc[u] = Tr<DT>::mma(kf, qf[u][ks], acc[u]);
        }
#pragma unroll
        for (int u = 0; u < ATT_RT; ++u) {
          if (t == ntile - 1) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (t * KT + res_row(r, g) >= total) acc[u][r] = -INFINITY;
          }
          st[u].update(acc[u], sl2);
        }
#pragma unroll
        for (int ks = 0; ks < C::PK; ++ks)
#pragma unroll
          for (int u = 0; u < ATT_RT; ++u) {
            const F pf = p_frag<DT>(acc[u], ks);
#pragma unroll
            for (int j = 0; j < C::NDV; ++j) st[u].o[j] = Tr<DT>::mma(vf.f[ks][j], pf, st[u].o[j]);
          }
      }
    };
    ga.lookup(0, total, L, pre, lst_off, perm);
    ga.issue(stage0, kin, vin, H, h, wave);
    if (ntile > 1) ga.lookup(KT, total, L, pre, lst_off, perm);
    for (int t = 0; t < ntile; t += 2) {
      step(t, stage0, stage1);
      if (t + 1 < ntile) step(t + 1, stage1, stage0);
    }
    dma_wait();
  }
}

// One workgroup per (ATT_ROWS-row chunk of a query block, head); grid = lpt rank x chunk x head.
template <int DT, int D>
__global__ __launch_bounds__(64 * ATT_WAVES) __attribute__((amdgpu_waves_per_eu(2))) void k_attend(
    const typename Tr<DT>::T* __restrict__ q, const typename Tr<DT>::T* __restrict__ kin,
    const typename Tr<DT>::T* __restrict__ vin, const typename Tr<DT>::T* __restrict__ gates,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ blk_off,
    const int32_t* __restrict__ blk_cell, const int32_t* __restrict__ cell_off,
    const int32_t* __restrict__ cell_blk, const int32_t* __restrict__ lpt,
    const int32_t* __restrict__ sel, const typename Tr<DT>::T* __restrict__ oc, int M, int H,
    int nchunk, int64_t N, int topk, float sl2, typename Tr<DT>::T* __restrict__ out) {
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  using F = typename Tr<DT>::frag;
  constexpr int NTH = 64 * ATT_WAVES;
  __shared__ __attribute__((aligned(1024))) T stage0[C::KTILE + C::VTILE];
  __shared__ __attribute__((aligned(1024))) T stage1[C::KTILE + C::VTILE];
  __shared__ int32_t pre[NTH + 1];
  __shared__ int32_t lst_off[NTH];
  __shared__ int32_t sel_lds[256];
  // the selected branch's weighted output, parked in LDS as fp16 while the window branch
  // runs (16-bit dtypes: the rounding is far below the output dtype's); fp32 keeps it in
  // registers
  constexpr bool PARK = DT != DT_F32;
  __shared__ _Float16 res_lds[PARK ? ATT_WAVES : 1][PARK ? ATT_RT * C::NDV * 16 : 1][64];
  ssa_f16v res[PARK ? 1 : ATT_RT][PARK ? 1 : C::NDV];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, c = lane & 31;
  const int h = blockIdx.x % H;
  const int chunk = (blockIdx.x / H) % nchunk;
  const int b = lpt[blockIdx.x / (H * nchunk)];
  const int r0 = blk_off[b], rows = blk_off[b + 1] - r0;
  if (chunk * ATT_ROWS >= rows) return;  // uniform across the workgroup
  int nsel = 0;
  const int32_t* srow = sel + ((int64_t)h * M + b) * topk;
  for (int t = 0; t < topk; ++t) nsel += srow[t] >= 0;
  for (int t = tid; t < nsel; t += NTH) sel_lds[t] = srow[t];
  const int cell = blk_cell[b];
  const int c0 = cell_off[cell], c1 = cell_off[cell + 1];

  const int wbase = chunk * ATT_ROWS + wave * 32 * ATT_RT;
  const bool wave_active = wbase < rows;
  F qf[ATT_RT][C::NKS];
  int64_t tok_q[ATT_RT];
  bool valid[ATT_RT];
#pragma unroll
  for (int u = 0; u < ATT_RT; ++u) {
    const int my_row = wbase + 32 * u + c;
    valid[u] = my_row < rows;
    tok_q[u] = valid[u] ? perm[r0 + my_row] : 0;
    load_q<DT, D>(qf[u], q + (tok_q[u] * H + h) * D, valid[u], lane);
  }
  Gather<DT, D> ga;
  ga.init(wave, lane);

  Online<C::NDV> st[ATT_RT];
  gathered_branch<DT, D>(st, ga, sel_lds, nsel, qf, kin, vin, perm, blk_off, H, h, sl2, wave_active,
                         stage0, stage1, pre, lst_off);
#pragma unroll
  for (int u = 0; u < ATT_RT; ++u) {
    const float g1 = valid[u] ? Tr<DT>::up(gates[(tok_q[u] * H + h) * 3 + 1]) : 0.f;
    const float f = g1 / xor32_sum(st[u].l);
#pragma unroll
    for (int j = 0; j < C::NDV; ++j) {
      if constexpr (PARK) {
#pragma unroll
        for (int r = 0; r < 16; ++r) res_lds[wave][(u * C::NDV + j) * 16 + r][lane] = (_Float16)(st[u].o[j][r] * f);
      } else {
        res[u][j] = st[u].o[j] * f;
      }
    }
  }
  gathered_branch<DT, D>(st, ga, cell_blk + c0, c1 - c0, qf, kin, vin, perm, blk_off, H, h, sl2,
                         wave_active, stage0, stage1, pre, lst_off);
#pragma unroll
  for (int u = 0; u < ATT_RT; ++u) {
    const float ltot = xor32_sum(st[u].l);
    const int my_row = wbase + 32 * u + c;
    if (wave_active && valid[u]) {
      const float g0 = Tr<DT>::up(gates[(tok_q[u] * H + h) * 3 + 0]);
      const float g2 = Tr<DT>::up(gates[(tok_q[u] * H + h) * 3 + 2]);
      const float f = g2 / ltot;
      const T* orow = oc + ((int64_t)h * N + r0 + my_row) * D;
      T* dst = out + (tok_q[u] * H + h) * D;
#pragma unroll
      for (int j = 0; j < C::NDV; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dv = 32 * j + res_row(r, g);
          float rs;
          if constexpr (PARK) rs = (float)res_lds[wave][(u * C::NDV + j) * 16 + r][lane];
          else rs = res[u][j][r];
          dst[dv] = Tr<DT>::cvt(rs + f * st[u].o[j][r] + g0 * Tr<DT>::up(orow[dv]));
        }
    }
  }
}

// ------------------------------------------------------------------ launchers
template <int DT, int D>
hipError_t run_pool(const ssa_plan_s* p, int H, const void* k, const void* v, const void* wk,
                    const void* wv, const FwdWs& w, hipStream_t s) {
  using T = typename Tr<DT>::T;
  const int Mp = (int)round_up(p->M, KT);
  hipLaunchKernelGGL((k_pool<DT, D>), dim3(Mp, H), dim3(256), 0, s, (const T*)k, (const T*)v,
                     (const T*)wk, (const T*)wv, p->perm, p->blk_off, (int)p->M, Mp, H, (T*)w.pooled);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t run_select(const ssa_plan_s* p, int H, int topk, float sl2, const void* q,
                      const FwdWs& w, int32_t* sel, hipStream_t s) {
  using T = typename Tr<DT>::T;
  const int Mp = (int)round_up(p->M, KT);
  const size_t shm = (size_t)Mp * sizeof(float);
  hipLaunchKernelGGL((k_select<DT, D>), dim3((unsigned)(p->M * H)), dim3(64 * SEL_WAVES), shm, s,
                     (const T*)q, (const T*)w.pooled, p->perm, p->blk_off, p->lpt, (int)p->M, Mp, H,
                     p->n, sl2, topk, (T*)w.oc, sel);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t run_attend(const ssa_plan_s* p, int H, int topk, float sl2, const void* q,
                      const void* k, const void* v, const void* gates, const FwdWs& w,
                      const int32_t* sel, void* out, hipStream_t s) {
  using T = typename Tr<DT>::T;
  const int nchunk = (p->max_rows + ATT_ROWS - 1) / ATT_ROWS;
  hipLaunchKernelGGL((k_attend<DT, D>), dim3((unsigned)(p->M * H * nchunk)), dim3(64 * ATT_WAVES), 0,
                     s, (const T*)q, (const T*)k, (const T*)v, (const T*)gates, p->perm, p->blk_off,
                     p->blk_cell, p->cell_off, p->cell_blk, p->lpt, sel, (const T*)w.oc, (int)p->M,
                     H, nchunk, p->n, topk, sl2, (T*)out);
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
