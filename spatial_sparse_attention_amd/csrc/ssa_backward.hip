// SSA backward for gfx950: gradients of the gated three-branch output with respect to Q,
// K, V and the gates, with the block selection held fixed (as the forward chose it) and no
// gradient through the importance scores or into W.
//
// For each branch x (compressed, selected, window) with probabilities P (recomputed from
// the forward's saved log-sum-exp), dO_x = g_x dO and o_x the branch output:
//   dgates[x] = <dO, o_x>,   D_x = <dO_x, o_x> = g_x dgates[x],
//   dS = P o (dO_x V^T - D_x),  dq += scale dS K,  dk += scale dS^T q,  dv += P^T dO_x.
// The compressed branch's keys are the pooled keys; their gradients flow back through
// W and the block mean: dK_i += (W_k dktil_b) / n_b, dV_i += (W_v dvtil_b) / n_b.
//
// Kernels: prep (dgates, D); dq (query-major, S^T layout as in the forward); the inverse
// selection (which query blocks selected each key block, by a stable radix sort, so every
// key-side sum runs in a fixed order); dk/dv of the selected and window branches
// (key-major, S layout so the queries are the MFMA contraction index); the compressed
// key side over query chunks; the pooling backward, which folds the chunk partials in
// order into one dK, dV term per (block, head), added by the dk/dv kernel as it writes.  No
// atomics: results are bitwise reproducible.
#include <hip/hip_runtime.h>
#include "ssa_internal.h"
#include "ssa_mfma.h"
#include "ssa_tiles.h"

namespace {

using namespace ssa_dev;
constexpr int BW = 4;           // waves per workgroup
constexpr int BROWS = 32 * BW;  // query rows (dq) or keys (dk/dv) per workgroup

struct BwdWs {
  float* D;                    // [3][H][N]
  uint32_t *ka, *kb;           // inverse-selection sort keys (E = H*M*topk)
  int32_t *va, *vb, *rank, *hist, *part;
  int32_t* inv_off;            // [H*M + 1]
  float *part_k, *part_v;      // [qch][H][Mp][d] compressed key-side partials
  float* ukv;                  // [2][H][Mp][d] per-block dK, dV terms of the compressed branch
  int qch;
};

int cmp_chunks(int64_t Mp, int H) {
  const int64_t groups = (Mp / KT + BW - 1) / BW * H;
  int64_t q = (1024 + groups - 1) / groups;
  return (int)(q < 1 ? 1 : (q > 64 ? 64 : q));
}

size_t carve(Carver& c, const ssa_plan_s* p, int H, int d, int topk, BwdWs* w) {
  const int64_t M = p->M > 0 ? p->M : 1, n1 = p->n > 0 ? p->n : 1;
  const int64_t Mp = pooled_rows(M);
  const int64_t E = (int64_t)H * M * topk;
  BwdWs t;
  t.qch = cmp_chunks(Mp, H);
  t.D = c.take<float>(3 * H * n1);
  t.ka = c.take<uint32_t>(E);
  t.kb = c.take<uint32_t>(E);
  t.va = c.take<int32_t>(E);
  t.vb = c.take<int32_t>(E);
  t.rank = c.take<int32_t>(E);
  t.hist = c.take<int32_t>(radix_hist_len(E));
  t.part = c.take<int32_t>(scan_part_len(radix_hist_len(E)));
  t.inv_off = c.take<int32_t>((int64_t)H * M + 1);
  t.part_k = c.take<float>((int64_t)t.qch * H * Mp * d);
  t.part_v = c.take<float>((int64_t)t.qch * H * Mp * d);
  t.ukv = c.take<float>((int64_t)2 * H * Mp * d);
  if (w) *w = t;
  return c.off;
}

// ------------------------------------------------------------------ prep
// dgates and D for the three branches.  A group of GS lanes per (sorted row r, head h): lane
// j of the group reads the j-th 16-byte chunk of dO's head row (and the matching fp32 chunks
// of the three saved branch outputs), so a group reads contiguous rows; the dot products are
// finished with shuffles inside the group.
template <int DT, int D>
__global__ __launch_bounds__(256) void k_bwd_prep(
    const typename Tr<DT>::T* __restrict__ dout, const typename Tr<DT>::T* __restrict__ gates,
    const float* __restrict__ obr, const int32_t* __restrict__ perm, int64_t N, int H,
    float* __restrict__ dgates, float* __restrict__ Dsave) {
  using T = typename Tr<DT>::T;
  constexpr int EPC = 16 / sizeof(T), CPR = D / EPC;
  constexpr int GS = CPR <= 16 ? 16 : (CPR <= 32 ? 32 : 64);  // lanes per head row
  static_assert(CPR <= GS, "one lane group per head row");
  const int64_t idx = ((int64_t)blockIdx.x * 256 + threadIdx.x) / GS;
  const int j = threadIdx.x & (GS - 1);
  const bool live = idx < N * H;
  const int64_t r = live ? idx / H : 0;
  const int h = live ? (int)(idx % H) : 0;
  const int64_t t = live ? perm[r] : 0;
  float acc[3] = {0.f, 0.f, 0.f};
  if (live && j < CPR) {
    const uint4 a = *reinterpret_cast<const uint4*>(dout + (t * H + h) * D + j * EPC);
    const T* ae = reinterpret_cast<const T*>(&a);
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const float* o = obr + (((int64_t)x * N + r) * H + h) * D + j * EPC;
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[x] += Tr<DT>::up(ae[e]) * o[e];
    }
  }
#pragma unroll
  for (int x = 0; x < 3; ++x)
#pragma unroll
    for (int off = GS / 2; off > 0; off >>= 1) acc[x] += __shfl_xor(acc[x], off, GS);
  if (live && j < 3) {
    const float v = j == 0 ? acc[0] : (j == 1 ? acc[1] : acc[2]);
    dgates[(t * H + h) * 3 + j] = v;
    Dsave[((int64_t)j * H + h) * N + r] = Tr<DT>::up(gates[(t * H + h) * 3 + j]) * v;
  }
}

// ------------------------------------------------------------------ list preparation
// Prefix offsets of a chunk (up to NTH entries) of a block list in LDS: lst_off[i] = first
// sorted row of block i, pre[i] = first set position of block i, pre[L] = set size.
template <int NTH>
__device__ inline int list_prefix(const int32_t* blist, int L, const int32_t* __restrict__ blk_off,
                                  int32_t* pre, int32_t* lst_off) {
  const int tid = threadIdx.x;
  __syncthreads();
  int sz = 0;
  if (tid < L) {
    const int bb = blist[tid];
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
  return pre[L];
}

// sorted row of set position j
__device__ inline int set_row(int j, int L, const int32_t* pre, const int32_t* lst_off) {
  int lo = 0, hi = L - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= j) lo = mid; else hi = mid - 1;
  }
  return lst_off[lo] + (j - pre[lo]);
}

// ------------------------------------------------------------------ dq (query-major)
// Per branch: tiles of keys; S^T = K Q^T, P^T from the saved lse, dP^T = V dO^T,
// dS^T = P^T o (g dP^T - D), dq^T += K^T dS^T.  The stage holds the K tile ([32][KROW])
// then the V tile ([32][VROW]).
template <int DT, int D>
struct DqState {
  using C = Cfg<DT, D>;
  using F = typename Tr<DT>::frag;
  F qf[C::NKS], dof[C::NKS];
  ssa_f16v dq[C::NDV];
  __device__ inline void tile(const typename Tr<DT>::T* st, int nvalid, float sl2, float lse,
                              float gx, float Dx, int lane) {
    const int g = lane >> 5;
    ssa_f16v s = st_tile<DT, D>(st, qf, zero16(), lane);
    // dP^T = V dO^T: the V tile rows are the A operand
    ssa_f16v dp = zero16();
    const typename Tr<DT>::T* vrow = st + C::KTILE + (lane & 31) * C::VROW + g * C::KPL;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) dp = Tr<DT>::mma(load_frag<DT>(vrow + ks * C::KS), dof[ks], dp);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = res_row(r, g) < nvalid ? fast_exp2(__builtin_fmaf(s[r], sl2, -lse)) : 0.f;
      s[r] = p * (gx * dp[r] - Dx);
    }
#pragma unroll
    for (int ks = 0; ks < C::PK; ++ks) {
      const F sf = p_frag<DT>(s, ks);
#pragma unroll
      for (int j = 0; j < C::NDV; ++j)
        dq[j] = Tr<DT>::mma(tr_frag<DT, C::KROW>(st, ks, j, lane), sf, dq[j]);
    }
  }
};

template <int DT, int D, bool BUF>
__global__ __launch_bounds__(64 * BW) void k_bwd_dq(
    const typename Tr<DT>::T* __restrict__ q, const typename Tr<DT>::T* __restrict__ kin,
    const typename Tr<DT>::T* __restrict__ vin, const typename Tr<DT>::T* __restrict__ gates,
    const typename Tr<DT>::T* __restrict__ dout, const typename Tr<DT>::T* __restrict__ pooled,
    const typename Tr<DT>::T* __restrict__ pooled_v, const float* __restrict__ lse3,
    const float* __restrict__ D3, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ blk_off, const int32_t* __restrict__ blk_cell,
    const int32_t* __restrict__ cell_off, const int32_t* __restrict__ cell_blk,
    const int32_t* __restrict__ lpt, const int32_t* __restrict__ sel, int M, int Mp, int H,
    int nchunk, int64_t N, int topk, float scale, float sl2, float* __restrict__ dq) {
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  constexpr int NTH = 64 * BW;
  __shared__ __attribute__((aligned(1024))) T stage[C::KTILE + C::VTILE];
  __shared__ int32_t pre[NTH + 1];
  __shared__ int32_t lst_off[NTH];
  __shared__ int32_t sel_lds[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, c = lane & 31;
  int unit, member;
  xcd_split(blockIdx.x, nchunk * H, unit, member);
  if (unit >= M) return;
  const int h = member % H, chunk = member / H;
  const int b = lpt[unit];
  const int r0 = blk_off[b], rows = blk_off[b + 1] - r0;
  if (chunk * BROWS >= rows) return;
  int nsel = 0;
  const int32_t* srow = sel + ((int64_t)h * M + b) * topk;
  for (int t = 0; t < topk; ++t) nsel += srow[t] >= 0;
  for (int t = tid; t < nsel; t += NTH) sel_lds[t] = srow[t];
  const int cell = blk_cell[b];
  const int cb0 = cell_off[cell], cb1 = cell_off[cell + 1];

  const int my_row = chunk * BROWS + wave * 32 + c;
  const bool valid = my_row < rows;
  const int64_t row = r0 + (valid ? my_row : 0);
  const int64_t tok = perm[row];
  DqState<DT, D> S;
  load_q<DT, D>(S.qf, q + (tok * H + h) * D, valid, lane);
  load_q<DT, D>(S.dof, dout + (tok * H + h) * D, valid, lane);
#pragma unroll
  for (int j = 0; j < C::NDV; ++j) S.dq[j] = zero16();
  float gx[3], lse[3], Dx[3];
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    gx[x] = valid ? Tr<DT>::up(gates[(tok * H + h) * 3 + x]) : 0.f;
    lse[x] = lse3[((int64_t)x * H + h) * N + row];
    Dx[x] = valid ? D3[((int64_t)x * H + h) * N + row] : 0.f;
  }

  // compressed branch, 32 pooled keys per tile: K = first (hi) pooled key plane of the
  // 64-key stage, V = the row-major pooled values
  const T* pst = pooled + (int64_t)h * (Mp / C::PT) * C::STAGE;
  const T* pvh = pooled_v + (int64_t)h * Mp * C::VROW;
  for (int t = 0; t * KT < M; ++t) {
    __syncthreads();
    const T* ksrc = pst + (int64_t)(t / 2) * C::STAGE + (t % 2) * KT * C::KROW;
    const T* vsrc = pvh + (int64_t)t * KT * C::VROW;
    dma_contiguous<BW>(stage, ksrc, C::KCH, wave, lane);
    dma_contiguous<BW>(stage + C::KTILE, vsrc, C::VCH, wave, lane);
    dma_wait();
    __syncthreads();
    S.tile(stage, min(KT, M - t * KT), sl2, lse[0], gx[0], Dx[0], lane);
  }
  // selected and window branches: gathered key tiles
  Gather<DT, D, BW> ga;
  ga.init(wave, lane);
#pragma unroll 1
  for (int x = 1; x <= 2; ++x) {
    const int32_t* blist = x == 1 ? sel_lds : cell_blk + cb0;
    const int nlist = x == 1 ? nsel : cb1 - cb0;
    for (int l0 = 0; l0 < nlist; l0 += NTH) {
      const int L = min(NTH, nlist - l0);
      const int total = list_prefix<NTH>(blist + l0, L, blk_off, pre, lst_off);
      for (int k0 = 0; k0 < total; k0 += KT) {
        __syncthreads();
        ga.lookup(k0, total, L, pre, lst_off, perm);
        ga.template issue<BUF>(stage, kin, vin, H, h, wave);
        dma_wait();
        __syncthreads();
        S.tile(stage, min(KT, total - k0), sl2, lse[x], gx[x], Dx[x], lane);
      }
    }
  }
  if (valid) {
    float* dst = dq + (tok * H + h) * D;
#pragma unroll
    for (int j = 0; j < C::NDV; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[32 * j + res_row(r, g)] = scale * S.dq[j][r];
  }
}

// ------------------------------------------------------------------ inverse selection
__global__ void k_inv_keys(const int32_t* __restrict__ sel, int64_t E, int M, int topk, int H,
                           uint32_t* __restrict__ key, int32_t* __restrict__ val) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int64_t hq = e / topk;  // h * M + query block
  const int h = (int)(hq / M);
  const int s = sel[e];
  key[e] = s >= 0 ? (uint32_t)(h * M + s) : (uint32_t)(H * M);
  val[e] = (int32_t)(hq % M);
}

__global__ void k_inv_off(const uint32_t* __restrict__ key, int64_t E, int nkeys,
                          int32_t* __restrict__ off) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k > nkeys) return;
  int64_t lo = 0, hi = E;  // first position with key >= k
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (key[mid] < (uint32_t)k) lo = mid + 1; else hi = mid;
  }
  off[k] = (int32_t)lo;
}

// ------------------------------------------------------------------ key side (S layout)
// A wave owns 32 keys: their K and V rows are B operands held in registers.  The queries
// that attend to the key block (the blocks of its window cell, then the query blocks whose
// selection holds it) form one stream of 32-row tiles: a stage holds the tile's Q rows (at
// 0, row stride KROW) and dO rows (at VOFF, row stride VROW); the stream runs through three
// stage buffers like the forward's key stream (copy of tile t + 2 issued at step t), with
// each query's sorted row, token and (lse, g, D) of its branch staged per segment in LDS.
// Per tile: S = Q K^T, P = exp2(S sl2 - lse), dP = dO V^T, dS = P o (g dP - D),
// dv += (g P)^T dO, dk += dS^T Q.
constexpr int QSEG = 1024;  // query rows staged per segment

template <int DT, int D>
struct KvState {
  using C = Cfg<DT, D>;
  using F = typename Tr<DT>::frag;
  F kf[C::NKS], vf[C::NKS];
  ssa_f16v dk[C::NDV], dv[C::NDV];
  // info[j] = {lse, g, D, 0} of tile query j
  __device__ inline void tile(const typename Tr<DT>::T* st, const float4* info, float sl2, int lane) {
    const int g = lane >> 5;
    ssa_f16v s = zero16(), dp = zero16();
    const typename Tr<DT>::T* qrow = st + (lane & 31) * C::KROW + g * C::KPL;
    const typename Tr<DT>::T* orow = st + C::KTILE + (lane & 31) * C::VROW + g * C::KPL;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      s = Tr<DT>::mma(load_frag<DT>(qrow + ks * C::KS), kf[ks], s);
      dp = Tr<DT>::mma(load_frag<DT>(orow + ks * C::KS), vf[ks], dp);
    }
    ssa_f16v pg;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float4 in = info[res_row(r, g)];
      const float p = fast_exp2(__builtin_fmaf(s[r], sl2, -in.x));
      pg[r] = in.y * p;
      s[r] = p * (in.y * dp[r] - in.z);
    }
#pragma unroll
    for (int ks = 0; ks < C::PK; ++ks) {
      const F pf = p_frag<DT>(pg, ks), sf = p_frag<DT>(s, ks);
#pragma unroll
      for (int j = 0; j < C::NDV; ++j) {
        dv[j] = Tr<DT>::mma(pf, tr_frag<DT, C::VROW>(st + C::KTILE, ks, j, lane), dv[j]);
        dk[j] = Tr<DT>::mma(sf, tr_frag<DT, C::KROW>(st, ks, j, lane), dk[j]);
      }
    }
  }
};

// per-query info of a tile of set positions k0 .. k0+31 (threads 0..31)
__device__ inline void fill_info(float4* info, int k0, int total, int L, const int32_t* pre,
                                 const int32_t* lst_off, const float* __restrict__ lse,
                                 const float* __restrict__ Dx, const void* gates, int dt16,
                                 const int32_t* __restrict__ perm, int H, int h, int x) {
  const int j = threadIdx.x;
  if (j >= KT) return;
  float4 v = make_float4(INFINITY, 0.f, 0.f, 0.f);
  if (k0 + j < total) {
    const int r = set_row(k0 + j, L, pre, lst_off);
    const int64_t gi = ((int64_t)perm[r] * H + h) * 3 + x;
    float gv;
    if (dt16 == 0) gv = reinterpret_cast<const float*>(gates)[gi];
    else if (dt16 == 1) gv = (float)reinterpret_cast<const _Float16*>(gates)[gi];
    else gv = (float)reinterpret_cast<const __bf16*>(gates)[gi];
    v = make_float4(lse[r], gv, Dx[r], 0.f);
  }
  info[j] = v;
}

// The query stream of a key-side kernel: `total` positions, position -> (sorted row r,
// branch x) by row_of.  Per segment of up to QSEG positions the tokens and (lse, g, D) of
// the branch go to LDS, then the segment's 32-row tiles (Q rows at 0, dO rows at VOFF) run
// through three stage buffers with copies two tiles ahead; per tile
//   S = Q K^T, P = exp2(S sl2 - lse), dP = dO V^T, dS = P o (g dP - D),
//   dv += (g P)^T dO, dk += dS^T Q
// (dS and g P with the queries as the contraction index, read back from registers).
template <int DT, int D, bool BUF, typename RowOf>
__device__ inline void kv_stream(KvState<DT, D>& S, TileCopy<DT, D, BW>& tc, typename Tr<DT>::T* buf0,
                                 typename Tr<DT>::T* buf1, typename Tr<DT>::T* buf2, int32_t* qtok,
                                 float4* qinf, int total, const typename Tr<DT>::T* __restrict__ q,
                                 const typename Tr<DT>::T* __restrict__ dout,
                                 const typename Tr<DT>::T* __restrict__ gates,
                                 const float* __restrict__ lse3, const float* __restrict__ D3,
                                 const int32_t* __restrict__ perm, int H, int h, int64_t N, float sl2,
                                 bool wave_active, int wave, int lane, RowOf row_of) {
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  using F = typename Tr<DT>::frag;
  using TC = TileCopy<DT, D, BW>;
  constexpr int NTH = 64 * BW;
  const int tid = threadIdx.x, g = lane >> 5;
  for (int s0 = 0; s0 < total; s0 += QSEG) {
    const int n = min(QSEG, total - s0);
    __syncthreads();  // the previous segment's tiles have been read
    for (int j = tid; j < n; j += NTH) {
      int r, x;
      row_of(s0 + j, r, x);
      const int64_t t = perm[r];
      qtok[j] = (int32_t)t;
      qinf[j] = make_float4(lse3[((int64_t)x * H + h) * N + r], Tr<DT>::up(gates[(t * H + h) * 3 + x]),
                            D3[((int64_t)x * H + h) * N + r], 0.f);
    }
    __syncthreads();
      const int ntile = (n + KT - 1) / KT;
      auto step = [&](int t, T* cur, T* nx2) __attribute__((always_inline)) {
        if (t + 1 < ntile) vm_wait<TC::NI>();  // tile t landed; tile t + 1 may be in flight
        else vm_wait<0>();
        __syncthreads();
        ssa_f16v ds = zero16(), pg = zero16();
        if (wave_active) {
          ssa_f16v sv = zero16(), dp = zero16();
          const T* qrow = cur + (lane & 31) * C::KROW + g * C::KPL;
          const T* orow = cur + TC::VOFF + (lane & 31) * C::VROW + g * C::KPL;
#pragma unroll
          for (int ks = 0; ks < C::NKS; ++ks) {
            sv = Tr<DT>::mma(load_frag<DT>(qrow + ks * C::KS), S.kf[ks], sv);
            dp = Tr<DT>::mma(load_frag<DT>(orow + ks * C::KS), S.vf[ks], dp);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = t * KT + res_row(r, g);
            const float4 in = j < n ? qinf[j] : make_float4(INFINITY, 0.f, 0.f, 0.f);
            const float pr = fast_exp2(__builtin_fmaf(sv[r], sl2, -in.x));
            ds[r] = pr * (in.y * dp[r] - in.z);
            pg[r] = in.y * pr;
          }
        }
        // transposed fragments of the tile, read before tile t + 2's copy is issued (the
        // transpose reads carry no alias information)
        F qt[C::PK][C::NDV], ot[C::PK][C::NDV];
        if (wave_active) {
#pragma unroll
          for (int ks = 0; ks < C::PK; ++ks)
#pragma unroll
            for (int jd = 0; jd < C::NDV; ++jd) {
              qt[ks][jd] = tr_frag<DT, C::KROW>(cur, ks, jd, lane);
              ot[ks][jd] = tr_frag<DT, C::VROW>(cur + TC::VOFF, ks, jd, lane);
            }
        }
        if (t + 2 < ntile) tc.template issue<BUF>(nx2, q, dout, H, h, wave);
        if (t + 3 < ntile) tc.fetch(qtok, (t + 3) * KT, n);
        if (wave_active) {
#pragma unroll
          for (int ks = 0; ks < C::PK; ++ks) {
            const F pf = p_frag<DT>(pg, ks), sf = p_frag<DT>(ds, ks);
#pragma unroll
            for (int jd = 0; jd < C::NDV; ++jd) {
              S.dv[jd] = Tr<DT>::mma(pf, ot[ks][jd], S.dv[jd]);
              S.dk[jd] = Tr<DT>::mma(sf, qt[ks][jd], S.dk[jd]);
            }
          }
        }
      };
      tc.fetch(qtok, 0, n);
      tc.template issue<BUF>(buf0, q, dout, H, h, wave);
      if (ntile > 1) {
        tc.fetch(qtok, KT, n);
        tc.template issue<BUF>(buf1, q, dout, H, h, wave);
      }
      if (ntile > 2) tc.fetch(qtok, 2 * KT, n);
      for (int t = 0; t < ntile; t += 3) {
        step(t, buf0, buf2);
        if (t + 1 < ntile) step(t + 1, buf1, buf0);
        if (t + 2 < ntile) step(t + 2, buf2, buf1);
      }
    }
}

template <int DT, int D, bool BUF>
__global__ __launch_bounds__(64 * BW) void k_bwd_dkdv(
    const typename Tr<DT>::T* __restrict__ q, const typename Tr<DT>::T* __restrict__ kin,
    const typename Tr<DT>::T* __restrict__ vin, const typename Tr<DT>::T* __restrict__ gates,
    const typename Tr<DT>::T* __restrict__ dout, const float* __restrict__ lse3,
    const float* __restrict__ D3, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ blk_off, const int32_t* __restrict__ blk_cell,
    const int32_t* __restrict__ cell_off, const int32_t* __restrict__ cell_blk,
    const int32_t* __restrict__ lpt, const int32_t* __restrict__ inv_off,
    const int32_t* __restrict__ inv_q, int M, int H, int nchunk, int64_t N, float scale, float sl2,
    const float* __restrict__ ukv, int Mp, float* __restrict__ dk, float* __restrict__ dv) {
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  using F = typename Tr<DT>::frag;
  using TC = TileCopy<DT, D, BW>;
  constexpr int NTH = 64 * BW;
  __shared__ __attribute__((aligned(1024))) T buf0[TC::ELEMS];
  __shared__ __attribute__((aligned(1024))) T buf1[TC::ELEMS];
  __shared__ __attribute__((aligned(1024))) T buf2[TC::ELEMS];
  __shared__ int32_t pre[NTH + 1];
  __shared__ int32_t lst_off[NTH];
  __shared__ int32_t ent_x[NTH];
  __shared__ int32_t qtok[QSEG];
  __shared__ float4 qinf[QSEG];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int unit, member;
  xcd_split(blockIdx.x, nchunk * H, unit, member);
  if (unit >= M) return;
  const int h = member % H, chunk = member / H;
  const int b = lpt[unit];
  const int r0 = blk_off[b], rows = blk_off[b + 1] - r0;
  if (chunk * BROWS >= rows) return;
  const int kbase = chunk * BROWS + wave * 32;
  const bool kvalid = kbase + c < rows;
  const bool wave_active = kbase < rows;
  const int64_t ktok = perm[r0 + (kvalid ? kbase + c : 0)];
  KvState<DT, D> S;
  load_q<DT, D>(S.kf, kin + (ktok * H + h) * D, kvalid, lane);
  load_q<DT, D>(S.vf, vin + (ktok * H + h) * D, kvalid, lane);
#pragma unroll
  for (int j = 0; j < C::NDV; ++j) S.dk[j] = S.dv[j] = zero16();
  const int cell = blk_cell[b];
  const int c0 = cell_off[cell], nwin = cell_off[cell + 1] - c0;
  const int i0 = inv_off[h * M + b], ninv = inv_off[h * M + b + 1] - i0;
  const int nent = nwin + ninv;  // window query blocks, then the selecting ones
  TC tc;
  tc.init(wave, lane);

  for (int e0 = 0; e0 < nent; e0 += NTH) {
    const int L = min(NTH, nent - e0);
    __syncthreads();  // the previous chunk's tables and stages are no longer read
    int sz = 0;
    if (tid < L) {
      const int e = e0 + tid;
      const int qb = e < nwin ? cell_blk[c0 + e] : inv_q[i0 + e - nwin];
      lst_off[tid] = blk_off[qb];
      sz = blk_off[qb + 1] - blk_off[qb];
      ent_x[tid] = e < nwin ? 2 : 1;
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
    kv_stream<DT, D, BUF>(S, tc, buf0, buf1, buf2, qtok, qinf, total, q, dout, gates, lse3, D3, perm,
                          H, h, N, sl2, wave_active, wave, lane,
                          [&](int pos, int& r, int& x) __attribute__((always_inline)) {
                            int lo = 0, hi = L - 1;  // last entry starting at or before pos
                            while (lo < hi) {
                              const int mid = (lo + hi + 1) >> 1;
                              if (pre[mid] <= pos) lo = mid; else hi = mid - 1;
                            }
                            r = lst_off[lo] + (pos - pre[lo]);
                            x = ent_x[lo];
                          });
  }
  // write, with the block's compressed-branch terms: lane holds column 32j + c of keys
  // res_row(r, g)
  const float* uk = ukv + ((int64_t)h * Mp + b) * D;
  const float* uv = ukv + (((int64_t)H + h) * Mp + b) * D;
  float ukc[C::NDV], uvc[C::NDV];
#pragma unroll
  for (int j = 0; j < C::NDV; ++j) {
    ukc[j] = uk[32 * j + c];
    uvc[j] = uv[32 * j + c];
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int kr = kbase + res_row(r, g);
    if (kr < rows) {
      const int64_t t = perm[r0 + kr];
#pragma unroll
      for (int j = 0; j < C::NDV; ++j) {
        dk[(t * H + h) * D + 32 * j + c] = scale * S.dk[j][r] + ukc[j];
        dv[(t * H + h) * D + 32 * j + c] = S.dv[j][r] + uvc[j];
      }
    }
  }
}

// ------------------------------------------------------------------ compressed key side
// Wave w of a workgroup owns pooled key tile blockIdx-group*BW + w; the workgroup streams the
// sorted query rows of its chunk (every query attends to every pooled key).  Partials per
// chunk: part[qc][h][key][d].
template <int DT, int D, bool BUF>
__global__ __launch_bounds__(64 * BW) void k_bwd_cmp(
    const typename Tr<DT>::T* __restrict__ q, const typename Tr<DT>::T* __restrict__ gates,
    const typename Tr<DT>::T* __restrict__ dout, const typename Tr<DT>::T* __restrict__ pooled,
    const typename Tr<DT>::T* __restrict__ pooled_v, const float* __restrict__ lse3,
    const float* __restrict__ D3, const int32_t* __restrict__ perm, int Mp, int H, int qch, int64_t N,
    float scale, float sl2, float* __restrict__ part_k, float* __restrict__ part_v) {
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  using TC = TileCopy<DT, D, BW>;
  __shared__ __attribute__((aligned(1024))) T buf0[TC::ELEMS];
  __shared__ __attribute__((aligned(1024))) T buf1[TC::ELEMS];
  __shared__ __attribute__((aligned(1024))) T buf2[TC::ELEMS];
  __shared__ int32_t qtok[QSEG];
  __shared__ float4 qinf[QSEG];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntile = Mp / KT;
  const int qc = blockIdx.x % qch;
  const int h = (blockIdx.x / qch) % H;
  const int kt = (blockIdx.x / (qch * H)) * BW + wave;
  const bool ktv = kt < ntile;
  const int ktc = ktv ? kt : 0;
  const T* krow = pooled + ((int64_t)h * (Mp / C::PT) + ktc / 2) * C::STAGE + ((ktc % 2) * KT + c) * C::KROW;
  const T* vrow = pooled_v + ((int64_t)h * Mp + ktc * KT + c) * C::VROW;
  KvState<DT, D> S;
  load_q<DT, D>(S.kf, krow, ktv, lane);
  load_q<DT, D>(S.vf, vrow, ktv, lane);
#pragma unroll
  for (int j = 0; j < C::NDV; ++j) S.dk[j] = S.dv[j] = zero16();
  const int64_t qlen = (N + qch - 1) / qch;
  const int64_t q0 = qc * qlen, q1 = min(N, q0 + qlen);
  const int total = (int)max((int64_t)0, q1 - q0);
  TC tc;
  tc.init(wave, lane);
  kv_stream<DT, D, BUF>(S, tc, buf0, buf1, buf2, qtok, qinf, total, q, dout, gates, lse3, D3, perm, H,
                        h, N, sl2, ktv, wave, lane,
                        [&](int pos, int& r, int& x) __attribute__((always_inline)) {
                          r = (int)q0 + pos;
                          x = 0;
                        });
  if (ktv) {
    float* pk = part_k + (((int64_t)qc * H + h) * Mp + kt * KT) * D;
    float* pv = part_v + (((int64_t)qc * H + h) * Mp + kt * KT) * D;
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int j = 0; j < C::NDV; ++j) {
        pk[res_row(r, g) * D + 32 * j + c] = scale * S.dk[j][r];
        pv[res_row(r, g) * D + 32 * j + c] = S.dv[j][r];
      }
  }
}

// ------------------------------------------------------------------ pooling backward
// grid (M, H): sum the chunk partials in order and map them through W^T and the mean: the
// compressed branch's dK, dV term shared by every token of the block.
template <int DT, int D>
__global__ __launch_bounds__(256) void k_bwd_pool(
    const typename Tr<DT>::T* __restrict__ wk, const typename Tr<DT>::T* __restrict__ wv,
    const float* __restrict__ part_k, const float* __restrict__ part_v,
    const int32_t* __restrict__ blk_off, int Mp, int H, int qch, float* __restrict__ ukv) {
  __shared__ float gk[D], gv[D];
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  for (int j = tid; j < 2 * D; j += 256) {
    const float* src = j < D ? part_k : part_v;
    const int c = j < D ? j : j - D;
    float s = 0.f;
    for (int qc = 0; qc < qch; ++qc) s += src[(((int64_t)qc * H + h) * Mp + b) * D + c];
    (j < D ? gk : gv)[c] = s;
  }
  __syncthreads();
  const float inv = 1.f / (float)(blk_off[b + 1] - blk_off[b]);
  for (int j = tid; j < 2 * D; j += 256) {
    const bool isk = j < D;
    const int i = isk ? j : j - D;
    const typename Tr<DT>::T* W = isk ? wk : wv;
    const float* gsrc = isk ? gk : gv;
    float s = 0.f;
    for (int c = 0; c < D; ++c) s += Tr<DT>::up(W[(int64_t)i * D + c]) * gsrc[c];
    ukv[(((int64_t)(isk ? 0 : 1) * H + h) * Mp + b) * D + i] = s * inv;
  }
}

template <int DT, int D>
hipError_t run_backward(const ssa_plan_s* p, int H, int topk, float scale, const void* q,
                        const void* k, const void* v, const void* wk, const void* wv,
                        const void* gates, const int32_t* sel, const void* dout, float* dq,
                        float* dk, float* dv, float* dgates, const FwdWs& fw, const BwdWs& w,
                        hipStream_t s) {
  using T = typename Tr<DT>::T;
  const int M = (int)p->M;
  const int Mp = (int)pooled_rows(M);
  const int64_t N = p->n;
  const float sl2 = scale * 1.4426950408889634f;
  const int nchunk = (p->max_rows + BROWS - 1) / BROWS;
  constexpr int PREP_GS = 16 / sizeof(T) * 16 >= D ? 16 : (16 / sizeof(T) * 32 >= D ? 32 : 64);
  hipLaunchKernelGGL((k_bwd_prep<DT, D>), dim3((unsigned)((N * H * PREP_GS + 255) / 256)), dim3(256), 0, s,
                     (const T*)dout, (const T*)gates, fw.obr, p->perm, N, H, dgates, w.D);
  const bool buf = buffer_addressable(N * H * D * (int64_t)sizeof(T));
  if (buf)
    hipLaunchKernelGGL((k_bwd_dq<DT, D, true>), dim3(xcd_grid(M, (int64_t)H * nchunk)), dim3(64 * BW), 0, s,
                     (const T*)q, (const T*)k, (const T*)v, (const T*)gates, (const T*)dout,
                     (const T*)fw.pooled, (const T*)fw.pooled_v, fw.lse, w.D, p->perm, p->blk_off, p->blk_cell,
                     p->cell_off, p->cell_blk, p->lpt, sel, M, Mp, H, nchunk, N, topk, scale, sl2, dq);
  else
    hipLaunchKernelGGL((k_bwd_dq<DT, D, false>), dim3(xcd_grid(M, (int64_t)H * nchunk)), dim3(64 * BW), 0, s,
                     (const T*)q, (const T*)k, (const T*)v, (const T*)gates, (const T*)dout,
                     (const T*)fw.pooled, (const T*)fw.pooled_v, fw.lse, w.D, p->perm, p->blk_off, p->blk_cell,
                     p->cell_off, p->cell_blk, p->lpt, sel, M, Mp, H, nchunk, N, topk, scale, sl2, dq);
  // inverse selection
  const int64_t E = (int64_t)H * M * topk;
  hipLaunchKernelGGL(k_inv_keys, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, s, sel, E, M, topk,
                     H, w.ka, w.va);
  uint32_t *ka = w.ka, *kb = w.kb;
  int32_t *va = w.va, *vb = w.vb;
  hipError_t e = ssa_sort::radix_sort(ka, va, kb, vb, (int)E, ssa_sort::bits_for((uint64_t)H * M),
                                      w.rank, w.hist, w.part, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_inv_off, dim3((unsigned)((H * M + 1 + 255) / 256)), dim3(256), 0, s, ka, E,
                     H * M, w.inv_off);
  const int groups = (Mp / KT + BW - 1) / BW;
  if (buf)
    hipLaunchKernelGGL((k_bwd_cmp<DT, D, true>), dim3((unsigned)(groups * H * w.qch)), dim3(64 * BW), 0, s,
                     (const T*)q, (const T*)gates, (const T*)dout, (const T*)fw.pooled,
                     (const T*)fw.pooled_v, fw.lse, w.D,
                     p->perm, Mp, H, w.qch, N, scale, sl2, w.part_k, w.part_v);
  else
    hipLaunchKernelGGL((k_bwd_cmp<DT, D, false>), dim3((unsigned)(groups * H * w.qch)), dim3(64 * BW), 0, s,
                     (const T*)q, (const T*)gates, (const T*)dout, (const T*)fw.pooled,
                     (const T*)fw.pooled_v, fw.lse, w.D,
                     p->perm, Mp, H, w.qch, N, scale, sl2, w.part_k, w.part_v);
  hipLaunchKernelGGL((k_bwd_pool<DT, D>), dim3(M, H), dim3(256), 0, s, (const T*)wk, (const T*)wv,
                     w.part_k, w.part_v, p->blk_off, Mp, H, w.qch, w.ukv);
  if (buf)
    hipLaunchKernelGGL((k_bwd_dkdv<DT, D, true>), dim3(xcd_grid(M, (int64_t)H * nchunk)), dim3(64 * BW), 0, s,
                     (const T*)q, (const T*)k, (const T*)v, (const T*)gates, (const T*)dout, fw.lse,
                     w.D, p->perm, p->blk_off, p->blk_cell, p->cell_off, p->cell_blk, p->lpt,
                     w.inv_off, va, M, H, nchunk, N, scale, sl2, w.ukv, Mp, dk, dv);
  else
    hipLaunchKernelGGL((k_bwd_dkdv<DT, D, false>), dim3(xcd_grid(M, (int64_t)H * nchunk)), dim3(64 * BW), 0, s,
                     (const T*)q, (const T*)k, (const T*)v, (const T*)gates, (const T*)dout, fw.lse,
                     w.D, p->perm, p->blk_off, p->blk_cell, p->cell_off, p->cell_blk, p->lpt,
                     w.inv_off, va, M, H, nchunk, N, scale, sl2, w.ukv, Mp, dk, dv);
  return hipGetLastError();
}

template <int DT>
hipError_t backward_d(int d, const ssa_plan_s* p, int H, int topk, float scale, const void* q,
                      const void* k, const void* v, const void* wk, const void* wv,
                      const void* gates, const int32_t* sel, const void* dout, float* dq,
                      float* dk, float* dv, float* dgates, const FwdWs& fw, const BwdWs& w,
                      hipStream_t s) {
  switch (d) {
    case 32: return run_backward<DT, 32>(p, H, topk, scale, q, k, v, wk, wv, gates, sel, dout, dq, dk, dv, dgates, fw, w, s);
    case 64: return run_backward<DT, 64>(p, H, topk, scale, q, k, v, wk, wv, gates, sel, dout, dq, dk, dv, dgates, fw, w, s);
    case 96: return run_backward<DT, 96>(p, H, topk, scale, q, k, v, wk, wv, gates, sel, dout, dq, dk, dv, dgates, fw, w, s);
    case 128: return run_backward<DT, 128>(p, H, topk, scale, q, k, v, wk, wv, gates, sel, dout, dq, dk, dv, dgates, fw, w, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t bwd_carve(Carver& c, const ssa_plan_s* p, int H, int d, int topk, void* w) {
  return carve(c, p, H, d, topk, static_cast<BwdWs*>(w));
}

hipError_t launch_backward(ssa_dtype dt, const ssa_plan_s* p, int H, int d, int topk, float scale,
                           const void* q, const void* k, const void* v, const void* wk,
                           const void* wv, const void* gates, const int32_t* sel, const void* dout,
                           float* dq, float* dk, float* dv, float* dgates, const FwdWs& fw,
                           void* ws, hipStream_t s) {
  Carver c(ws);
  c.off = (256 - (reinterpret_cast<uintptr_t>(ws) & 255)) & 255;
  BwdWs w;
  carve(c, p, H, d, topk, &w);
  switch (dt) {
    case SSA_F32: return backward_d<DT_F32>(d, p, H, topk, scale, q, k, v, wk, wv, gates, sel, dout, dq, dk, dv, dgates, fw, w, s);
    case SSA_F16: return backward_d<DT_F16>(d, p, H, topk, scale, q, k, v, wk, wv, gates, sel, dout, dq, dk, dv, dgates, fw, w, s);
    case SSA_BF16: return backward_d<DT_BF16>(d, p, H, topk, scale, q, k, v, wk, wv, gates, sel, dout, dq, dk, dv, dgates, fw, w, s);
  }
  return hipErrorInvalidValue;
}
