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
#include <algorithm>
#include "ssa_internal.h"
#include "ssa_mfma.h"
#include "ssa_tiles.h"

namespace {

using namespace ssa_dev;
constexpr int BW = 4;           // waves per workgroup (dq, compressed key side)
constexpr int BROWS = 32 * BW;  // query rows per dq workgroup
constexpr int KW = 4;           // waves per dk/dv workgroup
constexpr int KROWS = 32 * KW;  // keys per dk/dv workgroup

struct BwdWs {
  float* D;                    // [3][H][N]
  uint32_t *ka, *kb;           // inverse-selection sort keys (E = H*M*topk)
  int32_t *va, *vb, *rank, *hist, *part;
  int32_t* inv_off;            // [H*M + 1]
  float *part_k, *part_v;      // [qch][H][Mp][d] compressed key-side partials
  float* ukv;                  // [2][H][Mp][d] per-block dK, dV terms of the compressed branch
  int qch;
  // key-side schedule: (head, block) units in descending stream length, their work items
  uint32_t *ska, *skb;         // [H*M] sort keys
  int32_t *sva, *svb;          // [H*M] unit ids
  int4* sinfo;                 // [H*M] per sorted unit: {unit, pieces, partial row offset, -}
  int32_t* ioff;               // [H*M + 1] first item of each sorted unit
  int4* items;                 // [item_cap] {unit, key chunk, piece, partial row offset or -1},
                               // or {-(group + 1), group piece, 0, 0}
  int4* grp_meta;              // [H*M] per key group: {head, members, first member, keys}
  int4* grp_mem;               // [H*M] per member: {block, first key slot, partial row, rows}
  int32_t* ngrp;               // [1] key groups
  int32_t* xbase;              // [3 kinds][9]: list starts per XCD, then the kind's end
  float* kpart;                // [budget rows][2][d] partial dK, dV of split and tiny units
  int64_t item_cap;
};

// A key-side unit (head, key block) whose query stream has more than KV_EP query blocks
// (window blocks, then the selecting query blocks) is split into pieces of KV_EP blocks,
// while the partial sums of the pieces fit a fixed budget of key rows; the pieces' partial
// dK, dV are summed in piece order by k_kv_reduce.
//
// A tiny unit (at most KG_TINY keys, selected by some query block) instead keeps only its
// window part as an item (piece 0) and joins a key group: up to KG_KEYS keys of at most
// KG_MEM tiny units of one head, which streams the union of its members' selecting query
// blocks once, each row masked to the members that its block selected.  The union is cut
// into at most KG_GP ranges of at least KG_QB query blocks (group pieces 1, 2, ...).
constexpr int KV_EP = 8;
constexpr int KG_TINY = 32, KG_KEYS = 128, KG_MEM = 32, KG_QB = 16, KG_GP = 32;
__host__ __device__ inline int kg_pieces(int M) {
  const int p = (M + KG_QB - 1) / KG_QB;
  return p < KG_GP ? p : KG_GP;
}
__host__ __device__ inline int kg_qbp(int M) {  // query blocks per group piece
  const int gp = kg_pieces(M);
  return (M + gp - 1) / gp;
}
inline int64_t kv_budget_rows(int d) { return (int64_t)(256 << 20) / (8 * d); }

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
  const int64_t U = (int64_t)H * M;
  const int64_t nch = ((p->max_rows > 0 ? p->max_rows : 1) + KROWS - 1) / KROWS;
  t.ska = c.take<uint32_t>(U);
  t.skb = c.take<uint32_t>(U);
  t.sva = c.take<int32_t>(U);
  t.svb = c.take<int32_t>(U);
  t.sinfo = c.take<int4>(U);
  t.ioff = c.take<int32_t>(U + 1);
  // unsplit units give at most nch items each; split pieces and key-group pieces at most
  // one per partial row each (a piece's partial sums take at least one row)
  t.item_cap = U * nch + 2 * kv_budget_rows(d);
  t.items = c.take<int4>(t.item_cap);
  t.grp_meta = c.take<int4>(U);
  t.grp_mem = c.take<int4>(U);
  t.ngrp = c.take<int32_t>(1);
  t.xbase = c.take<int32_t>(3 * (NXCD + 1));
  t.kpart = c.take<float>(kv_budget_rows(d) * 2 * d);
  if (w) *w = t;
  return c.off;
}

// ------------------------------------------------------------------ prep
// dgates and D for the three branches.  A group of GS lanes per (sorted row r, head h): lane
// j of the group reads the j-th 16-byte chunk of dO's head row (and the matching chunks of
// the three saved branch outputs o0, o1, o2, sorted rows), so a group reads contiguous rows;
// the dot products are finished with shuffles inside the group.
template <int DT, int D>
__global__ __launch_bounds__(256) void k_bwd_prep(
    const typename Tr<DT>::T* __restrict__ dout, const typename Tr<DT>::T* __restrict__ gates,
    const typename SaveT<DT>::type* __restrict__ o0, const typename SaveT<DT>::type* __restrict__ o1,
    const typename SaveT<DT>::type* __restrict__ o2, const int32_t* __restrict__ perm, int64_t N, int H,
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
      const typename SaveT<DT>::type* o = (x == 0 ? o0 : (x == 1 ? o1 : o2)) + (r * H + h) * D + j * EPC;
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[x] += Tr<DT>::up(ae[e]) * (float)o[e];
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
// A wave owns 32 query rows: their Q and dO rows are B operands held in registers.  Per
// branch the keys form a stream of 32-key tiles -- the pooled keys, the selected blocks' keys,
// the window cell's keys -- copied through NB stage buffers (K rows at 0, V rows at VOFF),
// the copy of tile t + NB - 1 issued while tile t is in use.  Per tile, keys as rows:
//   S^T = K Q^T, P^T = exp2(S^T sl2 - lse), dP^T = V dO^T, dS^T = P^T o (g dP^T - D),
//   dq^T += K^T dS^T.
constexpr int DSEG = 2048;  // gathered keys staged per segment

template <int DT, int D>
struct DqState {
  using C = Cfg<DT, D>;
  using F = typename Tr<DT>::frag;
  F qf[C::NKS], dof[C::NKS];
  ssa_f16v dq[C::NDV];
};

// One branch's tile stream of n keys; fetch(t) readies tile t's copy addresses, issue(buf)
// starts that copy.
template <int DT, int D, int NB, typename Fetch, typename Issue>
__device__ inline void dq_stream(DqState<DT, D>& S, int n, float lse, float gx, float Dx, float sl2,
                                 bool wave_active, typename Tr<DT>::T* const* bufs, int lane, Fetch fetch,
                                 Issue issue) {
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  using F = typename Tr<DT>::frag;
  using TC = TileCopy<DT, D, BW>;
  const int g = lane >> 5;
  __syncthreads();  // the stage buffers' previous tiles have been read
  tile_pipeline<NB, TC::NI>(
      (n + KT - 1) / KT, bufs, fetch, issue,
      [&](int t, const T* cur, auto&& next) __attribute__((always_inline)) {
        ssa_f16v ds = zero16();
        constexpr bool PRE = C::KPL != 1;
        F kt[PRE ? C::PK : 1][C::NDV];
        if (wave_active) {
          ssa_f16v sv = zero16(), dp = zero16();
          const T* krow = cur + (lane & 31) * C::KROW + g * C::KPL;
          const T* vrow = cur + TC::VOFF + (lane & 31) * C::VROW + g * C::KPL;
          F ka[C::NKS], va[C::NKS];  // all fragment reads before the first MFMA
#pragma unroll
          for (int ks = 0; ks < C::NKS; ++ks) {
            ka[ks] = load_frag<DT>(krow + ks * C::KS);
            va[ks] = load_frag<DT>(vrow + ks * C::KS);
          }
#pragma unroll
          for (int ks = 0; ks < C::NKS; ++ks) {
            sv = Tr<DT>::mma(ka[ks], S.qf[ks], sv);
            dp = Tr<DT>::mma(va[ks], S.dof[ks], dp);
          }
          if constexpr (C::KPL != 1) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * C::NKS, 0);  // DS reads
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * C::NKS, 0);  // then MFMAs
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) ds[r] = fast_exp2(__builtin_fmaf(sv[r], sl2, -lse)) * (gx * dp[r] - Dx);
          if ((t + 1) * KT > n) {  // keys past n (finite rows) get no weight
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (t * KT + res_row(r, g) >= n) ds[r] = 0.f;
          }
          // 16-bit types: the K^T fragments are read before the next copy is issued (the
          // transpose reads carry no alias information); fp32 reads them in place (too many
          // registers) and issues the copy after its MFMAs
          if constexpr (PRE) {
#pragma unroll
            for (int ks = 0; ks < C::PK; ++ks)
#pragma unroll
              for (int j = 0; j < C::NDV; ++j) kt[ks][j] = tr_frag<DT, C::KROW>(cur, ks, j, lane);
          }
        }
        if constexpr (PRE) next();
        if (wave_active) {
#pragma unroll
          for (int ks = 0; ks < C::PK; ++ks) {
            const F sf = p_frag<DT>(ds, ks);
#pragma unroll
            for (int j = 0; j < C::NDV; ++j)
              S.dq[j] = Tr<DT>::mma(PRE ? kt[ks][j] : tr_frag<DT, C::KROW>(cur, ks, j, lane), sf, S.dq[j]);
          }
        }
        if constexpr (!PRE) next();
      });
}

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
  using TC = TileCopy<DT, D, BW>;
  constexpr int NTH = 64 * BW;
  // two workgroups per CU where the registers allow it
  constexpr int NB = stage_depth<DT, D, BW>(LDS_BYTES / 2 - 2048, DSEG * 4 + (2 * NTH + 257) * 4);
  SSA_STAGE_BUFFERS(T, TC::ELEMS, NB);
  __shared__ int32_t pre[NTH + 1];
  __shared__ int32_t lst_off[NTH];
  __shared__ int32_t sel_lds[256];
  __shared__ int32_t keytok[DSEG];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int unit, member;
  xcd_split(blockIdx.x, nchunk * H, unit, member);
  if (unit >= M) return;
  const int h = member % H, chunk = member / H;
  const int b = lpt[unit];
  const int r0 = blk_off[b], rows = blk_off[b + 1] - r0;
  if (chunk * BROWS >= rows) return;
  const int32_t* srow = sel + ((int64_t)h * M + b) * topk;
  const int sb = tid < topk ? srow[tid] : -1;  // selected ids ascend, -1 padded at the end
  if (sb >= 0) sel_lds[tid] = sb;
  const int nsel = __syncthreads_count(sb >= 0);
  const int cell = blk_cell[b];
  const int cb0 = cell_off[cell], cb1 = cell_off[cell + 1];

  const int wbase = chunk * BROWS + wave * 32;
  const bool wave_active = wbase < rows;
  const int my_row = wbase + c;
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
  TC tc;
  tc.init(wave, lane);

  // compressed branch: pooled key row r is row r % 64 of the first (hi) key plane of stage
  // r / 64; pooled values are row-major.  Rows past M are zero.
  {
    const T* kb = pooled + (int64_t)h * (Mp / C::PT) * C::STAGE;
    const T* vb = pooled_v + (int64_t)h * Mp * C::VROW;
    dq_stream<DT, D, NB>(S, M, lse[0], gx[0], Dx[0], sl2, wave_active, bufs, lane,
                     [&](int t) __attribute__((always_inline)) { tc.set_rows(t * KT); },
                     [&](T* dst) __attribute__((always_inline)) {
                       tc.template issue_rows<BUF>(
                           dst, kb, vb, [](int r) { return (r / C::PT) * C::STAGE + (r % C::PT) * C::KROW; },
                           [](int r) { return r * C::VROW; }, wave);
                     });
  }
  // selected and window branches: the list's blocks in order, staged DSEG keys at a time
#pragma unroll 1
  for (int x = 1; x <= 2; ++x) {
    const int32_t* blist = x == 1 ? sel_lds : cell_blk + cb0;
    const int nlist = x == 1 ? nsel : cb1 - cb0;
    for (int l0 = 0; l0 < nlist; l0 += NTH) {
      const int L = min(NTH, nlist - l0);
      const int total = list_prefix<NTH>(blist + l0, L, blk_off, pre, lst_off);
      for (int ks0 = 0; ks0 < total; ks0 += DSEG) {
        const int n = min(DSEG, total - ks0);
        __syncthreads();  // the previous segment's tiles have been fetched
        fill_tokens<DSEG / NTH, NTH>(keytok, n, [&](int j) { return set_row(ks0 + j, L, pre, lst_off); }, perm);
        __syncthreads();
        dq_stream<DT, D, NB>(S, n, x == 1 ? lse[1] : lse[2], x == 1 ? gx[1] : gx[2], x == 1 ? Dx[1] : Dx[2],
                             sl2, wave_active, bufs, lane,
                         [&](int t) __attribute__((always_inline)) { tc.fetch(keytok, t * KT, n); },
                         [&](T* dst) __attribute__((always_inline)) {
                           tc.template issue<BUF>(dst, kin, vin, H, h, wave);
                         });
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

// ------------------------------------------------------------------ key-side schedule
// Units u = h*M + b in head-major order, each head's units by descending stream length in
// query blocks (stable), are split into pieces and cut into work items (piece, key chunk).
// Sorted unit s goes to XCD s % 8; each XCD's items form one list, taken round-robin by the
// workgroups on that XCD, so the key chunks of a piece (which read the same query rows) run
// side by side on one L2, and the workgroups sweep the heads in order (one head's query rows
// at a time in the last-level cache).
__global__ void k_kv_keys(const int32_t* __restrict__ inv_off, const int32_t* __restrict__ blk_cell,
                          const int32_t* __restrict__ cell_off, int M, int U, uint32_t* __restrict__ key,
                          int32_t* __restrict__ val) {
  const int u = blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= U) return;
  const int cell = blk_cell[u % M];
  const int nent = cell_off[cell + 1] - cell_off[cell] + inv_off[u + 1] - inv_off[u];
  key[u] = (uint32_t)(u / M) * (uint32_t)(2 * M + 1) + (uint32_t)(2 * M - nent);  // nent <= 2M
  val[u] = u;
}

// Exclusive scan of one value per thread over a 1024-thread workgroup; returns the total.
template <typename V>
__device__ inline V wg_exclusive_scan(V x, V* sh) {
  const int tid = threadIdx.x;
  sh[tid] = x;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const V y = tid >= off ? sh[tid - off] : (V)0;
    __syncthreads();
    sh[tid] += y;
    __syncthreads();
  }
  const V incl = sh[tid], total = sh[1023];
  __syncthreads();
  sh[tid] = incl - x;
  return total;
}

// Item kinds, each run by its own key-side kernel: key-group pieces, units of more than 32
// keys (or all units where the narrow form is not built), narrow units (at most 32 keys).
constexpr int KV_GRP = 0, KV_UNIT = 1, KV_NARROW = 2, KV_KINDS = 3;

// One workgroup.  Per sorted unit: tiny (a key group member), split into pieces, or whole,
// taken in sorted order while the running partial demand (key rows) stays within its head's
// share of the budget; sinfo = {unit, pieces, partial row offset or -1, flags: 1 tiny, 2 narrow}.  Then,
// one thread per head, the head's tiny units in sorted order are packed into key groups.
// Items of kind k form 8 lists (one per XCD): list x of kind k holds items xbase[9k + x] ..
// xbase[9k + x + 1] - 1 (xbase[9k + 8] = end of kind k).  Group pieces and narrow items go
// to list i mod 8 by their index i; a wide unit's items stay together on XCD (sorted unit
// mod 8), ioff = its first item.  A narrow unit's ioff is its first narrow item index.
__global__ __launch_bounds__(1024) void k_kv_schedule(
    const int32_t* __restrict__ order, int U, int M, int H, int narrow_ok, const int32_t* __restrict__ inv_off,
    const int32_t* __restrict__ blk_cell, const int32_t* __restrict__ cell_off,
    const int32_t* __restrict__ blk_off, int64_t budget, int4* __restrict__ sinfo,
    int32_t* __restrict__ ioff, int32_t* __restrict__ xbase, int4* __restrict__ grp_meta,
    int4* __restrict__ grp_mem, int32_t* __restrict__ ngrp, int4* __restrict__ items) {
  __shared__ int64_t sh64[1024];
  __shared__ int32_t sh32[1024];
  __shared__ int32_t ubase[NXCD], ucount[NXCD];
  __shared__ int32_t s_ng, s_n2;
  const int tid = threadIdx.x;
  const int per = (U + 1023) / 1024;
  const int s0 = min(U, tid * per), s1 = min(U, s0 + per);
  const int GP = kg_pieces(M);
  auto unit_info = [&](int si, int& u, int& want, int& rows, bool& cand) {
    u = order[si];
    const int b = u % M, cell = blk_cell[b];
    const int ninv = inv_off[u + 1] - inv_off[u];
    const int nent = cell_off[cell + 1] - cell_off[cell] + ninv;
    want = (nent + KV_EP - 1) / KV_EP;
    rows = blk_off[b + 1] - blk_off[b];
    cand = rows <= KG_TINY && ninv > 0;
  };
  auto demand = [&](int want, int rows, bool cand) -> int64_t {
    return cand ? (int64_t)(1 + GP) * rows : (want > 1 ? (int64_t)want * rows : 0);
  };
  int64_t dsum = 0;
  for (int si = s0; si < s1; ++si) {
    int u, want, rows;
    bool cand;
    unit_info(si, u, want, rows, cand);
    dsum += demand(want, rows, cand);
  }
  wg_exclusive_scan<int64_t>(dsum, sh64);
  int64_t dpre = sh64[tid];
  // the budget is shared out by head (units are head-major, M per head; with more than 1024
  // heads it is one pool): each head's units, most entries first, take from its share, so
  // the long streams of every head are split or grouped, not only those of the first heads
  __shared__ int64_t hbase[1024];
  const bool per_head = H <= 1024;
  const int64_t share = per_head ? budget / H : budget;
  if (per_head) {
    int64_t run = dpre;
    for (int si = s0; si < s1; ++si) {
      if (si % M == 0) hbase[si / M] = run;
      int u, want, rows;
      bool cand;
      unit_info(si, u, want, rows, cand);
      run += demand(want, rows, cand);
    }
  }
  __syncthreads();
  int isum[NXCD];
#pragma unroll
  for (int x = 0; x < NXCD; ++x) isum[x] = 0;
  int nsum = 0;  // narrow items
  for (int si = s0; si < s1; ++si) {
    int u, want, rows;
    bool cand;
    unit_info(si, u, want, rows, cand);
    const int64_t dem = demand(want, rows, cand);
    const int64_t local = per_head ? dpre - hbase[si / M] : dpre;  // demand before it in its share
    const bool fits = dem > 0 && local + dem <= share;
    const bool tiny = cand && fits, split = !cand && fits;
    const bool narrow = narrow_ok && rows <= 32;
    const int pieces = tiny ? 1 + GP : (split ? want : 1);
    const int64_t prow = per_head ? (int64_t)(si / M) * share + local : dpre;  // partial rows
    sinfo[si] = make_int4(u, pieces, fits ? (int)prow : -1, (tiny ? 1 : 0) | (narrow ? 2 : 0));
    dpre += dem;
    const int n = tiny ? 1 : (rows + KROWS - 1) / KROWS * pieces;
    if (narrow) {
      nsum += n;
    } else {
#pragma unroll
      for (int x = 0; x < NXCD; ++x) isum[x] += (si % NXCD == x) ? n : 0;
    }
  }
  __syncthreads();  // sinfo is complete (global writes of this workgroup)
  // key groups: wave w packs the tiny units of heads w, w + 16, ... (sorted units h M ..
  // h M + M - 1 of head h) in order, a group never spanning two heads; the 64 units of a
  // chunk are read by the wave's lanes at once, then taken in order from the tiny ones'
  // ballot.  Pass 0 counts groups and members per wave, pass 1 writes them.
  const int wv = tid >> 6, ln = tid & 63;
  __shared__ int32_t wng[16], wnm[16], wgb[16], wmb[16];
  for (int pass = 0; pass < 2; ++pass) {
    int g = 0, m = 0;
    const int gb0 = pass ? wgb[wv] : 0, mb0 = pass ? wmb[wv] : 0;
    for (int h = wv; h < H; h += 16) {
      int keys = 0, mem = 0;
      for (int c0 = h * M; c0 < (h + 1) * M; c0 += 64) {
        const int si = c0 + ln;
        int4 in = make_int4(0, 0, -1, 0);
        int rows = 0;
        if (si < (h + 1) * M) {
          in = sinfo[si];
          if (in.w & 1) rows = blk_off[in.x % M + 1] - blk_off[in.x % M];
        }
        uint64_t bal = __builtin_amdgcn_ballot_w64((in.w & 1) != 0);
        while (bal) {
          const int l = __builtin_ctzll(bal);
          bal &= bal - 1;
          const int r = __builtin_amdgcn_readlane(rows, l);
          const int ub = __builtin_amdgcn_readlane(in.x, l) % M;
          const int po = __builtin_amdgcn_readlane(in.z, l);
          if (mem > 0 && (keys + r > KG_KEYS || mem == KG_MEM)) {  // close the open group
            if (pass && ln == 0) grp_meta[gb0 + g] = make_int4(h, mem, mb0 + m - mem, keys);
            ++g;
            keys = mem = 0;
          }
          if (pass && ln == 0) grp_mem[mb0 + m] = make_int4(ub, keys, po, r);
          keys += r;
          ++mem;
          ++m;
        }
      }
      if (mem > 0) {
        if (pass && ln == 0) grp_meta[gb0 + g] = make_int4(h, mem, mb0 + m - mem, keys);
        ++g;
      }
    }
    if (pass == 0) {
      if (ln == 0) {
        wng[wv] = g;
        wnm[wv] = m;
      }
      __syncthreads();
      if (tid == 0) {
        int ga = 0, ma = 0;
        for (int i = 0; i < 16; ++i) {
          wgb[i] = ga;
          wmb[i] = ma;
          ga += wng[i];
          ma += wnm[i];
        }
        s_ng = ga;
      }
      __syncthreads();
    }
  }
  __syncthreads();
  const int gtot = s_ng;
  const int n2tot = wg_exclusive_scan<int32_t>(nsum, sh32);
  int n2pre = sh32[tid];
  if (tid == 0) {
    *ngrp = gtot;
    s_n2 = n2tot;
  }
  __syncthreads();
  const int NGP = s_ng * GP, N2 = s_n2;
  int ipre[NXCD];
#pragma unroll
  for (int x = 0; x < NXCD; ++x) {
    const int tot = wg_exclusive_scan<int32_t>(isum[x], sh32);
    ipre[x] = sh32[tid];
    if (tid == 0) ucount[x] = tot;
    __syncthreads();
  }
  if (tid == 0) {
    int acc = 0;
    for (int x = 0; x < NXCD; ++x) {  // kind 0: group pieces
      xbase[KV_GRP * 9 + x] = acc;
      acc += (NGP + NXCD - 1 - x) / NXCD;
    }
    for (int x = 0; x < NXCD; ++x) {  // kind 1: wide units
      xbase[KV_UNIT * 9 + x] = acc;
      ubase[x] = acc;
      acc += ucount[x];
    }
    xbase[KV_GRP * 9 + 8] = xbase[KV_UNIT * 9];
    for (int x = 0; x < NXCD; ++x) {  // kind 2: narrow units
      xbase[KV_NARROW * 9 + x] = acc;
      acc += (N2 + NXCD - 1 - x) / NXCD;
    }
    xbase[KV_UNIT * 9 + 8] = xbase[KV_NARROW * 9];
    xbase[KV_NARROW * 9 + 8] = acc;
  }
  __syncthreads();
  for (int si = s0; si < s1; ++si) {
    const int4 in = sinfo[si];
    const int b = in.x % M, rows = blk_off[b + 1] - blk_off[b];
    const int n = (in.w & 1) ? 1 : (rows + KROWS - 1) / KROWS * in.y;
    if (in.w & 2) {
      ioff[si] = n2pre;
      n2pre += n;
    } else {
#pragma unroll
      for (int x = 0; x < NXCD; ++x) {
        if (si % NXCD == x) {
          ioff[si] = ubase[x] + ipre[x];
          ipre[x] += n;
        }
      }
    }
  }
  // group items: piece-major within a group (group g piece p = item i = g GP + p)
  for (int i = tid; i < NGP; i += 1024)
    items[xbase[KV_GRP * 9 + i % NXCD] + i / NXCD] = make_int4(-(i / GP) - 1, i % GP, 0, 0);
}

// Items of each sorted unit: piece-major, key chunks inner (a piece's chunks read the same
// query stream); a tiny unit has one item, its window part.
__global__ void k_kv_items(const int4* __restrict__ sinfo, const int32_t* __restrict__ ioff,
                           const int32_t* __restrict__ xbase, const int32_t* __restrict__ blk_off, int U, int M,
                           int4* __restrict__ items) {
  const int si = blockIdx.x * blockDim.x + threadIdx.x;
  if (si >= U) return;
  const int4 in = sinfo[si];
  const int b = in.x % M, rows = blk_off[b + 1] - blk_off[b];
  int i = ioff[si];
  // narrow item i goes to narrow list i mod 8; a wide unit's items are consecutive
  auto put = [&](int4 v) {
    if (in.w & 2) items[xbase[KV_NARROW * 9 + i % NXCD] + i / NXCD] = v;
    else items[i] = v;
    ++i;
  };
  if (in.w & 1) {  // tiny: the window part only (piece 0); the key group supplies the rest
    put(make_int4(in.x, 0, -1, in.z));
    return;
  }
  const int nch = (rows + KROWS - 1) / KROWS;
  for (int pc = 0; pc < in.y; ++pc)
    for (int ch = 0; ch < nch; ++ch) put(make_int4(in.x, ch, pc, in.z < 0 ? -1 : in.z + pc * rows));
}

// Split units: dK, dV = the pieces' partials summed in piece order, plus the block's
// compressed-branch terms.
template <int D>
__global__ __launch_bounds__(256) void k_kv_reduce(const int4* __restrict__ sinfo, const float* __restrict__ kpart,
                                                   const float* __restrict__ ukv, const int32_t* __restrict__ blk_off,
                                                   const int32_t* __restrict__ perm, int M, int Mp, int H,
                                                   float* __restrict__ dk, float* __restrict__ dv) {
  const int4 in = sinfo[blockIdx.x];
  if (in.y <= 1) return;
  const int h = in.x / M, b = in.x % M;
  const int r0 = blk_off[b], rows = blk_off[b + 1] - r0;
  const float* uk = ukv + ((int64_t)h * Mp + b) * D;
  const float* uv = ukv + (((int64_t)H + h) * Mp + b) * D;
  for (int idx = threadIdx.x; idx < rows * D; idx += 256) {
    const int kr = idx / D, c = idx % D;
    float sk = 0.f, sv = 0.f;  // in piece order; eight pieces' loads in flight at once
    for (int p0 = 0; p0 < in.y; p0 += 8) {
      float ak[8], av[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float* src = kpart + ((int64_t)in.z + (int64_t)(p0 + i) * rows + kr) * 2 * D;
        ak[i] = p0 + i < in.y ? src[c] : 0.f;
        av[i] = p0 + i < in.y ? src[D + c] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sk += ak[i];
        sv += av[i];
      }
    }
    const int64_t t = perm[r0 + kr];
    dk[(t * H + h) * D + c] = sk + uk[c];
    dv[(t * H + h) * D + c] = sv + uv[c];
  }
}

// ------------------------------------------------------------------ key side (S layout)
// A wave owns 32 keys: their K and V rows are B operands held in registers.  The queries
// that attend to the key block (the blocks of its window cell, then the query blocks whose
// selection holds it) form one stream of 32-row tiles: a stage holds the tile's Q rows (at
// 0, row stride KROW) and dO rows (at VOFF, row stride VROW); the stream runs through NB
// stage buffers like the forward's key stream (copy of tile t + NB - 1 issued at step t),
// with each query's sorted row, token and (lse, g, D) of its branch staged per segment in LDS.
// Per tile: S = Q K^T, P = exp2(S sl2 - lse), dP = dO V^T, dS = P o (g dP - D),
// dv += (g P)^T dO, dk += dS^T Q.
constexpr int QSEG = 1024;  // query rows staged per segment (a multiple of the workgroup size)
constexpr int QPAD = QSEG + KT;  // per-row table length: a segment and its last tile's padding

template <int DT, int D>
struct KvState {
  using C = Cfg<DT, D>;
  using F = typename Tr<DT>::frag;
  F kf[C::NKS], vf[C::NKS];
  ssa_f16v dk[C::NDV], dv[C::NDV];
};

// Token and (lse, g, D) tables of one segment: positions s0 .. s0 + n - 1 of a query stream
// (position -> sorted row r, branch x by row_of), three padded arrays of QPAD floats; the
// last tile's rows past n get probability 0.  MASK: row_of also gives the row's key mask
// (bit m: the row attends to the keys of key-group member m), a fourth array.  A thread's QSEG / NTH positions: rows first,
// then every load in flight at once.
template <int DT, int NTH, bool MASK = false, typename RowOf>
__device__ inline void fill_qtables(int32_t* qtok, float* qinf, int s0, int n, RowOf& row_of,
                                    const typename Tr<DT>::T* __restrict__ gates, const float* __restrict__ lse3,
                                    const float* __restrict__ D3, const int32_t* __restrict__ perm, int H,
                                    int h, int64_t N) {
  const int tid = threadIdx.x;
  constexpr int PER = QSEG / NTH;
  int rr[PER], xx[PER];
  uint32_t mk[PER];
  int64_t tk[PER];
  float ls[PER], dd[PER], gg[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    rr[i] = 0;
    xx[i] = 0;
    mk[i] = 0;
    if (tid + i * NTH < n) {
      if constexpr (MASK) row_of(s0 + tid + i * NTH, rr[i], xx[i], mk[i]);
      else row_of(s0 + tid + i * NTH, rr[i], xx[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const bool ok = tid + i * NTH < n;
    const int64_t o = ((int64_t)xx[i] * H + h) * N + rr[i];
    tk[i] = ok ? perm[rr[i]] : 0;
    ls[i] = ok ? lse3[o] : 0.f;
    dd[i] = ok ? D3[o] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i)
    gg[i] = tid + i * NTH < n ? Tr<DT>::up(gates[(tk[i] * H + h) * 3 + xx[i]]) : 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (tid + i * NTH < n) {
      qtok[tid + i * NTH] = (int32_t)tk[i];
      qinf[tid + i * NTH] = ls[i];
      qinf[QPAD + tid + i * NTH] = gg[i];
      qinf[2 * QPAD + tid + i * NTH] = dd[i];
      if constexpr (MASK) reinterpret_cast<uint32_t*>(qinf)[3 * QPAD + tid + i * NTH] = mk[i];
    }
  }
  if (tid < (KT - n % KT) % KT) {
    qinf[n + tid] = INFINITY;
    qinf[QPAD + n + tid] = 0.f;
    qinf[2 * QPAD + n + tid] = 0.f;
    if constexpr (MASK) reinterpret_cast<uint32_t*>(qinf)[3 * QPAD + n + tid] = 0u;
  }
}

// dS and g P of a 32-query tile (queries as rows res_row(r, g) of tile t of the segment)
// from its scores S and dP, with (lse, g, D) from the segment's tables.
// MASK: a row whose key mask lacks bit mlane (the lane's key's group member) gets no weight.
template <bool MASK = false>
__device__ inline void tile_ds_pg(const ssa_f16v& sv, const ssa_f16v& dp, const float* qinf, int t, int g,
                                  float sl2, ssa_f16v& ds, ssa_f16v& pg, int mlane = 0) {
  // rows t KT + res_row(r, g) = t KT + 8 (r / 4) + 4 g + r % 4
  const float* base = qinf + t * KT + 4 * g;
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const float4 l4 = *reinterpret_cast<const float4*>(base + 8 * r4);
    const float4 g4 = *reinterpret_cast<const float4*>(base + QPAD + 8 * r4);
    const float4 d4 = *reinterpret_cast<const float4*>(base + 2 * QPAD + 8 * r4);
    const float la[4] = {l4.x, l4.y, l4.z, l4.w}, da[4] = {d4.x, d4.y, d4.z, d4.w};
    float ga[4] = {g4.x, g4.y, g4.z, g4.w};
    if constexpr (MASK) {
      const uint4 m4 = *reinterpret_cast<const uint4*>(base + 3 * QPAD + 8 * r4);
      const uint32_t ma[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) ga[e] = (ma[e] >> mlane) & 1u ? ga[e] : 0.f;  // g = 0: dS = gP = 0
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * r4 + e;
      float pr = fast_exp2(__builtin_fmaf(sv[r], sl2, -la[e]));
      if constexpr (MASK) pr = ga[e] != 0.f ? pr : 0.f;
      ds[r] = pr * (ga[e] * dp[r] - da[e]);
      pg[r] = ga[e] * pr;
    }
  }
}

// The query stream of a key-side kernel: `total` positions, position -> (sorted row r,
// branch x) by row_of.  Per segment of up to QSEG positions the tokens and (lse, g, D) of
// the branch go to LDS, then the segment's 32-row tiles (Q rows at 0, dO rows at VOFF) run
// through NB stage buffers (copies NB - 1 tiles ahead); per tile
//   S = Q K^T, P = exp2(S sl2 - lse), dP = dO V^T, dS = P o (g dP - D),
//   dv += (g P)^T dO, dk += dS^T Q
// (dS and g P with the queries as the contraction index, read back from registers).
template <int DT, int D, bool BUF, int NB, int NW, bool MASK = false, typename RowOf>
__device__ inline void kv_stream(KvState<DT, D>& S, TileCopy<DT, D, NW>& tc, typename Tr<DT>::T* const* bufs,
                                 int32_t* qtok, float* qinf, int total, const typename Tr<DT>::T* __restrict__ q,
                                 const typename Tr<DT>::T* __restrict__ dout,
                                 const typename Tr<DT>::T* __restrict__ gates,
                                 const float* __restrict__ lse3, const float* __restrict__ D3,
                                 const int32_t* __restrict__ perm, int H, int h, int64_t N, float sl2,
                                 bool wave_active, int wave, int lane, RowOf row_of, int mlane = 0) {
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  using F = typename Tr<DT>::frag;
  using TC = TileCopy<DT, D, NW>;
  constexpr int NTH = 64 * NW;
  const int tid = threadIdx.x, g = lane >> 5;
  for (int s0 = 0; s0 < total; s0 += QSEG) {
    const int n = min(QSEG, total - s0);
    __syncthreads();  // the previous segment's tiles have been read
    fill_qtables<DT, NTH, MASK>(qtok, qinf, s0, n, row_of, gates, lse3, D3, perm, H, h, N);
    __syncthreads();
    // S = Q K^T and dP = dO V^T of a tile (waves without keys compute on zero key rows;
    // their results are not written)
    auto sdp = [&](const T* cur, ssa_f16v& sv, ssa_f16v& dp) __attribute__((always_inline)) {
      sv = zero16();
      dp = zero16();
      const T* qrow = cur + (lane & 31) * C::KROW + g * C::KPL;
      const T* orow = cur + TC::VOFF + (lane & 31) * C::VROW + g * C::KPL;
      // every fragment read is issued before the first MFMA (one LDS round trip, not one
      // per K step)
      F qa[C::NKS], oa[C::NKS];
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) {
        qa[ks] = load_frag<DT>(qrow + ks * C::KS);
        oa[ks] = load_frag<DT>(orow + ks * C::KS);
      }
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) {
        sv = Tr<DT>::mma(qa[ks], S.kf[ks], sv);
        dp = Tr<DT>::mma(oa[ks], S.vf[ks], dp);
      }
      if constexpr (C::KPL != 1) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * C::NKS, 0);  // DS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * C::NKS, 0);  // then MFMAs
      }
    };
    // the rest of a tile: dS, g P, then dK, dV
    auto finish = [&](int t, const T* cur, const ssa_f16v& sv, const ssa_f16v& dp, auto&& next)
                      __attribute__((always_inline)) {
      ssa_f16v ds, pg;
      tile_ds_pg<MASK>(sv, dp, qinf, t, g, sl2, ds, pg, mlane);
      // 16-bit types: the transposed fragments of the tile are read before the next copy is
      // issued (the transpose reads carry no alias information); fp32 reads them in place
      // (registers) and issues the copy after its MFMAs
      constexpr bool PRE = C::KPL != 1;
      F qt[PRE ? C::PK : 1][C::NDV], ot[PRE ? C::PK : 1][C::NDV];
      if constexpr (PRE) {
#pragma unroll
        for (int ks = 0; ks < C::PK; ++ks)
#pragma unroll
          for (int jd = 0; jd < C::NDV; ++jd) {
            qt[ks][jd] = tr_frag<DT, C::KROW>(cur, ks, jd, lane);
            ot[ks][jd] = tr_frag<DT, C::VROW>(cur + TC::VOFF, ks, jd, lane);
          }
        next();
      }
#pragma unroll
      for (int ks = 0; ks < C::PK; ++ks) {
        const F pf = p_frag<DT>(pg, ks), sf = p_frag<DT>(ds, ks);
#pragma unroll
        for (int jd = 0; jd < C::NDV; ++jd) {
          S.dv[jd] = Tr<DT>::mma(pf, PRE ? ot[ks][jd] : tr_frag<DT, C::VROW>(cur + TC::VOFF, ks, jd, lane),
                                 S.dv[jd]);
          S.dk[jd] = Tr<DT>::mma(sf, PRE ? qt[ks][jd] : tr_frag<DT, C::KROW>(cur, ks, jd, lane), S.dk[jd]);
        }
      }
      if constexpr (!PRE) next();
    };
    auto fetch = [&](int t) __attribute__((always_inline)) { tc.fetch(qtok, t * KT, n); };
    auto issue = [&](T* dst) __attribute__((always_inline)) { tc.template issue<BUF>(dst, q, dout, H, h, wave); };
    if constexpr (sizeof(T) == 2 && D <= 96) {  // (registers for the second slot)
      // S and dP of tile t + 1 run on the matrix cores while tile t is finished (two slots)
      ssa_f16v sv[2], dp[2];
      tile_pipeline_ahead<NB, TC::NI>(
          (n + KT - 1) / KT, bufs, fetch, issue,
          [&](int, const T* cur, auto sc) __attribute__((always_inline)) {
            sdp(cur, sv[decltype(sc)::value], dp[decltype(sc)::value]);
          },
          [&](int t, const T* cur, auto sc, auto&& next) __attribute__((always_inline)) {
            finish(t, cur, sv[decltype(sc)::value], dp[decltype(sc)::value], next);
          });
    } else {
      tile_pipeline<NB, TC::NI>((n + KT - 1) / KT, bufs, fetch, issue,
                                [&](int t, const T* cur, auto&& next) __attribute__((always_inline)) {
                                  ssa_f16v sv, dp;
                                  sdp(cur, sv, dp);
                                  finish(t, cur, sv, dp, next);
                                });
    }
  }
}

// Narrow key blocks (at most 32 keys): every wave holds the same 32 keys, and wave w takes
// the query tiles w, w + NW, w + 2 NW, ... of each segment, each wave copying its own tiles
// through its own two buffers (the copy of its next tile issued while it finishes the
// current one), with no workgroup barrier inside a segment.  The waves' dK, dV are partial
// sums over their tiles, added in wave order by the caller.
template <int DT, int D, bool BUF, int NW, typename RowOf>
__device__ inline void kv_stream_narrow(KvState<DT, D>& S, typename Tr<DT>::T* b0, typename Tr<DT>::T* b1,
                                        typename Tr<DT>::T* b2, typename Tr<DT>::T* b3, typename Tr<DT>::T* b4,
                                        typename Tr<DT>::T* b5, typename Tr<DT>::T* b6, typename Tr<DT>::T* b7,
                                        int32_t* qtok,
                                        float* qinf, int total, const typename Tr<DT>::T* __restrict__ q,
                                        const typename Tr<DT>::T* __restrict__ dout,
                                        const typename Tr<DT>::T* __restrict__ gates,
                                        const float* __restrict__ lse3, const float* __restrict__ D3,
                                        const int32_t* __restrict__ perm, int H, int h, int64_t N, float sl2,
                                        int wave, int lane, RowOf row_of) {
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  using F = typename Tr<DT>::frag;
  using T1 = TileCopy<DT, D, 1>;  // one wave copies a whole tile (the same layout)
  constexpr int NTH = 64 * NW;
  static_assert(T1::ELEMS <= TileCopy<DT, D, NW>::ELEMS, "a wave's tile fits a stage buffer");
  const int g = lane >> 5;
  // copy of the tile of segment rows k0 .. k0 + 31 into `stage`: instruction m covers 16-byte
  // positions 64 m .. 64 m + 63 of the K part (m < KI) or of the V part; row and chunk of a
  // lane are computed per instruction, the token read just before its copy
  auto copy_tile = [&](T* stage, int k0, int n) __attribute__((always_inline)) {
    int tk[T1::KI + T1::VI];
#pragma unroll
    for (int m = 0; m < T1::KI + T1::VI; ++m) {
      const bool isk = m < T1::KI;
      const int p = (isk ? m : m - T1::KI) * 64 + lane;
      const int rr = isk ? p / T1::KRC : p / T1::VRC;
      const int j = k0 + (rr < KT ? rr : 0);
      tk[m] = qtok[j < n ? j : 0];
    }
#pragma unroll
    for (int m = 0; m < T1::KI + T1::VI; ++m) {
      const bool isk = m < T1::KI;
      const int p = (isk ? m : m - T1::KI) * 64 + lane;
      const int ch = isk ? p % T1::KRC : p % T1::VRC;
      const int goff = ch < C::CPR ? ch * C::EPC : 0;  // padding lanes copy a valid chunk
      lds_void_t* dst = (lds_void_t*)(stage + m * 64 * C::EPC);
      if constexpr (BUF) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<T*>((isk ? q : dout) + h * D), 0, -1, 0x00020000);
        const uint32_t off = ((uint32_t)tk[m] * (uint32_t)(H * D) + (uint32_t)goff) * (uint32_t)sizeof(T);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, off, 0, 0, 0);
      } else {
        dma16((isk ? q : dout) + ((int64_t)tk[m] * H + h) * D + goff, stage + m * 64 * C::EPC);
      }
    }
  };
  for (int s0 = 0; s0 < total; s0 += QSEG) {
    const int n = min(QSEG, total - s0);
    __syncthreads();  // every wave is done with the previous segment
    fill_qtables<DT, NTH>(qtok, qinf, s0, n, row_of, gates, lse3, D3, perm, H, h, N);
    __syncthreads();
    const int ntile = (n + KT - 1) / KT;
    // one tile of this wave: stage `cur`, the next tile of the wave goes to `oth`
    auto step = [&](int t, T* cur, T* oth) __attribute__((always_inline)) {
      vm_wait<0>();  // tile t landed (the wave's only copy in flight)
      const T* qrow = cur + (lane & 31) * C::KROW + g * C::KPL;
      const T* orow = cur + T1::VOFF + (lane & 31) * C::VROW + g * C::KPL;
      ssa_f16v sv = zero16(), dp = zero16();
      {
        F qa[C::NKS], oa[C::NKS];  // all fragment reads before the first MFMA
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
          qa[ks] = load_frag<DT>(qrow + ks * C::KS);
          oa[ks] = load_frag<DT>(orow + ks * C::KS);
        }
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
          sv = Tr<DT>::mma(qa[ks], S.kf[ks], sv);
          dp = Tr<DT>::mma(oa[ks], S.vf[ks], dp);
        }
      }
      ssa_f16v ds, pg;
      tile_ds_pg(sv, dp, qinf, t, g, sl2, ds, pg);
      F qt[C::PK][C::NDV], ot[C::PK][C::NDV];  // read before the next copy is issued
#pragma unroll
      for (int ks = 0; ks < C::PK; ++ks)
#pragma unroll
        for (int jd = 0; jd < C::NDV; ++jd) {
          qt[ks][jd] = tr_frag<DT, C::KROW>(cur, ks, jd, lane);
          ot[ks][jd] = tr_frag<DT, C::VROW>(cur + T1::VOFF, ks, jd, lane);
        }
      if (t + NW < ntile) copy_tile(oth, (t + NW) * KT, n);
#pragma unroll
      for (int ks = 0; ks < C::PK; ++ks) {
        const F pf = p_frag<DT>(pg, ks), sf = p_frag<DT>(ds, ks);
#pragma unroll
        for (int jd = 0; jd < C::NDV; ++jd) {
          S.dv[jd] = Tr<DT>::mma(pf, ot[ks][jd], S.dv[jd]);
          S.dk[jd] = Tr<DT>::mma(sf, qt[ks][jd], S.dk[jd]);
        }
      }
    };
    auto run = [&](T* ba, T* bb) __attribute__((always_inline)) {
      if (wave >= ntile) return;
      copy_tile(ba, wave * KT, n);
      for (int t = wave; t < ntile; t += 2 * NW) {
        step(t, ba, bb);
        if (t + NW < ntile) step(t + NW, bb, ba);
      }
    };
    // static buffer pairs per wave (the compiler keeps each copy apart from the other reads)
    static_assert(NW == 4, "four waves, eight buffers");
    if (wave == 0) run(b0, b1);
    else if (wave == 1) run(b2, b3);
    else if (wave == 2) run(b4, b5);
    else run(b6, b7);
  }
}

// Resident workgroups (a multiple of 8) take their XCD's list of items of one kind
// round-robin.  KV_UNIT: an item is 128 keys of a unit's block and one piece of its query
// stream.  KV_NARROW: a unit of at most 32 keys, one piece (kv_stream_narrow).  KV_GRP: a
// key-group piece.  An unsplit unit writes dK, dV (with the block's compressed-branch
// terms); pieces write their partial sums to kpart.
template <int DT, int D, bool BUF, int MODE>
__global__ __launch_bounds__(64 * KW) void k_bwd_dkdv(
    const typename Tr<DT>::T* __restrict__ q, const typename Tr<DT>::T* __restrict__ kin,
    const typename Tr<DT>::T* __restrict__ vin, const typename Tr<DT>::T* __restrict__ gates,
    const typename Tr<DT>::T* __restrict__ dout, const float* __restrict__ lse3,
    const float* __restrict__ D3, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ blk_off, const int32_t* __restrict__ blk_cell,
    const int32_t* __restrict__ cell_off, const int32_t* __restrict__ cell_blk,
    const int4* __restrict__ items, const int32_t* __restrict__ xbase, const int32_t* __restrict__ inv_off,
    const int32_t* __restrict__ inv_q, const int32_t* __restrict__ sel, int topk,
    const int4* __restrict__ grp_meta, const int4* __restrict__ grp_mem, int M, int H, int64_t N,
    float scale, float sl2, const float* __restrict__ ukv, int Mp, float* __restrict__ kpart,
    float* __restrict__ dk, float* __restrict__ dv) {
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  using TC = TileCopy<DT, D, KW>;
  constexpr int NTH = 64 * KW;
  constexpr bool NARROW = MODE == KV_NARROW;  // eight stage buffers, two per wave
  constexpr bool MASK = MODE == KV_GRP;
  constexpr int QPLANES = MASK ? 4 : 3;
  constexpr int NB = NARROW ? 6
                            : stage_depth<DT, D, KW>(LDS_BYTES - 4096, QSEG * 4 + QPLANES * QPAD * 4 + (3 * NTH + 1) * 4);
  static_assert(!NARROW || KW == 4, "four waves with two buffers each");
  static_assert(!NARROW || 32 * D * 4 <= TC::ELEMS * (int)sizeof(T), "a wave's partial dK or dV fits a buffer");
  SSA_STAGE_BUFFERS(T, TC::ELEMS, NB);
  __shared__ __attribute__((aligned(NARROW ? 1024 : 16))) T buf6[NARROW ? TC::ELEMS : 16 / sizeof(T)];
  __shared__ __attribute__((aligned(NARROW ? 1024 : 16))) T buf7[NARROW ? TC::ELEMS : 16 / sizeof(T)];
  __shared__ int32_t pre[NTH + 1];
  __shared__ int32_t lst_off[NTH];
  __shared__ int32_t ent_x[NTH];  // an entry's branch, or a key-group entry's member mask
  __shared__ int32_t qtok[QSEG];
  __shared__ __attribute__((aligned(16))) float qinf[QPLANES * QPAD];  // lse, g, D (, mask)
  __shared__ int32_t gmb[MASK ? KG_MEM : 1], gko[MASK ? KG_MEM + 1 : 1], gpr[MASK ? KG_MEM : 1],
      grw[MASK ? KG_MEM : 1], wsum[KW];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int x = blockIdx.x % NXCD, nx = gridDim.x / NXCD;
  const int ib = xbase[MODE * 9 + x], ie = xbase[MODE * 9 + x + 1];
  TC tc;
  tc.init(wave, lane);
#pragma unroll 1
  for (int it = ib + (int)blockIdx.x / NXCD; it < ie; it += nx) {
    const int4 item = items[it];
    if constexpr (MODE == KV_GRP) {
      // ---- key group piece: members' keys in slots 0 .. keys - 1 (member m from slot
      // gko[m]); the query blocks of piece gp whose selection holds a member, each row masked
      // to those members
      const int4 gm = grp_meta[-item.x - 1];  // {head, members, first member, keys}
      const int gh = gm.x, nmem = gm.y, keys = gm.w, gp = item.y;
      __syncthreads();  // the previous item's tables are no longer read
      if (tid < nmem) {
        const int4 mm = grp_mem[gm.z + tid];  // {block, first slot, partial row, rows}
        gmb[tid] = mm.x;
        gko[tid] = mm.y;
        gpr[tid] = mm.z;
        grw[tid] = mm.w;
      }
      if (tid == 0) gko[nmem] = keys;
      __syncthreads();
      auto member_of = [&](int slot) __attribute__((always_inline)) {
        int m = 0;  // last member starting at or before the slot
        for (int i = 1; i < nmem; ++i) m = gko[i] <= slot ? i : m;
        return m;
      };
      const int slot = wave * 32 + c;
      const bool kvalid = slot < keys;
      const int mlane = kvalid ? member_of(slot) : 0;
      const int64_t ktok = kvalid ? perm[blk_off[gmb[mlane]] + slot - gko[mlane]] : 0;
      KvState<DT, D> S;
      load_q<DT, D>(S.kf, kin + (ktok * H + gh) * D, kvalid, lane);
      load_q<DT, D>(S.vf, vin + (ktok * H + gh) * D, kvalid, lane);
#pragma unroll
      for (int j = 0; j < C::NDV; ++j) S.dk[j] = S.dv[j] = zero16();
      const int qbp = kg_qbp(M);  // at most NTH (M is within the forward's limit)
      const int qb = gp * qbp + tid;
      uint32_t msk = 0;
      if (tid < qbp && qb < M) {
        const int32_t* srow = sel + ((int64_t)gh * M + qb) * topk;
        for (int t = 0; t < topk; ++t) {
          const int sb = srow[t];
          if (sb < 0) break;  // ids ascend, -1 padded at the end
          for (int i = 0; i < nmem; ++i) msk |= gmb[i] == sb ? 1u << i : 0u;
        }
      }
      // compaction in block order: wave ballots, then the waves' counts
      const uint64_t bal = __builtin_amdgcn_ballot_w64(msk != 0);
      if (lane == 0) wsum[wave] = __builtin_popcountll(bal);
      pre[tid + 1] = 0;
      if (tid == 0) pre[0] = 0;
      __syncthreads();
      int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
      int L = 0;
      for (int w2 = 0; w2 < KW; ++w2) {
        pos += w2 < wave ? wsum[w2] : 0;
        L += wsum[w2];
      }
      if (msk != 0) {
        lst_off[pos] = blk_off[qb];
        ent_x[pos] = (int)msk;
        pre[pos + 1] = blk_off[qb + 1] - blk_off[qb];
      }
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
      kv_stream<DT, D, BUF, NB, KW, true>(
          S, tc, bufs, qtok, qinf, total, q, dout, gates, lse3, D3, perm, H, gh, N, sl2, true, wave, lane,
          [&](int pos2, int& r, int& xb, uint32_t& mk) __attribute__((always_inline)) {
            int lo = 0, hi = L - 1;  // last entry starting at or before pos2
            while (lo < hi) {
              const int mid = (lo + hi + 1) >> 1;
              if (pre[mid] <= pos2) lo = mid; else hi = mid - 1;
            }
            r = lst_off[lo] + (pos2 - pre[lo]);
            xb = 1;
            mk = (uint32_t)ent_x[lo];
          },
          mlane);
      // partial sums: group piece gp is piece 1 + gp of each member; lane holds column
      // 32j + c of key slots wave 32 + res_row(r, g)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int sl = wave * 32 + res_row(r, g);
        if (sl < keys) {
          const int m = member_of(sl);
          float* dst = kpart + ((int64_t)gpr[m] + (int64_t)(1 + gp) * grw[m] + (sl - gko[m])) * 2 * D;
#pragma unroll
          for (int j = 0; j < C::NDV; ++j) {
            dst[32 * j + c] = scale * S.dk[j][r];
            dst[D + 32 * j + c] = S.dv[j][r];
          }
        }
      }
    } else {
      const int h = item.x / M, b = item.x % M, chunk = item.y, piece = item.z, prow = item.w;
      const int r0 = blk_off[b], rows = blk_off[b + 1] - r0;
      // narrow (at most 32 keys): every wave holds the block's keys and takes a share of the
      // query tiles
      const int kbase = NARROW ? 0 : chunk * KROWS + wave * 32;
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
      const int i0 = inv_off[item.x], ninv = inv_off[item.x + 1] - i0;
      const int nent = nwin + ninv;  // window query blocks, then the selecting ones
      // piece -1: a tiny unit's window part (its selecting query blocks are in a key group)
      const int e_lo = prow < 0 || piece < 0 ? 0 : piece * KV_EP;
      const int e_hi = prow < 0 ? nent : (piece < 0 ? nwin : min(nent, e_lo + KV_EP));

      for (int e0 = e_lo; e0 < e_hi; e0 += NTH) {
        const int L = min(NTH, e_hi - e0);
        __syncthreads();  // the previous tables and stages are no longer read
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
        auto row_of = [&](int pos, int& r, int& xb) __attribute__((always_inline)) {
          int lo = 0, hi = L - 1;  // last entry starting at or before pos
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] <= pos) lo = mid; else hi = mid - 1;
          }
          r = lst_off[lo] + (pos - pre[lo]);
          xb = ent_x[lo];
        };
        if constexpr (NARROW)
          kv_stream_narrow<DT, D, BUF, KW>(S, buf0, buf1, buf2, buf3, buf4, buf5, buf6, buf7, qtok, qinf, total, q,
                                           dout, gates, lse3, D3, perm, H, h, N, sl2, wave, lane, row_of);
        else
          kv_stream<DT, D, BUF, NB, KW>(S, tc, bufs, qtok, qinf, total, q, dout, gates, lse3, D3, perm, H, h, N,
                                        sl2, wave_active, wave, lane, row_of);
      }
      const float* uk = ukv + ((int64_t)h * Mp + b) * D;
      const float* uv = ukv + (((int64_t)H + h) * Mp + b) * D;
      if constexpr (NARROW) {
        // the waves' partial sums, added in wave order
        __syncthreads();  // every wave's stream is done: the buffers are free
        float* pk = reinterpret_cast<float*>(wave == 0 ? buf0 : wave == 1 ? buf1 : wave == 2 ? buf2 : buf3);
        float* pv = reinterpret_cast<float*>(wave == 0 ? buf4 : wave == 1 ? buf5 : wave == 2 ? buf6 : buf7);
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
          for (int j = 0; j < C::NDV; ++j) {
            pk[res_row(r, g) * D + 32 * j + c] = S.dk[j][r];
            pv[res_row(r, g) * D + 32 * j + c] = S.dv[j][r];
          }
        __syncthreads();
        for (int idx = tid; idx < rows * D; idx += NTH) {
          auto at = [&](const T* bf) __attribute__((always_inline)) { return reinterpret_cast<const float*>(bf)[idx]; };
          const float sk = ((at(buf0) + at(buf1)) + at(buf2)) + at(buf3);
          const float sv = ((at(buf4) + at(buf5)) + at(buf6)) + at(buf7);
          const int kr = idx / D, col = idx % D;
          if (prow < 0) {
            const int64_t t = perm[r0 + kr];
            dk[(t * H + h) * D + col] = scale * sk + uk[col];
            dv[(t * H + h) * D + col] = sv + uv[col];
          } else {
            float* dst = kpart + ((int64_t)prow + kr) * 2 * D;
            dst[col] = scale * sk;
            dst[D + col] = sv;
          }
        }
        __syncthreads();  // the buffers are read before the next item's copies
      } else if (prow < 0) {
        // lane holds column 32j + c of keys res_row(r, g)
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
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = kbase + res_row(r, g);
          if (kr < rows) {
            float* dst = kpart + ((int64_t)prow + kr) * 2 * D;
#pragma unroll
            for (int j = 0; j < C::NDV; ++j) {
              dst[32 * j + c] = scale * S.dk[j][r];
              dst[D + 32 * j + c] = S.dv[j][r];
            }
          }
        }
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
  constexpr int NB = stage_depth<DT, D, BW>(LDS_BYTES - 4096, QSEG * 20);
  SSA_STAGE_BUFFERS(T, TC::ELEMS, NB);
  __shared__ int32_t qtok[QSEG];
  __shared__ __attribute__((aligned(16))) float qinf[3 * QPAD];
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
  kv_stream<DT, D, BUF, NB, BW>(S, tc, bufs, qtok, qinf, total, q, dout, gates, lse3, D3, perm, H,
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
    float* __restrict__ part_k, float* __restrict__ part_v,
    const int32_t* __restrict__ blk_off, int Mp, int H, int qch, float* __restrict__ ukv, int conv) {
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
  if (conv) {  // no term shared by the block: each token's own position weight maps it later
    for (int j = tid; j < 2 * D; j += 256) {
      const bool isk = j < D;
      const int i = isk ? j : j - D;
      ukv[(((int64_t)(isk ? 0 : 1) * H + h) * Mp + b) * D + i] = 0.f;
      (isk ? part_k : part_v)[((int64_t)h * Mp + b) * D + i] = (isk ? gk : gv)[i] * inv;  // chunk 0's slot
    }
    return;
  }
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
                        hipStream_t s, int conv) {
  using T = typename Tr<DT>::T;
  const int M = (int)p->M;
  const int Mp = (int)pooled_rows(M);
  const int64_t N = p->n;
  const float sl2 = scale * 1.4426950408889634f;
  const int nchunk = (p->max_rows + BROWS - 1) / BROWS;
  constexpr int PREP_GS = 16 / sizeof(T) * 16 >= D ? 16 : (16 / sizeof(T) * 32 >= D ? 32 : 64);
  using ST = typename SaveT<DT>::type;
  const int64_t plane = N * H * D;  // f16: the compressed branch's plane is oc
  const ST* o0 = DT == DT_F16 ? (const ST*)fw.oc : (const ST*)fw.obr;
  const ST* o1 = (const ST*)fw.obr + (DT == DT_F16 ? 0 : plane);
  const ST* o2 = (const ST*)fw.obr + (DT == DT_F16 ? 1 : 2) * plane;
  hipLaunchKernelGGL((k_bwd_prep<DT, D>), dim3((unsigned)((N * H * PREP_GS + 255) / 256)), dim3(256), 0, s,
                     (const T*)dout, (const T*)gates, o0, o1, o2, p->perm, N, H, dgates, w.D);
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
                     w.part_k, w.part_v, p->blk_off, Mp, H, w.qch, w.ukv, conv);
  // key-side schedule
  const int U = H * M;
  hipLaunchKernelGGL(k_kv_keys, dim3((U + 255) / 256), dim3(256), 0, s, w.inv_off, p->blk_cell, p->cell_off, M,
                     U, w.ska, w.sva);
  uint32_t *sa = w.ska, *sb2 = w.skb;
  int32_t *oa = w.sva, *ob = w.svb;
  e = ssa_sort::radix_sort(sa, oa, sb2, ob, U, ssa_sort::bits_for((uint64_t)H * (2 * M + 1)), w.rank, w.hist,
                           w.part, s);
  if (e != hipSuccess) return e;
  // narrow units (at most 32 keys) where the eight-buffer form fits: 16-bit, d <= 96
  constexpr bool narrow_ok = sizeof(T) == 2 && D <= 96;
  hipLaunchKernelGGL(k_kv_schedule, dim3(1), dim3(1024), 0, s, oa, U, M, H, narrow_ok ? 1 : 0, w.inv_off,
                     p->blk_cell, p->cell_off, p->blk_off, kv_budget_rows(D), w.sinfo, w.ioff, w.xbase, w.grp_meta,
                     w.grp_mem, w.ngrp, w.items);
  hipLaunchKernelGGL(k_kv_items, dim3((U + 255) / 256), dim3(256), 0, s, w.sinfo, w.ioff, w.xbase, p->blk_off, U,
                     M, w.items);
  int dev = 0, cus = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  // one resident grid (a multiple of 8) per item kind; each kind's lists are read from xbase
  auto launch_kind = [&](auto kernel) -> hipError_t {
    int per_cu = 0;
    hipError_t e2 = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * KW, 0);
    if (e2 != hipSuccess) return e2;
    const unsigned grid = (unsigned)std::max<int64_t>(NXCD, (int64_t)cus * std::max(per_cu, 1) / NXCD * NXCD);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(64 * KW), 0, s, (const T*)q, (const T*)k, (const T*)v,
                       (const T*)gates, (const T*)dout, fw.lse, w.D, p->perm, p->blk_off, p->blk_cell, p->cell_off,
                       p->cell_blk, w.items, w.xbase, w.inv_off, va, sel, topk, w.grp_meta, w.grp_mem, M, H, N, scale,
                       sl2, w.ukv, Mp, w.kpart, dk, dv);
    return hipSuccess;
  };
  if (buf) {
    if ((e = launch_kind(k_bwd_dkdv<DT, D, true, KV_GRP>)) != hipSuccess) return e;
    if ((e = launch_kind(k_bwd_dkdv<DT, D, true, KV_UNIT>)) != hipSuccess) return e;
    if constexpr (narrow_ok)
      if ((e = launch_kind(k_bwd_dkdv<DT, D, true, KV_NARROW>)) != hipSuccess) return e;
  } else {
    if ((e = launch_kind(k_bwd_dkdv<DT, D, false, KV_GRP>)) != hipSuccess) return e;
    if ((e = launch_kind(k_bwd_dkdv<DT, D, false, KV_UNIT>)) != hipSuccess) return e;
    if constexpr (narrow_ok)
      if ((e = launch_kind(k_bwd_dkdv<DT, D, false, KV_NARROW>)) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_kv_reduce<D>), dim3(U), dim3(256), 0, s, w.sinfo, w.kpart, w.ukv, p->blk_off, p->perm,
                     M, Mp, H, dk, dv);
  if (conv) {  // the compressed branch's term through each token's own position weight
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_conv_term((ssa_dtype)DT, p, H, D, wk, wv, w.part_k, w.part_v, dk, dv, s);
  }
  return hipGetLastError();
}

template <int DT>
hipError_t backward_d(int d, const ssa_plan_s* p, int H, int topk, float scale, const void* q,
                      const void* k, const void* v, const void* wk, const void* wv,
                      const void* gates, const int32_t* sel, const void* dout, float* dq,
                      float* dk, float* dv, float* dgates, const FwdWs& fw, const BwdWs& w,
                      hipStream_t s, int conv) {
  switch (d) {
    case 32: return run_backward<DT, 32>(p, H, topk, scale, q, k, v, wk, wv, gates, sel, dout, dq, dk, dv, dgates, fw, w, s, conv);
    case 64: return run_backward<DT, 64>(p, H, topk, scale, q, k, v, wk, wv, gates, sel, dout, dq, dk, dv, dgates, fw, w, s, conv);
    case 96: return run_backward<DT, 96>(p, H, topk, scale, q, k, v, wk, wv, gates, sel, dout, dq, dk, dv, dgates, fw, w, s, conv);
    case 128: return run_backward<DT, 128>(p, H, topk, scale, q, k, v, wk, wv, gates, sel, dout, dq, dk, dv, dgates, fw, w, s, conv);
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
                           void* ws, hipStream_t s, int conv) {
  Carver c(ws);
  c.off = (256 - (reinterpret_cast<uintptr_t>(ws) & 255)) & 255;
  BwdWs w;
  carve(c, p, H, d, topk, &w);
  switch (dt) {
    case SSA_F32: return backward_d<DT_F32>(d, p, H, topk, scale, q, k, v, wk, wv, gates, sel, dout, dq, dk, dv, dgates, fw, w, s, conv);
    case SSA_F16: return backward_d<DT_F16>(d, p, H, topk, scale, q, k, v, wk, wv, gates, sel, dout, dq, dk, dv, dgates, fw, w, s, conv);
    case SSA_BF16: return backward_d<DT_BF16>(d, p, H, topk, scale, q, k, v, wk, wv, gates, sel, dout, dq, dk, dv, dgates, fw, w, s, conv);
  }
  return hipErrorInvalidValue;
}
