// The sparse-convolution compressor of SSA's compression branch, forward and backward.
//
// The nav.superapi.store Direct3D-S2 page ("Technical principles of Direct3D-S2") has the
// compression module extract block-level information by sparse 3D convolution and pooling.
// Reading: a convolution with kernel size and stride B over the occupied voxels -- every block
// is one output site and every voxel's weight depends on its position inside the block --
// followed by the mean over the block's occupied voxels:
//   ktil[h,b] = (1/n_b) sum_{i in b} k[i,h] Wc_k[o(i)]^T,  Wc [B^3][d_out][d_in],
// o(i) = (c_i mod B) as the x-major index (the plan's `pos`).  vtil likewise with Wc_v.
//
// Forward (k_pool_conv): per (block, group of up to 32 heads), the block's tokens are dealt to
// the waves; for each token a [heads x d_in] x [d_in x d_out] product on MFMA (A: the token's
// K rows, one head per row; B: its position's weight, read as contiguous runs of d_in)
// accumulates into the wave's tile; the waves' tiles are added in wave order through LDS,
// divided by n_b and stored exactly as the mean-pool kernel stores its result (fp32 key split
// into dtype planes, values transposed in the stage, row-major values).
// Backward (k_bwd_conv_term): dk[i,h] += g_k[h,b] Wc_k[o(i)] with g_k = dktil / n_b, added to
// the gradients the rest of the backward wrote (which carry no shared compressed term here).
#include <hip/hip_runtime.h>
#include "ssa_internal.h"
#include "ssa_mfma.h"
#include "ssa_tiles.h"

namespace {

using namespace ssa_dev;
constexpr int CV_WAVES = 4;

template <int DT, int D>
__global__ __launch_bounds__(64 * CV_WAVES) void k_pool_conv(
    const typename Tr<DT>::T* __restrict__ kin, const typename Tr<DT>::T* __restrict__ vin,
    const typename Tr<DT>::T* __restrict__ wck, const typename Tr<DT>::T* __restrict__ wcv,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ pos, const int32_t* __restrict__ blk_off,
    const int32_t* __restrict__ lpt, int M, int Mp, int H, typename Tr<DT>::T* __restrict__ pooled,
    typename Tr<DT>::T* __restrict__ pooled_v) {
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  using F = typename Tr<DT>::frag;
  constexpr int NS = C::NS, NDV = C::NDV, NKS = C::NKS;
  __shared__ float red[CV_WAVES][32 * D];  // every wave's [32 heads][D] tile
  const int nhg = (H + 31) / 32;
  const int unit = blockIdx.x / nhg, h0 = (blockIdx.x % nhg) * 32;
  const int hn = min(32, H - h0);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = unit < M ? lpt[unit] : unit;
  auto stage_of = [&](int h) { return pooled + ((int64_t)h * (Mp / C::PT) + b / C::PT) * C::STAGE; };
  if (b >= M) {  // zero padding block (as the mean-pool kernel writes it)
    for (int j = tid; j < hn * C::KROW; j += 64 * CV_WAVES) {
      const int h = h0 + j / C::KROW, cc = j % C::KROW;
      T* stg = stage_of(h);
      for (int s = 0; s < NS; ++s) stg[s * C::KPLANE + (b % C::PT) * C::KROW + cc] = (T)0.f;
      if (cc < D) {
        stg[NS * C::KPLANE + cc * C::VTROW + (b % C::PT)] = (T)0.f;
        pooled_v[((int64_t)h * Mp + b) * C::VROW + cc] = (T)0.f;
      }
    }
    return;
  }
  const int r0 = blk_off[b], r1 = blk_off[b + 1];
  const float inv = 1.f / (float)(r1 - r0);
  const int hh = h0 + c;  // this lane's head (A operand row)
  for (int kv = 0; kv < 2; ++kv) {
    const T* src = kv ? vin : kin;
    const T* wc = kv ? wcv : wck;
    ssa_f16v acc[NDV];
#pragma unroll
    for (int j = 0; j < NDV; ++j) acc[j] = zero16();
    for (int r = r0 + wave; r < r1; r += CV_WAVES) {
      const int tok = perm[r];
      const int o = pos[tok];
      const T* arow = src + ((int64_t)tok * H + (hh < H ? hh : 0)) * D + g * C::KPL;
      F af[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) af[ks] = hh < H ? load_frag<DT>(arow + ks * C::KS) : zero_frag<DT>();
      const T* wrow = wc + ((int64_t)o * D + c) * D + g * C::KPL;
#pragma unroll
      for (int j = 0; j < NDV; ++j)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          acc[j] = Tr<DT>::mma(af[ks], load_frag<DT>(wrow + (int64_t)32 * j * D + ks * C::KS), acc[j]);
    }
    // this wave's [head][out] tile to LDS, then the sum over waves in wave order
#pragma unroll
    for (int j = 0; j < NDV; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[wave][res_row(r, g) * D + 32 * j + c] = acc[j][r];
    __syncthreads();
    for (int e = tid; e < hn * D; e += 64 * CV_WAVES) {
      const int hl = e / D, cc = e % D, h = h0 + hl;
      float val = 0.f;
#pragma unroll
      for (int w = 0; w < CV_WAVES; ++w) val += red[w][hl * D + cc];
      val *= inv;
      T* stg = stage_of(h);
      if (kv == 0) {
        float rem = val;
        for (int s = 0; s < NS; ++s) {
          const T part = Tr<DT>::cvt(rem);
          stg[s * C::KPLANE + (b % C::PT) * C::KROW + cc] = part;
          rem -= Tr<DT>::up(part);
        }
        if (cc < C::KROW - D)
          for (int s = 0; s < NS; ++s) stg[s * C::KPLANE + (b % C::PT) * C::KROW + D + cc] = (T)0.f;
      } else {
        const T vv = Tr<DT>::cvt(val);
        stg[NS * C::KPLANE + cc * C::VTROW + (b % C::PT)] = vv;
        pooled_v[((int64_t)h * Mp + b) * C::VROW + cc] = vv;
      }
    }
    __syncthreads();  // LDS reused by the values
  }
}

// dk[i,h,:] += g_k[h, b(i), :] Wc_k[o(i)] (d_out -> d_in), dv likewise; g already divided by n_b.
// One workgroup per token; thread e covers (tensor, head, d_in) entries e, e + 256, ...
template <int DT, int D>
__global__ __launch_bounds__(256) void k_bwd_conv_term(
    const typename Tr<DT>::T* __restrict__ wck, const typename Tr<DT>::T* __restrict__ wcv,
    const float* __restrict__ gk, const float* __restrict__ gv, const int32_t* __restrict__ tok2blk,
    const int32_t* __restrict__ pos, int Mp, int H, float* __restrict__ dk, float* __restrict__ dv) {
  __shared__ float gl[2][32 * D];
  const int64_t tok = blockIdx.x;
  const int b = tok2blk[tok], o = pos[tok];
  for (int h0 = 0; h0 < H; h0 += 32) {
    const int hn = min(32, H - h0);
    __syncthreads();
    for (int e = threadIdx.x; e < 2 * hn * D; e += 256) {
      const int kv = e / (hn * D), r = e % (hn * D), hl = r / D, cc = r % D;
      gl[kv][hl * D + cc] = (kv ? gv : gk)[((int64_t)(h0 + hl) * Mp + b) * D + cc];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 2 * hn * D; e += 256) {
      const int kv = e / (hn * D), r = e % (hn * D), hl = r / D, in = r % D;
      const typename Tr<DT>::T* W = (kv ? wcv : wck) + (int64_t)o * D * D + in;
      const float* g = gl[kv] + hl * D;
      float s0 = 0.f, s1 = 0.f;
#pragma unroll 8
      for (int out = 0; out < D; out += 2) {
        s0 += g[out] * Tr<DT>::up(W[(int64_t)out * D]);
        s1 += g[out + 1] * Tr<DT>::up(W[(int64_t)(out + 1) * D]);
      }
      float* dst = (kv ? dv : dk) + (tok * H + h0 + hl) * D + in;
      *dst += s0 + s1;
    }
  }
}

template <int DT, int D>
hipError_t run_pool_conv(const ssa_plan_s* p, int H, const void* k, const void* v, const void* wck,
                         const void* wcv, const FwdWs& w, hipStream_t s) {
  using T = typename Tr<DT>::T;
  const int Mp = (int)pooled_rows(p->M);
  const int nhg = (H + 31) / 32;
  hipLaunchKernelGGL((k_pool_conv<DT, D>), dim3((unsigned)(Mp * nhg)), dim3(64 * CV_WAVES), 0, s, (const T*)k,
                     (const T*)v, (const T*)wck, (const T*)wcv, p->perm, p->pos, p->blk_off, p->lpt, (int)p->M,
                     Mp, H, (T*)w.pooled, (T*)w.pooled_v);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t run_conv_term(const ssa_plan_s* p, int H, const void* wck, const void* wcv, const float* gk,
                         const float* gv, float* dk, float* dv, hipStream_t s) {
  using T = typename Tr<DT>::T;
  hipLaunchKernelGGL((k_bwd_conv_term<DT, D>), dim3((unsigned)p->n), dim3(256), 0, s, (const T*)wck,
                     (const T*)wcv, gk, gv, p->tok2blk, p->pos, (int)pooled_rows(p->M), H, dk, dv);
  return hipGetLastError();
}

template <int DT>
hipError_t pool_conv_d(int d, const ssa_plan_s* p, int H, const void* k, const void* v, const void* wck,
                       const void* wcv, const FwdWs& w, hipStream_t s) {
  switch (d) {
    case 32: return run_pool_conv<DT, 32>(p, H, k, v, wck, wcv, w, s);
    case 64: return run_pool_conv<DT, 64>(p, H, k, v, wck, wcv, w, s);
    case 96: return run_pool_conv<DT, 96>(p, H, k, v, wck, wcv, w, s);
    case 128: return run_pool_conv<DT, 128>(p, H, k, v, wck, wcv, w, s);
  }
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t conv_term_d(int d, const ssa_plan_s* p, int H, const void* wck, const void* wcv, const float* gk,
                       const float* gv, float* dk, float* dv, hipStream_t s) {
  switch (d) {
    case 32: return run_conv_term<DT, 32>(p, H, wck, wcv, gk, gv, dk, dv, s);
    case 64: return run_conv_term<DT, 64>(p, H, wck, wcv, gk, gv, dk, dv, s);
    case 96: return run_conv_term<DT, 96>(p, H, wck, wcv, gk, gv, dk, dv, s);
    case 128: return run_conv_term<DT, 128>(p, H, wck, wcv, gk, gv, dk, dv, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_pool_conv(ssa_dtype dt, const ssa_plan_s* p, int H, int d, const void* k, const void* v,
                            const void* wck, const void* wcv, const FwdWs& w, hipStream_t s) {
  switch (dt) {
    case SSA_F32: return pool_conv_d<DT_F32>(d, p, H, k, v, wck, wcv, w, s);
    case SSA_F16: return pool_conv_d<DT_F16>(d, p, H, k, v, wck, wcv, w, s);
    case SSA_BF16: return pool_conv_d<DT_BF16>(d, p, H, k, v, wck, wcv, w, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_conv_term(ssa_dtype dt, const ssa_plan_s* p, int H, int d, const void* wck, const void* wcv,
                            const float* gk, const float* gv, float* dk, float* dv, hipStream_t s) {
  switch (dt) {
    case SSA_F32: return conv_term_d<DT_F32>(d, p, H, wck, wcv, gk, gv, dk, dv, s);
    case SSA_F16: return conv_term_d<DT_F16>(d, p, H, wck, wcv, gk, gv, dk, dv, s);
    case SSA_BF16: return conv_term_d<DT_BF16>(d, p, H, wck, wcv, gk, gv, dk, dv, s);
  }
  return hipErrorInvalidValue;
}
