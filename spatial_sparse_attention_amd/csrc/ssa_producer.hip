// The step before SSA: each token's queries, keys, values and gates from its features, in one
// kernel (a projection GEMM on MFMA whose epilogue applies the per-head RMS norm and the 3D
// rotary embedding to q and k and the sigmoid to the gates).
//
// The Sparc3D/Hi3D pipeline page ("Stage 3") names RMS normalisation of the self-attention
// queries and keys and rotary position embeddings; the nav.superapi.store Direct3D-S2 page
// ("Technical principles of Direct3D-S2") sums SSA's branches with per-branch gates that the
// model predicts.  Definitions (ssa.h, ssa_qkv_gates): y = x W^T with W in linear-layer layout
// [out_features, C]; q = rope(rmsnorm(y_q) * gamma_q), k likewise, v = y_v, gates =
// sigmoid(x W_g^T + b_g); rope rotates pair i of axis a (dimensions 2Pa + 2i, 2Pa + 2i + 1,
// P = floor(d / 6)) by c_a * base^(-i / P).
//
// Layout of the product: Y^T = W X^T, so the MFMA's A operand is a tile of weight rows
// (output features) and its B operand a tile of token rows, both read as contiguous 16-byte
// runs; in the result a lane holds one token and its registers hold features, so the
// per-head sum of squares is register-local (plus one swap with the other half-wave) and the
// rotary pairs (features 2i, 2i + 1) sit in neighbouring registers of the same lane.
#include <hip/hip_runtime.h>
#include <math.h>
#include "ssa_internal.h"
#include "ssa_mfma.h"
#include "ssa_tiles.h"

namespace {

using namespace ssa_dev;
constexpr int PR_WAVES = 4;              // waves per workgroup, 32 tokens each
constexpr int PR_TOK = 32 * PR_WAVES;    // tokens per workgroup
constexpr int PR_KC = 64;                // features of x per K chunk
constexpr int PR_ROW = PR_KC + 8;        // LDS row stride (elements)

// One workgroup per (tile of PR_TOK tokens, tile of D output features); a feature tile is
// one head of q, k or v, or D consecutive gate features.  Tiles of one token range are
// consecutive workgroups of one XCD (xcd_split), so their x rows stay in that XCD's L2.
template <int DT, int D>
__global__ __launch_bounds__(64 * PR_WAVES) void k_qkv_gates(
    const typename Tr<DT>::T* __restrict__ x, const typename Tr<DT>::T* __restrict__ wqkv,
    const typename Tr<DT>::T* __restrict__ wg, const typename Tr<DT>::T* __restrict__ bg,
    const typename Tr<DT>::T* __restrict__ gq, const typename Tr<DT>::T* __restrict__ gk,
    const int32_t* __restrict__ coords, int64_t N, int Cdim, int H, int nft, int ntt, float log2_base,
    float eps, typename Tr<DT>::T* __restrict__ q, typename Tr<DT>::T* __restrict__ k,
    typename Tr<DT>::T* __restrict__ v, typename Tr<DT>::T* __restrict__ gates) {
  using T = typename Tr<DT>::T;
  using F = typename Tr<DT>::frag;
  constexpr int NDV = D / 32;
  constexpr int NTH = 64 * PR_WAVES;
  constexpr int WCH = D * (PR_KC / 8), XCH = PR_TOK * (PR_KC / 8);  // 16-byte chunks per tile
  constexpr int WPT = (WCH + NTH - 1) / NTH, XPT = (XCH + NTH - 1) / NTH;
  __shared__ __attribute__((aligned(16))) T wl[2][D * PR_ROW];
  __shared__ __attribute__((aligned(16))) T xl[2][PR_TOK * PR_ROW];

  int tt, ft;
  xcd_split(blockIdx.x, nft, tt, ft);
  if (tt >= ntt) return;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tok0 = (int64_t)tt * PR_TOK;
  // weight rows of this feature tile (rows past the gate features read row 0, unused)
  const int G3 = 3 * H;
  const bool is_gate = ft >= 3 * H;
  const int fg0 = is_gate ? (ft - 3 * H) * D : 0;
  const T* wbase = is_gate ? wg : wqkv + (int64_t)ft * D * Cdim;
  auto wrow = [&](int f) __attribute__((always_inline)) {
    return is_gate ? wbase + (int64_t)(fg0 + f < G3 ? fg0 + f : 0) * Cdim : wbase + (int64_t)f * Cdim;
  };

  uint4 wr[WPT], xr[XPT];
  auto load_chunk = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < WPT; ++m) {
      const int p = tid + m * NTH, row = p / (PR_KC / 8), col = (p % (PR_KC / 8)) * 8;
      const bool ok = p < WCH && k0 + col < Cdim;
      wr[m] = ok ? *reinterpret_cast<const uint4*>(wrow(row) + k0 + col) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < XPT; ++m) {
      const int p = tid + m * NTH, row = p / (PR_KC / 8), col = (p % (PR_KC / 8)) * 8;
      const bool ok = p < XCH && tok0 + row < N && k0 + col < Cdim;
      xr[m] = ok ? *reinterpret_cast<const uint4*>(x + (tok0 + row) * Cdim + k0 + col) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_chunk = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < WPT; ++m) {
      const int p = tid + m * NTH;
      if (p < WCH) *reinterpret_cast<uint4*>(&wl[b][(p / (PR_KC / 8)) * PR_ROW + (p % (PR_KC / 8)) * 8]) = wr[m];
    }
#pragma unroll
    for (int m = 0; m < XPT; ++m) {
      const int p = tid + m * NTH;
      if (p < XCH) *reinterpret_cast<uint4*>(&xl[b][(p / (PR_KC / 8)) * PR_ROW + (p % (PR_KC / 8)) * 8]) = xr[m];
    }
  };

  ssa_f16v acc[NDV];
#pragma unroll
  for (int j = 0; j < NDV; ++j) acc[j] = zero16();
  const int nch = (Cdim + PR_KC - 1) / PR_KC;
  load_chunk(0);
  for (int ch = 0; ch < nch; ++ch) {
    const int b = ch & 1;
    store_chunk(b);
    __syncthreads();  // chunk ch is in LDS; every wave has finished chunk ch - 1 (the other buffer)
    if (ch + 1 < nch) load_chunk((ch + 1) * PR_KC);
    const T* xs = &xl[b][(wave * 32 + c) * PR_ROW + g * 8];
    const T* ws = &wl[b][c * PR_ROW + g * 8];
#pragma unroll
    for (int ks = 0; ks < PR_KC / 16; ++ks) {
      const F xf = *reinterpret_cast<const F*>(xs + ks * 16);
#pragma unroll
      for (int j = 0; j < NDV; ++j) {
        const F wf = *reinterpret_cast<const F*>(ws + j * 32 * PR_ROW + ks * 16);
        acc[j] = Tr<DT>::mma(wf, xf, acc[j]);
      }
    }
  }

  // ---- epilogue: this lane's token, features 32 j + res_row(r, g) of the tile
  const int64_t tok = tok0 + wave * 32 + c;
  if (tok >= N) return;
  if (is_gate) {
#pragma unroll
    for (int j = 0; j < NDV; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int fg = fg0 + 32 * j + res_row(r, g);
        if (fg < G3) {
          const float z = acc[j][r] + (bg ? Tr<DT>::up(bg[fg]) : 0.f);
          gates[tok * G3 + fg] = Tr<DT>::cvt(1.f / (1.f + __expf(-z)));
        }
      }
    return;
  }
  const int kind = ft / H, h = ft % H;  // 0 q, 1 k, 2 v
  T* dst = (kind == 0 ? q : kind == 1 ? k : v) + (tok * H + h) * D;
  if (kind < 2) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NDV; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) ss += acc[j][r] * acc[j][r];
    ss = xor32_sum(ss);  // the other half of the head's features sits in lane c ^ 32
    const float inv = 1.f / sqrtf(ss / (float)D + eps);
    const T* gam = kind == 0 ? gq : gk;
    constexpr int P = D / 6;
    const float cx = (float)coords[3 * tok], cy = (float)coords[3 * tok + 1], cz = (float)coords[3 * tok + 2];
#pragma unroll
    for (int j = 0; j < NDV; ++j)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const int f = 32 * j + res_row(r, g);  // even; its pair partner f + 1 is register r + 1
        float u = acc[j][r] * inv * Tr<DT>::up(gam[f]);
        float w = acc[j][r + 1] * inv * Tr<DT>::up(gam[f + 1]);
        if (f < 6 * P) {
          const int a = f / (2 * P), i = (f % (2 * P)) / 2;
          const float ang = (a == 0 ? cx : a == 1 ? cy : cz) * exp2f(-(float)i / (float)P * log2_base);
          float sn, cs;
          sincosf(ang, &sn, &cs);
          const float u2 = u * cs - w * sn;
          w = u * sn + w * cs;
          u = u2;
        }
        acc[j][r] = u;
        acc[j][r + 1] = w;
      }
  }
#pragma unroll
  for (int j = 0; j < NDV; ++j)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      typedef unsigned u2 __attribute__((ext_vector_type(2)));
      const T e[4] = {Tr<DT>::cvt(acc[j][4 * r4]), Tr<DT>::cvt(acc[j][4 * r4 + 1]), Tr<DT>::cvt(acc[j][4 * r4 + 2]),
                      Tr<DT>::cvt(acc[j][4 * r4 + 3])};
      *reinterpret_cast<u2*>(dst + 32 * j + 8 * r4 + 4 * g) = __builtin_bit_cast(u2, e);
    }
}

template <int DT, int D>
hipError_t run_qkv(int64_t N, int C, int H, const void* x, const void* wqkv, const void* wg, const void* bg,
                   const void* gq, const void* gk, const int32_t* coords, float base, float eps, void* q, void* k,
                   void* v, void* gates, hipStream_t s) {
  using T = typename Tr<DT>::T;
  const int nft = 3 * H + (3 * H + D - 1) / D;
  const int ntt = (int)((N + PR_TOK - 1) / PR_TOK);
  hipLaunchKernelGGL((k_qkv_gates<DT, D>), dim3(xcd_grid(ntt, nft)), dim3(64 * PR_WAVES), 0, s, (const T*)x,
                     (const T*)wqkv, (const T*)wg, (const T*)bg, (const T*)gq, (const T*)gk, coords, N, C, H, nft,
                     ntt, log2f(base), eps, (T*)q, (T*)k, (T*)v, (T*)gates);
  return hipGetLastError();
}

template <int DT>
hipError_t qkv_d(int d, int64_t N, int C, int H, const void* x, const void* wqkv, const void* wg, const void* bg,
                 const void* gq, const void* gk, const int32_t* coords, float base, float eps, void* q, void* k,
                 void* v, void* gates, hipStream_t s) {
  switch (d) {
    case 32: return run_qkv<DT, 32>(N, C, H, x, wqkv, wg, bg, gq, gk, coords, base, eps, q, k, v, gates, s);
    case 64: return run_qkv<DT, 64>(N, C, H, x, wqkv, wg, bg, gq, gk, coords, base, eps, q, k, v, gates, s);
    case 96: return run_qkv<DT, 96>(N, C, H, x, wqkv, wg, bg, gq, gk, coords, base, eps, q, k, v, gates, s);
    case 128: return run_qkv<DT, 128>(N, C, H, x, wqkv, wg, bg, gq, gk, coords, base, eps, q, k, v, gates, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

extern "C" ssa_status ssa_qkv_gates(ssa_dtype dt, int64_t n, int32_t C, int32_t H, int32_t d, const void* x,
                                    const void* w_qkv, const void* w_gate, const void* b_gate,
                                    const void* gamma_q, const void* gamma_k, const int32_t* coords,
                                    float rope_base, float eps, void* q, void* k, void* v, void* gates,
                                    hipStream_t stream) {
  if (!abi_enum_in(&dt, 0, 2)) return SSA_ERR_INVALID_ARG;
  if (n < 0 || C < 1 || H < 1 || d < 1) return SSA_ERR_INVALID_ARG;
  if (!(rope_base >= 0.f) || isinf(rope_base) || !(eps >= 0.f) || isinf(eps)) return SSA_ERR_INVALID_ARG;
  if (dt == SSA_F32) return SSA_ERR_UNSUPPORTED;
  if (!(d == 32 || d == 64 || d == 96 || d == 128) || C % 8 != 0) return SSA_ERR_UNSUPPORTED;
  // element offsets of q, k, v stay below 2^31 and those of x below 2^40 (divisions: no overflow)
  if (n > (((int64_t)1 << 31) - 1) / ((int64_t)H * d) || n > (((int64_t)1 << 40) - 1) / C)
    return SSA_ERR_UNSUPPORTED;
  if (n == 0) return SSA_OK;
  if (!x || !w_qkv || !w_gate || !gamma_q || !gamma_k || !coords || !q || !k || !v || !gates)
    return SSA_ERR_INVALID_ARG;
  RoctxRange r("ssa_qkv_gates");
  const float base = rope_base == 0.f ? 10000.f : rope_base;
  const float e = eps == 0.f ? 1e-6f : eps;
  const hipError_t err = dt == SSA_F16
                             ? qkv_d<DT_F16>(d, n, C, H, x, w_qkv, w_gate, b_gate, gamma_q, gamma_k, coords, base, e,
                                             q, k, v, gates, stream)
                             : qkv_d<DT_BF16>(d, n, C, H, x, w_qkv, w_gate, b_gate, gamma_q, gamma_k, coords, base,
                                              e, q, k, v, gates, stream);
  return err == hipSuccess ? SSA_OK : SSA_ERR_HIP;
}
