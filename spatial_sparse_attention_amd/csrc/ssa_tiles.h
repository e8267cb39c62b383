// Tile geometry and MFMA building blocks shared by the forward and backward kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <type_traits>
#include "ssa_mfma.h"

namespace ssa_dev {

constexpr int KT = 32;                // keys (or queries) per tile
constexpr float RESCALE_SLACK = 8.f;  // log2 units the running max may lag the true max

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
  static constexpr int PK = KT / KS;                    // K steps over a 32-key tile (PV)
  // pooled stage: NS key planes [64][KROW], then the values transposed [D][VTROW]
  static constexpr int PT = 64;
  static constexpr int VTROW = sizeof(T) == 4 ? PT + 1 : PT + 4;
  static constexpr int KPLANE = PT * KROW;
  static constexpr int STAGE = NS * KPLANE + D * VTROW;
};


// ------------------------------------------------------------------ stage-buffer reads in asm
// Reads of a stage buffer while copies into other stage buffers are in flight.  Written as
// plain loads, the compiler makes the wave wait for every copy into LDS still in flight
// (vmcnt(0)) before them, wherever it loses track of which copy wrote which buffer (at the
// joins of the stream's control flow), and so drains the copy pipeline at every tile.  The
// stream's own wait and barrier already guarantee that this buffer's copy has landed, so
// these reads are issued from asm, all at once, and waited for (lgkmcnt) inside the same
// statement; the outputs are early-clobber so that no output shares the address register.
__device__ inline uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
template <int S, typename V>
__device__ inline void lds_rd_b128_x2(uint32_t a, V (&o)[2]) {
  asm volatile("ds_read_b128 %0, %2 offset:%3\n\t"
               "ds_read_b128 %1, %2 offset:%4\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(o[0]), "=&v"(o[1])
               : "v"(a), "i"(0 * S), "i"(1 * S));
}
template <int S, typename V>
__device__ inline void lds_rd_b128_x4(uint32_t a, V (&o)[4]) {
  asm volatile("ds_read_b128 %0, %4 offset:%5\n\t"
               "ds_read_b128 %1, %4 offset:%6\n\t"
               "ds_read_b128 %2, %4 offset:%7\n\t"
               "ds_read_b128 %3, %4 offset:%8\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
               : "v"(a), "i"(0 * S), "i"(1 * S), "i"(2 * S), "i"(3 * S));
}
template <int S, typename V>
__device__ inline void lds_rd_b128_x6(uint32_t a, V (&o)[6]) {
  asm volatile("ds_read_b128 %0, %6 offset:%7\n\t"
               "ds_read_b128 %1, %6 offset:%8\n\t"
               "ds_read_b128 %2, %6 offset:%9\n\t"
               "ds_read_b128 %3, %6 offset:%10\n\t"
               "ds_read_b128 %4, %6 offset:%11\n\t"
               "ds_read_b128 %5, %6 offset:%12\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5])
               : "v"(a), "i"(0 * S), "i"(1 * S), "i"(2 * S), "i"(3 * S), "i"(4 * S), "i"(5 * S));
}
template <int S, typename V>
__device__ inline void lds_rd_b128_x8(uint32_t a, V (&o)[8]) {
  asm volatile("ds_read_b128 %0, %8 offset:%9\n\t"
               "ds_read_b128 %1, %8 offset:%10\n\t"
               "ds_read_b128 %2, %8 offset:%11\n\t"
               "ds_read_b128 %3, %8 offset:%12\n\t"
               "ds_read_b128 %4, %8 offset:%13\n\t"
               "ds_read_b128 %5, %8 offset:%14\n\t"
               "ds_read_b128 %6, %8 offset:%15\n\t"
               "ds_read_b128 %7, %8 offset:%16\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
               : "v"(a), "i"(0 * S), "i"(1 * S), "i"(2 * S), "i"(3 * S), "i"(4 * S), "i"(5 * S), "i"(6 * S), "i"(7 * S));
}
template <int ROW>
__device__ inline void lds_rd_tr_ndv1(uint32_t a, ssa_s4 (&o)[4]) {
  asm volatile("ds_read_b64_tr_b16 %0, %4 offset:%5\n\t"
               "ds_read_b64_tr_b16 %1, %4 offset:%6\n\t"
               "ds_read_b64_tr_b16 %2, %4 offset:%7\n\t"
               "ds_read_b64_tr_b16 %3, %4 offset:%8\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
               : "v"(a), "i"(((16 * 0 + 8 * 0) * ROW + 32 * 0) * 2),
                 "i"(((16 * 0 + 8 * 1) * ROW + 32 * 0) * 2),
                 "i"(((16 * 1 + 8 * 0) * ROW + 32 * 0) * 2),
                 "i"(((16 * 1 + 8 * 1) * ROW + 32 * 0) * 2));
}
template <int ROW>
__device__ inline void lds_rd_tr_ndv2(uint32_t a, ssa_s4 (&o)[8]) {
  asm volatile("ds_read_b64_tr_b16 %0, %8 offset:%9\n\t"
               "ds_read_b64_tr_b16 %1, %8 offset:%10\n\t"
               "ds_read_b64_tr_b16 %2, %8 offset:%11\n\t"
               "ds_read_b64_tr_b16 %3, %8 offset:%12\n\t"
               "ds_read_b64_tr_b16 %4, %8 offset:%13\n\t"
               "ds_read_b64_tr_b16 %5, %8 offset:%14\n\t"
               "ds_read_b64_tr_b16 %6, %8 offset:%15\n\t"
               "ds_read_b64_tr_b16 %7, %8 offset:%16\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
               : "v"(a), "i"(((16 * 0 + 8 * 0) * ROW + 32 * 0) * 2),
                 "i"(((16 * 0 + 8 * 1) * ROW + 32 * 0) * 2),
                 "i"(((16 * 0 + 8 * 0) * ROW + 32 * 1) * 2),
                 "i"(((16 * 0 + 8 * 1) * ROW + 32 * 1) * 2),
                 "i"(((16 * 1 + 8 * 0) * ROW + 32 * 0) * 2),
                 "i"(((16 * 1 + 8 * 1) * ROW + 32 * 0) * 2),
                 "i"(((16 * 1 + 8 * 0) * ROW + 32 * 1) * 2),
                 "i"(((16 * 1 + 8 * 1) * ROW + 32 * 1) * 2));
}
template <int ROW>
__device__ inline void lds_rd_tr_ndv3(uint32_t a, ssa_s4 (&o)[12]) {
  asm volatile("ds_read_b64_tr_b16 %0, %12 offset:%13\n\t"
               "ds_read_b64_tr_b16 %1, %12 offset:%14\n\t"
               "ds_read_b64_tr_b16 %2, %12 offset:%15\n\t"
               "ds_read_b64_tr_b16 %3, %12 offset:%16\n\t"
               "ds_read_b64_tr_b16 %4, %12 offset:%17\n\t"
               "ds_read_b64_tr_b16 %5, %12 offset:%18\n\t"
               "ds_read_b64_tr_b16 %6, %12 offset:%19\n\t"
               "ds_read_b64_tr_b16 %7, %12 offset:%20\n\t"
               "ds_read_b64_tr_b16 %8, %12 offset:%21\n\t"
               "ds_read_b64_tr_b16 %9, %12 offset:%22\n\t"
               "ds_read_b64_tr_b16 %10, %12 offset:%23\n\t"
               "ds_read_b64_tr_b16 %11, %12 offset:%24\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]), "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11])
               : "v"(a), "i"(((16 * 0 + 8 * 0) * ROW + 32 * 0) * 2),
                 "i"(((16 * 0 + 8 * 1) * ROW + 32 * 0) * 2),
                 "i"(((16 * 0 + 8 * 0) * ROW + 32 * 1) * 2),
                 "i"(((16 * 0 + 8 * 1) * ROW + 32 * 1) * 2),
                 "i"(((16 * 0 + 8 * 0) * ROW + 32 * 2) * 2),
                 "i"(((16 * 0 + 8 * 1) * ROW + 32 * 2) * 2),
                 "i"(((16 * 1 + 8 * 0) * ROW + 32 * 0) * 2),
                 "i"(((16 * 1 + 8 * 1) * ROW + 32 * 0) * 2),
                 "i"(((16 * 1 + 8 * 0) * ROW + 32 * 1) * 2),
                 "i"(((16 * 1 + 8 * 1) * ROW + 32 * 1) * 2),
                 "i"(((16 * 1 + 8 * 0) * ROW + 32 * 2) * 2),
                 "i"(((16 * 1 + 8 * 1) * ROW + 32 * 2) * 2));
}
template <int ROW>
__device__ inline void lds_rd_tr_ndv4(uint32_t a, ssa_s4 (&o)[16]) {
  asm volatile("ds_read_b64_tr_b16 %0, %16 offset:%17\n\t"
               "ds_read_b64_tr_b16 %1, %16 offset:%18\n\t"
               "ds_read_b64_tr_b16 %2, %16 offset:%19\n\t"
               "ds_read_b64_tr_b16 %3, %16 offset:%20\n\t"
               "ds_read_b64_tr_b16 %4, %16 offset:%21\n\t"
               "ds_read_b64_tr_b16 %5, %16 offset:%22\n\t"
               "ds_read_b64_tr_b16 %6, %16 offset:%23\n\t"
               "ds_read_b64_tr_b16 %7, %16 offset:%24\n\t"
               "ds_read_b64_tr_b16 %8, %16 offset:%25\n\t"
               "ds_read_b64_tr_b16 %9, %16 offset:%26\n\t"
               "ds_read_b64_tr_b16 %10, %16 offset:%27\n\t"
               "ds_read_b64_tr_b16 %11, %16 offset:%28\n\t"
               "ds_read_b64_tr_b16 %12, %16 offset:%29\n\t"
               "ds_read_b64_tr_b16 %13, %16 offset:%30\n\t"
               "ds_read_b64_tr_b16 %14, %16 offset:%31\n\t"
               "ds_read_b64_tr_b16 %15, %16 offset:%32\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]), "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]), "=&v"(o[12]), "=&v"(o[13]), "=&v"(o[14]), "=&v"(o[15])
               : "v"(a), "i"(((16 * 0 + 8 * 0) * ROW + 32 * 0) * 2),
                 "i"(((16 * 0 + 8 * 1) * ROW + 32 * 0) * 2),
                 "i"(((16 * 0 + 8 * 0) * ROW + 32 * 1) * 2),
                 "i"(((16 * 0 + 8 * 1) * ROW + 32 * 1) * 2),
                 "i"(((16 * 0 + 8 * 0) * ROW + 32 * 2) * 2),
                 "i"(((16 * 0 + 8 * 1) * ROW + 32 * 2) * 2),
                 "i"(((16 * 0 + 8 * 0) * ROW + 32 * 3) * 2),
                 "i"(((16 * 0 + 8 * 1) * ROW + 32 * 3) * 2),
                 "i"(((16 * 1 + 8 * 0) * ROW + 32 * 0) * 2),
                 "i"(((16 * 1 + 8 * 1) * ROW + 32 * 0) * 2),
                 "i"(((16 * 1 + 8 * 0) * ROW + 32 * 1) * 2),
                 "i"(((16 * 1 + 8 * 1) * ROW + 32 * 1) * 2),
                 "i"(((16 * 1 + 8 * 0) * ROW + 32 * 2) * 2),
                 "i"(((16 * 1 + 8 * 1) * ROW + 32 * 2) * 2),
                 "i"(((16 * 1 + 8 * 0) * ROW + 32 * 3) * 2),
                 "i"(((16 * 1 + 8 * 1) * ROW + 32 * 3) * 2));
}
// N 16-byte fragments at byte offsets i * S from p (one asm statement).
template <int N, int S, typename V>
__device__ inline void lds_frags_b128(const void* p, V (&o)[N]) {
  const uint32_t a = lds_u32(p);
  if constexpr (N == 2) lds_rd_b128_x2<S>(a, o);
  else if constexpr (N == 4) lds_rd_b128_x4<S>(a, o);
  else if constexpr (N == 6) lds_rd_b128_x6<S>(a, o);
  else if constexpr (N == 8) lds_rd_b128_x8<S>(a, o);
  else static_assert(N == 2, "fragment count");
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
// MFMA operand fragment from a row-major 32-row tile in LDS (tile[row][col], row stride ROW
// elements), K step ks over the rows, output columns 32*j .. 32*j+31: lane l supplies
// column 32j + l%32 at the rows held by result registers ks*KPL .. ks*KPL + KPL - 1 of a
// score tile, i.e. rows 16ks + 4g + {0..3} and 16ks + 8 + 4g + {0..3} (g = l/32) for
// 16-bit types.  It is the A operand V^T of O^T += V^T P^T and equally the B operand X of
// Y += P^T X when the rows are the contraction index.
template <int DT, int ROW>
__device__ inline typename Tr<DT>::frag tr_frag(const typename Tr<DT>::T* tile, int ks, int j, int lane) {
  if constexpr (Tr<DT>::KPL == 1) {
    return tile[res_row(ks, lane >> 5) * ROW + 32 * j + (lane & 31)];
  } else {
    const int i = lane & 15, G = lane >> 4;
    const typename Tr<DT>::T* p =
        tile + (16 * ks + 4 * (G >> 1) + (i >> 2)) * ROW + 32 * j + 16 * (G & 1) + 4 * (i & 3);
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    const u2 a = __builtin_bit_cast(u2, lds_read_tr16(p));
    const u2 b = __builtin_bit_cast(u2, lds_read_tr16(p + 8 * ROW));
    const u4 u = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(typename Tr<DT>::frag, u);
  }
}

template <int DT, int D>
__device__ inline typename Tr<DT>::frag vt_frag(const typename Tr<DT>::T* vt, int ks, int j, int lane) {
  return tr_frag<DT, Cfg<DT, D>::VROW>(vt, ks, j, lane);
}

// The same A operand (V^T, output columns 32j..32j+31, K step ks) from a transposed value
// tile vtt[dv][key] (row stride VTROW) whose 32-key sub-tile starts at key kb: ordinary
// 8-byte LDS reads of keys kb + 16ks + 4g + {0..3} and kb + 16ks + 8 + 4g + {0..3}.
template <int DT, int D>
__device__ inline typename Tr<DT>::frag vtt_frag(const typename Tr<DT>::T* vtt, int kb, int ks, int j,
                                                 int lane) {
  using C = Cfg<DT, D>;
  const int g = lane >> 5;
  const typename Tr<DT>::T* row = vtt + (32 * j + (lane & 31)) * C::VTROW + kb;
  if constexpr (C::KPL == 1) {
    return row[res_row(ks, g)];
  } else {
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    const u2 a = *reinterpret_cast<const u2*>(row + 16 * ks + 4 * g);
    const u2 b = *reinterpret_cast<const u2*>(row + 16 * ks + 8 + 4 * g);
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
    using C = Cfg<DT, D>;
    if constexpr (C::KPL != 1 && C::PK == 2) {  // 16-bit: the tr_frag reads in one asm statement
      const int i = lane & 15, G = lane >> 4;
      const typename Tr<DT>::T* p = vt + (4 * (G >> 1) + (i >> 2)) * C::VROW + 16 * (G & 1) + 4 * (i & 3);
      ssa_s4 o[4 * C::NDV];
      const uint32_t a = lds_u32(p);
      if constexpr (C::NDV == 1) lds_rd_tr_ndv1<C::VROW>(a, o);
      else if constexpr (C::NDV == 2) lds_rd_tr_ndv2<C::VROW>(a, o);
      else if constexpr (C::NDV == 3) lds_rd_tr_ndv3<C::VROW>(a, o);
      else lds_rd_tr_ndv4<C::VROW>(a, o);
      typedef unsigned u2 __attribute__((ext_vector_type(2)));
      typedef unsigned u4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int ks = 0; ks < C::PK; ++ks)
#pragma unroll
        for (int j = 0; j < C::NDV; ++j) {
          const u2 x = __builtin_bit_cast(u2, o[(ks * C::NDV + j) * 2]);
          const u2 y = __builtin_bit_cast(u2, o[(ks * C::NDV + j) * 2 + 1]);
          const u4 u = {x.x, x.y, y.x, y.y};
          f[ks][j] = __builtin_bit_cast(typename Tr<DT>::frag, u);
        }
    } else {
#pragma unroll
      for (int ks = 0; ks < C::PK; ++ks)
#pragma unroll
        for (int j = 0; j < C::NDV; ++j) f[ks][j] = vt_frag<DT, D>(vt, ks, j, lane);
    }
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
  // Two 16-score sets of the same row (a 64-key tile).  Returns p in s0, s1.
  __device__ inline void update2(ssa_f16v& s0, ssa_f16v& s1, float sl2) {
    float mt0 = fmaxf(s0[0], s0[1]), mt1 = fmaxf(s1[0], s1[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) {
      mt0 = fmaxf(mt0, fmaxf(s0[r], s0[r + 1]));
      mt1 = fmaxf(mt1, fmaxf(s1[r], s1[r + 1]));
    }
    const float mt = xor32_max(fmaxf(mt0, mt1)) * sl2;
    if (__builtin_amdgcn_ballot_w64(mt > m + RESCALE_SLACK)) {
      const float mn = fmaxf(m, mt);
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int j = 0; j < NDV; ++j) o[j] *= alpha;
      m = mn;
    }
    float sum0 = 0.f, sum1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = fast_exp2(__builtin_fmaf(s0[r], sl2, -m));
      s1[r] = fast_exp2(__builtin_fmaf(s1[r], sl2, -m));
      sum0 += s0[r];
      sum1 += s1[r];
    }
    l += sum0 + sum1;
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
// ------------------------------------------------------------------ XCD-aware work order
// gfx950 dispatches workgroup i of a grid to XCD i % 8, and each XCD has its own L2.  Work
// comes in units of `per` workgroups that read the same rows (the heads and chunks of one
// query block); units are dealt to the XCDs round-robin and a unit's members run on one XCD,
// consecutively, so they share that XCD's L2.  Grid: xcd_grid(nunits, per) workgroups;
// unit >= nunits means no work.
constexpr int NXCD = 8;
__device__ inline void xcd_split(int id, int per, int& unit, int& member) {
  const int x = id % NXCD, k = id / NXCD;
  unit = (k / per) * NXCD + x;
  member = k % per;
}

// ------------------------------------------------------------------ gathered token tiles
// Copies of one gathered 32-key tile from the caller's K and V into LDS, 16 bytes per lane
// and instruction: the K rows ([32][KROW]) at the start of the stage, the V rows ([32][VROW])
// at VOFF.  K and V copies never share an instruction, so each instruction reads through one
// (wave-uniform) buffer descriptor, and every wave issues the same NI instructions per tile,
// so a wave can wait for all but its newest tile's copies with one count.  Lanes on a row's
// padding chunk, past a part's chunks or past the tile copy a valid chunk into a spot nobody
// reads (the row padding, the gap before VOFF, or the buffer's tail).
template <int DT, int D, int NW>
struct TileCopy {
  using C = Cfg<DT, D>;
  using T = typename Tr<DT>::T;
  static constexpr int KRC = C::KCH / KT, VRC = C::VCH / KT;  // chunks per padded row
  static constexpr int KI = (C::KCH + 63) / 64, VI = (C::VCH + 63) / 64;  // instructions
  static constexpr int NI = (KI + VI + NW - 1) / NW;
  static constexpr int ELEMS = NI * NW * 64 * C::EPC;  // stage buffer, tail included
  static constexpr int VOFF = KI * 64 * C::EPC;         // V rows' offset in the stage
  int32_t row[NI];   // tile row (key) of each copy
  int32_t goff[NI];  // element offset inside the token's head row
  int32_t tok[NI];
  __device__ inline void init(int wave, int lane) {
#pragma unroll
    for (int m = 0; m < NI; ++m) {
      const int i = wave + m * NW;
      const bool isk = i < KI;
      const int p = (isk ? i : i - KI) * 64 + lane;
      const int rr = isk ? p / KRC : p / VRC, ch = isk ? p % KRC : p % VRC;
      const bool ok = (isk ? p < C::KCH : (i < KI + VI && p < C::VCH)) && ch < C::CPR;
      row[m] = ok ? rr : 0;
      goff[m] = ok ? ch * C::EPC : 0;
    }
  }
  // tokens of the tile starting at key k0 of a staged segment of n keys (rows past n: key 0)
  __device__ inline void fetch(const int32_t* keytok, int k0, int n) {
#pragma unroll
    for (int m = 0; m < NI; ++m) {
      const int j = k0 + row[m];
      tok[m] = keytok[j < n ? j : 0];
    }
  }
  template <bool BUF>
  __device__ inline void issue(T* stage, const T* kin, const T* vin, int H, int h, int wave) const {
    if constexpr (BUF) {
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(kin + h * D), 0, -1, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(vin + h * D), 0, -1, 0x00020000);
#pragma unroll
      for (int m = 0; m < NI; ++m) {
        const uint32_t off = ((uint32_t)tok[m] * (uint32_t)(H * D) + (uint32_t)goff[m]) * (uint32_t)sizeof(T);
        lds_void_t* dst = (lds_void_t*)(stage + (wave + m * NW) * 64 * C::EPC);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wave + m * NW < KI ? rk : rv, dst, 16, off, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int m = 0; m < NI; ++m) {
        const T* src = (wave + m * NW < KI ? kin : vin) + ((int64_t)tok[m] * H + h) * D + goff[m];
        dma16(src, stage + (wave + m * NW) * 64 * C::EPC);
      }
    }
  }
  // The same copies from two row-addressed sources: row r of the K part at kb + ko(r) and of
  // the V part at vb + vo(r) (element offsets), for the rows r0 + tile row (set_rows).
  __device__ inline void set_rows(int r0) {
#pragma unroll
    for (int m = 0; m < NI; ++m) tok[m] = r0 + row[m];
  }
  template <bool BUF, typename KO, typename VO>
  __device__ inline void issue_rows(T* stage, const T* kb, const T* vb, KO ko, VO vo, int wave) const {
    if constexpr (BUF) {
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(kb), 0, -1, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(vb), 0, -1, 0x00020000);
#pragma unroll
      for (int m = 0; m < NI; ++m) {
        const bool isk = wave + m * NW < KI;
        const uint32_t off = ((uint32_t)(isk ? ko(tok[m]) : vo(tok[m])) + (uint32_t)goff[m]) * (uint32_t)sizeof(T);
        lds_void_t* dst = (lds_void_t*)(stage + (wave + m * NW) * 64 * C::EPC);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(isk ? rk : rv, dst, 16, off, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int m = 0; m < NI; ++m) {
        const bool isk = wave + m * NW < KI;
        const T* src = isk ? kb + ko(tok[m]) + goff[m] : vb + vo(tok[m]) + goff[m];
        dma16(src, stage + (wave + m * NW) * 64 * C::EPC);
      }
    }
  }
};

// keytok[j] = perm[row(j)] for j < n <= PER * NT (NT threads): a thread's PER rows first,
// then all of its loads in flight at once.
template <int PER, int NT, typename Row>
__device__ inline void fill_tokens(int32_t* keytok, int n, Row row, const int32_t* __restrict__ perm) {
  const int tid = threadIdx.x;
  constexpr int nt = NT;
  int r[PER], v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) r[i] = tid + i * nt < n ? row(tid + i * nt) : -1;
#pragma unroll
  for (int i = 0; i < PER; ++i) v[i] = r[i] >= 0 ? perm[r[i]] : 0;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (r[i] >= 0) keytok[tid + i * nt] = v[i];
}

// Waits until at most N of this wave's vector memory operations are outstanding (vmcnt is
// six bits: 3:0 and 15:14 of the immediate).
template <int N>
__device__ inline void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier of the copy pipelines: this wave's LDS accesses complete, then s_barrier,
// in one asm statement whose memory clobber keeps the compiler from moving any memory access
// across it.  __syncthreads() would not do here: its workgroup release fence makes the
// compiler wait for every copy into LDS still in flight (vmcnt(0)), which drains the pipeline
// at each step.  The caller has already waited (vm_wait) for the copies that the next step
// reads, and the steps share data through LDS only.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Waits until at most k tiles' copies (NI instructions each) are outstanding, k <= 4.
template <int NI>
__device__ inline void vm_wait_tiles(int k) {
  switch (k) {
    case 0: vm_wait<0>(); break;
    case 1: vm_wait<NI>(); break;
    case 2: vm_wait<2 * NI>(); break;
    case 3: vm_wait<3 * NI>(); break;
    default: vm_wait<4 * NI>(); break;
  }
}

// Stage buffers that fit an LDS budget next to `other` bytes of tables: 3 to 6.
template <int DT, int D, int NW>
constexpr int stage_depth(int budget, int other) {
  const int n = (budget - other) / (TileCopy<DT, D, NW>::ELEMS * (int)sizeof(typename Tr<DT>::T));
  return n < 3 ? 3 : (n > 6 ? 6 : n);
}

// A stream of ntile tiles through NB stage buffers (separate LDS arrays, so the compiler
// knows a copy into one does not touch reads of another): the copies of tiles 0 .. NB-2 are
// issued up front, and step t, once tile t has landed and every wave has passed the
// barrier, runs body(t, stage, next) where next() issues tile t + NB - 1 into the buffer
// tile t - 1 used and readies tile t + NB's addresses.  fetch(t) readies tile t's copy
// addresses, issue(buffer) starts the copy (NI instructions per wave).
template <int NB, int NI, typename T, typename Fetch, typename Issue, typename Body>
__device__ inline void tile_pipeline(int ntile, T* const* bufs, Fetch&& fetch, Issue&& issue, Body&& body) {
  static_assert(NB >= 2 && NB <= 6, "stage depth");
  if (ntile <= 0) return;
#pragma unroll
  for (int u = 0; u < NB - 1; ++u) {
    if (u < ntile) {
      fetch(u);
      issue(bufs[u]);
    }
  }
  if (NB - 1 < ntile) fetch(NB - 1);
  for (int t0 = 0; t0 < ntile; t0 += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int t = t0 + u;
      if (t < ntile) {
        vm_wait_tiles<NI>(min(NB - 2, ntile - 1 - t));
        lds_barrier();
        body(t, bufs[u], [&]() __attribute__((always_inline)) {
          if (t + NB - 1 < ntile) issue(bufs[(u + NB - 1) % NB]);
          if (t + NB < ntile) fetch(t + NB);
        });
      }
    }
  }
}

// Calls f(std::integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Waits until at most kt * NI + nf * E of this wave's vector memory operations are
// outstanding, for kt, nf in [0, K].
template <int NI, int E, int K>
__device__ inline void vm_wait_kn(int kt, int nf) {
  static_for<0, K + 1>([&](auto a) __attribute__((always_inline)) {
    static_for<0, K + 1>([&](auto b) __attribute__((always_inline)) {
      constexpr int A = decltype(a)::value, B = decltype(b)::value;
      if (kt == A && nf == B) vm_wait<A * NI + B * E>();
    });
  });
}

// The same stream with a one-tile lookahead inside each wave: step t first runs
// ahead(t + 1, stage of t + 1, slot (t + 1) % 2) -- the MFMAs whose results step t + 1 needs
// -- and then body(t, stage of t, slot t % 2, next), so the matrix cores work on tile t + 1
// while the vector units finish tile t.  Tile t + 1 must have landed at step t, so NB - 3
// tiles stay in flight beyond it.  The caller keeps two state slots.
template <int NB, int NI, typename T, typename Fetch, typename Issue, typename Ahead, typename Body>
__device__ inline void tile_pipeline_ahead(int ntile, T* const* bufs, Fetch&& fetch, Issue&& issue, Ahead&& ahead,
                                           Body&& body) {
  static_assert(NB >= 3 && NB <= 6, "stage depth");
  constexpr int UN = NB % 2 == 0 ? NB : 2 * NB;  // unrolled steps: buffer and slot both static
  if (ntile <= 0) return;
#pragma unroll
  for (int u = 0; u < NB - 1; ++u) {
    if (u < ntile) {
      fetch(u);
      issue(bufs[u]);
    }
  }
  if (NB - 1 < ntile) fetch(NB - 1);
  vm_wait_tiles<NI>(min(NB - 2, ntile - 1));
  lds_barrier();
  ahead(0, bufs[0], std::integral_constant<int, 0>{});
  for (int t0 = 0; t0 < ntile; t0 += UN) {
    static_for<0, UN>([&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      const int t = t0 + u;
      if (t < ntile) {
        if (t + 1 < ntile) {
          vm_wait_tiles<NI>(min(NB - 3, ntile - 2 - t));  // tile t + 1 landed
          lds_barrier();
          ahead(t + 1, bufs[(u + 1) % NB], std::integral_constant<int, (u + 1) % 2>{});
        }
        body(t, bufs[u % NB], std::integral_constant<int, u % 2>{}, [&]() __attribute__((always_inline)) {
          if (t + NB - 1 < ntile) issue(bufs[(u + NB - 1) % NB]);
          if (t + NB < ntile) fetch(t + NB);
        });
      }
    });
  }
}

// Copy of nchunks 16-byte chunks (a whole pooled stage) from global g to LDS, spread over NW
// waves in exactly NI instructions per wave, so that a wave can wait for a given number of
// stages by counting instructions: a wave with fewer real instructions repeats the last one
// (the same bytes to the same place).  Lane l of instruction i writes LDS base + 1024 i + 16 l.
template <int NW, int NI>
__device__ inline void dma_stage(void* lds, const void* g, int nchunks, int wave, int lane) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g), 0, nchunks * 16, 0x00020000);
  const int last = (nchunks - 1) >> 6;
#pragma unroll
  for (int m = 0; m < NI; ++m) {
    const int i = min(wave + m * NW, last);
    const int p = i * 64 + lane;
    if (p < nchunks) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)((char*)lds + i * 1024), 16, p * 16, 0, 0, 0);
  }
}

// Declares the stage buffers buf0 .. buf5 of a kernel (those past NB are 16-byte stubs) and
// the pointer table `bufs`.
#define SSA_STAGE_BUFFERS(T, ELEMS, NB)                                                          \
  __shared__ __attribute__((aligned(1024))) T buf0[ELEMS];                                     \
  __shared__ __attribute__((aligned(1024))) T buf1[ELEMS];                                     \
  __shared__ __attribute__((aligned((NB) > 2 ? 1024 : 16))) T buf2[(NB) > 2 ? (ELEMS) : 16 / sizeof(T)]; \
  __shared__ __attribute__((aligned((NB) > 3 ? 1024 : 16))) T buf3[(NB) > 3 ? (ELEMS) : 16 / sizeof(T)]; \
  __shared__ __attribute__((aligned((NB) > 4 ? 1024 : 16))) T buf4[(NB) > 4 ? (ELEMS) : 16 / sizeof(T)]; \
  __shared__ __attribute__((aligned((NB) > 5 ? 1024 : 16))) T buf5[(NB) > 5 ? (ELEMS) : 16 / sizeof(T)]; \
  T* const bufs[6] = {buf0, buf1, buf2, buf3, buf4, buf5}

}  // namespace ssa_dev
