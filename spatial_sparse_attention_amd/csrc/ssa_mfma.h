// Device-side helpers: dtype traits and MFMA fragments for gfx950 (wave64).
//
// 32x32 MFMA tiles.  For A (MxK) the lane l supplies row l%32; for B (KxN) the
// lane supplies column l%32; the K slice of lane l is group g = l/32, elements
// [g*KPL, g*KPL+KPL) of the KS-wide step (KPL = 8 for 16-bit types, 1 for fp32).
// Result register r of lane l holds D[8*(r/4) + 4*g + r%4][l%32].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 ssa_half8 __attribute__((ext_vector_type(8)));
typedef __bf16 ssa_bf8 __attribute__((ext_vector_type(8)));
typedef float ssa_f16v __attribute__((ext_vector_type(16)));
typedef float ssa_f4v __attribute__((ext_vector_type(4)));

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };
template <int DT> struct Tr;
// element type of the saved branch outputs: f16 for f16 inputs, else fp32
template <int DT> struct SaveT { using type = float; };
template <> struct SaveT<DT_F16> { using type = _Float16; };

template <int DT> struct Tr;

template <> struct Tr<DT_F16> {
  using T = _Float16;
  using frag = ssa_half8;
  static constexpr int KS = 16, KPL = 8, NSPLIT = 2;
  __device__ static inline ssa_f16v mma(frag a, frag b, ssa_f16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static inline T cvt(float x) { return (T)x; }
  __device__ static inline float up(T x) { return (float)x; }
};

template <> struct Tr<DT_BF16> {
  using T = __bf16;
  using frag = ssa_bf8;
  static constexpr int KS = 16, KPL = 8, NSPLIT = 3;
  __device__ static inline ssa_f16v mma(frag a, frag b, ssa_f16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline T cvt(float x) { return (T)x; }
  __device__ static inline float up(T x) { return (float)x; }
};

template <> struct Tr<DT_F32> {
  using T = float;
  using frag = float;
  static constexpr int KS = 2, KPL = 1, NSPLIT = 1;
  __device__ static inline ssa_f16v mma(frag a, frag b, ssa_f16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline T cvt(float x) { return x; }
  __device__ static inline float up(T x) { return x; }
};

// Load the KPL elements of one K step from a row (16-byte or 4-byte load).
template <int DT>
__device__ inline typename Tr<DT>::frag load_frag(const typename Tr<DT>::T* p) {
  return *reinterpret_cast<const typename Tr<DT>::frag*>(p);
}

// Key index held by result register r of lane group g in a 32-key tile.
__device__ inline int res_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// gfx950 LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// source lane i = 4t + a points at 4 consecutive 16-bit values S[i][0..3];
// destination lane j receives S[4t + j/4][j%4] for t = 0..3.  Pointing source lane
// 4t + a at row (r0 + t), column (c0 + 4a) of a row-major matrix gives lane j the
// column c0 + j of rows r0..r0+3.
typedef short ssa_s4 __attribute__((ext_vector_type(4)));
__device__ inline ssa_s4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) ssa_s4*)(p));
}
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
