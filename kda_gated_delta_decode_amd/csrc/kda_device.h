// kda_device.h -- device helpers shared by the decode and prefill kernels:
// vector types and the cross-lane sums built on DPP and the gfx950
// permlane swaps.  Internal header.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kda {

using f2 = float __attribute__((ext_vector_type(2)));
using f4 = float __attribute__((ext_vector_type(4)));
using h4 = _Float16 __attribute__((ext_vector_type(4)));
using h8 = _Float16 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Cross-lane sums.  Each returns x_i + x_(i xor m) in lane i: the same two
// operands in every lane of a pair, so all lanes of a group end with
// identical bits after the full butterfly.
// ---------------------------------------------------------------------------

// DPP controls (GCN/CDNA encoding): quad_perm selectors, row_half_mirror,
// row_ror:8 (a rotate by 8 inside a 16-lane row is the xor-8 partner).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppQuadXor3 = 0x1B;     // quad_perm [3,2,1,0]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float sum_xor1(float x) { return x + dpp<kDppQuadXor1>(x); }
__device__ __forceinline__ float sum_xor2(float x) { return x + dpp<kDppQuadXor2>(x); }
// half-row mirror sends lane i to i^7 (within 8 lanes); a quad xor-3 of that
// is i^4.
__device__ __forceinline__ float sum_xor4(float x) {
  return x + dpp<kDppQuadXor3>(dpp<kDppRowHalfMirror>(x));
}
__device__ __forceinline__ float sum_xor8(float x) { return x + dpp<kDppRowRor8>(x); }
// permlane16_swap(x, x) returns rows (0,0,2,2) and (1,1,3,3) of x.
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// permlane32_swap(x, x) returns halves (lo,lo) and (hi,hi) of x.
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_sum(float x) {
  return sum_xor32(sum_xor16(sum_xor8(sum_xor4(sum_xor2(sum_xor1(x))))));
}
// Sum over the row groups of a wave: the lanes that hold the same columns,
// i.e. lane bits log2(LPR) .. 5.
template <int LPR>
__device__ __forceinline__ float rowgroup_sum(float x) {
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "8, 16 or 32 lanes per row");
  if constexpr (LPR == 8) x = sum_xor8(x);
  if constexpr (LPR <= 16) x = sum_xor16(x);
  return sum_xor32(x);
}

// Reduce-scatter over the row groups, for tiles whose per-wave sums then
// meet in LDS.  The gfx950 permlane swaps exchange halves of TWO registers,
// so one swap and one add reduce two values at once: after the swap over
// lane bit 5 (and bit 4, unless LPR == 32) each lane quadrant q holds the
// full sums of orig[q * M + j], j < M, in out[j].  With LPR == 8 the lanes
// are first all-reduced over bit 3 (DPP), which leaves duplicates that only
// the bit-3-clear lanes store.  Orig is laid out so each quadrant's values
// are contiguous.
template <int LPR>
constexpr int rs_quadrants() { return LPR == 32 ? 2 : 4; }

template <int LPR, int N>
__device__ __forceinline__ void rowgroup_reduce_scatter(const float (&orig)[N],
                                                        float (&out)[N / rs_quadrants<LPR>()]) {
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "8, 16 or 32 lanes per row");
  constexpr int Q = rs_quadrants<LPR>();
  constexpr int M = N / Q;
  float x[N];
#pragma unroll
  for (int j = 0; j < M; ++j) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      float v = orig[q * M + j];
      if constexpr (LPR == 8) v = sum_xor8(v);
      x[Q * j + q] = v;
    }
  }
  float y[N / 2];
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[2 * i]),
                                                    __float_as_uint(x[2 * i + 1]), false, false);
    y[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (Q == 2) {
#pragma unroll
    for (int i = 0; i < M; ++i) out[i] = y[i];
  } else {
#pragma unroll
    for (int j = 0; j < M; ++j) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(y[2 * j]),
                                                      __float_as_uint(y[2 * j + 1]), false, false);
      out[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  }
}

// Reduce-scatter of 64 values over the 64 lanes of a wave: every lane
// passes v[0..63]; lane l returns the sum over all lanes of v[bitrev6(l)]
// (bitrev6 reverses the 6 lane-id bits).  Two permlane swaps of register
// pairs halve the values per lane at lane bits 5 and 4; DPP exchanges with
// a select do the same at bits 3..0.  63 exchange-adds in all, against 384
// for 64 separate full-wave sums.
__device__ __forceinline__ float wave_reduce_scatter64(const float (&v)[64], int lane) {
  float y[32], z[16], w[8], u[4], p[2];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[2 * i]),
                                                    __float_as_uint(v[2 * i + 1]), false, false);
    y[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(y[2 * i]),
                                                    __float_as_uint(y[2 * i + 1]), false, false);
    z[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const bool b3 = (lane & 8) != 0, b2 = (lane & 4) != 0, b1 = (lane & 2) != 0, b0 = (lane & 1) != 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float keep = b3 ? z[2 * i + 1] : z[2 * i], send = b3 ? z[2 * i] : z[2 * i + 1];
    w[i] = keep + dpp<kDppRowRor8>(send);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float keep = b2 ? w[2 * i + 1] : w[2 * i], send = b2 ? w[2 * i] : w[2 * i + 1];
    u[i] = keep + dpp<kDppQuadXor3>(dpp<kDppRowHalfMirror>(send));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float keep = b1 ? u[2 * i + 1] : u[2 * i], send = b1 ? u[2 * i] : u[2 * i + 1];
    p[i] = keep + dpp<kDppQuadXor2>(send);
  }
  const float keep = b0 ? p[1] : p[0], send = b0 ? p[0] : p[1];
  return keep + dpp<kDppQuadXor1>(send);
}

__device__ __forceinline__ int bitrev6(int l) {
  return ((l & 1) << 5) | ((l & 2) << 3) | ((l & 4) << 1) | ((l & 8) >> 1) | ((l & 16) >> 3) |
         ((l & 32) >> 5);
}

}  // namespace kda
