// Device-side helpers shared by the kernel files: vector types, the
// per-row active-key interval of every mode, and the token-major index map.
#pragma once

#include "svg_internal.h"

namespace svg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define SVG_LDS __attribute__((address_space(3)))

// A sampled query row as read from a caller's row list, clamped into the
// video rows [T, L): the list is trusted to hold ascending distinct video
// rows, and the clamp keeps any other contents from addressing outside the
// tensors (they give unspecified labels instead).
__device__ __forceinline__ int sampled_row(const KGeom& g, int x) { return min(max(x, g.T), g.L - 1); }

// Active keys of query row x in the head's working layout are
// [0, T) U [lo, hi) (text keys, then one contiguous run of video keys).
// Closed forms (u = x - T, video index; rebuttal answer to Weakness 1):
//   SPATIAL  frame-major, frames i2 with |i2 - i| < a1: whole frames
//            [max(0, i-a1+1), min(N, i+a1)) * F.
//   TEMPORAL token-major (u = j*N + i), positions j2 with |j2 - j| < a2:
//            [max(0, j-a2+1), min(F, j+a2)) * N  -- the slashes of the
//            frame-major map become one band after the layout change.
//   WINDOW   |u2 - u| < window.   STRIPE  u2 < stripe.   FULL every key.
// Text rows (x < T) see every key.  SKIP has no keys (lo = hi = 0, and
// callers never reach here for it).
__device__ __forceinline__ void row_interval(const KGeom& g, int mode, int x, int& lo, int& hi) {
  if (x < g.T) {
    lo = 0;
    hi = g.L;
    return;
  }
  const long long u = x - g.T, NF = (long long)g.N * g.F;
  long long a, b;
  switch (mode) {
    case SVG_SPATIAL: {
      long long i = fastdiv((int32_t)u, g.divF_mul, g.divF_shift);
      a = i - g.a1 + 1;
      b = i + g.a1;
      a = a < 0 ? 0 : a;
      b = b > g.N ? g.N : b;
      a *= g.F;
      b *= g.F;
      break;
    }
    case SVG_TEMPORAL: {
      long long j = fastdiv((int32_t)u, g.divN_mul, g.divN_shift);
      a = j - g.a2 + 1;
      b = j + g.a2;
      a = a < 0 ? 0 : a;
      b = b > g.F ? g.F : b;
      a *= g.N;
      b *= g.N;
      break;
    }
    case SVG_WINDOW:
      a = u - g.window + 1;
      b = u + g.window;
      a = a < 0 ? 0 : a;
      b = b > NF ? NF : b;
      break;
    case SVG_STRIPE:
      a = 0;
      b = g.stripe < NF ? g.stripe : NF;
      break;
    case SVG_FULL:
      a = 0;
      b = NF;
      break;
    default:
      lo = hi = 0;
      return;
  }
  lo = (int)(g.T + a);
  hi = (int)(g.T + b);
}

// Frame-major row of token-major row xp (identity on text rows).
__device__ __forceinline__ int perm_inv_row(const KGeom& g, int xp) {
  if (xp < g.T) return xp;
  int up = xp - g.T;
  int j = fastdiv(up, g.divN_mul, g.divN_shift);
  int i = up - j * g.N;
  return g.T + i * g.F + j;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// Value of lane l^32 combined with the own value (v_permlane32_swap swaps
// the upper half of its first operand with the lower half of its second;
// with both operands equal, each lane ends up holding both halves' values).
__device__ __forceinline__ float half_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace svg
