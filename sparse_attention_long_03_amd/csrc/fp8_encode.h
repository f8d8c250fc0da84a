// FP8 (OCP e4m3fn) encoding shared by the kernels that quantise a token's
// vector with one float32 scale ("DeepSeek V3.2-Exp Cuts Prolonged-Context
// Costs With DeepSeek Sparse Consideration (DSA)", part (1): the indexer
// works in FP8): the cache write (index keys) and the indexer projection
// (index queries).
#pragma once

#include "common.h"

namespace dsa {

// float32 -> e4m3fn code, round to nearest even, for |y| <= 448 (finite).
// Normal range (|y| >= 2^-6, exponent e): the magnitude in units of the
// code step 2^(e-3) rounds to an integer m in [8, 16], and the code is
// (e + 7) * 8 + (m - 8) -- m = 16 carries into the next exponent by itself.
// Below 2^-6 the step is 2^-9 and the code is the rounded count m in [0, 8]
// (m = 8 is the smallest normal, code 0x08).  rintf rounds ties to even.
__device__ __forceinline__ u32 e4m3fn_code(float y) {
  const u32 u = __float_as_uint(y);
  const u32 sign = (u >> 31) << 7;
  const float a = __uint_as_float(u & 0x7FFFFFFFu);
  u32 mag;
  if (a < 0.015625f) {  // 2^-6
    mag = (u32)rintf(a * 512.f);
  } else {
    const int e = (int)((u >> 23) & 0xFF) - 127;                      // floor(log2 a), in [-6, 8]
    const float m = rintf(a * __uint_as_float((u32)(127 + 3 - e) << 23));  // a * 2^(3-e), exact
    mag = (u32)((e + 7) * 8) + (u32)m - 8u;
  }
  return sign | mag;
}

// The per-token scale: max(amax / 448, 2^-126), an exactly rounded float32
// division.
__device__ __forceinline__ float e4m3fn_scale(float amax) { return fmaxf(amax / 448.f, 1.17549435e-38f); }

// The code of x under a token's scale: e4m3fn(clamp(x / scale, +-448)).
__device__ __forceinline__ u32 e4m3fn_quantise(float x, float scale) {
  return e4m3fn_code(fminf(fmaxf(x / scale, -448.f), 448.f));
}

}  // namespace dsa
