// Arithmetic of the lightning indexer on gfx950 FP8 matrix cores, shared by
// the kernel that writes the logits and the kernel that selects from them on
// the fly, so that both compute every logit with the same operations in the
// same order (and therefore the same fp32 value).
//
// "DeepSeek V3.2-Exp Cuts Prolonged-Context Costs With DeepSeek Sparse
// Consideration (DSA)", part (1): per query token, a few small FP8 indexer
// heads with a ReLU score every earlier token:
//   I[t,s] = qs[t] * ks[s] * sum_j w[t,j] * ReLU(q8[t,j,:] . k8[s,:])
//
// Mapping.  One query token's heads form the M side of the MFMA (16 heads per
// M tile), keys form N (16 keys per N tile) and the head dim is K, so one
// v_mfma_f32_16x16x128_f8f6f4 computes 16 heads x 16 keys of dot products
// (D_I = 64 uses two 16x16x32 fp8 MFMAs).  In the 16x16 result a lane holds
// one key (column) and four heads (rows), so the ReLU and the per-head
// weights are applied in registers and the sum over heads needs only three
// cross-lane swaps for all 64 keys of a group (lanes n, n+16, n+32, n+48).
//
// Each lane group g (lanes 16g..16g+15) feeds the same byte range of the head
// dim for both operands; the contraction is a plain sum over the K index, so
// any consistent assignment of bytes to K slots gives the same result.
#pragma once

#include "common.h"

namespace dsa {

// ReLU as one integer max on the float's bits: a set sign bit (negative
// values and -0) makes the word negative, so max(bits, 0) gives +0; any other
// value is returned unchanged.  Unlike fmaxf it needs no NaN canonicalisation.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

template <int H_I, int D_I>
struct KeyFrag;

// D_I = 128: 32 bytes per lane (one f8f6f4 MFMA)
template <int H_I>
struct KeyFrag<H_I, 128> {
  v8i v;
  __device__ __forceinline__ void load(const uint8_t* row_base, int g) {
    const v4i* p = reinterpret_cast<const v4i*>(row_base + 32 * g);
    v4i a = p[0], b = p[1];
    v = v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  __device__ __forceinline__ void zero() { v = v8i{0, 0, 0, 0, 0, 0, 0, 0}; }
  __device__ __forceinline__ static v4f mma(const KeyFrag& a, const KeyFrag& b) {
    v4f c = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a.v, b.v, c, 0, 0, 0, 0, 0, 0);
  }
};

// D_I = 64: 16 bytes per lane (two 16x16x32 fp8 MFMAs)
template <int H_I>
struct KeyFrag<H_I, 64> {
  v4i v;
  __device__ __forceinline__ void load(const uint8_t* row_base, int g) {
    v = *reinterpret_cast<const v4i*>(row_base + 16 * g);
  }
  __device__ __forceinline__ void zero() { v = v4i{0, 0, 0, 0}; }
  __device__ __forceinline__ static v4f mma(const KeyFrag& a, const KeyFrag& b) {
    v4f c = {0.f, 0.f, 0.f, 0.f};
    long a0 = (long)(((unsigned long)(u32)a.v[1] << 32) | (u32)a.v[0]);
    long a1 = (long)(((unsigned long)(u32)a.v[3] << 32) | (u32)a.v[2]);
    long b0 = (long)(((unsigned long)(u32)b.v[1] << 32) | (u32)b.v[0]);
    long b1 = (long)(((unsigned long)(u32)b.v[3] << 32) | (u32)b.v[2]);
    c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a0, b0, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a1, b1, c, 0, 0, 0);
    return c;
  }
};

// The query side of one token in registers: its heads as MFMA A operands
// (row = head mt*16 + n) and the weights of the heads whose results this lane
// holds (mt*16 + 4g + i).  Heads past H_I are zero.
template <int H_I, int D_I>
struct IndexerQuery {
  static constexpr int MT = (H_I + 15) / 16;
  KeyFrag<H_I, D_I> qa[MT];
  float wv[MT][4];
  float qscale;

  __device__ __forceinline__ void load(const uint8_t* __restrict__ q8, const float* __restrict__ qs,
                                       const float* __restrict__ w, int t, int n, int g) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int h = mt * 16 + n;
      if (h < H_I)
        qa[mt].load(q8 + ((int64_t)t * H_I + h) * D_I, g);
      else
        qa[mt].zero();
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = mt * 16 + 4 * g + i;
        wv[mt][i] = (h < H_I) ? w[(int64_t)t * H_I + h] : 0.f;
      }
    qscale = qs[t];
  }

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      qa[mt].zero();
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[mt][i] = 0.f;
    }
    qscale = 0.f;
  }
};

// Head-weighted ReLU sums of one query against 64 keys (4 N tiles of 16):
// lane 16j + n returns the sum for key 16j + n of the group.  Within a lane,
// each 16-head tile sums its four heads in a short chain of its own and the
// tiles are added pairwise, so the dependent adds stay few; that leaves each
// lane (group g, column n) with p[j], its four heads' share of key 16j + n,
// for the four key groups j.  The sum over the four lane groups then ends in
// lane group j for key group j, by recursive halving on gfx950's VALU row
// swaps (a ds_bpermute shuffle would count on the in-order LDS counter and
// wait behind the key-fragment reads in flight):
//   permlane16_swap(p[0], p[1]) swaps the odd rows (lane groups) of its first
//   operand with the even rows of its second, so in lane group g the two
//   results are p[g & 1] of groups g and g ^ 1: their sum is key group g & 1
//   over that pair of lane groups; the same for p[2], p[3] (key group
//   2 + (g & 1));
//   permlane32_swap(u, v) swaps the upper half of u with the lower half of v,
//   so the two results are u (lower half) or v (upper half) of lane groups g
//   and g ^ 2: their sum is key group g over all four lane groups.
// Every key is the sum (groups 0 + 1) + (groups 2 + 3), in one order or the
// other of each addition, which gives the same value.
//
// The chain is spelled out (one product, then fused multiply-adds in head
// order) and contraction is off: left to itself the compiler may fuse either
// product of w0*r0 + w1*r1, and it chooses per unrolled copy, so copies (and
// kernels) would round the same key differently.
template <int H_I, int D_I>
__device__ __forceinline__ float group_scores(const IndexerQuery<H_I, D_I>& q, const KeyFrag<H_I, D_I> (&kb)[4]) {
#pragma clang fp contract(off)
  constexpr int MT = IndexerQuery<H_I, D_I>::MT;
  float p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v4f acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = KeyFrag<H_I, D_I>::mma(q.qa[mt], kb[j]);
    float pm[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      pm[mt] = q.wv[mt][0] * relu(acc[mt][0]);
#pragma unroll
      for (int i = 1; i < 4; ++i) pm[mt] = __builtin_fmaf(q.wv[mt][i], relu(acc[mt][i]), pm[mt]);
    }
#pragma unroll
    for (int w = 1; w < MT; w *= 2)
#pragma unroll
      for (int mt = 0; mt + w < MT; mt += 2 * w) pm[mt] += pm[mt + w];
    p[j] = pm[0];
  }
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(p[0]), __float_as_uint(p[1]), false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(p[2]), __float_as_uint(p[3]), false, false);
  const float u = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const float v = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(u), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// The logit from the head sum and the two per-token scales.
__device__ __forceinline__ float scaled_logit(float res, float qscale, float kscale) { return (res * qscale) * kscale; }

}  // namespace dsa
