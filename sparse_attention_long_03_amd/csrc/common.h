// Device-side helpers shared by the gfx950 kernels of the DSA path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32;

constexpr int kWave = 64;

// Token row of a cache, contiguous or paged.  Paged: physical page from the
// block table, row within the page.
struct Layout {
  const int32_t* block_table;
  int64_t seq_capacity;
  int32_t max_pages;
  int32_t paged;
};

__device__ __forceinline__ int64_t token_row(const Layout& L, int b, int s) {
  if (L.paged) {
    int page = L.block_table[(int64_t)b * L.max_pages + (s >> 6)];
    return (int64_t)page * 64 + (s & 63);
  }
  return (int64_t)b * L.seq_capacity + s;
}

// Order-preserving map float -> u32: a > b as floats <=> key(a) > key(b),
// with -0 mapped to the key of +0.
__device__ __forceinline__ u32 order_key(float f) {
  u32 u = __float_as_uint(f);
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave-wide inclusive prefix sum of a u32 (64 lanes).
__device__ __forceinline__ u32 wave_incl_scan(u32 v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    u32 o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// Block-wide inclusive prefix sum for NT threads (NT multiple of 64, <= 1024).
// `scratch` must hold NT/64 + 1 u32 in LDS.  Returns the inclusive prefix;
// *total receives the block total.  Contains two barriers.
template <int NT>
__device__ __forceinline__ u32 block_incl_scan(u32 v, u32* scratch, u32* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  u32 incl = wave_incl_scan(v);
  if (lane == 63) scratch[wid] = incl;
  __syncthreads();
  u32 off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    u32 s = scratch[i];
    off += (i < wid) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return incl + off;
}

}  // namespace dsa
