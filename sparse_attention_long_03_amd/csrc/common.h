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

// Wave-wide inclusive prefix sum of a u32 (64 lanes), on DPP: four row
// shifts give the sums within each row of 16 lanes, then row_bcast:15 adds row
// r-1's total to rows 1 and 3 and row_bcast:31 adds the first two rows' total
// to rows 2 and 3.  Lanes whose DPP source lies outside the row, or whose row
// is masked off, read 0.
__device__ __forceinline__ u32 wave_incl_scan(u32 v) {
  v += (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  v += (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
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
