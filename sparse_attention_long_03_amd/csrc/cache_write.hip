// Cache write: store new tokens' index keys (quantised to FP8) and latent rows.
//
// "DeepSeek V3.2-Exp Cuts Prolonged-Context Costs With DeepSeek Sparse
// Consideration (DSA)", part (1): the indexer scores in FP8, so every token's
// index key is kept as e4m3fn codes with one float32 scale per token:
//   scale = max(amax / 448, 2^-126),  code_i = e4m3fn(clamp(x_i / scale, +-448))
// with round to nearest, ties to even.  The latent row (576 bf16) is copied
// as is.  One wave per token: the key's amax is a wave reduction, each lane
// encodes D_I/64 elements, and the row copy is 72 chunks of 16 bytes.
#include "fp8_encode.h"
#include "launch.h"

namespace dsa {

constexpr int CW_WAVES = 4;

template <int D_I>
__global__ __launch_bounds__(CW_WAVES * 64) void cache_write_kernel(const int32_t* __restrict__ seq_id,
                                                                     const int32_t* __restrict__ pos, int T,
                                                                     Layout lay, const float* __restrict__ k_new,
                                                                     const uint8_t* __restrict__ kv_new,
                                                                     uint8_t* __restrict__ k8, float* __restrict__ ks,
                                                                     uint8_t* __restrict__ kv) {
  constexpr int EPL = D_I / 64;  // elements per lane
  const int t = blockIdx.x * CW_WAVES + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const int64_t row = token_row(lay, seq_id[t], pos[t]);

  float x[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) x[e] = k_new[(int64_t)t * D_I + EPL * lane + e];
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
  const float scale = e4m3fn_scale(amax);

  u32 packed = 0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) packed |= e4m3fn_quantise(x[e], scale) << (8 * e);
  uint8_t* krow = k8 + row * D_I + EPL * lane;
  if (EPL == 2)
    *reinterpret_cast<uint16_t*>(krow) = (uint16_t)packed;
  else
    *krow = (uint8_t)packed;
  if (lane == 0) ks[row] = scale;

  if (kv_new != nullptr) {
    const uint8_t* src = kv_new + (int64_t)t * 1152;
    uint8_t* dst = kv + row * 1152;
    *reinterpret_cast<v4i*>(dst + 16 * lane) = *reinterpret_cast<const v4i*>(src + 16 * lane);
    if (lane < 8) *reinterpret_cast<v4i*>(dst + 1024 + 16 * lane) = *reinterpret_cast<const v4i*>(src + 1024 + 16 * lane);
  }
}

hipError_t launch_cache_write(int T, int D_I, const int32_t* seq_id, const int32_t* pos, const Layout& lay,
                              const float* k_new, const uint16_t* kv_new, uint8_t* k8, float* ks, uint16_t* kv,
                              hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + CW_WAVES - 1) / CW_WAVES);
  const uint8_t* kvn = reinterpret_cast<const uint8_t*>(kv_new);
  uint8_t* kvc = reinterpret_cast<uint8_t*>(kv);
  if (D_I == 128)
    hipLaunchKernelGGL(cache_write_kernel<128>, grid, dim3(CW_WAVES * 64), 0, stream, seq_id, pos, T, lay, k_new, kvn,
                       k8, ks, kvc);
  else if (D_I == 64)
    hipLaunchKernelGGL(cache_write_kernel<64>, grid, dim3(CW_WAVES * 64), 0, stream, seq_id, pos, T, lay, k_new, kvn,
                       k8, ks, kvc);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dsa
