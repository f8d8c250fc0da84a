// Lightning indexer logits on gfx950 FP8 matrix cores.
//
// "DeepSeek V3.2-Exp Cuts Prolonged-Context Costs With DeepSeek Sparse
// Consideration (DSA)", part (1).  The per-tile arithmetic (heads on the MFMA
// M side, keys on N, ReLU and head weights in registers) lives in
// indexer_math.h; this kernel streams the keys and writes the logits.
//
// Decode is bound by HBM (one 128-byte key row feeds 64 heads x 128 MACs =
// 128 flop/byte, far under the FP8 ridge), so the kernel streams keys with
// wide loads and keeps many 8 KB wave tiles in flight.
//
// When `hist` is given, the epilogue also counts the top 11 bits of each
// stored logit's order-preserving key into a per-row 2048-bin histogram (LDS
// per workgroup, then one global atomic per non-empty bin): the first level
// of the top-k radix select, obtained without reading the logits again.
#include "indexer_math.h"
#include "launch.h"

namespace dsa {

constexpr int IDX_WAVES = 4;
constexpr int IDX_ITERS = 4;                                    // 64-key groups per wave
constexpr int IDX_KEYS_PER_WG = IDX_WAVES * IDX_ITERS * 64;     // 1024 keys per workgroup

template <int H_I, int D_I>
__global__ __launch_bounds__(IDX_WAVES * 64) void indexer_kernel(const uint8_t* __restrict__ q8,
                                                                 const float* __restrict__ qs,
                                                                 const float* __restrict__ w,
                                                                 const uint8_t* __restrict__ k8,
                                                                 const float* __restrict__ ks,
                                                                 const int32_t* __restrict__ seq_id,
                                                                 const int32_t* __restrict__ pos, Layout lay,
                                                                 float* __restrict__ logits, int64_t ld,
                                                                 u32* __restrict__ hist) {
  __shared__ u32 h_lds[2048];
  using Frag = KeyFrag<H_I, D_I>;

  const int t = blockIdx.y;
  const int p = pos[t];
  const int wg_base = blockIdx.x * IDX_KEYS_PER_WG;
  if (wg_base > p) return;
  const int b = seq_id[t];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int n = lane & 15;
  const int g = lane >> 4;

  IndexerQuery<H_I, D_I> qq;
  qq.load(q8, qs, w, t, n, g);
  float* __restrict__ out_row = logits + (int64_t)t * ld;
  if (hist != nullptr) {
    for (int i = threadIdx.x; i < 2048; i += IDX_WAVES * 64) h_lds[i] = 0;
    __syncthreads();
  }

  // Groups of 64 keys this wave handles: base(it) = first + it*WAVES*64.
  // Every group is loaded (groups past p re-read the group holding p, and
  // store nothing), so the number of loads in flight is the same on every
  // path and the next group's keys stay in flight while this one is reduced.
  const int first = wg_base + wid * 64;
  const int last_group = p & ~63;  // 64-aligned group holding position p
  // The key scales load with their keys: a load issued after a logit store
  // cannot complete before it (the counter is in order), so nothing the math
  // waits for may be issued after the previous group's store.
  Frag kb[2][4];
  float ksb[2];
  auto issue = [&](int it, int slot) {
    const int base = min(first + it * IDX_WAVES * 64, last_group);  // one page when paged
    const int64_t row0 = token_row(lay, b, base);
    const uint8_t* grp = k8 + row0 * D_I;  // wave-uniform base of the 64 rows
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = min(base + 16 * j + n, p);  // positions past p read p
      kb[slot][j].load(grp + (u32)(s - base) * D_I, g);
    }
    ksb[slot] = ks[row0 + (min(base + lane, p) - base)];
  };
  issue(0, 0);
#pragma unroll
  for (int it = 0; it < IDX_ITERS; ++it) {
    const int cur = it & 1;
    if (it + 1 < IDX_ITERS) issue(it + 1, cur ^ 1);
    const int base = first + it * IDX_WAVES * 64;
    const int s_me = base + lane;
    const float ksv = ksb[cur];
    const float res = group_scores<H_I, D_I>(qq, kb[cur], g);
    if (s_me <= p) {
      const float v = scaled_logit(res, qq.qscale, ksv);
      out_row[s_me] = v;
      if (hist != nullptr) atomicAdd(&h_lds[order_key(v) >> 21], 1u);
    }
  }
  if (hist != nullptr) {
    __syncthreads();
    u32* g = hist + (int64_t)t * 2048;
    for (int i = threadIdx.x; i < 2048; i += IDX_WAVES * 64) {
      const u32 c = h_lds[i];
      if (c) atomicAdd(&g[i], c);
    }
  }
}

bool indexer_supported(int H_I, int D_I) {
  return (H_I == 64 || H_I == 4) && (D_I == 128 || D_I == 64);
}

template <int H_I, int D_I>
static hipError_t launch_t(int T, int max_len, const uint8_t* q8, const float* qs, const float* w, const uint8_t* k8,
                           const float* ks, const int32_t* seq_id, const int32_t* pos, const Layout& lay,
                           float* logits, int64_t ld, u32* hist, hipStream_t stream) {
  dim3 grid((max_len + IDX_KEYS_PER_WG - 1) / IDX_KEYS_PER_WG, T);
  hipLaunchKernelGGL((indexer_kernel<H_I, D_I>), grid, dim3(IDX_WAVES * 64), 0, stream, q8, qs, w, k8, ks, seq_id,
                     pos, lay, logits, ld, hist);
  return hipGetLastError();
}

hipError_t launch_indexer(int T, int max_len, int H_I, int D_I, const uint8_t* q8, const float* qs, const float* w,
                          const uint8_t* k8, const float* ks, const int32_t* seq_id, const int32_t* pos,
                          const Layout& lay, float* logits, int64_t ld, u32* hist, hipStream_t stream) {
  if (T == 0 || max_len == 0) return hipSuccess;
#define DSA_IDX_CASE(HH, DD) \
  if (H_I == HH && D_I == DD) \
    return launch_t<HH, DD>(T, max_len, q8, qs, w, k8, ks, seq_id, pos, lay, logits, ld, hist, stream);
  DSA_IDX_CASE(64, 128)
  DSA_IDX_CASE(64, 64)
  DSA_IDX_CASE(4, 128)
  DSA_IDX_CASE(4, 64)
#undef DSA_IDX_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsa
