// Per-query top-k selection by radix select on order-preserving keys.
//
// "DeepSeek V3.2-Exp Cuts Prolonged-Context Costs With DeepSeek Sparse
// Consideration (DSA)", part (2): each query keeps only its top-k (k = 2048)
// key-value entries.  Result: the positions of the k largest logits of the
// row; equal logits are taken lowest position first; -0 equals +0.
//
// One 1024-thread workgroup per row:
//   pass 1  histogram of the top 11 key bits (2048 bins, LDS atomics);
//           the bin holding the k-th largest value is found by a block scan;
//   pass 2  one ordered sweep of the row: positions whose bin is above the
//           threshold bin are written to the output at once, positions inside
//           it are appended, in position order, to a candidate list;
//   pass 3  two more histogram rounds over the candidates (bits 20..10, then
//           9..0) give the exact k-th key v* and how many ties at v* to keep;
//   pass 4  an ordered sweep of the candidates writes keys above v* and the
//           first ties at v*.
// Ordered compaction uses wave prefix sums and one block scan per 4096
// elements, so the output is deterministic: the positions above the
// threshold bin in ascending order, then the selected candidates ascending.
#include "launch.h"

namespace dsa {

constexpr int TK_NT = 1024;
constexpr int TK_E = 4;
constexpr int TK_CHUNK = TK_NT * TK_E;

// Threshold search: bins are visited from the top; returns the bin holding
// the `need`-th largest element and the count of elements in higher bins.
template <int NB>
__device__ __forceinline__ void find_threshold(const u32* hist, u32 need, u32* scratch, u32* out_bin,
                                               u32* out_above) {
  constexpr int BPT = NB / TK_NT;  // bins per thread: 2 or 1
  const int tid = threadIdx.x;
  u32 c[BPT];
  u32 tot_mine = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    c[i] = hist[NB - 1 - (tid * BPT + i)];
    tot_mine += c[i];
  }
  u32 total;
  const u32 incl = block_incl_scan<TK_NT>(tot_mine, scratch, &total);
  u32 excl = incl - tot_mine;
  if (excl < need && incl >= need) {
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (excl + c[i] >= need) {
        *out_bin = NB - 1 - (tid * BPT + i);
        *out_above = excl;
        break;
      }
      excl += c[i];
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(TK_NT) void topk_kernel(const float* __restrict__ logits, int64_t ld,
                                                     const int32_t* __restrict__ valid_len, int len_add, int k,
                                                     int32_t* __restrict__ idx, u32* __restrict__ cand_key,
                                                     int32_t* __restrict__ cand_pos) {
  __shared__ u32 hist[2048];
  __shared__ u32 scratch[TK_NT / 64 + 1];
  __shared__ u32 sh_bin, sh_above;

  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = valid_len[t] + len_add;
  int32_t* __restrict__ out = idx + (int64_t)t * k;
  if (n <= k) {
    for (int i = tid; i < k; i += TK_NT) out[i] = (i < n) ? i : -1;
    return;
  }
  const float* __restrict__ row = logits + (int64_t)t * ld;
  u32* __restrict__ ckey = cand_key + (int64_t)t * ld;
  int32_t* __restrict__ cpos = cand_pos + (int64_t)t * ld;

  // ---- pass 1: histogram of bits 31..21
  for (int i = tid; i < 2048; i += TK_NT) hist[i] = 0;
  __syncthreads();
  for (int i0 = tid * TK_E; i0 < n; i0 += TK_CHUNK) {
    if (i0 + TK_E <= n) {
      const float4 v = *reinterpret_cast<const float4*>(row + i0);
      atomicAdd(&hist[order_key(v.x) >> 21], 1u);
      atomicAdd(&hist[order_key(v.y) >> 21], 1u);
      atomicAdd(&hist[order_key(v.z) >> 21], 1u);
      atomicAdd(&hist[order_key(v.w) >> 21], 1u);
    } else {
      for (int i = i0; i < n; ++i) atomicAdd(&hist[order_key(row[i]) >> 21], 1u);
    }
  }
  __syncthreads();
  find_threshold<2048>(hist, (u32)k, scratch, &sh_bin, &sh_above);
  const u32 b1 = sh_bin;
  const u32 above1 = sh_above;
  const u32 n_cand = hist[b1];
  __syncthreads();

  // ---- pass 2: ordered sweep; emit bins above b1, collect bin b1
  u32 emit_base = 0, cand_base = 0;
  for (int c0 = 0; c0 < n; c0 += TK_CHUNK) {
    const int i0 = c0 + tid * TK_E;
    u32 kk[TK_E];
    bool ok[TK_E];
    if (i0 + TK_E <= n) {
      const float4 v = *reinterpret_cast<const float4*>(row + i0);
      kk[0] = order_key(v.x);
      kk[1] = order_key(v.y);
      kk[2] = order_key(v.z);
      kk[3] = order_key(v.w);
#pragma unroll
      for (int e = 0; e < TK_E; ++e) ok[e] = true;
    } else {
#pragma unroll
      for (int e = 0; e < TK_E; ++e) {
        ok[e] = (i0 + e) < n;
        kk[e] = ok[e] ? order_key(row[i0 + e]) : 0u;
      }
    }
    u32 ne = 0, nc = 0;
#pragma unroll
    for (int e = 0; e < TK_E; ++e) {
      const u32 bin = kk[e] >> 21;
      ne += (ok[e] && bin > b1) ? 1u : 0u;
      nc += (ok[e] && bin == b1) ? 1u : 0u;
    }
    const u32 packed = (nc << 16) | ne;
    u32 tot;
    const u32 incl = block_incl_scan<TK_NT>(packed, scratch, &tot);
    const u32 excl = incl - packed;
    u32 eo = emit_base + (excl & 0xFFFFu);
    u32 co = cand_base + (excl >> 16);
#pragma unroll
    for (int e = 0; e < TK_E; ++e) {
      if (!ok[e]) continue;
      const u32 bin = kk[e] >> 21;
      if (bin > b1) {
        out[eo++] = i0 + e;
      } else if (bin == b1) {
        ckey[co] = kk[e];
        cpos[co] = i0 + e;
        ++co;
      }
    }
    emit_base += tot & 0xFFFFu;
    cand_base += tot >> 16;
  }
  // candidates written by other threads of this workgroup are re-read below
  __threadfence();
  __syncthreads();

  // ---- pass 3: resolve the exact k-th key among the candidates
  const u32 need1 = (u32)k - above1;
  for (int i = tid; i < 2048; i += TK_NT) hist[i] = 0;
  __syncthreads();
  for (u32 j = tid; j < n_cand; j += TK_NT) atomicAdd(&hist[(ckey[j] >> 10) & 0x7FFu], 1u);
  __syncthreads();
  find_threshold<2048>(hist, need1, scratch, &sh_bin, &sh_above);
  const u32 b2 = sh_bin;
  const u32 need2 = need1 - sh_above;
  __syncthreads();
  for (int i = tid; i < 1024; i += TK_NT) hist[i] = 0;
  __syncthreads();
  const u32 hi2 = (b1 << 11) | b2;  // bits 31..10 of the keys still in play
  for (u32 j = tid; j < n_cand; j += TK_NT) {
    const u32 key = ckey[j];
    if ((key >> 10) == hi2) atomicAdd(&hist[key & 0x3FFu], 1u);
  }
  __syncthreads();
  find_threshold<1024>(hist, need2, scratch, &sh_bin, &sh_above);
  const u32 vstar = (hi2 << 10) | sh_bin;
  const u32 ties = need2 - sh_above;  // how many keys equal to vstar to keep (>= 1)

  // ---- pass 4: ordered sweep of the candidates
  u32 gt_base = 0, eq_base = 0;
  for (u32 c0 = 0; c0 < n_cand; c0 += TK_CHUNK) {
    const u32 j0 = c0 + tid * TK_E;
    u32 kk[TK_E];
    u32 ngt = 0, neq = 0;
#pragma unroll
    for (int e = 0; e < TK_E; ++e) {
      kk[e] = (j0 + e < n_cand) ? ckey[j0 + e] : 0u;
      const bool ok = (j0 + e) < n_cand;
      ngt += (ok && kk[e] > vstar) ? 1u : 0u;
      neq += (ok && kk[e] == vstar) ? 1u : 0u;
    }
    const u32 packed = (neq << 16) | ngt;
    u32 tot;
    const u32 incl = block_incl_scan<TK_NT>(packed, scratch, &tot);
    const u32 excl = incl - packed;
    u32 gt_before = gt_base + (excl & 0xFFFFu);
    u32 eq_before = eq_base + (excl >> 16);
#pragma unroll
    for (int e = 0; e < TK_E; ++e) {
      if (j0 + e >= n_cand) continue;
      const u32 key = kk[e];
      if (key > vstar) {
        out[above1 + gt_before + min(eq_before, ties)] = cpos[j0 + e];
        ++gt_before;
      } else if (key == vstar) {
        if (eq_before < ties) out[above1 + gt_before + eq_before] = cpos[j0 + e];
        ++eq_before;
      }
    }
    gt_base += tot & 0xFFFFu;
    eq_base += tot >> 16;
  }
}

size_t topk_workspace_bytes(int T, int64_t ld) {
  return 2 * align256((size_t)T * (size_t)ld * 4);
}

hipError_t launch_topk(const float* logits, int64_t ld, const int32_t* valid_len, int len_add, int T, int k,
                       int32_t* idx, void* ws, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  u32* cand_key = reinterpret_cast<u32*>(ws);
  int32_t* cand_pos = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + align256((size_t)T * ld * 4));
  hipLaunchKernelGGL(topk_kernel, dim3(T), dim3(TK_NT), 0, stream, logits, ld, valid_len, len_add, k, idx, cand_key,
                     cand_pos);
  return hipGetLastError();
}

}  // namespace dsa
