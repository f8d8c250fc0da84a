// Per-query top-k selection by radix select on order-preserving keys.
//
// "DeepSeek V3.2-Exp Cuts Prolonged-Context Costs With DeepSeek Sparse
// Consideration (DSA)", part (2): each query keeps only its top-k (k = 2048)
// key-value entries.  Result: the positions of the k largest logits of the
// row; equal logits are taken lowest position first; -0 equals +0.
//
// A 128K-long row is 512 KB, so one workgroup per row would leave most of the
// chip idle.  The selection is split over three launches:
//   histogram  a per-row count of the top 11 key bits (2048 bins); in
//              dsa_forward the indexer builds it in its epilogue, so the
//              logits are not read for it;
//   chunk      many workgroups per row (4096 positions each) find the bin
//              that holds the k-th largest key from the histogram, and sweep
//              their chunk once: positions in higher bins go to a per-chunk
//              "above" list, positions in the threshold bin to a per-chunk
//              candidate list, both in position order;
//   resolve    one workgroup per row concatenates the above lists, finds the
//              exact k-th key among the candidates with two more histogram
//              rounds (bits 20..10, 9..0), and appends the candidates above it
//              plus the first ties at it.
// Everything is written at positions derived from counts, never from atomics,
// so the output is deterministic: above-threshold-bin positions ascending,
// then the selected candidates ascending.
#include "launch.h"

namespace dsa {

constexpr int TK_CH = 4096;  // positions per chunk
constexpr int TK_CHUNK_NT = 512;
constexpr int TK_RES_NT = 1024;
constexpr int TK_BINS = 2048;
constexpr int TK_MAX_CHUNKS = TK_RES_NT;  // rows up to 4M positions
constexpr int TK_RES_STAGE = 12288;       // candidates staged in LDS (96 KB)

// Valid length of row t, clamped to the stated bound max_len (so a length
// past it never reaches beyond the launched chunks or the workspace).
__device__ __forceinline__ int row_len(const int32_t* valid_len, int len_add, int t, int max_len) {
  return min(valid_len[t] + len_add, max_len);
}

// Threshold search over NB bins visited from the top with NT threads: the bin
// holding the `need`-th largest element and the count in higher bins.
template <int NB, int NT>
__device__ __forceinline__ void find_threshold(const u32* hist, u32 need, u32* scratch, u32* out_bin,
                                               u32* out_above) {
  constexpr int BPT = NB / NT;
  const int tid = threadIdx.x;
  u32 c[BPT];
  u32 mine = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    c[i] = hist[NB - 1 - (tid * BPT + i)];
    mine += c[i];
  }
  u32 total;
  const u32 incl = block_incl_scan<NT>(mine, scratch, &total);
  u32 excl = incl - mine;
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

__global__ void zero_u32_kernel(u32* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

// Histogram of the top 11 key bits of each row (standalone selection).
__global__ __launch_bounds__(TK_CHUNK_NT) void topk_hist_kernel(const float* __restrict__ logits, int64_t ld,
                                                                const int32_t* __restrict__ valid_len, int len_add,
                                                                int max_len, int k, u32* __restrict__ hist) {
  __shared__ u32 h[TK_BINS];
  const int t = blockIdx.y;
  const int n = row_len(valid_len, len_add, t, max_len);
  const int c0 = blockIdx.x * TK_CH;
  if (n <= k || c0 >= n) return;
  for (int i = threadIdx.x; i < TK_BINS; i += TK_CHUNK_NT) h[i] = 0;
  __syncthreads();
  const float* row = logits + (int64_t)t * ld;
  const int c1 = min(n, c0 + TK_CH);
  for (int i = c0 + threadIdx.x; i < c1; i += TK_CHUNK_NT) atomicAdd(&h[order_key(row[i]) >> 21], 1u);
  __syncthreads();
  u32* g = hist + (int64_t)t * TK_BINS;
  for (int i = threadIdx.x; i < TK_BINS; i += TK_CHUNK_NT)
    if (h[i]) atomicAdd(&g[i], h[i]);
}

struct TopkWs {
  u32* hist;      // [T, 2048]
  u32* counts;    // [T, nch, 2]   (above, candidates) per chunk
  int32_t* above; // [T, nch, cap_above]
  u32* ckey;      // [T, nch, TK_CH]
  int32_t* cpos;  // [T, nch, TK_CH]
  int nch;
  int cap_above;
};

__global__ __launch_bounds__(TK_CHUNK_NT) void topk_chunk_kernel(const float* __restrict__ logits, int64_t ld,
                                                                 const int32_t* __restrict__ valid_len, int len_add,
                                                                 int max_len, int k, TopkWs ws) {
  constexpr int NT = TK_CHUNK_NT;
  constexpr int E = TK_CH / NT;  // 8 positions per thread
  __shared__ u32 scratch[NT / 64 + 1];
  __shared__ u32 sh_bin, sh_above;
  const int t = blockIdx.y;
  const int c = blockIdx.x;
  const int n = row_len(valid_len, len_add, t, max_len);
  const int c0 = c * TK_CH;
  if (n <= k || c0 >= n) return;
  // the chunk's logits are loaded first: their latency overlaps the threshold search
  const float* row = logits + (int64_t)t * ld;
  const int i0 = c0 + threadIdx.x * E;
  u32 kk[E];
#pragma unroll
  for (int q = 0; q < E / 4; ++q) {
    const int i = i0 + 4 * q;
    if (i + 4 <= n) {
      const float4 v = *reinterpret_cast<const float4*>(row + i);
      kk[4 * q + 0] = order_key(v.x);
      kk[4 * q + 1] = order_key(v.y);
      kk[4 * q + 2] = order_key(v.z);
      kk[4 * q + 3] = order_key(v.w);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) kk[4 * q + e] = (i + e < n) ? order_key(row[i + e]) : 0u;
    }
  }
  find_threshold<TK_BINS, NT>(ws.hist + (int64_t)t * TK_BINS, (u32)k, scratch, &sh_bin, &sh_above);
  const u32 b1 = sh_bin;
  u32 na = 0, nc = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool ok = (i0 + e) < n;
    const u32 bin = kk[e] >> 21;
    na += (ok && bin > b1) ? 1u : 0u;
    nc += (ok && bin == b1) ? 1u : 0u;
  }
  const u32 packed = (nc << 16) | na;
  u32 tot;
  const u32 incl = block_incl_scan<NT>(packed, scratch, &tot);
  const u32 excl = incl - packed;
  const int64_t slot = (int64_t)t * ws.nch + c;
  int32_t* abv = ws.above + slot * ws.cap_above;
  u32* ck = ws.ckey + slot * TK_CH;
  int32_t* cp = ws.cpos + slot * TK_CH;
  u32 ao = excl & 0xFFFFu, co = excl >> 16;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (i0 + e >= n) continue;
    const u32 bin = kk[e] >> 21;
    if (bin > b1) {
      abv[ao++] = i0 + e;
    } else if (bin == b1) {
      ck[co] = kk[e];
      cp[co] = i0 + e;
      ++co;
    }
  }
  if (threadIdx.x == 0) {
    ws.counts[slot * 2 + 0] = tot & 0xFFFFu;
    ws.counts[slot * 2 + 1] = tot >> 16;
  }
}

// The exact selection among C threshold-bin candidates (their key bits
// 20..0 and positions, in position order, read through cand_key / cand_pos):
// the need1-th largest key via two more histogram rounds (bits 20..10, then
// 9..0), then one ordered sweep that writes to out the candidates above it
// and the first ties at it, in position order.  `hist` holds TK_BINS words of
// LDS; every thread of the block takes part.
template <int NT, class KeyF, class PosF>
__device__ __forceinline__ void select_candidates(u32 C, u32 need1, int32_t* __restrict__ out, KeyF cand_key,
                                                  PosF cand_pos, u32* hist, u32* scratch, u32* sh_bin,
                                                  u32* sh_above) {
  const int tid = threadIdx.x;
  for (u32 j = tid; j < C; j += NT) atomicAdd(&hist[cand_key(j) >> 10], 1u);
  __syncthreads();
  find_threshold<TK_BINS, NT>(hist, need1, scratch, sh_bin, sh_above);
  const u32 b2 = *sh_bin;
  const u32 need2 = need1 - *sh_above;
  __syncthreads();
  for (int i = tid; i < 1024; i += NT) hist[i] = 0;
  __syncthreads();
  for (u32 j = tid; j < C; j += NT) {
    const u32 key = cand_key(j);
    if ((key >> 10) == b2) atomicAdd(&hist[key & 0x3FFu], 1u);
  }
  __syncthreads();
  find_threshold<1024, NT>(hist, need2, scratch, sh_bin, sh_above);
  const u32 low = (b2 << 10) | *sh_bin;  // bits 20..0 of the k-th key
  const u32 ties = need2 - *sh_above;    // keys equal to it that are kept (>= 1)

  // ordered sweep of the candidates (their order = position order).  Up to
  // 4 per thread, each thread takes a contiguous run, so one block scan
  // places them all.
  if (C <= 4u * NT) {
    const u32 R = (C + NT - 1) / NT;
    const u32 j0 = (u32)tid * R;
    u32 key[4];
    u32 gt = 0, eq = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const u32 j = j0 + r;
      key[r] = ((u32)r < R && j < C) ? cand_key(j) : 0u;
      const bool ok = (u32)r < R && j < C;
      gt += (ok && key[r] > low) ? 1u : 0u;
      eq += (ok && key[r] == low) ? 1u : 0u;
    }
    u32 bt;
    const u32 packed = (eq << 16) | gt;
    const u32 excl = block_incl_scan<NT>(packed, scratch, &bt) - packed;
    u32 gt_before = excl & 0xFFFFu, eq_before = excl >> 16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const u32 j = j0 + r;
      if ((u32)r >= R || j >= C) continue;
      if (key[r] > low) {
        out[gt_before + min(eq_before, ties)] = cand_pos(j);
        ++gt_before;
      } else if (key[r] == low) {
        if (eq_before < ties) out[gt_before + eq_before] = cand_pos(j);
        ++eq_before;
      }
    }
    return;
  }
  u32 gt_base = 0, eq_base = 0;
  for (u32 j0 = 0; j0 < C; j0 += NT) {
    const u32 j = j0 + tid;
    const bool ok = j < C;
    const u32 key = ok ? cand_key(j) : 0u;
    const u32 gt = (ok && key > low) ? 1u : 0u;
    const u32 eq = (ok && key == low) ? 1u : 0u;
    const u32 packed = (eq << 16) | gt;
    u32 bt;
    const u32 bincl = block_incl_scan<NT>(packed, scratch, &bt);
    const u32 excl = bincl - packed;
    const u32 gt_before = gt_base + (excl & 0xFFFFu);
    const u32 eq_before = eq_base + (excl >> 16);
    if (gt) out[gt_before + min(eq_before, ties)] = cand_pos(j);
    else if (eq && eq_before < ties) out[gt_before + eq_before] = cand_pos(j);
    gt_base += bt & 0xFFFFu;
    eq_base += bt >> 16;
  }
}

// Largest c in [0, n) with off[c] <= j (off ascending, off[0] = 0).
__device__ __forceinline__ int chunk_of(const u32* off, int n, u32 j) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= j) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// chunk_of for U indices at once: the same fixed sequence of steps for all,
// so their LDS reads are in flight together.  `top` is the largest power of
// two below n (0 when n == 1).
template <int U>
__device__ __forceinline__ void chunk_of_n(const u32* off, int n, int top, const u32 (&j)[U], int (&lo)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u) lo[u] = 0;
  for (int step = top; step > 0; step >>= 1) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (lo[u] + step < n && off[lo[u] + step] <= j[u]) lo[u] += step;
  }
}

__global__ __launch_bounds__(TK_RES_NT) void topk_resolve_kernel(const int32_t* __restrict__ valid_len, int len_add,
                                                                 int max_len, int k, int32_t* __restrict__ idx,
                                                                 TopkWs ws) {
  constexpr int NT = TK_RES_NT;
  __shared__ u32 hist[TK_BINS];
  __shared__ u32 scratch[NT / 64 + 1];
  __shared__ u32 sh_bin, sh_above;
  __shared__ u32 s_aoff[TK_MAX_CHUNKS], s_coff[TK_MAX_CHUNKS];
  __shared__ u32 s_ckey[TK_RES_STAGE];
  __shared__ int32_t s_cpos[TK_RES_STAGE];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = row_len(valid_len, len_add, t, max_len);
  int32_t* __restrict__ out = idx + (int64_t)t * k;
  if (n <= k) {
    for (int i = tid; i < k; i += NT) out[i] = (i < n) ? i : -1;
    return;
  }
  const int nch = (n + TK_CH - 1) / TK_CH;  // <= TK_MAX_CHUNKS (checked on the host)
  const int64_t slot0 = (int64_t)t * ws.nch;
  // the lists are only read here and `out` only written: no aliasing, so the
  // list loads may run ahead of the stores
  const int32_t* __restrict__ above = ws.above;
  const u32* __restrict__ ckey = ws.ckey;
  const int32_t* __restrict__ cpos = ws.cpos;

  // ---- per-chunk counts -> exclusive offsets (one chunk per thread)
  const u32 my_a = (tid < nch) ? ws.counts[(slot0 + tid) * 2 + 0] : 0u;
  const u32 my_c = (tid < nch) ? ws.counts[(slot0 + tid) * 2 + 1] : 0u;
  u32 tot;
  const u32 incl = block_incl_scan<NT>((my_c << 16) | my_a, scratch, &tot);
  // counts per chunk are <= 4096, but totals may exceed 16 bits: rescan separately if needed
  u32 a_excl, c_excl, A, C;
  if (nch * TK_CH < 65536) {
    a_excl = (incl - ((my_c << 16) | my_a)) & 0xFFFFu;
    c_excl = (incl - ((my_c << 16) | my_a)) >> 16;
    A = tot & 0xFFFFu;
    C = tot >> 16;
  } else {
    const u32 ia = block_incl_scan<NT>(my_a, scratch, &A);
    const u32 ic = block_incl_scan<NT>(my_c, scratch, &C);
    a_excl = ia - my_a;
    c_excl = ic - my_c;
  }
  if (tid < nch) {
    s_aoff[tid] = a_excl;
    s_coff[tid] = c_excl;
  }
  __syncthreads();

  // ---- above lists, concatenated in chunk order
  for (u32 j = tid; j < A; j += NT) {
    const int c = chunk_of(s_aoff, nch, j);
    out[j] = above[(slot0 + c) * ws.cap_above + (j - s_aoff[c])];
  }
  const u32 need1 = (u32)k - A;

  // ---- candidates: stage (key bits 20..0, position) in LDS when they fit
  const bool staged = C <= TK_RES_STAGE;
  if (staged) {
    // four candidates per thread per round: their chunk lookups share one
    // search, and all eight loads are in flight before any is used
    const int top = nch > 1 ? 1 << (31 - __builtin_clz((u32)(nch - 1))) : 0;
    for (u32 j0 = 0; j0 < C; j0 += 4 * NT) {
      u32 j[4];
      int c[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) j[u] = j0 + u * NT + tid;
      chunk_of_n<4>(s_coff, nch, top, j, c);
      u32 kv[4];
      int32_t pv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        // past C the lane reads the row's first slot instead (never out of range)
        const int64_t g = j[u] < C ? (slot0 + c[u]) * TK_CH + (j[u] - s_coff[c[u]]) : slot0 * TK_CH;
        kv[u] = ckey[g];
        pv[u] = cpos[g];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (j[u] < C) {
          s_ckey[j[u]] = kv[u] & 0x1FFFFFu;
          s_cpos[j[u]] = pv[u];
        }
      }
    }
  }
  for (int i = tid; i < TK_BINS; i += NT) hist[i] = 0;
  __syncthreads();
  auto cand_key = [&](u32 j) -> u32 {
    if (staged) return s_ckey[j];
    const int c = chunk_of(s_coff, nch, j);
    return ckey[(slot0 + c) * TK_CH + (j - s_coff[c])] & 0x1FFFFFu;
  };
  auto cand_pos = [&](u32 j) -> int32_t {
    if (staged) return s_cpos[j];
    const int c = chunk_of(s_coff, nch, j);
    return cpos[(slot0 + c) * TK_CH + (j - s_coff[c])];
  };

  select_candidates<NT>(C, need1, out + A, cand_key, cand_pos, hist, scratch, &sh_bin, &sh_above);
}

// Chunk slots per row: enough for the longest valid row (max_len); the row
// stride of the logits plays no part in the workspace.
static int topk_nch(int64_t max_len) {
  const int64_t c = (max_len + TK_CH - 1) / TK_CH;
  return c > 0 ? (int)c : 1;
}

WsLayout topk_layout(int T, int64_t max_len, int k) {
  WsLayout L;
  const size_t slots = (size_t)T * topk_nch(max_len);
  const size_t cap_above = k < TK_CH ? k : TK_CH;
  L.add("hist", (size_t)T * TK_BINS * 4);  // first: the indexer's fused histogram lives here
  L.add("counts", slots * 2 * 4);
  L.add("above", slots * cap_above * 4);
  L.add("ckey", slots * TK_CH * 4);
  L.add("cpos", slots * TK_CH * 4);
  return L;
}

static TopkWs carve(void* ws, int T, int64_t max_len, int k) {
  const WsLayout L = topk_layout(T, max_len, k);
  TopkWs w;
  w.nch = topk_nch(max_len);
  w.cap_above = k < TK_CH ? k : TK_CH;
  w.hist = static_cast<u32*>(L.at(ws, 0));
  w.counts = static_cast<u32*>(L.at(ws, 1));
  w.above = static_cast<int32_t*>(L.at(ws, 2));
  w.ckey = static_cast<u32*>(L.at(ws, 3));
  w.cpos = static_cast<int32_t*>(L.at(ws, 4));
  return w;
}

size_t topk_workspace_bytes(int T, int64_t max_len, int k) { return topk_layout(T, max_len, k).total; }

u32* topk_hist_buffer(void* ws) { return static_cast<u32*>(ws); }

hipError_t launch_topk_zero_hist(void* ws, int T, hipStream_t stream) {
  const int64_t n = (int64_t)T * TK_BINS;
  const int64_t want = (n + 255) / 256;
  const int blocks = (int)(want < 1024 ? want : 1024);
  hipLaunchKernelGGL(zero_u32_kernel, dim3(blocks), dim3(256), 0, stream, topk_hist_buffer(ws), n);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int64_t ld, const int32_t* valid_len, int len_add, int T, int max_len,
                       int k, int32_t* idx, void* ws, bool hist_ready, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  TopkWs w = carve(ws, T, max_len, k);
  const int nch = w.nch;
  if (!hist_ready) {
    hipError_t e = launch_topk_zero_hist(ws, T, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_hist_kernel, dim3(nch, T), dim3(TK_CHUNK_NT), 0, stream, logits, ld, valid_len, len_add,
                       max_len, k, w.hist);
  }
  hipLaunchKernelGGL(topk_chunk_kernel, dim3(nch, T), dim3(TK_CHUNK_NT), 0, stream, logits, ld, valid_len, len_add,
                     max_len, k, w);
  hipLaunchKernelGGL(topk_resolve_kernel, dim3(T), dim3(TK_RES_NT), 0, stream, valid_len, len_add, max_len, k, idx, w);
  return hipGetLastError();
}

}  // namespace dsa
