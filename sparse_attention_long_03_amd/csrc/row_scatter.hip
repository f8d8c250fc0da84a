// Scatter-add of bf16 rows into an fp32 table through a sort.
//
// Used by the training side ("DeepSeek V3.2-Exp Cuts Prolonged-Context Costs
// With DeepSeek Sparse Consideration (DSA)", "Teaching signal"): the sparse
// attention's key/value gradient and the indexer's key gradient reach each
// selected cache row once per query that selected it.
//
// Many producers (query tokens) each emit one gradient row per selected
// cache row; a cache row selected by several queries must receive the sum.
// fp32 atomics reach only about a fifth of the store bandwidth on this GPU,
// so instead of one atomic per value and producer, the (row, slot) list is
// sorted by row with a stable LSD radix sort (8-bit digits, one pass per
// byte of the largest row id), and a wave then walks 256 consecutive sorted
// entries, sums each run of equal rows in fp32 and adds the run to the table
// with one atomic per value (a run crossing a chunk edge is added by both
// waves).  Within a chunk the sum runs in slot order; the order of the
// atomics across chunks is not fixed.
#include "launch.h"

namespace dsa {

constexpr u32 SLOT_NONE = 0xFFFFFFFFu;

// ---------------------------------------------------------------------------
// stable LSD radix sort of the row list (8-bit digits)
// ---------------------------------------------------------------------------

constexpr int RS_NT = 256;
constexpr int RS_ROUNDS = 16;
constexpr int RS_BLOCK = RS_NT * RS_ROUNDS;  // elements per block

// per-block digit counts, digit-major: hist[d * nblocks + block]
__global__ __launch_bounds__(RS_NT) void radix_hist_kernel(const u32* __restrict__ keys, int N, int shift,
                                                            u32* __restrict__ hist, int nblocks) {
  __shared__ u32 h[256];
  const int tid = threadIdx.x;
  h[tid] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * RS_BLOCK;
#pragma unroll 4
  for (int r = 0; r < RS_ROUNDS; ++r) {
    const int64_t i = base + r * RS_NT + tid;
    if (i < N) atomicAdd(&h[(keys[i] >> shift) & 255u], 1u);
  }
  __syncthreads();
  hist[(int64_t)tid * nblocks + blockIdx.x] = h[tid];
}

// one workgroup per digit: exclusive scan of its counts over the blocks
__global__ __launch_bounds__(RS_NT) void radix_scan_kernel(u32* __restrict__ hist, int nblocks,
                                                            u32* __restrict__ totals) {
  __shared__ u32 scratch[RS_NT / 64 + 1];
  u32* row = hist + (int64_t)blockIdx.x * nblocks;
  u32 carry = 0;
  for (int i0 = 0; i0 < nblocks; i0 += RS_NT) {
    const int i = i0 + threadIdx.x;
    const u32 v = (i < nblocks) ? row[i] : 0u;
    u32 tot;
    const u32 incl = block_incl_scan<RS_NT>(v, scratch, &tot);
    if (i < nblocks) row[i] = carry + incl - v;
    carry += tot;
  }
  if (threadIdx.x == 0) totals[blockIdx.x] = carry;
}

// Scatter in a stable order: each round takes RS_NT consecutive elements;
// lanes with equal digits find each other with 8 ballots, and the waves of
// a round are ranked in order through per-wave digit counts in LDS.
__global__ __launch_bounds__(RS_NT) void radix_scatter_kernel(const u32* __restrict__ keys_in,
                                                               const u32* __restrict__ vals_in, int N, int shift,
                                                               const u32* __restrict__ hist,
                                                               const u32* __restrict__ totals, int nblocks,
                                                               u32* __restrict__ keys_out,
                                                               u32* __restrict__ vals_out) {
  constexpr int NWV = RS_NT / 64;
  __shared__ u32 s_base[256];
  __shared__ u32 s_wcnt[NWV][256];
  __shared__ u32 scratch[NWV + 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  {
    const u32 tot_d = totals[tid];
    u32 all;
    const u32 incl = block_incl_scan<RS_NT>(tot_d, scratch, &all);
    s_base[tid] = incl - tot_d + hist[(int64_t)tid * nblocks + blockIdx.x];
#pragma unroll
    for (int w = 0; w < NWV; ++w) s_wcnt[w][tid] = 0;
  }
  __syncthreads();
  const unsigned long long below = (1ull << lane) - 1ull;
  const int64_t base = (int64_t)blockIdx.x * RS_BLOCK;
  for (int r = 0; r < RS_ROUNDS; ++r) {
    const int64_t i = base + r * RS_NT + tid;
    const bool valid = i < N;
    const u32 key = valid ? keys_in[i] : 0u;
    const u32 val = valid ? (vals_in ? vals_in[i] : (u32)i) : 0u;
    const u32 dig = (key >> shift) & 255u;
    unsigned long long peers = __builtin_amdgcn_ballot_w64(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool set = (dig >> bit) & 1u;
      const unsigned long long bb = __builtin_amdgcn_ballot_w64(set);
      peers &= set ? bb : ~bb;
    }
    const u32 rank = (u32)__popcll(peers & below);
    if (valid && rank == 0) s_wcnt[wid][dig] = (u32)__popcll(peers);
    __syncthreads();
    if (valid) {
      u32 pos = s_base[dig] + rank;
      for (int w = 0; w < wid; ++w) pos += s_wcnt[w][dig];
      keys_out[pos] = key;
      vals_out[pos] = val;
    }
    __syncthreads();
    u32 add = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      add += s_wcnt[w][tid];
      s_wcnt[w][tid] = 0;
    }
    s_base[tid] += add;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// segmented reduction
// ---------------------------------------------------------------------------

constexpr int RD_CHUNK = 256;  // sorted entries per wave

__device__ __forceinline__ void add_bf16x8(float* acc, v4i x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] += __uint_as_float((u32)x[i] << 16);
    acc[2 * i + 1] += __uint_as_float((u32)x[i] & 0xFFFF0000u);
  }
}

// Rows of W bf16 values = C chunks of 16 bytes: lane l sums chunk l (l < C)
// and chunk 64 + l (64 + l < C); other lanes load a valid chunk and drop it.
template <int W>
__global__ __launch_bounds__(256) void row_reduce_kernel(const u32* __restrict__ keys, const u32* __restrict__ vals,
                                                         int N, const uint16_t* __restrict__ src_rows,
                                                         float* __restrict__ dst) {
  constexpr int C = W / 8;
  const int lane = threadIdx.x & 63;
  const int64_t base = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RD_CHUNK;
  if (base >= N) return;
  const bool has0 = lane < C, has1 = 64 + lane < C;
  const int c0 = lane % C, c1 = (64 + lane < C) ? 64 + lane : c0;
  float a0[8], a1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a0[i] = a1[i] = 0.f;
  u32 cur = SLOT_NONE;
  bool done = false;
  auto flush = [&]() {
    float* row = dst + (int64_t)cur * W;
    if (has0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) __hip_atomic_fetch_add(row + 8 * c0 + i, a0[i], __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
    }
    if (has1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) __hip_atomic_fetch_add(row + 8 * c1 + i, a1[i], __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) a0[i] = a1[i] = 0.f;
  };
  for (int sub = 0; sub < RD_CHUNK / 64; ++sub) {
    const int64_t j = base + 64 * sub + lane;
    const u32 kj = (j < N) ? keys[j] : SLOT_NONE;
    const u32 vj = (j < N) ? vals[j] : 0u;
    if (__builtin_amdgcn_readfirstlane(kj) == SLOT_NONE) break;  // the rest of the list is past the end
#pragma unroll 1
    for (int e0 = 0; e0 < 64 && !done; e0 += 8) {
      v4i x0[8], x1[8];
      u32 ke[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        ke[u] = __builtin_amdgcn_readlane(kj, e0 + u);
        const u32 ve = __builtin_amdgcn_readlane(vj, e0 + u);
        const uint16_t* src = src_rows + (int64_t)(ke[u] == SLOT_NONE ? 0u : ve) * W;
        x0[u] = *reinterpret_cast<const v4i*>(src + 8 * c0);
        if (C > 64) x1[u] = *reinterpret_cast<const v4i*>(src + 8 * c1);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (ke[u] == SLOT_NONE) {
          done = true;
          break;
        }
        if (ke[u] != cur) {
          if (cur != SLOT_NONE) flush();
          cur = ke[u];
        }
        add_bf16x8(a0, x0[u]);
        if (C > 64 && has1) add_bf16x8(a1, x1[u]);
      }
    }
    if (done) break;
  }
  if (cur != SLOT_NONE) flush();
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static int sort_passes(int64_t num_rows) {
  int bits = 0;
  while (bits < 32 && (int64_t(1) << bits) <= num_rows) ++bits;  // bit length of num_rows
  return (bits + 7) / 8;
}

struct ScatterWorkspace {
  u32 *keys_b, *vals_a, *vals_b, *hist, *totals;
};

WsLayout scatter_layout(int64_t N) {
  WsLayout L;
  const size_t nblocks = ((size_t)N + RS_BLOCK - 1) / RS_BLOCK;
  L.add("keys_b", (size_t)N * 4);
  L.add("vals_a", (size_t)N * 4);
  L.add("vals_b", (size_t)N * 4);
  L.add("hist", 256 * nblocks * 4);
  L.add("totals", 256 * 4);
  return L;
}

static void carve_scatter(int64_t N, void* base, ScatterWorkspace* w) {
  const WsLayout L = scatter_layout(N);
  w->keys_b = static_cast<u32*>(L.at(base, 0));
  w->vals_a = static_cast<u32*>(L.at(base, 1));
  w->vals_b = static_cast<u32*>(L.at(base, 2));
  w->hist = static_cast<u32*>(L.at(base, 3));
  w->totals = static_cast<u32*>(L.at(base, 4));
}

size_t row_scatter_workspace_bytes(int64_t N) { return scatter_layout(N).total; }

hipError_t launch_row_scatter_add(u32* rows, int N, int64_t num_rows, const uint16_t* src_rows, int W, float* dst,
                                  void* ws, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  ScatterWorkspace w;
  carve_scatter(N, ws, &w);
  const int nblocks = (N + RS_BLOCK - 1) / RS_BLOCK;
  hipError_t e;
  const int passes = sort_passes(num_rows);
  u32 *kin = rows, *kout = w.keys_b, *vin = nullptr, *vout = w.vals_a;
  for (int p = 0; p < passes; ++p) {
    hipLaunchKernelGGL(radix_hist_kernel, dim3(nblocks), dim3(RS_NT), 0, stream, kin, N, 8 * p, w.hist, nblocks);
    hipLaunchKernelGGL(radix_scan_kernel, dim3(256), dim3(RS_NT), 0, stream, w.hist, nblocks, w.totals);
    hipLaunchKernelGGL(radix_scatter_kernel, dim3(nblocks), dim3(RS_NT), 0, stream, kin, vin, N, 8 * p, w.hist,
                       w.totals, nblocks, kout, vout);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    std::swap(kin, kout);
    vin = vout;
    vout = (vout == w.vals_a) ? w.vals_b : w.vals_a;
  }
  const int chunks = (N + RD_CHUNK - 1) / RD_CHUNK;
  const dim3 grid((chunks + 3) / 4);
  if (W == 576)
    hipLaunchKernelGGL(row_reduce_kernel<576>, grid, dim3(256), 0, stream, kin, vin, N, src_rows, dst);
  else if (W == 128)
    hipLaunchKernelGGL(row_reduce_kernel<128>, grid, dim3(256), 0, stream, kin, vin, N, src_rows, dst);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dsa
