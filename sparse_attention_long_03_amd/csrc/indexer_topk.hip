// Lightning indexer fused with the top-k selection, for batches with many
// query tokens (prefill): the logits are consumed as they are produced and
// never stored.
//
// "DeepSeek V3.2-Exp Cuts Prolonged-Context Costs With DeepSeek Sparse
// Consideration (DSA)", parts (1) and (2): score every earlier token with the
// indexer, keep the k highest-scoring ones (lowest position first among
// equal scores, -0 equal to +0).
//
// Work split.  A workgroup takes 4 consecutive query tokens, one per wave,
// and streams the keys of their sequence from position 0 in tiles of 64 keys
// staged through LDS (one global read of a tile serves all 4 tokens).  With
// one token a wave fits in 168 registers (a 20-byte spill outside the tile
// loop), so three waves share each SIMD; two tokens a wave took 250 registers
// and two waves per SIMD, and ran 2% slower at the 64K prefill.  Each wave
// computes its token's logits for the tile with the same arithmetic as the
// logits kernel (indexer_math.h), so every logit is bit-identical to the one
// dsa_indexer_logits would store.
//
// Streaming selection.  Per token, the wave keeps a candidate list in the
// workspace: (order key, position) pairs in increasing position, plus a
// threshold key `tau`.  A logit enters the list when its key is above tau.
// When the list nears its capacity, the wave finds the exact k-th largest key
// K* of the list (radix select over key bits 31..21, 20..10, 9..0) and keeps,
// in order, the entries above K* and the first entries equal to K*, k in all;
// tau becomes K*.  This is exact: a dropped entry is beaten by k kept ones,
// and a later logit equal to K* loses to the kept ties, which all sit at
// lower positions -- so the strict test against tau also carries the tie
// rule.  After the last tile the same select writes the k positions (or all
// of them, padded with -1, when the row is not longer than k).
//
// Tokens of different sequences in one workgroup are handled in one pass over
// the keys per sequence.
#include "indexer_math.h"
#include "launch.h"

namespace dsa {

constexpr int FT_WAVES = 4;
constexpr int FT_QPW = 1;                 // query tokens per wave
constexpr int FT_QB = FT_WAVES * FT_QPW;  // query tokens per workgroup
constexpr int FT_TILE = 64;               // keys per tile
constexpr int FT_AHEAD = 4;               // key tiles in flight (register stages)
constexpr int FT_CAP_MAX = 12288;         // candidate slots per token
constexpr int FT_BINS = 2048;

// Memory fence for one wave's own LDS and global traffic: waits until this
// wave's earlier accesses are done, so lanes see each other's writes.
__device__ __forceinline__ void wave_sync() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup"); }

#ifndef LDS_AS
#define LDS_AS __attribute__((address_space(3)))
#endif

// A wave's selection histogram lives in LDS.  Its pointer carries the LDS
// address space in every signature below, so each access is an LDS
// instruction whether or not the helpers are inlined.
typedef LDS_AS u32 lds_u32;

__device__ __forceinline__ void lds_inc(lds_u32* p) {
  __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ u32 lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((u32)(m >> 32), __builtin_amdgcn_mbcnt_lo((u32)m, 0u));
}

// Wave-level threshold search over NB bins from the top: the bin holding the
// need-th largest entry (1 <= need <= total) and the count in higher bins.
template <int NB>
__device__ __forceinline__ void wave_threshold(const lds_u32* hist, u32 need, u32& bin, u32& above) {
  constexpr int BPL = NB / 64;
  const int lane = threadIdx.x & 63;
  const lds_u32* run = hist + NB - 1 - lane * BPL;  // this lane's bins, from the top: run[0], run[-1], ...
  u32 mine = 0;
#pragma unroll 8
  for (int i = 0; i < BPL; ++i) mine += run[-i];
  const u32 incl = wave_incl_scan(mine);
  const u32 excl = incl - mine;
  const bool here = excl < need && incl >= need;
  // first bin of this lane's run where the running count reaches need
  // (branch-free; only the lane that holds it uses the result)
  u32 e = excl, b = 0, a = 0;
  bool found = false;
#pragma unroll 8
  for (int i = 0; i < BPL; ++i) {
    const u32 e2 = e + run[-i];
    const bool hit = !found && e2 >= need;
    b = hit ? (u32)(NB - 1 - (lane * BPL + i)) : b;
    a = hit ? e : a;
    found = found || hit;
    e = e2;
  }
  const int src = __builtin_ctzll(__ballot(here));
  bin = __shfl(b, src, 64);
  above = __shfl(a, src, 64);
}

// Adds 1 to hist[f(key)] for every list entry whose key passes `sel`.
template <typename Sel, typename Bin>
__device__ __forceinline__ void wave_count(const u32* __restrict__ key, int n, lds_u32* hist, Sel sel, Bin bin) {
  const int lane = threadIdx.x & 63;
  int j = lane;
  // eight loads in flight per step: the list sits in L2, MALL or HBM
  for (; j + 448 < n; j += 512) {
    u32 kk[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) kk[u] = key[j + 64 * u];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (sel(kk[u])) lds_inc(&hist[bin(kk[u])]);
  }
  for (; j < n; j += 64) {
    const u32 k0 = key[j];
    if (sel(k0)) lds_inc(&hist[bin(k0)]);
  }
}

// Exact k-th largest key of a list of n > k entries, by one wave: kstar, and
// how many entries equal to it are kept (ties >= 1).
__device__ __forceinline__ void wave_kth(const u32* __restrict__ key, int n, int k, lds_u32* hist, u32& kstar,
                                         u32& ties) {
  const int lane = threadIdx.x & 63;
  wave_sync();  // the list entries this wave appended are visible
  for (int i = lane; i < FT_BINS; i += 64) hist[i] = 0;
  wave_sync();
  wave_count(key, n, hist, [](u32) { return true; }, [](u32 x) { return x >> 21; });
  wave_sync();
  u32 b1, a1;
  wave_threshold<FT_BINS>(hist, (u32)k, b1, a1);
  u32 need = (u32)k - a1;
  wave_sync();
  for (int i = lane; i < FT_BINS; i += 64) hist[i] = 0;
  wave_sync();
  wave_count(key, n, hist, [b1](u32 x) { return (x >> 21) == b1; }, [](u32 x) { return (x >> 10) & 0x7FFu; });
  wave_sync();
  u32 b2, a2;
  wave_threshold<FT_BINS>(hist, need, b2, a2);
  need -= a2;
  const u32 pre = (b1 << 11) | b2;
  wave_sync();
  for (int i = lane; i < 1024; i += 64) hist[i] = 0;
  wave_sync();
  wave_count(key, n, hist, [pre](u32 x) { return (x >> 10) == pre; }, [](u32 x) { return x & 0x3FFu; });
  wave_sync();
  u32 b3, a3;
  wave_threshold<1024>(hist, need, b3, a3);
  kstar = (pre << 10) | b3;
  ties = need - a3;
  wave_sync();
}

// Writes, in list order, the entries with key > kstar and the first `ties`
// entries with key == kstar: to (okey, opos) when okey is given (which may be
// the list itself: every entry moves to a lower or equal index), else only the
// positions to opos.  Exactly k entries qualify; writes stop at index k.
__device__ __forceinline__ void wave_emit(const u32* key, const int32_t* pos, int n, int k, u32 kstar, u32 ties,
                                          u32* okey, int32_t* opos) {
  const int lane = threadIdx.x & 63;
  u32 taken = 0, eq_seen = 0;
  // four 64-entry chunks per step, all loaded before any is written: an
  // entry only moves to a lower or equal index, so in-place compaction
  // never overwrites an entry that is still to be read
  for (int j0 = 0; j0 < n; j0 += 256) {
    u32 kk[4];
    int32_t pp[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + 64 * u + lane;
      kk[u] = (j < n) ? key[j] : 0u;
      pp[u] = (j < n) ? pos[j] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool ok = j0 + 64 * u + lane < n;
      const bool gt = ok && kk[u] > kstar;
      const bool eq = ok && kk[u] == kstar;
      const uint64_t meq = __ballot(eq);
      const bool take = gt || (eq && eq_seen + lanes_below(meq) < ties);
      const uint64_t mt = __ballot(take);
      const u32 d = taken + lanes_below(mt);
      if (take && d < (u32)k) {
        if (okey != nullptr) okey[d] = kk[u];
        opos[d] = pp[u];
      }
      taken += (u32)__popcll(mt);
      eq_seen += (u32)__popcll(meq);
    }
  }
}

// Staging of one 64-key tile: 4 threads per key row, D_I/4 bytes each.
template <int D_I>
struct TileRegs;
template <>
struct TileRegs<128> {
  v4i a, b;
  __device__ __forceinline__ void load(const uint8_t* src) {
    const v4i* p = reinterpret_cast<const v4i*>(src);
    a = p[0];
    b = p[1];
  }
  __device__ __forceinline__ void store(uint8_t* dst) const {
    v4i* p = reinterpret_cast<v4i*>(dst);
    p[0] = a;
    p[1] = b;
  }
};
template <>
struct TileRegs<64> {
  v4i a;
  __device__ __forceinline__ void load(const uint8_t* src) { a = *reinterpret_cast<const v4i*>(src); }
  __device__ __forceinline__ void store(uint8_t* dst) const { *reinterpret_cast<v4i*>(dst) = a; }
};

// PAGED: the layout, fixed per launch, so the contiguous loop keeps no page
// lookup or layout select.
template <int H_I, int D_I, bool PAGED>
__global__ __launch_bounds__(FT_WAVES * 64, 3) void indexer_topk_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, const float* __restrict__ ks, const int32_t* __restrict__ seq_id,
    const int32_t* __restrict__ pos, Layout lay, int T, int max_len, int k, int cap, int32_t* __restrict__ idx,
    u32* __restrict__ ckey, int32_t* __restrict__ cpos) {
  constexpr int STRIDE = D_I + 16;  // padded LDS row: rotates banks between rows
  constexpr int CPT = D_I / 4;      // staged bytes per thread
  __shared__ __align__(16) uint8_t tile[2][FT_TILE * STRIDE];
  __shared__ u32 hist[FT_WAVES][FT_BINS];
  __shared__ int32_t s_seq[FT_QB], s_pos[FT_QB];

  // the longest rows first (prefill: position grows with the token index)
  const int t0 = (gridDim.x - 1 - blockIdx.x) * FT_QB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  if (tid < FT_QB) {
    const int t = t0 + tid;
    s_seq[tid] = (t < T) ? seq_id[t] : -1;
    s_pos[tid] = (t < T) ? min(pos[t], max_len - 1) : -1;  // clamped to the stated bound
  }
  __syncthreads();

  // this wave's tokens: rows wid*2 + qi of the workgroup
  IndexerQuery<H_I, D_I> qq[FT_QPW];
  int my_seq[FT_QPW], my_pos[FT_QPW], cnt[FT_QPW];
  u32 tau[FT_QPW];
  u32* lkey[FT_QPW];
  int32_t* lpos[FT_QPW];
#pragma unroll
  for (int qi = 0; qi < FT_QPW; ++qi) {
    const int r = wid * FT_QPW + qi;
    const int t = t0 + r;
    my_seq[qi] = s_seq[r];
    my_pos[qi] = s_pos[r];
    if (my_seq[qi] >= 0)
      qq[qi].load(q8, qs, w, t, n, g);
    else
      qq[qi].zero();
    cnt[qi] = 0;
    tau[qi] = 0u;  // accepts every key (the smallest key of a number is above 0)
    const int64_t tt = (t < T) ? t : 0;
    lkey[qi] = ckey + tt * cap;
    lpos[qi] = cpos + tt * cap;
  }
  lds_u32* my_hist = (lds_u32*)&hist[wid][0];

  const int sr = tid >> 2;         // staged key row
  const int sc = (tid & 3) * CPT;  // staged byte offset in the row
  u32 done = 0;
  while (true) {
    // next pass: the sequence of the first token not yet handled
    int seq = -1;
    for (int r = 0; r < FT_QB; ++r)
      if (!((done >> r) & 1u) && s_seq[r] >= 0) {
        seq = s_seq[r];
        break;
      }
    if (seq < 0) break;
    u32 act = 0;
    int pmax = 0;
    for (int r = 0; r < FT_QB; ++r)
      if (!((done >> r) & 1u) && s_seq[r] == seq) {
        act |= 1u << r;
        pmax = max(pmax, s_pos[r]);
      }
    done |= act;
    bool row_on[FT_QPW];
    bool wave_on = false;
#pragma unroll
    for (int qi = 0; qi < FT_QPW; ++qi) {
      row_on[qi] = (act >> (wid * FT_QPW + qi)) & 1u;
      wave_on |= row_on[qi];
    }
    const int ntiles = pmax / FT_TILE + 1;

    // Key tiles load FT_AHEAD tiles ahead into a ring of register stages
    // (stage j holds the next tile of residue j), so the loop body covers
    // FT_AHEAD tiles.  Loads past the last tile re-read it, and tiles past it
    // are computed but never taken (their positions exceed every row's
    // end): every path issues the same loads, so the waits stay partial.
    struct Stage {
      TileRegs<D_I> r;
      float ks;
      int pg;  // physical page of the stage's next tile (paged layout)
    };
    // A tile is one 64-token page when paged.  Each stage looks up the page
    // of its next tile right after issuing its current loads, FT_AHEAD steps
    // before it is needed: loads complete in issue order, so a lookup issued
    // just before its use would make that wait drain every stage.
    const int32_t* pg_src = PAGED ? lay.block_table + (int64_t)seq * lay.max_pages : nullptr;
    auto page = [&](int i) -> int { return PAGED ? pg_src[min(i, ntiles - 1)] : 0; };
    // contiguous: the sequence's first key row and scale; a row within the
    // sequence is a 32-bit byte offset from them (max_len <= 4M, so
    // max_len * D_I < 2^32)
    const uint8_t* k8_seq = k8 + (int64_t)seq * lay.seq_capacity * D_I;
    const float* ks_seq = ks + (int64_t)seq * lay.seq_capacity;
    auto load = [&](Stage& S, int i) {  // S.pg is the page of tile i
      const int base = min(i, ntiles - 1) * FT_TILE;
      if (PAGED) {
        const int64_t row0 = (int64_t)S.pg * 64;
        S.r.load(k8 + (row0 + (min(base + sr, pmax) - base)) * D_I + sc);
        S.ks = ks[row0 + (min(base + lane, pmax) - base)];
        S.pg = page(i + FT_AHEAD);
      } else {
        S.r.load(k8_seq + (u32)(min(base + sr, pmax) * D_I + sc));
        S.ks = *reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(ks_seq) + (u32)(4 * min(base + lane, pmax)));
      }
    };
    float ksv;
    auto step = [&](int i, Stage& S) {  // S holds tile i+1
      if (wave_on) {
        KeyFrag<H_I, D_I> kb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) kb[j].load(&tile[i & 1][(16 * j + n) * STRIDE], g);
        const int s = i * FT_TILE + lane;
#pragma unroll
        for (int qi = 0; qi < FT_QPW; ++qi) {
          if (!row_on[qi]) continue;
          const float res = group_scores<H_I, D_I>(qq[qi], kb);
          const u32 key = order_key(scaled_logit(res, qq[qi].qscale, ksv));
          const bool take = s <= my_pos[qi] && key > tau[qi];
          const uint64_t m = __ballot(take);
          if (m == 0) continue;
          if (take) {  // entry d < cap <= 12288: a 32-bit byte offset from the list bases
            const u32 off = 4u * (u32)(cnt[qi] + (int)lanes_below(m));
            *reinterpret_cast<u32*>(reinterpret_cast<uint8_t*>(lkey[qi]) + off) = key;
            *reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(lpos[qi]) + off) = s;
          }
          cnt[qi] += __popcll(m);
        }
      }
      S.r.store(&tile[(i + 1) & 1][sr * STRIDE + sc]);
      ksv = S.ks;
      load(S, i + 1 + FT_AHEAD);
      __syncthreads();
    };
    Stage s0, s1, s2, s3;
    s0.pg = page(0);
    s1.pg = page(1);
    s2.pg = page(2);
    s3.pg = page(3);
    load(s0, 0);  // tile 0, then its stage's next tile 4 (page looked up by load)
    s0.r.store(&tile[0][sr * STRIDE + sc]);
    ksv = s0.ks;
    load(s1, 1);
    load(s2, 2);
    load(s3, 3);
    load(s0, 4);
    __syncthreads();
    for (int it = 0; it < ntiles; it += FT_AHEAD) {
      step(it + 0, s1);
      step(it + 1, s2);
      step(it + 2, s3);
      step(it + 3, s0);
      // a list compacts once it could not take FT_AHEAD more tiles
#pragma unroll
      for (int qi = 0; qi < FT_QPW; ++qi) {
        if (cnt[qi] > cap - FT_AHEAD * FT_TILE) {
          u32 kstar, ties;
          wave_kth(lkey[qi], cnt[qi], k, my_hist, kstar, ties);
          wave_emit(lkey[qi], lpos[qi], cnt[qi], k, kstar, ties, lkey[qi], lpos[qi]);
          cnt[qi] = k;
          tau[qi] = kstar;
        }
      }
    }
  }

  // final selection of this wave's tokens
#pragma unroll
  for (int qi = 0; qi < FT_QPW; ++qi) {
    if (my_seq[qi] < 0) continue;
    int32_t* out = idx + (int64_t)(t0 + wid * FT_QPW + qi) * k;
    const int c = cnt[qi];
    if (c <= k) {
      wave_sync();
      for (int j = lane; j < k; j += 64) out[j] = (j < c) ? lpos[qi][j] : -1;
    } else {
      u32 kstar, ties;
      wave_kth(lkey[qi], c, k, my_hist, kstar, ties);
      wave_emit(lkey[qi], lpos[qi], c, k, kstar, ties, nullptr, out);
    }
  }
}

// A capacity is a whole number of tiles (fused_topk_cap_from_bytes takes it
// that way from a workspace size), so the minimum k + 320 is rounded up.
int fused_topk_cap(int max_len, int k) {
  int c = ((max_len + FT_TILE - 1) / FT_TILE) * FT_TILE + FT_AHEAD * FT_TILE;  // no compaction needed
  if (c > FT_CAP_MAX) c = FT_CAP_MAX;
  const int min_cap = ((k + (FT_AHEAD + 1) * FT_TILE + FT_TILE - 1) / FT_TILE) * FT_TILE;
  if (c < min_cap) c = min_cap;
  return c;
}

int fused_topk_cap_from_bytes(int T, size_t bytes) {
  if (T <= 0) return FT_CAP_MAX;
  size_t c = bytes / (8 * (size_t)T);  // key + position per slot and token
  if (c > (size_t)FT_CAP_MAX) c = FT_CAP_MAX;
  return (int)(c & ~size_t(FT_TILE - 1));
}

// keys then positions; T * cap * 4 is a multiple of 256 (cap is a multiple of 64)
WsLayout fused_topk_layout(int T, int cap) {
  WsLayout L;
  L.add("ckey", (size_t)T * cap * 4);
  L.add("cpos", (size_t)T * cap * 4);
  return L;
}

size_t fused_topk_workspace_bytes(int T, int cap) { return fused_topk_layout(T, cap).total; }

// a compacted list (k entries) must take FT_AHEAD more tiles before the next
// check, plus one tile of margin
bool fused_topk_cap_ok(int cap, int k) {
  return cap >= k + (FT_AHEAD + 1) * FT_TILE && cap <= FT_CAP_MAX && cap % FT_TILE == 0;
}

template <int H_I, int D_I>
static hipError_t launch_fused_t(int T, int max_len, const uint8_t* q8, const float* qs, const float* w, const uint8_t* k8,
                                 const float* ks, const int32_t* seq_id, const int32_t* pos, const Layout& lay,
                                 int k, int cap, int32_t* idx, void* ws, hipStream_t stream) {
  const WsLayout L = fused_topk_layout(T, cap);
  u32* ckey = static_cast<u32*>(L.at(ws, 0));
  int32_t* cpos = static_cast<int32_t*>(L.at(ws, 1));
  const int blocks = (T + FT_QB - 1) / FT_QB;
  if (lay.paged)
    hipLaunchKernelGGL((indexer_topk_kernel<H_I, D_I, true>), dim3(blocks), dim3(FT_WAVES * 64), 0, stream, q8, qs, w,
                       k8, ks, seq_id, pos, lay, T, max_len, k, cap, idx, ckey, cpos);
  else
    hipLaunchKernelGGL((indexer_topk_kernel<H_I, D_I, false>), dim3(blocks), dim3(FT_WAVES * 64), 0, stream, q8, qs,
                       w, k8, ks, seq_id, pos, lay, T, max_len, k, cap, idx, ckey, cpos);
  return hipGetLastError();
}

hipError_t launch_indexer_topk(int T, int max_len, int H_I, int D_I, const uint8_t* q8, const float* qs, const float* w,
                               const uint8_t* k8, const float* ks, const int32_t* seq_id, const int32_t* pos,
                               const Layout& lay, int k, int cap, int32_t* idx, void* ws, hipStream_t stream) {
  if (T == 0) return hipSuccess;
#define DSA_FT_CASE(HH, DD) \
  if (H_I == HH && D_I == DD) \
    return launch_fused_t<HH, DD>(T, max_len, q8, qs, w, k8, ks, seq_id, pos, lay, k, cap, idx, ws, stream);
  DSA_FT_CASE(64, 128)
  DSA_FT_CASE(64, 64)
  DSA_FT_CASE(4, 128)
  DSA_FT_CASE(4, 64)
#undef DSA_FT_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsa
