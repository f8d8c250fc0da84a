// Lightning indexer logits on gfx950 FP8 matrix cores.
//
// "DeepSeek V3.2-Exp Cuts Prolonged-Context Costs With DeepSeek Sparse
// Consideration (DSA)", part (1).  The per-tile arithmetic (heads on the MFMA
// M side, keys on N, ReLU and head weights in registers) lives in
// indexer_math.h; this kernel streams the keys and writes the logits.
//
// Decode is bound by HBM (one 128-byte key row feeds 64 heads x 128 MACs =
// 128 flop/byte, far under the FP8 ridge), so the kernel streams keys with
// wide loads and keeps an 8 KB group per wave in flight.
//
// Key loads cover whole 128-byte lines.  An MFMA fragment wants 16 key rows
// across 16 lanes, each lane 32 contiguous bytes of its row, which no single
// load instruction can fill with whole lines; so each wave writes its group
// into its own LDS slab and reads the fragments back from there.  (Loading
// fragments straight from HBM reads each line in two halves through two
// instructions.)  On a contiguous cache the loads are nontemporal; on a paged
// one, where every group is a separately placed page, they are plain: on one
// MI355X the streaming hint takes the 128K contiguous decode from 57.7 to
// 50.6 us but the paged ragged batch from 270 to 320 us.
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

#ifndef LDS_AS
#define LDS_AS __attribute__((address_space(3)))
#endif

// One 64-key group on its way from HBM to MFMA fragments.  Lane l of load
// instruction i takes 16-byte chunk l % CPR of row RPI*i + l / CPR, so an
// instruction covers RPI whole rows.  In the wave's LDS slab, chunk c of row r
// sits at slot c ^ swz(r) of the row: the 16 rows a fragment read touches then
// fall on 16 distinct bank groups, and a row still fills its own bytes.
template <int H_I, int D_I>
struct GroupStage {
  static constexpr int CPR = D_I / 16;  // 16-byte chunks per row (8 or 4)
  static constexpr int RPI = 64 / CPR;  // rows per load instruction (8 or 16)
  static constexpr int NI = 64 / RPI;   // load instructions per group (8 or 4)
  v4i v[NI];

  __device__ __forceinline__ static int swz(int r) { return D_I == 128 ? (r >> 1) & 7 : (r >> 2) & 3; }

  // rows base..base+63 of a group whose first row is at grp; rows past p
  // read p.  STREAM: nontemporal loads.
  template <bool STREAM>
  __device__ __forceinline__ void load(const uint8_t* __restrict__ grp, int base, int p, int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = RPI * i + lane / CPR;
      const int sp = min(base + r, p);
      const v4i* src = reinterpret_cast<const v4i*>(grp + (u32)(sp - base) * D_I + 16 * (lane % CPR));
      v[i] = STREAM ? __builtin_nontemporal_load(src) : *src;
    }
  }
  __device__ __forceinline__ void store(LDS_AS uint8_t* slab, int lane) const {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = RPI * i + lane / CPR;
      *reinterpret_cast<LDS_AS v4i*>(slab + r * D_I + 16 * ((lane % CPR) ^ swz(r))) = v[i];
    }
  }
  // the fragment of key tile j for lane (n, g): row 16j + n, bytes of lane group g
  __device__ __forceinline__ static KeyFrag<H_I, D_I> frag(const LDS_AS uint8_t* slab, int j, int n, int g) {
    const int r = 16 * j + n;
    const LDS_AS uint8_t* row = slab + r * D_I;
    KeyFrag<H_I, D_I> f;
    if constexpr (D_I == 128) {
      const v4i a = *reinterpret_cast<const LDS_AS v4i*>(row + 16 * ((2 * g) ^ swz(r)));
      const v4i b = *reinterpret_cast<const LDS_AS v4i*>(row + 16 * ((2 * g + 1) ^ swz(r)));
      f.v = v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
      f.v = *reinterpret_cast<const LDS_AS v4i*>(row + 16 * (g ^ swz(r)));
    }
    return f;
  }
};

template <int H_I, int D_I, bool STREAM>
__global__ __launch_bounds__(IDX_WAVES * 64) void indexer_kernel(const uint8_t* __restrict__ q8,
                                                                 const float* __restrict__ qs,
                                                                 const float* __restrict__ w,
                                                                 const uint8_t* __restrict__ k8,
                                                                 const float* __restrict__ ks,
                                                                 const int32_t* __restrict__ seq_id,
                                                                 const int32_t* __restrict__ pos, Layout lay,
                                                                 float* __restrict__ logits, int64_t ld,
                                                                 u32* __restrict__ hist, int max_len) {
  __shared__ __attribute__((aligned(16))) uint8_t slabs[IDX_WAVES][64 * D_I];
  __shared__ u32 h_lds[2048];
  using Stage = GroupStage<H_I, D_I>;

  const int t = blockIdx.y;
  // a position past the stated bound is taken as the last one it allows, so
  // no store leaves the row or the launched grid
  const int p = min(pos[t], max_len - 1);
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
  // path.  The next group's loads are issued as soon as the current group is
  // in the slab, and stay in flight while it is reduced.
  const int first = wg_base + wid * 64;
  const int last_group = p & ~63;  // 64-aligned group holding position p
  LDS_AS uint8_t* slab = (LDS_AS uint8_t*)&slabs[wid][0];
  Stage st;
  float ksr;
  auto issue = [&](int it) {
    const int base = min(first + it * IDX_WAVES * 64, last_group);  // one page when paged
    const int64_t row0 = token_row(lay, b, base);
    st.template load<STREAM>(k8 + row0 * D_I, base, p, lane);
    ksr = ks[row0 + (min(base + lane, p) - base)];
  };
  issue(0);
#pragma unroll
  for (int it = 0; it < IDX_ITERS; ++it) {
    st.store(slab, lane);  // the wave's own slab: LDS accesses of one wave stay in order
    const float ksv = ksr;
    if (it + 1 < IDX_ITERS) issue(it + 1);
    KeyFrag<H_I, D_I> kb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kb[j] = Stage::frag(slab, j, n, g);
    const int base = first + it * IDX_WAVES * 64;
    const int s_me = base + lane;
    const float res = group_scores<H_I, D_I>(qq, kb);
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
  if (lay.paged)
    hipLaunchKernelGGL((indexer_kernel<H_I, D_I, false>), grid, dim3(IDX_WAVES * 64), 0, stream, q8, qs, w, k8, ks,
                       seq_id, pos, lay, logits, ld, hist, max_len);
  else
    hipLaunchKernelGGL((indexer_kernel<H_I, D_I, true>), grid, dim3(IDX_WAVES * 64), 0, stream, q8, qs, w, k8, ks,
                       seq_id, pos, lay, logits, ld, hist, max_len);
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
