// Tile staging shared by the sparse attention kernels (forward and
// backward): a tile is 32 latent rows of 576 bf16 gathered from the cache
// into LDS, the 512 no-rope values of a row stored row-major in padded rows
// and the 64 rope values with their 16-byte chunks XOR-swizzled by row.
// The rows are MLA latent entries shared by every query head ("DeepSeek
// V3.2-Exp Cuts Prolonged-Context Costs With DeepSeek Sparse Consideration
// (DSA)", "Instantiation"), so one staged tile serves all heads of a
// workgroup.
#pragma once

#include "common.h"

namespace dsa {

constexpr int AT_TILE = 32;
constexpr int AT_D = 576;
constexpr int AT_DV = 512;
constexpr int AT_ROW_BYTES = AT_D * 2;              // 1152
constexpr int NOPE_STRIDE = 1040;                   // 1024 B + 16 B: rotates LDS banks per row
constexpr int NOPE_BYTES = AT_TILE * NOPE_STRIDE;   // 33280
constexpr int ROPE_BYTES = AT_TILE * 128;           // 4096
constexpr int BUF_BYTES = NOPE_BYTES + ROPE_BYTES;  // 37376
constexpr int AT_MAX_SPLIT = 2048;                  // rows per split (k <= 2048)
constexpr u32 ROW_INVALID = 0x80000000u;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

// s_waitcnt immediates (gfx9 encoding): at most N vector-memory loads of
// this wave outstanding / every LDS access of this wave done; nothing else
#define DSA_VMCNT(N) (((N) & 0xF) | (((N) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
#define DSA_LGKMCNT0 (0xF | (0x3 << 14) | (0x7 << 4))

// float -> bf16 bits, round to nearest even (gfx950 converts natively)
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses,
// not for its global loads, so the next tile's loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(DSA_LGKMCNT0);
  __builtin_amdgcn_s_barrier();
}

// A tile is 32 rows x 72 chunks of 16 bytes.  With NT threads, TPR = NT/32
// threads share a row: thread tid takes row tid/TPR and chunks tid%TPR + TPR*r.
// Every address is one row base plus an immediate offset; a wave reads whole
// 128-byte lines of 64/TPR rows per load.
template <int NT>
struct TileStage {
  static constexpr int TPR = NT / AT_TILE;
  static constexpr int PER = (72 + TPR - 1) / TPR;
  v4i v[PER];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ kv, const u32* rows, int tid) {
    const int c0 = tid % TPR;
    const u32 phys = rows[tid / TPR] & ~ROW_INVALID;
    const uint8_t* src = kv + (int64_t)phys * AT_ROW_BYTES + 16 * c0;
#pragma unroll
    for (int r = 0; r < PER; ++r)
      if (72 % TPR == 0 || c0 + TPR * r < 72) v[r] = *reinterpret_cast<const v4i*>(src + 16 * TPR * r);
  }
  // no-rope chunks row-major (padded rows); rope chunk cc of row r in slot cc^(r&7)
  __device__ __forceinline__ void store(LDS_AS uint8_t* buf, int tid) const {
    const int row = tid / TPR, c0 = tid % TPR;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int c = c0 + TPR * r;
      if (c < 64)
        *reinterpret_cast<LDS_AS v4i*>(buf + row * NOPE_STRIDE + 16 * c) = v[r];
      else if (c < 72)
        *reinterpret_cast<LDS_AS v4i*>(buf + NOPE_BYTES + row * 128 + 16 * ((c - 64) ^ (row & 7))) = v[r];
    }
  }
};

// Physical rows of n selected entries sel[0..n) of sequence b, compacted in
// order with the padding entries (-1) dropped: s_row[c] for c < nvalid, then
// the tail of the last tile filled with a valid row of the sequence flagged
// ROW_INVALID; s_valid[it] has bit j set when row j of tile it is selected.
// Returns nvalid.  `scan_scratch` holds NT/64 words; the caller issues a
// barrier before reading s_row / s_valid.  `after_first_load` runs once the
// first chunk of sel is requested, so the caller can put its own loads in
// flight beside it: the scan's barriers wait for LDS traffic only, so those
// loads stay outstanding through it.
template <int NT, class F>
__device__ __forceinline__ int compact_selection(const int32_t* __restrict__ sel, int n, const Layout& lay, int b,
                                                 u32* s_row, u32* s_valid, u32* scan_scratch, int tid,
                                                 F&& after_first_load) {
  constexpr int NW = NT / 64;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  int s_next = (tid < n) ? sel[tid] : -1;
  after_first_load();
  int nvalid = 0;
  for (int i0 = 0; i0 < n; i0 += NT) {
    const int s = s_next;
    if (i0 + NT < n) s_next = (i0 + NT + tid < n) ? sel[i0 + NT + tid] : -1;
    const u32 incl = wave_incl_scan(s >= 0 ? 1u : 0u);
    if (lane == 63) scan_scratch[wid] = incl;
    lds_barrier();
    u32 off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const u32 c = scan_scratch[w];
      off += (w < wid) ? c : 0u;
      tot += c;
    }
    lds_barrier();  // scan_scratch is rewritten by the next chunk
    if (s >= 0) s_row[nvalid + (int)(off + incl) - 1] = (u32)token_row(lay, b, s);
    nvalid += (int)tot;
  }
  const int ntiles = (nvalid + AT_TILE - 1) / AT_TILE;
  const u32 safe_row = (u32)token_row(lay, b, 0);
  for (int i = nvalid + tid; i < ntiles * AT_TILE; i += NT) s_row[i] = safe_row | ROW_INVALID;
  for (int it = tid; it < ntiles; it += NT) {
    const int left = nvalid - it * AT_TILE;
    s_valid[it] = left >= AT_TILE ? 0xFFFFFFFFu : ((1u << left) - 1u);
  }
  return nvalid;
}

}  // namespace dsa
