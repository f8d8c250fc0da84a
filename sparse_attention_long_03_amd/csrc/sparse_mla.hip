// Sparse attention under MLA in MQA mode, on gfx950 bf16 matrix cores.
//
// "DeepSeek V3.2-Exp Cuts Prolonged-Context Costs With DeepSeek Sparse
// Consideration (DSA)", part (2): standard attention runs only over the
// selected subset; "Instantiation": MLA in MQA mode, every latent KV row is
// shared by all query heads.  A latent row has 576 bf16 values; the key is
// the whole row, the value its first 512 entries.
//
// Work split.  A workgroup takes one query token, 4 waves of 16 heads each
// and one slice ("split") of the selected rows; the splits are merged by a
// log-sum-exp combine.  A wave holds its heads' O accumulator (512 x 16 fp32
// = 128 registers per lane) and Q operand (72 registers).
//
// Per tile of 32 selected rows:
//   gather   the rows' 16-byte chunks are loaded into registers while the
//            previous tile is computed, then written to the other of two LDS
//            buffers; the 512 no-rope values of a row are stored row-major in
//            padded rows, the 64 rope values with their chunks XOR-swizzled by
//            row, so the score reads avoid LDS bank conflicts;
//   scores   S^T = K Q^T on 16x16x32 bf16 MFMAs: keys on M, the wave's 16
//            heads on N, the 576 dims on K.  A lane ends up holding one head
//            and 8 keys, so the online-softmax max/sum need only two xor
//            steps across the four lane groups;
//   values   O^T += V^T P^T: dims on M (32 tiles of 16), heads on N, keys on
//            K.  V^T comes from the row-major tile through ds_read_b64_tr_b16
//            (the LDS transpose read of gfx950), and P already sits in the
//            B-operand layout, so P never leaves registers.
// The exponentials use exp2 with log2(e) folded into the scale.
#include "attn_tile.h"
#include "launch.h"

namespace dsa {

// Online-softmax reference maximum: P = exp2(z - m_ref) may grow to
// 2^RESCALE_SLACK before O and l are rescaled to a new reference, so the
// accumulator is rescaled only when a head's maximum grows by more than that
// -- a few times per split instead of every tile.  The result is exact: the
// normalisation divides by l accumulated against the same reference.
constexpr float RESCALE_SLACK = 8.f;

// Maximum over the four lanes n, n+16, n+32, n+48 (one head's lane groups).
// The row swaps of gfx950 run on the VALU: a ds_bpermute shuffle counts on
// the LDS counter, and waiting for it also waits for every LDS read issued
// before it.
__device__ __forceinline__ float max_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Scores, online softmax and value product for one tile held in `buf`.
// `valid` has bit j set when row j of the tile is a selected row.
__device__ __forceinline__ void attend_tile(const LDS_AS uint8_t* __restrict__ buf, u32 valid, const v8bf* qf,
                                           float scale_log2, int n, int g, float& m_ref, float& l_part, v4f* o) {
  const LDS_AS uint8_t* nope = buf;
  const LDS_AS uint8_t* rope = buf + NOPE_BYTES;
  // ---- scores S^T (keys x heads): K fragments of keys n and 16+n, dims
  // 32ks + 8g..+8 (no-rope rows for ks < 16, the swizzled rope block after).
  // The reads run SPIPE steps ahead of the MFMAs that use them, in a ring of
  // registers, so LDS latency overlaps the matrix work.
  constexpr int SPIPE = 4;
  auto frag = [&](int ks, int r) -> v8bf {
    if (ks < 16) return *reinterpret_cast<const LDS_AS v8bf*>(nope + r * NOPE_STRIDE + 64 * ks + 16 * g);
    const int c = 4 * (ks - 16) + g;  // rope chunk
    return *reinterpret_cast<const LDS_AS v8bf*>(rope + r * 128 + 16 * (c ^ (r & 7)));
  };
  v8bf ra0[SPIPE], ra1[SPIPE];
#pragma unroll
  for (int j = 0; j < SPIPE; ++j) {
    ra0[j] = frag(j, n);
    ra1[j] = frag(j, 16 + n);
  }
  v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < AT_D / 32; ++ks) {
    const int slot = ks % SPIPE;
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra0[slot], qf[ks], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra1[slot], qf[ks], s1, 0, 0, 0);
    if (ks + SPIPE < AT_D / 32) {
      ra0[slot] = frag(ks + SPIPE, n);
      ra1[slot] = frag(ks + SPIPE, 16 + n);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the ring order
  }
  // lane holds head n: s0[i] -> key 4g+i, s1[i] -> key 16+4g+i
  float z[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z[i] = ((valid >> (4 * g + i)) & 1u) ? s0[i] * scale_log2 : -INFINITY;
    z[4 + i] = ((valid >> (16 + 4 * g + i)) & 1u) ? s1[i] * scale_log2 : -INFINITY;
  }
  float mx = z[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = fmaxf(mx, z[i]);
  mx = max_over_groups(mx);
  // move the reference only when this tile would exceed the slack
  if (__builtin_amdgcn_ballot_w64(mx > m_ref + RESCALE_SLACK) != 0) {
    const float m_new = (mx > m_ref + RESCALE_SLACK) ? mx : m_ref;
    const float corr = (m_ref == -INFINITY) ? 0.f : exp2f(m_ref - m_new);
    l_part *= corr;
#pragma unroll
    for (int mt = 0; mt < AT_DV / 16; ++mt) o[mt] *= corr;
    m_ref = m_new;
  }
  const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
  v8bf pb;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = __builtin_amdgcn_exp2f(z[i] - m_use);  // v_exp_f32; results below 2^-126 flush to 0
    l_part += p;
    pb[i] = (__bf16)p;
  }

  // ---- values O^T += V^T P^T; V^T rows through the LDS transpose read:
  // source lane s of group g points at keys kb + s/4, dims 16mt + 4(s%4)..+3
  const LDS_AS uint8_t* vsrc0 = nope + (4 * g + (n >> 2)) * NOPE_STRIDE + 8 * (n & 3);
  const LDS_AS uint8_t* vsrc1 = vsrc0 + 16 * NOPE_STRIDE;
#pragma unroll
  for (int mt = 0; mt < AT_DV / 16; ++mt) {
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)(vsrc0 + 32 * mt));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)(vsrc1 + 32 * mt));
    const v8bf av = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, o[mt], 0, 0, 0);
    if ((mt & 7) == 7) __builtin_amdgcn_sched_barrier(0);
  }
}

// DENSE = false: the rows are the selected positions idx[t, :], gathered.
// DENSE = true (the masked dense variant): the rows are all positions
// 0..pos[t] of the token's sequence, read in order, and a row counts only if
// its position is among idx[t, :] -- the same set, reached over contiguous
// rows.  Splits then run over positions (at most 2048 per split).
template <int NW, bool DENSE>
__global__ __launch_bounds__(NW * 64) void sparse_mla_kernel(const uint16_t* __restrict__ q,
                                                             const uint8_t* __restrict__ kv,
                                                             const int32_t* __restrict__ idx,
                                                             const int32_t* __restrict__ seq_id,
                                                             const int32_t* __restrict__ pos, Layout lay, int H,
                                                             int k, int split_len, int n_splits, float scale_log2,
                                                             uint16_t* __restrict__ out, float* __restrict__ lse,
                                                             uint16_t* __restrict__ ws_o, float* __restrict__ ws_ml,
                                                             int n_tokens) {
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BUF_BYTES];
  __shared__ u32 s_row[AT_MAX_SPLIT];
  __shared__ u32 s_valid[AT_MAX_SPLIT / AT_TILE];

  // Workgroup -> (token, split, head group).  Workgroups are dealt to the 8
  // XCDs round-robin by linear id; the head groups of one (token, split)
  // take consecutive slots of one XCD, so the second gathers its rows from
  // that XCD's L2 right after the first brought them from HBM.
  const int n_hg = H / (16 * NW) > 0 ? H / (16 * NW) : 1;
  const int lin = blockIdx.x;
  const int xcd = lin & 7;
  const int slot = lin >> 3;
  const int pair = xcd + 8 * (slot / n_hg);  // (token, split) index
  const int hg = slot - (slot / n_hg) * n_hg;
  const int t = pair / n_splits;
  const int split = pair - t * n_splits;
  if (t >= n_tokens) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int n = lane & 15;
  const int g = lane >> 4;
  const int h0 = hg * (16 * NW) + wid * 16;  // first head of this wave
  const bool has_heads = h0 < H;             // waves past H only help stage rows
  const int b = seq_id[t];
  const int32_t* __restrict__ idx_row = idx + (int64_t)t * k;

  const int j_begin = split * split_len;
  const int j_end = DENSE ? min(pos[t] + 1, j_begin + split_len) : min(k, j_begin + split_len);
  const int nrows = max(0, j_end - j_begin);
  int ntiles = (nrows + AT_TILE - 1) / AT_TILE;

  // Q^T operand: head h0+n, dims 32*ks + 8g .. +8 (waves past H read head 0
  // and discard their results: uniform control flow keeps O in registers);
  // requested beside the first selection load
  v8bf qf[AT_D / 32];
  auto load_q = [&] {
    const uint16_t* qrow = q + ((int64_t)t * H + (has_heads ? h0 : 0) + n) * AT_D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < AT_D / 32; ++ks) qf[ks] = *reinterpret_cast<const v8bf*>(qrow + 32 * ks);
  };

  // physical rows of this split (padding and the ragged tail load a valid
  // row of the sequence and are masked), and one validity bit per row
  const int64_t safe_row = token_row(lay, b, 0);
  if (!DENSE) {
    // selected positions, compacted in order (padding entries -1 dropped:
    // rows shorter than k carry many), then the tail of the last tile masked
    __shared__ u32 scan_scratch[NT / 64 + 1];
    const int nvalid =
        compact_selection<NT>(idx_row + j_begin, nrows, lay, b, s_row, s_valid, scan_scratch, tid, load_q);
    ntiles = (nvalid + AT_TILE - 1) / AT_TILE;
  } else {
    load_q();
    for (int i = tid; i < ntiles * AT_TILE; i += NT)
      s_row[i] = (i < nrows) ? (u32)token_row(lay, b, j_begin + i) : ((u32)safe_row | ROW_INVALID);
    for (int i = tid; i < AT_MAX_SPLIT / AT_TILE; i += NT) s_valid[i] = 0;
    __syncthreads();
    for (int j = tid; j < k; j += NT) {
      const int s = idx_row[j];
      if (s >= j_begin && s < j_end) atomicOr(&s_valid[(s - j_begin) >> 5], 1u << ((s - j_begin) & 31));
    }
  }

  float m_ref = -INFINITY;  // reference max (log2 units) of head h0+n
  float l_part = 0.f;       // partial sum over this lane's keys
  v4f o[AT_DV / 16];
#pragma unroll
  for (int mt = 0; mt < AT_DV / 16; ++mt) o[mt] = v4f{0.f, 0.f, 0.f, 0.f};

  LDS_AS uint8_t* lds = (LDS_AS uint8_t*)smem;
  lds_barrier();  // s_row / s_valid visible; the Q loads stay in flight
  // Two tiles in flight: while a tile is computed from one LDS buffer, the
  // next two load into two register stages (A: odd distance, B: even), so the
  // loop runs over pairs of tiles.  Every path issues the same loads -- tiles
  // past the last one re-read it (an L2 hit; a padding tile of an odd count is
  // masked out, contributing exactly nothing) -- so the waits stay partial.
  TileStage<NT> sa, sb;
  auto tile_rows = [&](int i) { return s_row + min(i, ntiles - 1) * AT_TILE; };
  if (ntiles > 0) {
    sa.load(kv, tile_rows(0), tid);
    sa.store(lds, tid);
    sa.load(kv, tile_rows(1), tid);
    sb.load(kv, tile_rows(2), tid);
  }
  // Q and the first tile are in; only the two stages' loads stay outstanding
  __builtin_amdgcn_s_waitcnt(DSA_VMCNT(2 * TileStage<NT>::PER));
  for (int it = 0; it < ntiles; it += 2) {
    lds_barrier();  // tile `it` is in buffer 0; buffer 1 is free
    attend_tile(lds, s_valid[it], qf, scale_log2, n, g, m_ref, l_part, o);
    sa.store(lds + BUF_BYTES, tid);
    sa.load(kv, tile_rows(it + 3), tid);
    lds_barrier();  // tile `it+1` is in buffer 1; buffer 0 is free
    attend_tile(lds + BUF_BYTES, (it + 1 < ntiles) ? s_valid[it + 1] : 0u, qf, scale_log2, n, g, m_ref, l_part, o);
    sb.store(lds, tid);
    sb.load(kv, tile_rows(it + 4), tid);
  }

  if (!has_heads) return;
  // ---- finish: sum l over the four lane groups
  float l = l_part;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  const int h = h0 + n;
  if (n_splits == 1) {
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    uint16_t* orow = out + ((int64_t)t * H + h) * AT_DV + 4 * g;
#pragma unroll
    for (int mt = 0; mt < AT_DV / 16; ++mt) {
      v2i pk;
      pk[0] = (int)((u32)f2bf(o[mt][0] * inv) | ((u32)f2bf(o[mt][1] * inv) << 16));
      pk[1] = (int)((u32)f2bf(o[mt][2] * inv) | ((u32)f2bf(o[mt][3] * inv) << 16));
      *reinterpret_cast<v2i*>(orow + 16 * mt) = pk;
    }
    if (lse != nullptr && g == 0)
      lse[(int64_t)t * H + h] = (l > 0.f) ? (m_ref + log2f(l)) * 0.69314718055994531f : -INFINITY;
  } else {
    // split partial: O normalised by its own l, as bf16 (a convex combination
    // of value rows, so bf16 keeps the range), plus (reference max, l).  The
    // wave's 16 heads x 512 dims are stored in fragment order, [mt/2][lane][8]
    // (tiles mt and mt+1 of a lane side by side), so each store instruction
    // writes 1 KB contiguous.
    const int64_t slot_o = ((int64_t)t * n_splits + split) * H + h;
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    uint16_t* orow = ws_o + (slot_o - n) * AT_DV + 8 * lane;
#pragma unroll
    for (int mp = 0; mp < AT_DV / 32; ++mp) {
      v4i pk;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const v4f& a = o[2 * mp + i];
        pk[2 * i] = (int)((u32)f2bf(a[0] * inv) | ((u32)f2bf(a[1] * inv) << 16));
        pk[2 * i + 1] = (int)((u32)f2bf(a[2] * inv) | ((u32)f2bf(a[3] * inv) << 16));
      }
      *reinterpret_cast<v4i*>(orow + 512 * mp) = pk;
    }
    if (g == 0) {
      ws_ml[slot_o * 2 + 0] = m_ref;
      ws_ml[slot_o * 2 + 1] = l;
    }
  }
}

// Merge the splits: with o_s the normalised partial of split s,
//   O = sum_s w_s o_s / sum_s w_s,   w_s = 2^(m_s - M) l_s,   M = max_s m_s.
// The partials are in the attention kernel's fragment order (per 16 heads:
// [mt/2][lane][8], lane = n + 16g holding head n, dims 16mt + 4g..+3 of tiles
// mt and mt+1), so a wave takes one token, one group of 16 heads and one pair
// of dim tiles with the same lane mapping: each load instruction reads 1 KB
// contiguous of a split.  Each lane derives the split weights of its head.
constexpr int AT_MAX_SPLITS = 8;

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ ws_o,
                                                      const float* __restrict__ ws_ml, int T, int H, int n_splits,
                                                      uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int PAIRS = AT_DV / 32;
  const int n_hg = H / 16;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= T * n_hg * PAIRS) return;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int mp = item % PAIRS;
  const int th = item / PAIRS;
  const int t = th / n_hg;
  const int h = (th - t * n_hg) * 16 + n;
  const int64_t slot0 = (int64_t)t * n_splits * H + h;  // split s: slot0 + s*H

  // the splits' partials, requested first so they overlap the weights below
  const uint16_t* src = ws_o + (slot0 - n) * AT_DV + 8 * lane + 512 * mp;
  const int64_t split_stride = (int64_t)H * AT_DV;
  v4i x[AT_MAX_SPLITS];
#pragma unroll
  for (int sp = 0; sp < AT_MAX_SPLITS; ++sp)
    x[sp] = (sp < n_splits) ? *reinterpret_cast<const v4i*>(src + sp * split_stride) : v4i{0, 0, 0, 0};

  // (reference max, l) of every split of head h; M over the non-empty ones
  float ms[AT_MAX_SPLITS], ls[AT_MAX_SPLITS];
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < AT_MAX_SPLITS; ++sp) {
    ms[sp] = -INFINITY;
    ls[sp] = 0.f;
    if (sp < n_splits) {
      const v2f ml = *reinterpret_cast<const v2f*>(ws_ml + (slot0 + (int64_t)sp * H) * 2);
      ms[sp] = ml[0];
      ls[sp] = ml[1];
    }
    if (ls[sp] > 0.f) M = fmaxf(M, ms[sp]);
  }
  float wgt[AT_MAX_SPLITS];
  float L = 0.f;
#pragma unroll
  for (int sp = 0; sp < AT_MAX_SPLITS; ++sp) {
    wgt[sp] = (ls[sp] > 0.f) ? exp2f(ms[sp] - M) * ls[sp] : 0.f;
    L += wgt[sp];
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < AT_MAX_SPLITS; ++sp) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += wgt[sp] * __uint_as_float((u32)x[sp][i] << 16);
      acc[2 * i + 1] += wgt[sp] * __uint_as_float((u32)x[sp][i] & 0xFFFF0000u);
    }
  }
  uint16_t* orow = out + ((int64_t)t * H + h) * AT_DV + 4 * g + 32 * mp;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    v2i pk;
    pk[0] = (int)((u32)f2bf(acc[4 * i] * inv) | ((u32)f2bf(acc[4 * i + 1] * inv) << 16));
    pk[1] = (int)((u32)f2bf(acc[4 * i + 2] * inv) | ((u32)f2bf(acc[4 * i + 3] * inv) << 16));
    *reinterpret_cast<v2i*>(orow + 16 * i) = pk;
  }
  if (lse != nullptr && mp == 0 && g == 0)
    lse[(int64_t)t * H + h] = (L > 0.f) ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

bool attn_supported(int H) { return H == 16 || H == 32 || H == 64 || H == 128; }

// waves per workgroup: 4 (64 heads; 128 heads take two workgroups, and with
// fewer heads the spare waves only stage rows).  Eight waves covering all 128
// heads do not fit: their prefetch registers spill.
static int attn_waves(int H) { return 4; }
static int head_groups(int H) { return H > 16 * attn_waves(H) ? H / (16 * attn_waves(H)) : 1; }

int attn_splits(int T, int H, int k) {
  const int base = T * head_groups(H);
  const int tiles = (k + AT_TILE - 1) / AT_TILE;
  int s = 1;
  // keep >= 4 tiles per split; stop once the grid reaches 256 workgroups
  while (base * s < 256 && tiles / (2 * s) >= 4 && 2 * s <= AT_MAX_SPLITS) s *= 2;
  return s;
}

// masked dense variant: splits over positions, at most AT_MAX_SPLIT each
static int dense_splits(int T, int H, int max_len) {
  const int tiles = (max_len + AT_TILE - 1) / AT_TILE;
  int s = 1;
  while (s * AT_MAX_SPLIT < max_len) s *= 2;
  while (T * head_groups(H) * s < 256 && tiles / (2 * s) >= 4 && 2 * s <= AT_MAX_SPLITS) s *= 2;
  return s;
}

bool dense_attn_supported(int max_len) { return max_len <= AT_MAX_SPLITS * AT_MAX_SPLIT; }

// split partials (bf16, normalised) and their (max, sum) pairs; none with one split
static WsLayout split_layout(int T, int H, int s) {
  WsLayout L;
  if (s == 1) return L;
  const size_t slots = (size_t)T * s * H;
  L.add("o", slots * AT_DV * 2);
  L.add("ml", slots * 2 * 4);
  return L;
}

WsLayout attn_layout(int T, int H, int k) { return split_layout(T, H, attn_splits(T, H, k)); }
WsLayout dense_attn_layout(int T, int H, int max_len) { return split_layout(T, H, dense_splits(T, H, max_len)); }
size_t attn_workspace_bytes(int T, int H, int k) { return attn_layout(T, H, k).total; }
size_t dense_attn_workspace_bytes(int T, int H, int max_len) { return dense_attn_layout(T, H, max_len).total; }

template <bool DENSE>
static hipError_t launch_attn_t(int T, int H, const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                                const int32_t* seq_id, const int32_t* pos, const Layout& lay, int k, int max_len,
                                float sm_scale, uint16_t* out, float* lse, void* ws, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int n_hg = head_groups(H);
  const int n_splits = DENSE ? dense_splits(T, H, max_len) : attn_splits(T, H, k);
  const int span = DENSE ? max_len : k;
  const int tiles = (span + AT_TILE - 1) / AT_TILE;
  const int split_len = ((tiles + n_splits - 1) / n_splits) * AT_TILE;
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  uint16_t* ws_o = nullptr;
  float* ws_ml = nullptr;
  if (n_splits > 1) {
    const WsLayout L = split_layout(T, H, n_splits);
    ws_o = static_cast<uint16_t*>(L.at(ws, 0));
    ws_ml = static_cast<float*>(L.at(ws, 1));
  }
  // (token, split) pairs rounded up to a multiple of 8 (one per XCD per slot)
  const int pairs = T * n_splits;
  const int blocks = ((pairs + 7) / 8) * 8 * n_hg;
  const uint8_t* kvb = reinterpret_cast<const uint8_t*>(kv);
  hipLaunchKernelGGL((sparse_mla_kernel<4, DENSE>), dim3(blocks), dim3(4 * 64), 0, stream, q, kvb, idx, seq_id, pos,
                     lay, H, k, split_len, n_splits, scale_log2, out, lse, ws_o, ws_ml, T);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_splits == 1) return e;
  const int waves = T * (H / 16) * (AT_DV / 32);
  hipLaunchKernelGGL(combine_kernel, dim3((waves + 3) / 4), dim3(256), 0, stream, ws_o, ws_ml, T, H, n_splits, out,
                     lse);
  return hipGetLastError();
}

hipError_t launch_attn(int T, int H, const uint16_t* q, const uint16_t* kv, const int32_t* idx, const int32_t* seq_id,
                       const Layout& lay, int k, float sm_scale, uint16_t* out, float* lse, void* ws,
                       hipStream_t stream) {
  return launch_attn_t<false>(T, H, q, kv, idx, seq_id, nullptr, lay, k, 0, sm_scale, out, lse, ws, stream);
}

hipError_t launch_dense_attn(int T, int H, const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                             const int32_t* seq_id, const int32_t* pos, const Layout& lay, int k, int max_len,
                             float sm_scale, uint16_t* out, float* lse, void* ws, hipStream_t stream) {
  return launch_attn_t<true>(T, H, q, kv, idx, seq_id, pos, lay, k, max_len, sm_scale, out, lse, ws, stream);
}

}  // namespace dsa
