// Sparse attention under MLA in MQA mode, on gfx950 bf16 matrix cores.
//
// "DeepSeek V3.2-Exp Cuts Prolonged-Context Costs With DeepSeek Sparse
// Consideration (DSA)", part (2): standard attention runs only over the
// selected subset; "Instantiation": MLA in MQA mode, every latent KV row is
// shared by all query heads.  A latent row has 576 bf16 values; the key is
// the whole row, the value its first 512 entries.
//
// Work split.  A workgroup takes one query token, 4 waves of 16 heads each
// (two head groups cover 128 heads; with fewer than 64 heads the spare waves
// only help stage rows) and one slice ("split") of the selected rows; the
// splits are merged afterwards by a log-sum-exp combine.  The O accumulator
// of a wave's 16 heads is 512 x 16 fp32 (128 registers per lane) and its Q
// operand 72 registers, so one wave per SIMD holds them with room for the
// staged next tile.
//
// Per tile of 32 selected rows:
//   gather   the rows' 16-byte chunks are loaded into registers while the
//            previous tile is computed, then written to the other of two LDS
//            buffers (double buffering); the 512 no-rope values of a row are
//            stored row-major with padded rows, the 64 rope values with their
//            chunks XOR-swizzled by row, so the score reads avoid LDS bank
//            conflicts;
//   scores   S^T = K Q^T on 16x16x32 bf16 MFMAs: keys on M, the wave's 16
//            heads on N, the 576 dims on K.  A lane ends up holding one head
//            and 8 keys, so the online-softmax max/sum need only two xor
//            steps across the four lane groups;
//   values   O^T += V^T P^T: dims on M (32 tiles of 16), heads on N, keys on
//            K.  V^T comes from the row-major tile through ds_read_b64_tr_b16
//            (the LDS transpose read of gfx950), and P already sits in the
//            B-operand layout, so P never leaves registers and the per-head
//            rescale of O is in-lane.
// The exponentials use exp2 with log2(e) folded into the scale.
#include "launch.h"

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
#define LDS_AS __attribute__((address_space(3)))

__device__ __forceinline__ uint16_t f2bf(float f) {
  // round to nearest even (inputs here are finite)
  u32 u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// waits for every LDS access of this wave, and for nothing else
#define DSA_LGKMCNT0 (0xF | (0x3 << 14) | (0x7 << 4))

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses,
// not for its global loads, so the next tile's loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(DSA_LGKMCNT0);
  __builtin_amdgcn_s_barrier();
}

// A tile is 32 rows x 72 chunks of 16 bytes.  Thread tid stages chunks
// tid + NT*r: consecutive threads read consecutive chunks of a row.
template <int NT>
struct TileStage {
  static constexpr int CHUNKS = AT_TILE * 72;
  static constexpr int PER_THREAD = (CHUNKS + NT - 1) / NT;
  v4i v[PER_THREAD];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ kv, const u32* rows, int tid) {
#pragma unroll
    for (int r = 0; r < PER_THREAD; ++r) {
      const int c = tid + NT * r;
      if (CHUNKS % NT == 0 || c < CHUNKS) {
        const int row = c / 72, col = c - row * 72;
        const u32 phys = rows[row] & ~ROW_INVALID;
        v[r] = *reinterpret_cast<const v4i*>(kv + (int64_t)phys * AT_ROW_BYTES + 16 * col);
      }
    }
  }
  // no-rope chunks row-major (padded rows); rope chunk cc of row r in slot cc^(r&7)
  __device__ __forceinline__ void store(LDS_AS uint8_t* buf, int tid) const {
#pragma unroll
    for (int r = 0; r < PER_THREAD; ++r) {
      const int c = tid + NT * r;
      if (CHUNKS % NT == 0 || c < CHUNKS) {
        const int row = c / 72, col = c - row * 72;
        LDS_AS uint8_t* dst = (col < 64) ? buf + row * NOPE_STRIDE + 16 * col
                                         : buf + NOPE_BYTES + row * 128 + 16 * ((col - 64) ^ (row & 7));
        *reinterpret_cast<LDS_AS v4i*>(dst) = v[r];
      }
    }
  }
};

// Scores, online softmax and value product for one tile held in `buf`.
__device__ __forceinline__ void attend_tile(const LDS_AS uint8_t* __restrict__ buf, const u32* rows, const v8bf* qf,
                                           float scale_log2, int n, int g, float& m_run, float& l_part, v4f* o) {
  const LDS_AS uint8_t* nope = buf;
  const LDS_AS uint8_t* rope = buf + NOPE_BYTES;
  // ---- scores S^T (keys x heads)
  v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const v8bf a0 = *reinterpret_cast<const LDS_AS v8bf*>(nope + n * NOPE_STRIDE + 64 * ks + 16 * g);
    const v8bf a1 = *reinterpret_cast<const LDS_AS v8bf*>(nope + (16 + n) * NOPE_STRIDE + 64 * ks + 16 * g);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ks], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ks], s1, 0, 0, 0);
    if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int ks = 16; ks < 18; ++ks) {
    const int c = 4 * (ks - 16) + g;  // rope chunk
    const int r0 = n, r1 = 16 + n;
    const v8bf a0 = *reinterpret_cast<const LDS_AS v8bf*>(rope + r0 * 128 + 16 * (c ^ (r0 & 7)));
    const v8bf a1 = *reinterpret_cast<const LDS_AS v8bf*>(rope + r1 * 128 + 16 * (c ^ (r1 & 7)));
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ks], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ks], s1, 0, 0, 0);
  }
  // lane holds head n: s0[i] -> key 4g+i, s1[i] -> key 16+4g+i
  float z[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z[i] = (rows[4 * g + i] & ROW_INVALID) ? -INFINITY : s0[i] * scale_log2;
    z[4 + i] = (rows[16 + 4 * g + i] & ROW_INVALID) ? -INFINITY : s1[i] * scale_log2;
  }
  float mx = z[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = fmaxf(mx, z[i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float m_new = fmaxf(m_run, mx);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float corr = exp2f(m_run - m_use);
  float psum = 0.f;
  float pz[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    pz[i] = exp2f(z[i] - m_use);
    psum += pz[i];
  }
  l_part = l_part * corr + psum;
  m_run = m_new;
  v8bf pb;
#pragma unroll
  for (int i = 0; i < 8; ++i) pb[i] = __builtin_bit_cast(__bf16, f2bf(pz[i]));

  // ---- values O^T += V^T P^T; V^T rows through the LDS transpose read:
  // source lane s of group g points at keys kb + s/4, dims 16mt + 4(s%4)..+3
  const LDS_AS uint8_t* vsrc0 = nope + (4 * g + (n >> 2)) * NOPE_STRIDE + 8 * (n & 3);
  const LDS_AS uint8_t* vsrc1 = vsrc0 + 16 * NOPE_STRIDE;
#pragma unroll
  for (int mt = 0; mt < AT_DV / 16; ++mt) {
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)(vsrc0 + 32 * mt));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)(vsrc1 + 32 * mt));
    const v8bf av = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    v4f acc = o[mt] * corr;
    o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, acc, 0, 0, 0);
    // bound the read-ahead of the transpose reads (register pressure)
    if ((mt & 7) == 7) __builtin_amdgcn_sched_barrier(0);
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void sparse_mla_kernel(const uint16_t* __restrict__ q,
                                                             const uint8_t* __restrict__ kv,
                                                             const int32_t* __restrict__ idx,
                                                             const int32_t* __restrict__ seq_id, Layout lay, int H,
                                                             int k, int split_len, int n_splits, float scale_log2,
                                                             uint16_t* __restrict__ out, float* __restrict__ lse,
                                                             float* __restrict__ ws_o, float* __restrict__ ws_ml,
                                                             int n_tokens) {
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BUF_BYTES];
  __shared__ u32 s_row[AT_MAX_SPLIT];

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
  const int j_end = min(k, j_begin + split_len);
  const int nrows = max(0, j_end - j_begin);
  const int ntiles = (nrows + AT_TILE - 1) / AT_TILE;

  // physical rows of this split (padding and the ragged tail load a valid
  // row of the sequence and are masked)
  const int64_t safe_row = token_row(lay, b, 0);
  for (int i = tid; i < ntiles * AT_TILE; i += NT) {
    const int j = j_begin + i;
    const int s = (i < nrows) ? idx_row[j] : -1;
    s_row[i] = (s >= 0) ? (u32)token_row(lay, b, s) : ((u32)safe_row | ROW_INVALID);
  }

  // Q^T operand: head h0+n, dims 32*ks + 8g .. +8
  v8bf qf[AT_D / 32];
  {
    const uint16_t* qrow = q + ((int64_t)t * H + (has_heads ? h0 : 0) + n) * AT_D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < AT_D / 32; ++ks) qf[ks] = *reinterpret_cast<const v8bf*>(qrow + 32 * ks);
  }
  float m_run = -INFINITY;  // running max (log2 units) of head h0+n
  float l_part = 0.f;       // partial sum over this lane's keys
  v4f o[AT_DV / 16];
#pragma unroll
  for (int mt = 0; mt < AT_DV / 16; ++mt) o[mt] = v4f{0.f, 0.f, 0.f, 0.f};

  LDS_AS uint8_t* lds = (LDS_AS uint8_t*)smem;
  __syncthreads();  // s_row visible
  TileStage<NT> stage;
  if (ntiles > 0) {
    stage.load(kv, s_row, tid);
    stage.store(lds, tid);
  }
  for (int it = 0; it < ntiles; ++it) {
    LDS_AS uint8_t* cur = lds + (it & 1) * BUF_BYTES;
    const bool more = it + 1 < ntiles;
    if (more) stage.load(kv, s_row + (it + 1) * AT_TILE, tid);  // in flight during this tile
    lds_barrier();  // tile `it` is in `cur`; the other buffer is free
    // waves without heads compute on head 0's query and discard the result:
    // uniform control flow keeps the accumulators in registers
    attend_tile(cur, s_row + it * AT_TILE, qf, scale_log2, n, g, m_run, l_part, o);
    if (more) stage.store(lds + ((it + 1) & 1) * BUF_BYTES, tid);
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
      lse[(int64_t)t * H + h] = (l > 0.f) ? (m_run + log2f(l)) * 0.69314718055994531f : -INFINITY;
  } else {
    const int64_t slot = ((int64_t)t * n_splits + split) * H + h;
    float* orow = ws_o + slot * AT_DV + 4 * g;
#pragma unroll
    for (int mt = 0; mt < AT_DV / 16; ++mt) *reinterpret_cast<v4f*>(orow + 16 * mt) = o[mt];
    if (g == 0) {
      ws_ml[slot * 2 + 0] = m_run;
      ws_ml[slot * 2 + 1] = l;
    }
  }
}

// Merge the splits: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// One wave per (token, head); each lane owns 8 of the 512 value dims.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
                                                      int TH, int H, int n_splits, uint16_t* __restrict__ out,
                                                      float* __restrict__ lse) {
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= TH) return;
  const int lane = threadIdx.x & 63;
  const int t = item / H;
  const int h = item - t * H;
  float M = -INFINITY;
  for (int s = 0; s < n_splits; ++s) {
    const int64_t slot = ((int64_t)t * n_splits + s) * H + h;
    if (ws_ml[slot * 2 + 1] > 0.f) M = fmaxf(M, ws_ml[slot * 2]);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int s = 0; s < n_splits; ++s) {
    const int64_t slot = ((int64_t)t * n_splits + s) * H + h;
    const float ls = ws_ml[slot * 2 + 1];
    if (!(ls > 0.f)) continue;
    const float wgt = exp2f(ws_ml[slot * 2] - M);
    L += wgt * ls;
    const v4f* src = reinterpret_cast<const v4f*>(ws_o + slot * AT_DV + 8 * lane);
    const v4f x0 = src[0], x1 = src[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] += wgt * x0[i];
      acc[4 + i] += wgt * x1[i];
    }
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  v4i pk;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    pk[i] = (int)((u32)f2bf(acc[2 * i] * inv) | ((u32)f2bf(acc[2 * i + 1] * inv) << 16));
  *reinterpret_cast<v4i*>(out + ((int64_t)t * H + h) * AT_DV + 8 * lane) = pk;
  if (lse != nullptr && lane == 0)
    lse[(int64_t)t * H + h] = (L > 0.f) ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

bool attn_supported(int H) { return H == 16 || H == 32 || H == 64 || H == 128; }

constexpr int AT_NW = 4;  // 4 waves x 16 heads per workgroup

static int head_groups(int H) { return H > 16 * AT_NW ? H / (16 * AT_NW) : 1; }

int attn_splits(int T, int H, int k) {
  const int base = T * head_groups(H);
  const int tiles = (k + AT_TILE - 1) / AT_TILE;
  int s = 1;
  // keep >= 4 tiles per split; stop once the grid reaches 256 workgroups
  while (base * s < 256 && tiles / (2 * s) >= 4) s *= 2;
  return s;
}

size_t attn_workspace_bytes(int T, int H, int k) {
  const int s = attn_splits(T, H, k);
  if (s == 1) return 0;
  const size_t slots = (size_t)T * s * H;
  return align256(slots * AT_DV * 4) + align256(slots * 2 * 4);
}

hipError_t launch_attn(int T, int H, const uint16_t* q, const uint16_t* kv, const int32_t* idx, const int32_t* seq_id,
                       const Layout& lay, int k, float sm_scale, uint16_t* out, float* lse, void* ws,
                       hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int n_hg = head_groups(H);
  const int n_splits = attn_splits(T, H, k);
  const int tiles = (k + AT_TILE - 1) / AT_TILE;
  const int split_len = ((tiles + n_splits - 1) / n_splits) * AT_TILE;
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  float* ws_o = nullptr;
  float* ws_ml = nullptr;
  if (n_splits > 1) {
    const size_t slots = (size_t)T * n_splits * H;
    ws_o = reinterpret_cast<float*>(ws);
    ws_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + align256(slots * AT_DV * 4));
  }
  // (token, split) pairs rounded up to a multiple of 8 (one per XCD per slot)
  const int pairs = T * n_splits;
  const int blocks = ((pairs + 7) / 8) * 8 * n_hg;
  hipLaunchKernelGGL((sparse_mla_kernel<AT_NW>), dim3(blocks), dim3(AT_NW * 64), 0, stream, q,
                     reinterpret_cast<const uint8_t*>(kv), idx, seq_id, lay, H, k, split_len, n_splits, scale_log2,
                     out, lse, ws_o, ws_ml, T);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_splits == 1) return e;
  const int TH = T * H;
  hipLaunchKernelGGL(combine_kernel, dim3((TH + 3) / 4), dim3(256), 0, stream, ws_o, ws_ml, TH, H, n_splits, out, lse);
  return hipGetLastError();
}

}  // namespace dsa
