// The indexer's training signal: KL divergence to the attention distribution.
//
// "DeepSeek V3.2-Exp Cuts Prolonged-Context Costs With DeepSeek Sparse
// Consideration (DSA)", "Teaching signal": the indexer learns to imitate the
// main attention's head-summed distribution through a KL divergence, the
// target taking no gradient.  Over the selected entries j of query t (the
// sparse stage; the dense warm-up is the same with every position selected):
//   target  p[t,j] = (1/H) sum_h exp(z[t,h,j] - lse[t,h])   (kl_target_kernel)
//   indexer q[t,j] = softmax_j I[t, idx[t,j]]
//   loss    L_t = sum_j p (log p - log q),   dL/dI = q - p
// and back through I = sum_h w_h ReLU(qd_h . kd_j) (qd = qs * q8, kd = ks * k8,
// the FP8 quantisation taken as the identity):
//   dw_h  = sum_j dI_j ReLU(qd_h . kd_j)
//   dqd_h = w_h sum_j dI_j [qd_h . kd_j > 0] kd_j
//   dkd_j = dI_j sum_h w_h [qd_h . kd_j > 0] qd_h      (added per cache row)
#include "attn_tile.h"
#include "indexer_math.h"
#include "launch.h"

namespace dsa {


namespace {
constexpr u32 SLOT_NONE = 0xFFFFFFFFu;
constexpr float LOG2E = 1.4426950408889634f;
}  // namespace

// ---------------------------------------------------------------------------
// target: head-mean attention probability of each selected entry
// ---------------------------------------------------------------------------

// Workgroup = one query token, 8 waves of 16 heads (waves past H only stage
// rows).  The selection is taken in its own order (entry j of idx[t, :] is
// slot j; padding entries load a valid row and are masked), 32 entries per
// tile, through the forward's gather pipeline.  Per tile a wave forms
// S^T = K Q^T for its heads, P = exp(z - lse), and sums P over its 16 heads
// with four xor steps; the waves' sums meet in LDS and the next tile's first
// 32 threads write their total / H.
//
// The dense warm-up (every position 0..pos[t] of the sequence) runs the same
// tile loop over contiguous positions, split into chunks of up to 2048 per
// workgroup (blockIdx.y), in two launches:
//   KT_DENSE_LSE     per chunk and head, the running maximum m (log2 units)
//                    and the sum l of exp2(z - m) over the chunk's positions;
//   KT_DENSE_TARGET  every lane first merges the chunks' (m, l) of its head
//                    into the dense lse (the warm-up's attention runs over
//                    every position), then the target of each position.
// When the caller has the dense lse already (the warm-up's dense attention
// forward returns it), KT_DENSE_GIVEN takes it as input and runs the second
// launch alone: every row is read once instead of twice.
constexpr int KT_NW = 8;
enum KtMode { KT_SELECTED = 0, KT_DENSE_LSE = 1, KT_DENSE_TARGET = 2, KT_DENSE_GIVEN = 3 };

// Sum over the 16 lanes of each row of the wave (every lane ends with its
// row's sum): row rotations by 8, 4, 2 and 1 lanes.
__device__ __forceinline__ float row_sum16(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror:8
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror:4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false));  // row_ror:2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false));  // row_ror:1
  return v;
}

template <int MODE>
__global__ __launch_bounds__(KT_NW * 64) void kl_target_kernel(const uint16_t* __restrict__ q,
                                                             const uint8_t* __restrict__ kv,
                                                             const int32_t* __restrict__ idx,
                                                             const int32_t* __restrict__ seq_id,
                                                             const int32_t* __restrict__ pos, Layout lay, int H,
                                                             int k, float scale_log2, const float* __restrict__ lse,
                                                             float* __restrict__ target, int64_t ld_target,
                                                             float* __restrict__ ml, int n_chunks,
                                                             float* __restrict__ lse_out, int n_tokens) {
  constexpr bool DENSE = MODE != KT_SELECTED;
  constexpr int NT = KT_NW * 64;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BUF_BYTES];
  __shared__ u32 s_row[AT_MAX_SPLIT];
  __shared__ u32 s_valid[AT_MAX_SPLIT / AT_TILE];
  __shared__ float s_part[2][KT_NW][AT_TILE];
  const int t = blockIdx.x;
  if (t >= n_tokens) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int h0 = wid * 16;
  const bool has_heads = h0 < H;
  const int nw_heads = H / 16;
  const int b = seq_id[t];
  const int32_t* __restrict__ idx_row = DENSE ? nullptr : idx + (int64_t)t * k;
  // the entries of this workgroup: the selection, or one chunk of positions
  const int j_begin = DENSE ? blockIdx.y * AT_MAX_SPLIT : 0;
  const int n_ent = DENSE ? min(pos[t] + 1 - j_begin, AT_MAX_SPLIT) : k;
  if (n_ent <= 0) return;  // (dense) the chunk lies past the query's position
  const int ntiles = (n_ent + AT_TILE - 1) / AT_TILE;

  const u32 safe_row = (u32)token_row(lay, b, 0);
  for (int i = tid; i < ntiles * AT_TILE; i += NT) {
    int s;
    if constexpr (DENSE)
      s = (i < n_ent) ? j_begin + i : -1;
    else
      s = (i < k) ? idx_row[i] : -1;
    s_row[i] = (s >= 0) ? (u32)token_row(lay, b, s) : (safe_row | ROW_INVALID);
  }
  __syncthreads();
  for (int it = tid; it < ntiles; it += NT) {
    u32 m = 0;
    for (int r = 0; r < AT_TILE; ++r) m |= ((s_row[it * AT_TILE + r] & ROW_INVALID) ? 0u : 1u) << r;
    s_valid[it] = m;
  }

  const int hq = (has_heads ? h0 : 0) + n;
  v8bf qf[AT_D / 32];
  {
    const uint16_t* qrow = q + ((int64_t)t * H + hq) * AT_D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < AT_D / 32; ++ks) qf[ks] = *reinterpret_cast<const v8bf*>(qrow + 32 * ks);
  }
  // lse of head hq in log2 units: given (the forward's), or merged from the
  // dense chunks' (m, l)
  float lse2 = 0.f;
  if constexpr (MODE == KT_SELECTED || MODE == KT_DENSE_GIVEN) {
    lse2 = lse[(int64_t)t * H + hq] * LOG2E;
  } else if constexpr (MODE == KT_DENSE_TARGET) {
    const int nch = min(n_chunks, (pos[t] + AT_MAX_SPLIT) / AT_MAX_SPLIT);
    const float* mlq = ml + ((int64_t)t * n_chunks * H + hq) * 2;
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, mlq[(int64_t)c * H * 2]);
    float L = 0.f;
    for (int c = 0; c < nch; ++c) L += mlq[(int64_t)c * H * 2 + 1] * exp2f(mlq[(int64_t)c * H * 2] - M);
    lse2 = M + log2f(L);
    if (lse_out != nullptr && blockIdx.y == 0 && g == 0 && has_heads)
      lse_out[(int64_t)t * H + hq] = lse2 * 0.69314718055994531f;
  }
  const float inv_h = 1.f / (float)H;
  float m_run = -INFINITY, l_run = 0.f;  // KT_DENSE_LSE: this lane's keys of head hq

  LDS_AS uint8_t* lds = (LDS_AS uint8_t*)smem;
  __syncthreads();  // s_row / s_valid visible

  // Scores of one tile; then the head sum (to s_part[it & 1]) or the lane's
  // running (m, l).
  auto tile = [&](const LDS_AS uint8_t* buf, int it) {
    constexpr int SPIPE = 4;
    auto frag = [&](int ks, int r) -> v8bf {
      if (ks < 16) return *reinterpret_cast<const LDS_AS v8bf*>(buf + r * NOPE_STRIDE + 64 * ks + 16 * g);
      const int c = 4 * (ks - 16) + g;
      return *reinterpret_cast<const LDS_AS v8bf*>(buf + NOPE_BYTES + r * 128 + 16 * (c ^ (r & 7)));
    };
    v8bf ra0[SPIPE], ra1[SPIPE];
#pragma unroll
    for (int j = 0; j < SPIPE; ++j) {
      ra0[j] = frag(j, n);
      ra1[j] = frag(j, 16 + n);
    }
    v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int ks = 0; ks < AT_D / 32; ++ks) {
      const int slot = ks % SPIPE;
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra0[slot], qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra1[slot], qf[ks], s1, 0, 0, 0);
      if (ks + SPIPE < AT_D / 32) {
        ra0[slot] = frag(ks + SPIPE, n);
        ra1[slot] = frag(ks + SPIPE, 16 + n);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (MODE == KT_DENSE_LSE) {
      // lane holds head n: s0[i] -> key 4g+i, s1[i] -> key 16+4g+i
      const u32 valid = s_valid[it];
      float z[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[i] = ((valid >> (4 * g + i)) & 1u) ? s0[i] * scale_log2 : -INFINITY;
        z[4 + i] = ((valid >> (16 + 4 * g + i)) & 1u) ? s1[i] * scale_log2 : -INFINITY;
      }
      float mx = m_run;
#pragma unroll
      for (int i = 0; i < 8; ++i) mx = fmaxf(mx, z[i]);
      if (mx > -INFINITY) {
        // v_exp_f32: arguments are <= 0, and results below 2^-126 flush to 0
        // (terms under 2^-126 of the running maximum's)
        float add = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) add += __builtin_amdgcn_exp2f(z[i] - mx);
        l_run = l_run * __builtin_amdgcn_exp2f(m_run - mx) + add;  // exp2(-inf) = 0 on the first tile
        m_run = mx;
      }
    } else {
      float p[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(s0[i] * scale_log2 - lse2);
        p[4 + i] = __builtin_amdgcn_exp2f(s1[i] * scale_log2 - lse2);
      }
      // sum over the 16 heads of the lane group: rotations within each row
      // of 16 lanes (DPP, on the VALU, not through LDS); lane n = 0 ends
      // with the row's sum
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = row_sum16(p[i]);
      if (n == 0 && has_heads) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s_part[it & 1][wid][4 * g + i] = p[i];
          s_part[it & 1][wid][16 + 4 * g + i] = p[4 + i];
        }
      }
    }
  };
  // the sums of tile it, written once every wave has stored its part
  auto finish = [&](int it) {
    if constexpr (MODE != KT_DENSE_LSE) {
      if (tid < AT_TILE && it >= 0 && it < ntiles) {
        float v = 0.f;
        for (int w = 0; w < nw_heads; ++w) v += s_part[it & 1][w][tid];
        const int j = it * AT_TILE + tid;
        if constexpr (DENSE) {
          if (j < n_ent) target[(int64_t)t * ld_target + j_begin + j] = v * inv_h;
        } else {
          if (j < k) target[(int64_t)t * k + j] = ((s_valid[it] >> tid) & 1u) ? v * inv_h : 0.f;
        }
      }
    }
  };

  TileStage<NT> sa, sb;
  auto tile_rows = [&](int i) { return s_row + min(i, ntiles - 1) * AT_TILE; };
  sa.load(kv, tile_rows(0), tid);
  sa.store(lds, tid);
  sa.load(kv, tile_rows(1), tid);
  sb.load(kv, tile_rows(2), tid);
  __builtin_amdgcn_s_waitcnt(DSA_VMCNT(2 * TileStage<NT>::PER));
  for (int it = 0; it < ntiles; it += 2) {
    lds_barrier();  // tile it in buffer 0; tile it-1's sums stored
    finish(it - 1);
    tile(lds, it);
    sa.store(lds + BUF_BYTES, tid);
    sa.load(kv, tile_rows(it + 3), tid);
    lds_barrier();
    finish(it);
    if (it + 1 < ntiles) tile(lds + BUF_BYTES, it + 1);
    sb.store(lds, tid);
    sb.load(kv, tile_rows(it + 4), tid);
  }
  __syncthreads();
  finish(ntiles - 1);  // (with an odd tile count already written once: the same values)

  if constexpr (MODE == KT_DENSE_LSE) {
    // merge the four lane groups of head hq (lanes n, n+16, n+32, n+48)
#pragma unroll
    for (int d = 16; d < 64; d <<= 1) {
      const float mo = __shfl_xor(m_run, d, 64);
      const float lo = __shfl_xor(l_run, d, 64);
      const float mm = fmaxf(m_run, mo);
      l_run = (mm == -INFINITY) ? 0.f : l_run * exp2f(m_run - mm) + lo * exp2f(mo - mm);
      m_run = mm;
    }
    if (g == 0 && has_heads) {
      float* o = ml + (((int64_t)t * n_chunks + blockIdx.y) * H + hq) * 2;
      o[0] = m_run;
      o[1] = l_run;
    }
  }
}

// ---------------------------------------------------------------------------
// loss and gradients (H_I = 64, D_I = 128)
// ---------------------------------------------------------------------------

constexpr int KL_HI = 64;
constexpr int KL_DI = 128;
constexpr int KL_TILE = 64;                  // selection entries per wave step
constexpr int KL_MAXK = 2048;
constexpr int MT_STRIDE = KL_HI * 2 + 16;    // mask tile row: 64 heads, bf16 0/1 (+16 B)
constexpr int KT_STRIDE = KL_DI * 2 + 16;    // key tile row: 128 dims, bf16 (+16 B)
constexpr int KL_WAVE_LDS = KL_TILE * (MT_STRIDE + KT_STRIDE);  // 26624 B per wave

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v += __shfl_xor(v, d, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}

// Workgroup = one query token, 4 waves; wave w takes the selection's 64-entry
// tiles w, w+4, ...  Pass 1 scores the tile's entries with the indexer's own
// per-tile arithmetic (indexer_math.h) into LDS; the softmax, the loss and
// dI = q - p follow over the whole selection.  Pass 2 recomputes the
// per-head dot products r (4 FP8 MFMAs per 16 entries: lane (n, g) holds
// heads mt*16+4g+i of entry 16j+n) and forms, per tile:
//   dw      from ReLU(r) in registers;
//   a mask tile M[entry][head] = [r > 0] (bf16 0/1) and a key tile
//   Kt[entry][dim] = dI * ks * k8 (bf16), both in the wave's LDS;
//   dk^T[dim][entry] = (w q8)^T M^T  -- A = (w * q8)^T fragments kept in
//     registers for the token, B = mask rows; scaled by dI * qs per entry and
//     stored as one bf16 row of 128 per slot;
//   dq[head][dim] += M^T Kt           -- both operands through the LDS
//     transpose read; accumulated over the wave's tiles, then summed over the
//     waves with LDS float atomics and scaled by w.
__global__ __launch_bounds__(256) void indexer_kl_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, const float* __restrict__ ks, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ seq_id, Layout lay, int k, int kp, const float* __restrict__ target,
    float* __restrict__ loss, float* __restrict__ dq, float* __restrict__ dw, uint16_t* __restrict__ slot_dk,
    u32* __restrict__ rows_out, int n_tokens) {
  __shared__ float s_lg[KL_MAXK];  // logits, then dI
  __shared__ u32 s_row[KL_MAXK];
  __shared__ __attribute__((aligned(16))) uint8_t s_wave[4 * KL_WAVE_LDS];  // later: dq sums (32 KB)
  __shared__ float s_red[8];
  __shared__ float s_dw[KL_HI];
  const int t = blockIdx.x;
  if (t >= n_tokens) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int b = seq_id[t];
  const int ntiles = (k + KL_TILE - 1) / KL_TILE;
  const u32 safe_row = (u32)token_row(lay, b, 0);
  for (int j = tid; j < ntiles * KL_TILE; j += 256) {
    const int s = (j < k) ? idx[(int64_t)t * k + j] : -1;
    const u32 row = (s >= 0) ? (u32)token_row(lay, b, s) : (safe_row | ROW_INVALID);
    s_row[j] = row;
    if (j < kp) rows_out[(int64_t)t * kp + j] = (s >= 0) ? row : SLOT_NONE;
  }
  if (tid < KL_HI) s_dw[tid] = 0.f;

  IndexerQuery<KL_HI, KL_DI> qy;
  qy.load(q8, qs, w, t, n, g);
  // A operand of dk^T: (w_h * q8[h][d])^T, lane (m = dim, g) holding heads
  // 32ks + 8g .. +7 of dim 16dt + m, through LDS (the token's q8 rows)
  v8bf xw[2][8];
  {
    LDS_AS uint8_t* qst = (LDS_AS uint8_t*)s_wave;
    for (int c = tid; c < KL_HI * KL_DI / 16; c += 256)
      *reinterpret_cast<LDS_AS v4i*>(qst + 16 * c) =
          *reinterpret_cast<const v4i*>(q8 + (int64_t)t * KL_HI * KL_DI + 16 * c);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int d = 16 * dt + n;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int h = 32 * kk + 8 * g + i;
          const u32 byte = qst[h * KL_DI + d];
          xw[kk][dt][i] = (__bf16)(w[(int64_t)t * KL_HI + h] * __builtin_amdgcn_cvt_f32_fp8((int)byte, 0));
        }
      }
    __syncthreads();
  }
  const float qscale = qy.qscale;

  auto load_keys = [&](int it, KeyFrag<KL_HI, KL_DI> (&kb)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32 row = s_row[it * KL_TILE + 16 * j + n] & ~ROW_INVALID;
      kb[j].load(k8 + (int64_t)row * KL_DI, g);
    }
  };

  // ---- pass 1: logits of the selected entries
  for (int it = wid; it < ntiles; it += 4) {
    KeyFrag<KL_HI, KL_DI> kb[4];
    load_keys(it, kb);
    const int e = it * KL_TILE + lane;
    const u32 row = s_row[e];
    const float ksv = ks[row & ~ROW_INVALID];
    const float res = group_scores<KL_HI, KL_DI>(qy, kb);
    s_lg[e] = (row & ROW_INVALID) ? -INFINITY : scaled_logit(res, qscale, ksv);
  }
  __syncthreads();

  // ---- softmax over the selection, loss, dI = q - p
  float mx = -INFINITY;
  for (int j = tid; j < k; j += 256) mx = fmaxf(mx, s_lg[j]);
  mx = wave_max(mx);
  if (lane == 0) s_red[wid] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  __syncthreads();
  float z = 0.f;
  if (mx != -INFINITY)
    for (int j = tid; j < k; j += 256) z += __builtin_amdgcn_exp2f((s_lg[j] - mx) * LOG2E);
  z = wave_sum(z);
  if (lane == 0) s_red[wid] = z;
  __syncthreads();
  z = s_red[0] + s_red[1] + s_red[2] + s_red[3];
  const float inv_z = (z > 0.f) ? 1.f / z : 0.f;
  const float log_z = (z > 0.f) ? logf(z) : 0.f;
  float lsum = 0.f;
  for (int j = tid; j < ntiles * KL_TILE; j += 256) {
    float di = 0.f;
    if (j < k && !(s_row[j] & ROW_INVALID)) {
      const float lg = s_lg[j];
      const float qv = __builtin_amdgcn_exp2f((lg - mx) * LOG2E) * inv_z;
      const float p = target[(int64_t)t * k + j];
      if (p > 0.f) lsum += p * (logf(p) - (lg - mx - log_z));
      di = qv - p;
    }
    s_lg[j] = di;
  }
  lsum = wave_sum(lsum);
  __syncthreads();  // every s_lg read done before s_red is reused
  if (lane == 0) s_red[4 + wid] = lsum;
  __syncthreads();
  if (tid == 0) loss[t] = s_red[4] + s_red[5] + s_red[6] + s_red[7];

  // ---- pass 2: gradients
  LDS_AS uint8_t* mt_lds = (LDS_AS uint8_t*)s_wave + wid * KL_WAVE_LDS;
  LDS_AS uint8_t* kt_lds = mt_lds + KL_TILE * MT_STRIDE;
  v4f dqa[4][8];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 8; ++c) dqa[a][c] = v4f{0.f, 0.f, 0.f, 0.f};
  float dwa[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) dwa[a][i] = 0.f;

  for (int it = wid; it < ntiles; it += 4) {
    KeyFrag<KL_HI, KL_DI> kb[4];
    load_keys(it, kb);
    const int e = it * KL_TILE + lane;
    const float di = s_lg[e];
    const float cks = di * ks[s_row[e] & ~ROW_INVALID];  // dI * ks of entry `lane`
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float c = __shfl(cks, 16 * j + n, 64);      // entry 16j + n
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const v4f r = KeyFrag<KL_HI, KL_DI>::mma(qy.qa[mt], kb[j]);
        v4s mb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dwa[mt][i] += c * relu(r[i]);
          mb[i] = (r[i] > 0.f) ? (short)0x3F80 : (short)0;  // bf16 1.0 / 0.0
        }
        *reinterpret_cast<LDS_AS v4s*>(mt_lds + (16 * j + n) * MT_STRIDE + 2 * (16 * mt + 4 * g)) = mb;
      }
      // dI * ks * k8 of entry 16j + n, dims 32g .. 32g + 31
      LDS_AS uint8_t* krow = kt_lds + (16 * j + n) * KT_STRIDE + 2 * 32 * g;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        v8bf o;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int word = kb[j].v[2 * q4 + h];
          const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
          const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
          o[4 * h + 0] = (__bf16)(c * lo[0]);
          o[4 * h + 1] = (__bf16)(c * lo[1]);
          o[4 * h + 2] = (__bf16)(c * hi[0]);
          o[4 * h + 3] = (__bf16)(c * hi[1]);
        }
        *reinterpret_cast<LDS_AS v8bf*>(krow + 16 * q4) = o;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");  // the wave's tile writes before its reads

    // dk^T[dim][entry] = sum_h (w q8)^T[dim][h] M[entry][h], per 16 entries
    const float dsc = di * qscale;  // dI * qs of entry `lane`
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      v8bf mrow[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        mrow[kk] = *reinterpret_cast<const LDS_AS v8bf*>(mt_lds + (16 * kt + n) * MT_STRIDE + 2 * (32 * kk + 8 * g));
      const float sc = __shfl(dsc, 16 * kt + n, 64);
      uint16_t* out = slot_dk + ((int64_t)t * kp + it * KL_TILE + 16 * kt + n) * KL_DI + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xw[0][dt], mrow[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xw[1][dt], mrow[1], acc, 0, 0, 0);
        v2i pk;
        pk[0] = (int)((u32)f2bf(acc[0] * sc) | ((u32)f2bf(acc[1] * sc) << 16));
        pk[1] = (int)((u32)f2bf(acc[2] * sc) | ((u32)f2bf(acc[3] * sc) << 16));
        *reinterpret_cast<v2i*>(out + 16 * dt) = pk;
      }
    }

    // dq[head][dim] += M^T Kt over the tile's 64 entries (two K steps of 32)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int r0 = 32 * kk + 8 * g + (n >> 2);
      v8bf am[4], bk[8];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const LDS_AS uint8_t* p = mt_lds + r0 * MT_STRIDE + 2 * 16 * mt + 8 * (n & 3);
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)p);
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)(p + 4 * MT_STRIDE));
        am[mt] = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const LDS_AS uint8_t* p = kt_lds + r0 * KT_STRIDE + 2 * 16 * dt + 8 * (n & 3);
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)p);
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)(p + 4 * KT_STRIDE));
        bk[dt] = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          dqa[mt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am[mt], bk[dt], dqa[mt][dt], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");  // reads done before the next tile's writes
  }

  // ---- dw: over the wave's entries (lanes n), then over the waves
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = dwa[mt][i];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      v += __shfl_xor(v, 8, 64);
      if (n == 0) atomicAdd(&s_dw[16 * mt + 4 * g + i], v);
    }
  // ---- dq: the waves' partial sums meet in LDS (the tiles' space)
  __syncthreads();
  float* s_dq = reinterpret_cast<float*>(s_wave);
  for (int i = tid; i < KL_HI * KL_DI; i += 256) s_dq[i] = 0.f;
  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(&s_dq[(16 * mt + 4 * g + i) * KL_DI + 16 * dt + n], dqa[mt][dt][i]);
  __syncthreads();
  for (int i = tid; i < KL_HI * KL_DI; i += 256) {
    const int h = i / KL_DI;
    dq[(int64_t)t * KL_HI * KL_DI + i] = s_dq[i] * w[(int64_t)t * KL_HI + h];
  }
  if (tid < KL_HI) dw[(int64_t)t * KL_HI + tid] = s_dw[tid] * qscale;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

bool kl_supported(int H_I, int D_I) { return H_I == KL_HI && D_I == KL_DI; }

static int kl_kp(int k) { return ((k + KL_TILE - 1) / KL_TILE) * KL_TILE; }

WsLayout kl_layout(int T, int k) {
  WsLayout L;
  if (T == 0) return L;
  const size_t N = (size_t)T * kl_kp(k);
  L.add("slot_dk", N * KL_DI * 2);
  L.add("rows", N * 4);
  L.add_sub("scatter", scatter_layout(N));
  return L;
}

size_t kl_workspace_bytes(int T, int k) { return kl_layout(T, k).total; }

bool kl_size_ok(int T, int k) { return (int64_t)T * kl_kp(k) < (int64_t(1) << 31); }

hipError_t launch_kl_target(int T, int H, const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                            const int32_t* seq_id, const Layout& lay, int k, float sm_scale, const float* lse,
                            float* target, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(kl_target_kernel<KT_SELECTED>, dim3(T), dim3(KT_NW * 64), 0, stream, q,
                     reinterpret_cast<const uint8_t*>(kv), idx, seq_id, nullptr, lay, H, k, sm_scale * LOG2E, lse,
                     target, (int64_t)k, nullptr, 0, nullptr, T);
  return hipGetLastError();
}

static int dense_target_chunks(int max_len) { return (max_len + AT_MAX_SPLIT - 1) / AT_MAX_SPLIT; }

WsLayout kl_target_dense_layout(int T, int H, int max_len) {
  WsLayout L;
  L.add("ml", (size_t)T * dense_target_chunks(max_len) * H * 2 * 4);  // per chunk and head: max, sum
  return L;
}

size_t kl_target_dense_workspace_bytes(int T, int H, int max_len) { return kl_target_dense_layout(T, H, max_len).total; }

hipError_t launch_kl_target_dense(int T, int H, int max_len, const uint16_t* q, const uint16_t* kv,
                                  const int32_t* seq_id, const int32_t* pos, const Layout& lay, float sm_scale,
                                  float* target, int64_t ld, float* lse_out, void* ws, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int nch = dense_target_chunks(max_len);
  float* ml = static_cast<float*>(kl_target_dense_layout(T, H, max_len).at(ws, 0));
  const uint8_t* kvb = reinterpret_cast<const uint8_t*>(kv);
  hipLaunchKernelGGL(kl_target_kernel<KT_DENSE_LSE>, dim3(T, nch), dim3(KT_NW * 64), 0, stream, q, kvb, nullptr,
                     seq_id, pos, lay, H, 0, sm_scale * LOG2E, nullptr, nullptr, (int64_t)0, ml, nch, nullptr, T);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kl_target_kernel<KT_DENSE_TARGET>, dim3(T, nch), dim3(KT_NW * 64), 0, stream, q, kvb, nullptr,
                     seq_id, pos, lay, H, 0, sm_scale * LOG2E, nullptr, target, ld, ml, nch, lse_out, T);
  return hipGetLastError();
}

hipError_t launch_kl_target_dense_lse(int T, int H, int max_len, const uint16_t* q, const uint16_t* kv,
                                      const int32_t* seq_id, const int32_t* pos, const Layout& lay, float sm_scale,
                                      const float* lse, float* target, int64_t ld, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int nch = dense_target_chunks(max_len);
  const uint8_t* kvb = reinterpret_cast<const uint8_t*>(kv);
  hipLaunchKernelGGL(kl_target_kernel<KT_DENSE_GIVEN>, dim3(T, nch), dim3(KT_NW * 64), 0, stream, q, kvb, nullptr,
                     seq_id, pos, lay, H, 0, sm_scale * LOG2E, lse, target, ld, nullptr, nch, nullptr, T);
  return hipGetLastError();
}

hipError_t launch_kl(int T, const uint8_t* q8, const float* qs, const float* w, const uint8_t* k8, const float* ks,
                     const int32_t* idx, const int32_t* seq_id, const Layout& lay, int64_t num_rows, int k,
                     const float* target, float* loss, float* dq, float* dw, float* dk, void* ws,
                     hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int kp = kl_kp(k);
  const size_t N = (size_t)T * kp;
  const WsLayout L = kl_layout(T, k);
  uint16_t* slot_dk = static_cast<uint16_t*>(L.at(ws, 0));
  u32* rows = static_cast<u32*>(L.at(ws, 1));
  void* scatter_ws = L.at(ws, 2);
  hipLaunchKernelGGL(indexer_kl_kernel, dim3(T), dim3(256), 0, stream, q8, qs, w, k8, ks, idx, seq_id, lay, k, kp,
                     target, loss, dq, dw, slot_dk, rows, T);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_row_scatter_add(rows, (int)N, num_rows, slot_dk, KL_DI, dk, scatter_ws, stream);
}

}  // namespace dsa
