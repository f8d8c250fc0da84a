// Backward of the sparse attention under MLA in MQA mode, on gfx950.
//
// "DeepSeek V3.2-Exp Cuts Prolonged-Context Costs With DeepSeek Sparse
// Consideration (DSA)", opening paragraph and "Teaching signal": the sparse
// path is trained, so gradients flow through the selected rows.  For query t,
// head h and its selected rows i (z = scale q.kv_i, P = softmax(z) restored
// from the forward's log-sum-exp, V = kv[:, :512], dO the output gradient):
//   dP_i = dO . V_i,  D = dO . O,  dS_i = P_i (dP_i - D)
//   dq   = scale sum_i dS_i kv_i
//   dkv_i += scale sum_h dS_hi q_h   (+ sum_h P_hi dO_h on the first 512)
// Every query's heads share its rows (MQA), so a row's gradient is a
// contraction over heads, and a cache row selected by several queries
// collects all their contributions.
//
// Three steps, chosen for the memory system of the MI355X:
//   1. dq kernel, per (token, 64 heads): the forward's row gather and tile
//      pipeline; per tile it rebuilds S and dP (the no-rope K fragments feed
//      both), then P and dS in registers, accumulates dq^T += K^T dS^T with
//      K^T read through the LDS transpose read, and stores P and scale*dS as
//      bf16 per (token, head, slot) together with the token's row list.
//   2. slot kernel, per token, all heads: the gradient of each selected slot,
//      [scale dS; P]^T [q; dO] -- a contraction over 2H stacked rows -- on
//      bf16 MFMAs.  q and dO are constant per token, so each wave keeps its
//      slice of [q; dO]^T in registers (read once through the LDS transpose
//      read) and streams the P / dS tiles; one bf16 row of 576 per slot.
//   3. the per-slot rows are added into dkv through a sort of the row list
//      (row_scatter.hip): one fp32 atomic per (run of equal rows, value)
//      instead of one per (slot, value).
#include "attn_tile.h"
#include "launch.h"

namespace dsa {

constexpr u32 SLOT_NONE = 0xFFFFFFFFu;  // row list entry past a token's selected slots (sorts last)
constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// 1. dq, P and dS
// ---------------------------------------------------------------------------

// One tile in `buf`: rebuild S and dP, form P and dS, store them, and add
// K^T dS^T to the dq accumulator.  Lane (n, g) holds head n; its score
// registers cover keys 4g..4g+3 and 16+4g..16+4g+3 of the tile.
__device__ __forceinline__ void dq_tile(const LDS_AS uint8_t* __restrict__ buf, u32 valid, const v8bf* qf,
                                        const v8bf* dof, float scale_log2, float lse2, float dsum, float sm_scale,
                                        int n, int g, v4f* acc, uint16_t* __restrict__ ds_row,
                                        uint16_t* __restrict__ p_row, bool store) {
  const LDS_AS uint8_t* nope = buf;
  const LDS_AS uint8_t* rope = buf + NOPE_BYTES;
  constexpr int SPIPE = 4;
  auto frag = [&](int ks, int r) -> v8bf {
    if (ks < 16) return *reinterpret_cast<const LDS_AS v8bf*>(nope + r * NOPE_STRIDE + 64 * ks + 16 * g);
    const int c = 4 * (ks - 16) + g;
    return *reinterpret_cast<const LDS_AS v8bf*>(rope + r * 128 + 16 * (c ^ (r & 7)));
  };
  v8bf ra0[SPIPE], ra1[SPIPE];
#pragma unroll
  for (int j = 0; j < SPIPE; ++j) {
    ra0[j] = frag(j, n);
    ra1[j] = frag(j, 16 + n);
  }
  // S^T = K Q^T and dP^T = V dO^T; the no-rope fragments (V) serve both
  v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, d0 = s0, d1 = s0;
#pragma unroll
  for (int ks = 0; ks < AT_D / 32; ++ks) {
    const int slot = ks % SPIPE;
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra0[slot], qf[ks], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra1[slot], qf[ks], s1, 0, 0, 0);
    if (ks < AT_DV / 32) {
      d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra0[slot], dof[ks], d0, 0, 0, 0);
      d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra1[slot], dof[ks], d1, 0, 0, 0);
    }
    if (ks + SPIPE < AT_D / 32) {
      ra0[slot] = frag(ks + SPIPE, n);
      ra1[slot] = frag(ks + SPIPE, 16 + n);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // P = exp(z - lse) (0 for masked rows) and scale * dS = scale * P (dP - D)
  v8bf pb, db;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // v_exp_f32 (values below 2^-126 flush to 0, far below bf16's resolution of P)
    const float p0 = ((valid >> (4 * g + i)) & 1u) ? __builtin_amdgcn_exp2f(s0[i] * scale_log2 - lse2) : 0.f;
    const float p1 = ((valid >> (16 + 4 * g + i)) & 1u) ? __builtin_amdgcn_exp2f(s1[i] * scale_log2 - lse2) : 0.f;
    pb[i] = (__bf16)p0;
    pb[4 + i] = (__bf16)p1;
    db[i] = (__bf16)(p0 * (d0[i] - dsum) * sm_scale);
    db[4 + i] = (__bf16)(p1 * (d1[i] - dsum) * sm_scale);
  }
  if (store) {
    const v4i pv = __builtin_bit_cast(v4i, pb), dv = __builtin_bit_cast(v4i, db);
    *reinterpret_cast<v2i*>(p_row + 4 * g) = v2i{pv[0], pv[1]};
    *reinterpret_cast<v2i*>(p_row + 16 + 4 * g) = v2i{pv[2], pv[3]};
    *reinterpret_cast<v2i*>(ds_row + 4 * g) = v2i{dv[0], dv[1]};
    *reinterpret_cast<v2i*>(ds_row + 16 + 4 * g) = v2i{dv[2], dv[3]};
  }
  // dq^T += K^T (scale dS)^T: K^T through the LDS transpose read.  Source
  // lane n of group g points at rows 4g + n/4 (and 16 rows on), dims
  // 16mt + 4(n%4)..+3, so the fragment's K order is the keys' order in db.
  // Fragments 32..35 are the rope dims, with the rope block's chunk swizzle.
  // The reads run DPIPE fragments ahead of the MFMAs that use them.
  const LDS_AS uint8_t* vsrc0 = nope + (4 * g + (n >> 2)) * NOPE_STRIDE + 8 * (n & 3);
  const int rr = 4 * g + (n >> 2);
  auto kt = [&](int mt) -> v8bf {
    const LDS_AS uint8_t* p0;
    int step;
    if (mt < AT_DV / 16) {
      p0 = vsrc0 + 32 * mt;
      step = 16 * NOPE_STRIDE;
    } else {
      const int c = 2 * (mt - AT_DV / 16) + ((n & 3) >> 1);
      p0 = rope + rr * 128 + 16 * (c ^ (rr & 7)) + 8 * (n & 1);
      step = 16 * 128;
    }
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)p0);
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)(p0 + step));
    return __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  constexpr int DPIPE = 6;
  constexpr int NKT = AT_D / 16;
  v8bf ring[DPIPE];
#pragma unroll
  for (int j = 0; j < DPIPE; ++j) ring[j] = kt(j);
#pragma unroll
  for (int mt = 0; mt < NKT; ++mt) {
    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[mt % DPIPE], db, acc[mt], 0, 0, 0);
    if (mt + DPIPE < NKT) ring[mt % DPIPE] = kt(mt + DPIPE);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Workgroup = (token, 16*NW heads); 16 heads per wave.  Outputs: dq, the
// P / scale*dS rows of the token (dsp: [T][2H][kp], rows h: scale*dS of head
// h, rows H+h: P), and, from head group 0, the token's compacted row list
// (rows_out[t*kp + c], SLOT_NONE past the selected slots) and count.
template <int NW>
__global__ __launch_bounds__(NW * 64) void sparse_mla_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ seq_id, Layout lay, int H, int k, int kp, float sm_scale,
    const uint16_t* __restrict__ out, const float* __restrict__ lse, const uint16_t* __restrict__ dout,
    float* __restrict__ dq, uint16_t* __restrict__ dsp, u32* __restrict__ rows_out, int32_t* __restrict__ cnt_out,
    int n_tokens) {
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BUF_BYTES];
  __shared__ u32 s_row[AT_MAX_SPLIT];
  __shared__ u32 s_valid[AT_MAX_SPLIT / AT_TILE];
  __shared__ u32 scan_scratch[NW + 1];

  // head groups of one token on one XCD, in consecutive slots (shared rows
  // come from that XCD's L2 for the second)
  const int n_hg = H / (16 * NW) > 0 ? H / (16 * NW) : 1;
  const int lin = blockIdx.x;
  const int slot = lin >> 3;
  const int t = (lin & 7) + 8 * (slot / n_hg);
  const int hg = slot - (slot / n_hg) * n_hg;
  if (t >= n_tokens) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int h0 = hg * (16 * NW) + wid * 16;
  const bool has_heads = h0 < H;
  const int b = seq_id[t];

  const int nvalid = compact_selection<NT>(idx + (int64_t)t * k, k, lay, b, s_row, s_valid, scan_scratch, tid, [] {});
  const int ntiles = (nvalid + AT_TILE - 1) / AT_TILE;

  // Q^T and dO^T operands of head h0+n (dims 32ks + 8g..+8), and D = dO . O
  const int hq = (has_heads ? h0 : 0) + n;
  const int64_t th = (int64_t)t * H + hq;
  v8bf qf[AT_D / 32], dof[AT_DV / 32];
#pragma unroll
  for (int ks = 0; ks < AT_D / 32; ++ks) qf[ks] = *reinterpret_cast<const v8bf*>(q + th * AT_D + 32 * ks + 8 * g);
  float dsum = 0.f;
#pragma unroll
  for (int ks = 0; ks < AT_DV / 32; ++ks) {
    dof[ks] = *reinterpret_cast<const v8bf*>(dout + th * AT_DV + 32 * ks + 8 * g);
    const v8bf o = *reinterpret_cast<const v8bf*>(out + th * AT_DV + 32 * ks + 8 * g);
#pragma unroll
    for (int i = 0; i < 8; ++i) dsum += (float)dof[ks][i] * (float)o[i];
  }
  dsum += __shfl_xor(dsum, 16, 64);
  dsum += __shfl_xor(dsum, 32, 64);
  const float lse2 = lse[th] * LOG2E;
  const float scale_log2 = sm_scale * LOG2E;
  uint16_t* ds_base = dsp + ((int64_t)t * 2 * H + hq) * kp;
  uint16_t* p_base = ds_base + (int64_t)H * kp;

  v4f acc[AT_D / 16];
#pragma unroll
  for (int mt = 0; mt < AT_D / 16; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};

  LDS_AS uint8_t* lds = (LDS_AS uint8_t*)smem;
  __syncthreads();  // s_row / s_valid visible
  if (hg == 0) {
    for (int c = tid; c < kp; c += NT) rows_out[(int64_t)t * kp + c] = (c < nvalid) ? s_row[c] : SLOT_NONE;
    if (tid == 0) cnt_out[t] = nvalid;
  }
  // the forward's two-stage gather pipeline (tiles past the last re-read it
  // and are masked out)
  TileStage<NT> sa, sb;
  auto tile_rows = [&](int i) { return s_row + min(i, ntiles - 1) * AT_TILE; };
  if (ntiles > 0) {
    sa.load(kv, tile_rows(0), tid);
    sa.store(lds, tid);
    sa.load(kv, tile_rows(1), tid);
    sb.load(kv, tile_rows(2), tid);
  }
  __builtin_amdgcn_s_waitcnt(DSA_VMCNT(2 * TileStage<NT>::PER));
  for (int it = 0; it < ntiles; it += 2) {
    lds_barrier();
    dq_tile(lds, s_valid[it], qf, dof, scale_log2, lse2, dsum, sm_scale, n, g, acc, ds_base + it * AT_TILE,
            p_base + it * AT_TILE, has_heads);
    sa.store(lds + BUF_BYTES, tid);
    sa.load(kv, tile_rows(it + 3), tid);
    lds_barrier();
    dq_tile(lds + BUF_BYTES, (it + 1 < ntiles) ? s_valid[it + 1] : 0u, qf, dof, scale_log2, lse2, dsum, sm_scale, n,
            g, acc, ds_base + (it + 1) * AT_TILE, p_base + (it + 1) * AT_TILE, has_heads && it + 1 < ntiles);
    sb.store(lds, tid);
    sb.load(kv, tile_rows(it + 4), tid);
  }
  if (!has_heads) return;
  // lane (n, g) holds dq^T[16mt + 4g + i][head n]
  float* dq_row = dq + th * AT_D + 4 * g;
#pragma unroll
  for (int mt = 0; mt < AT_D / 16; ++mt) *reinterpret_cast<v4f*>(dq_row + 16 * mt) = acc[mt];
}

// ---------------------------------------------------------------------------
// 2. per-slot gradients
// ---------------------------------------------------------------------------

constexpr int XS_STRIDE = AT_ROW_BYTES + 16;  // staged [q; dO] row in LDS (1168 B)
constexpr int DT_STRIDE = 80;                 // staged P / dS row of a tile: 64 B + 16

// Workgroup = one token; wave w owns the gradient dims 128w..128w+127 (no
// rope) and 512+16w..+15 (rope).  With X = [scale-free q rows; dO rows]
// (2H rows of 576, dO's rope part zero) and Dt = [scale dS; P] (2H rows per
// slot): grad^T[dims x slots] = X^T Dt.  A = X^T fragments stay in
// registers; B = Dt fragments come from the staged tile.
template <int H>
__global__ __launch_bounds__(256) void sparse_mla_bwd_slot_kernel(const uint16_t* __restrict__ q,
                                                                  const uint16_t* __restrict__ dout,
                                                                  const uint16_t* __restrict__ dsp,
                                                                  const int32_t* __restrict__ cnt, int kp,
                                                                  uint16_t* __restrict__ slot_grad, int n_tokens) {
  constexpr int KS = 2 * H / 32;        // K steps over the stacked rows
  constexpr int KSR = (H + 31) / 32;    // K steps that reach q rows (rope)
  constexpr int XBYTES = 32 * XS_STRIDE;
  constexpr int DBYTES = 2 * H * DT_STRIDE;
  constexpr int DCHUNKS = 2 * H * 4;     // 16-byte chunks of a Dt tile
  constexpr int DCH = (DCHUNKS + 255) / 256;
  __shared__ __attribute__((aligned(16))) uint8_t smem[XBYTES > 2 * DBYTES ? XBYTES : 2 * DBYTES];
  const int t = blockIdx.x;
  if (t >= n_tokens) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  LDS_AS uint8_t* lds = (LDS_AS uint8_t*)smem;

  // ---- X^T fragments: 32 stacked rows at a time through LDS
  v8bf xa[KS][8], xr[KSR];
  for (int kb = 0; kb < KS; ++kb) {
    for (int c = tid; c < 32 * 72; c += 256) {
      const int r = c / 72, ch = c - r * 72;
      const int kappa = 32 * kb + r;
      v4i v = v4i{0, 0, 0, 0};
      if (kappa < H)
        v = *reinterpret_cast<const v4i*>(q + ((int64_t)t * H + kappa) * AT_D + 8 * ch);
      else if (ch < 64)
        v = *reinterpret_cast<const v4i*>(dout + ((int64_t)t * H + kappa - H) * AT_DV + 8 * ch);
      *reinterpret_cast<LDS_AS v4i*>(lds + r * XS_STRIDE + 16 * ch) = v;
    }
    __syncthreads();
    // source lane n of group g: rows 8g + n/4 (+4), dims d0 + 4(n%4)..+3
    const LDS_AS uint8_t* src = lds + (8 * g + (n >> 2)) * XS_STRIDE + 8 * (n & 3);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int d0 = 128 * wid + 16 * m;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)(src + 2 * d0));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)(src + 4 * XS_STRIDE + 2 * d0));
      xa[kb][m] = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    if (kb < KSR) {
      const int d0 = AT_DV + 16 * wid;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)(src + 2 * d0));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)(src + 4 * XS_STRIDE + 2 * d0));
      xr[kb] = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    __syncthreads();
  }

  // ---- tiles of 32 slots: Dt rows (2H x 64 B) staged in one of two buffers
  const int ntiles = (cnt[t] + AT_TILE - 1) / AT_TILE;
  const uint16_t* dt = dsp + (int64_t)t * 2 * H * kp;
  v4i st[DCH];
  auto load_tile = [&](int it) {
    const int itc = min(it, max(ntiles - 1, 0));
#pragma unroll
    for (int j = 0; j < DCH; ++j) {
      const int c = min(tid + 256 * j, DCHUNKS - 1);
      st[j] = *reinterpret_cast<const v4i*>(dt + (int64_t)(c >> 2) * kp + AT_TILE * itc + 8 * (c & 3));
    }
  };
  auto store_tile = [&](LDS_AS uint8_t* buf) {
#pragma unroll
    for (int j = 0; j < DCH; ++j) {
      const int c = tid + 256 * j;
      if (DCHUNKS % 256 == 0 || c < DCHUNKS)
        *reinterpret_cast<LDS_AS v4i*>(buf + (c >> 2) * DT_STRIDE + 16 * (c & 3)) = st[j];
    }
  };
  if (ntiles > 0) {
    load_tile(0);
    store_tile(lds);
    load_tile(1);
  }
  uint16_t* out_base = slot_grad + (int64_t)t * kp * AT_D;
  for (int it = 0; it < ntiles; ++it) {
    LDS_AS uint8_t* cur = lds + (it & 1) * DBYTES;
    __syncthreads();  // tile `it` staged; the other buffer is free
    if (it + 1 < ntiles) store_tile(lds + ((it + 1) & 1) * DBYTES);
    load_tile(it + 2);
    v4f acc[9][2];
#pragma unroll
    for (int m = 0; m < 9; ++m) acc[m][0] = acc[m][1] = v4f{0.f, 0.f, 0.f, 0.f};
    const LDS_AS uint8_t* src = cur + (8 * g + (n >> 2)) * DT_STRIDE + 8 * (n & 3);
#pragma unroll
    for (int kb = 0; kb < KS; ++kb) {
      v8bf bfr[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const LDS_AS uint8_t* p = src + 32 * kb * DT_STRIDE + 32 * nt;
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)p);
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)(p + 4 * DT_STRIDE));
        bfr[nt] = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[m][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[kb][m], bfr[nt], acc[m][nt], 0, 0, 0);
      if (kb < KSR)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[8][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xr[kb], bfr[nt], acc[8][nt], 0, 0, 0);
    }
    // lane (n, g): dims d0 + 4g..+3 of slot 32it + 16nt + n
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      uint16_t* row = out_base + (int64_t)(AT_TILE * it + 16 * nt + n) * AT_D + 4 * g;
#pragma unroll
      for (int m = 0; m < 9; ++m) {
        const int d0 = m < 8 ? 128 * wid + 16 * m : AT_DV + 16 * wid;
        v2i pk;
        pk[0] = (int)((u32)f2bf(acc[m][nt][0]) | ((u32)f2bf(acc[m][nt][1]) << 16));
        pk[1] = (int)((u32)f2bf(acc[m][nt][2]) | ((u32)f2bf(acc[m][nt][3]) << 16));
        *reinterpret_cast<v2i*>(row + d0) = pk;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------

bool attn_bwd_supported(int H) { return H == 16 || H == 32 || H == 64 || H == 128; }

static int bwd_kp(int k) { return ((k + AT_TILE - 1) / AT_TILE) * AT_TILE; }

struct BwdWorkspace {
  uint16_t* dsp;
  uint16_t* slot_grad;
  u32* rows;
  int32_t* cnt;
  void* scatter;
};

WsLayout attn_bwd_layout(int T, int H, int k) {
  WsLayout L;
  if (T == 0) return L;
  const size_t N = (size_t)T * bwd_kp(k);
  L.add("dsp", N * 2 * H * 2);
  L.add("slot_grad", N * AT_D * 2);
  L.add("rows", N * 4);
  L.add("cnt", (size_t)T * 4);
  L.add_sub("scatter", scatter_layout(N));
  return L;
}

static void carve_bwd(int T, int H, int k, void* base, BwdWorkspace* w) {
  const WsLayout L = attn_bwd_layout(T, H, k);
  w->dsp = static_cast<uint16_t*>(L.at(base, 0));
  w->slot_grad = static_cast<uint16_t*>(L.at(base, 1));
  w->rows = static_cast<u32*>(L.at(base, 2));
  w->cnt = static_cast<int32_t*>(L.at(base, 3));
  w->scatter = L.at(base, 4);
}

size_t attn_bwd_workspace_bytes(int T, int H, int k) { return attn_bwd_layout(T, H, k).total; }

bool attn_bwd_size_ok(int T, int k) { return (int64_t)T * bwd_kp(k) < (int64_t(1) << 31); }

hipError_t launch_attn_bwd_dq(int T, int H, const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                              const int32_t* seq_id, const Layout& lay, int k, float sm_scale, const uint16_t* out,
                              const float* lse, const uint16_t* dout, float* dq, void* ws, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  BwdWorkspace w;
  carve_bwd(T, H, k, ws, &w);
  const int kp = bwd_kp(k);
  const int n_hg = H > 64 ? H / 64 : 1;
  const int blocks = ((T + 7) / 8) * 8 * n_hg;
  hipLaunchKernelGGL(sparse_mla_bwd_dq_kernel<4>, dim3(blocks), dim3(256), 0, stream, q,
                     reinterpret_cast<const uint8_t*>(kv), idx, seq_id, lay, H, k, kp, sm_scale, out, lse, dout, dq,
                     w.dsp, w.rows, w.cnt, T);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dkv(int T, int H, const uint16_t* q, const uint16_t* dout, int64_t num_rows, int k,
                               float* dkv, void* ws, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  BwdWorkspace w;
  carve_bwd(T, H, k, ws, &w);
  const int kp = bwd_kp(k);
  const int N = T * kp;
  hipError_t e;

  // per-slot gradients
  switch (H) {
    case 16: hipLaunchKernelGGL(sparse_mla_bwd_slot_kernel<16>, dim3(T), dim3(256), 0, stream, q, dout, w.dsp, w.cnt,
                                kp, w.slot_grad, T); break;
    case 32: hipLaunchKernelGGL(sparse_mla_bwd_slot_kernel<32>, dim3(T), dim3(256), 0, stream, q, dout, w.dsp, w.cnt,
                                kp, w.slot_grad, T); break;
    case 64: hipLaunchKernelGGL(sparse_mla_bwd_slot_kernel<64>, dim3(T), dim3(256), 0, stream, q, dout, w.dsp, w.cnt,
                                kp, w.slot_grad, T); break;
    case 128: hipLaunchKernelGGL(sparse_mla_bwd_slot_kernel<128>, dim3(T), dim3(256), 0, stream, q, dout, w.dsp,
                                 w.cnt, kp, w.slot_grad, T); break;
    default: return hipErrorInvalidValue;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // the per-slot rows into dkv, through the sort of the row list
  return launch_row_scatter_add(w.rows, N, num_rows, w.slot_grad, AT_D, dkv, w.scatter, stream);
}

}  // namespace dsa
