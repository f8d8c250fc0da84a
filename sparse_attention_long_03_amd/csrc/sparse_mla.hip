// Sparse attention under MLA in MQA mode, on gfx950 bf16 matrix cores.
//
// "DeepSeek V3.2-Exp Cuts Prolonged-Context Costs With DeepSeek Sparse
// Consideration (DSA)", part (2): standard attention runs only over the
// selected subset; "Instantiation": MLA in MQA mode, every latent KV row is
// shared by all query heads.  A latent row has 576 bf16 values; the key is
// the whole row, the value its first 512 entries.
//
// Work split.  A workgroup takes one query token, a group of 16*NW heads and
// one slice ("split") of the selected rows; the splits are merged afterwards
// by a log-sum-exp combine.  Per tile of 32 selected rows:
//   gather   the rows (1152 B each) go into LDS twice: row-major for the
//            scores, and the 512 value columns transposed (keys contiguous)
//            for the value product;
//   scores   S^T = K Q^T on 16x16x32 bf16 MFMAs: keys on M, this wave's 16
//            heads on N, the 576 dims on K.  A lane ends up holding one head
//            and 8 keys, so the online softmax max/sum need no shuffles
//            except two xor steps across the four lane groups;
//   values   O^T += V^T P^T: dims on M (32 tiles of 16), heads on N, the 32
//            keys on K.  The probabilities already sit in the B-operand
//            layout (one head per lane), so P never leaves registers, and the
//            per-head rescale of O is in-lane.
// The exponentials use exp2 with log2(e) folded into the scale.
#include "launch.h"

namespace dsa {

constexpr int AT_TILE = 32;
constexpr int AT_D = 576;
constexpr int AT_DV = 512;
constexpr int KS_STRIDE = 1168;  // bytes per row-major row in LDS (1152 + 16: rotates banks per row)
constexpr int VT_STRIDE = 72;    // bytes per transposed value row (32 keys * 2 + 8)
constexpr int KS_BYTES = AT_TILE * KS_STRIDE;
constexpr int VT_BYTES = AT_DV * VT_STRIDE;

__device__ __forceinline__ uint16_t f2bf(float f) {
  // round to nearest even (inputs here are finite)
  u32 u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int NW>
__global__ __launch_bounds__(NW * 64, 2) void sparse_mla_kernel(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ kv,
                                                               const int32_t* __restrict__ idx,
                                                               const int32_t* __restrict__ seq_id, Layout lay,
                                                               int H, int k, int split_len, int n_splits,
                                                               float scale_log2, uint16_t* __restrict__ out,
                                                               float* __restrict__ lse, float* __restrict__ ws_o,
                                                               float* __restrict__ ws_ml) {
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) uint8_t smem[KS_BYTES + VT_BYTES];
  __shared__ int s_valid[AT_TILE];
  uint8_t* const Ks = smem;
  uint8_t* const Vt = smem + KS_BYTES;

  const int split = blockIdx.x;
  const int t = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int h0 = blockIdx.y * (16 * NW) + wid * 16;  // first head of this wave
  const int b = seq_id[t];
  const int32_t* __restrict__ idx_row = idx + (int64_t)t * k;

  // Q^T operand: head h0+n, dims 32*ks + 8g .. +8
  v8bf qf[AT_D / 32];
  {
    const uint16_t* qrow = q + ((int64_t)t * H + h0 + n) * AT_D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < AT_D / 32; ++ks) qf[ks] = *reinterpret_cast<const v8bf*>(qrow + 32 * ks);
  }

  float m_run = -INFINITY;  // running max (log2 units) of head h0+n
  float l_part = 0.f;       // partial sum over this lane's keys
  v4f o[AT_DV / 16];
#pragma unroll
  for (int mt = 0; mt < AT_DV / 16; ++mt) o[mt] = v4f{0.f, 0.f, 0.f, 0.f};

  const int j_begin = split * split_len;
  const int j_end = min(k, j_begin + split_len);

  for (int j0 = j_begin; j0 < j_end; j0 += AT_TILE) {
    __syncthreads();  // previous tile fully consumed
    // ---- gather 32 rows: value part as (4 keys x 8 dims) groups, rope part row-major only
#pragma unroll
    for (int r = 0; r < (8 * 64) / NT; ++r) {
      const int gi = tid + NT * r;
      const int kq = gi & 7;   // key quad
      const int oc = gi >> 3;  // dim octet 0..63
      v4i c[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int j = j0 + 4 * kq + rr;
        int s = (j < j_end) ? idx_row[j] : -1;
        s = (s < 0) ? 0 : s;
        const int64_t row = token_row(lay, b, s);
        c[rr] = *reinterpret_cast<const v4i*>(kv + row * AT_D + 8 * oc);
        *reinterpret_cast<v4i*>(Ks + (4 * kq + rr) * KS_STRIDE + 16 * oc) = c[rr];
      }
      // transpose: dim 8*oc + d gets keys 4kq..4kq+3 (8 bytes)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const u32 a0 = (u32)c[0][m], a1 = (u32)c[1][m], a2 = (u32)c[2][m], a3 = (u32)c[3][m];
        v2i lo, hi;
        lo[0] = (int)((a0 & 0xFFFFu) | (a1 << 16));
        lo[1] = (int)((a2 & 0xFFFFu) | (a3 << 16));
        hi[0] = (int)((a0 >> 16) | (a1 & 0xFFFF0000u));
        hi[1] = (int)((a2 >> 16) | (a3 & 0xFFFF0000u));
        *reinterpret_cast<v2i*>(Vt + (8 * oc + 2 * m) * VT_STRIDE + 8 * kq) = lo;
        *reinterpret_cast<v2i*>(Vt + (8 * oc + 2 * m + 1) * VT_STRIDE + 8 * kq) = hi;
      }
    }
#pragma unroll
    for (int r = 0; r < (AT_TILE * 8) / NT; ++r) {
      const int gi = tid + NT * r;
      const int rowi = gi >> 3;
      const int oc = 64 + (gi & 7);
      const int j = j0 + rowi;
      int s = (j < j_end) ? idx_row[j] : -1;
      s = (s < 0) ? 0 : s;
      const int64_t row = token_row(lay, b, s);
      *reinterpret_cast<v4i*>(Ks + rowi * KS_STRIDE + 16 * oc) =
          *reinterpret_cast<const v4i*>(kv + row * AT_D + 8 * oc);
    }
    if (tid < AT_TILE) {
      const int j = j0 + tid;
      s_valid[tid] = (j < j_end) && (idx_row[j] >= 0);
    }
    __syncthreads();

    // ---- scores S^T (keys x heads)
    v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < AT_D / 32; ++ks) {
      const v8bf a0 = *reinterpret_cast<const v8bf*>(Ks + n * KS_STRIDE + 64 * ks + 16 * g);
      const v8bf a1 = *reinterpret_cast<const v8bf*>(Ks + (16 + n) * KS_STRIDE + 64 * ks + 16 * g);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ks], s1, 0, 0, 0);
    }
    // lane holds head n: s0[i] -> key 4g+i, s1[i] -> key 16+4g+i
    float z[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = s_valid[4 * g + i] ? s0[i] * scale_log2 : -INFINITY;
      z[4 + i] = s_valid[16 + 4 * g + i] ? s1[i] * scale_log2 : -INFINITY;
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

    // ---- values O^T += V^T P^T
#pragma unroll
    for (int mt = 0; mt < AT_DV / 16; ++mt) {
      const uint8_t* vrow = Vt + (mt * 16 + n) * VT_STRIDE;
      const v2i lo = *reinterpret_cast<const v2i*>(vrow + 8 * g);
      const v2i hi = *reinterpret_cast<const v2i*>(vrow + 32 + 8 * g);
      const v4i av = v4i{lo[0], lo[1], hi[0], hi[1]};
      v4f acc = o[mt] * corr;
      o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av), pb, acc, 0, 0, 0);
    }
  }

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

static int heads_per_wg(int H) { return H >= 64 ? 64 : H; }

int attn_splits(int T, int H, int k) {
  const int base = T * (H / heads_per_wg(H));
  const int tiles = (k + AT_TILE - 1) / AT_TILE;
  int s = 1;
  // each split keeps >= 8 tiles; stop once the grid reaches 256 workgroups
  while (base * s < 256 && tiles / (2 * s) >= 8) s *= 2;
  return s;
}

size_t attn_workspace_bytes(int T, int H, int k) {
  const int s = attn_splits(T, H, k);
  if (s == 1) return 0;
  const size_t slots = (size_t)T * s * H;
  return align256(slots * AT_DV * 4) + align256(slots * 2 * 4);
}

template <int NW>
static void launch_main(dim3 grid, hipStream_t stream, const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                        const int32_t* seq_id, const Layout& lay, int H, int k, int split_len, int n_splits,
                        float scale_log2, uint16_t* out, float* lse, float* ws_o, float* ws_ml) {
  hipLaunchKernelGGL((sparse_mla_kernel<NW>), grid, dim3(NW * 64), 0, stream, q, kv, idx, seq_id, lay, H, k,
                     split_len, n_splits, scale_log2, out, lse, ws_o, ws_ml);
}

hipError_t launch_attn(int T, int H, const uint16_t* q, const uint16_t* kv, const int32_t* idx, const int32_t* seq_id,
                       const Layout& lay, int k, float sm_scale, uint16_t* out, float* lse, void* ws,
                       hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int hpw = heads_per_wg(H);
  const int nw = hpw / 16;
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
  dim3 grid(n_splits, H / hpw, T);
  switch (nw) {
    case 1: launch_main<1>(grid, stream, q, kv, idx, seq_id, lay, H, k, split_len, n_splits, scale_log2, out, lse, ws_o, ws_ml); break;
    case 2: launch_main<2>(grid, stream, q, kv, idx, seq_id, lay, H, k, split_len, n_splits, scale_log2, out, lse, ws_o, ws_ml); break;
    case 4: launch_main<4>(grid, stream, q, kv, idx, seq_id, lay, H, k, split_len, n_splits, scale_log2, out, lse, ws_o, ws_ml); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_splits == 1) return e;
  const int TH = T * H;
  hipLaunchKernelGGL(combine_kernel, dim3((TH + 3) / 4), dim3(256), 0, stream, ws_o, ws_ml, TH, H, n_splits, out, lse);
  return hipGetLastError();
}

}  // namespace dsa
