// The indexer's inputs from a token's hidden state, on gfx950 bf16 matrix
// cores.
//
// "DeepSeek V3.2-Exp Cuts Prolonged-Context Costs With DeepSeek Sparse
// Consideration (DSA)", part (1): for each query token h_t the indexer forms
// a few small heads q[t, j] and one weight w[t, j] per head, and every token
// has its own index key.  Read as linear maps of h_t without bias:
//   q[t] = Wq h_t (H_I * D_I values, head-major), w[t] = Ww h_t, k[t] = Wk h_t,
// with q then stored like an index key: e4m3fn codes and one float32 scale
// per token over all of its H_I * D_I values.
//
// Two kernels.
//   proj_gemm_kernel   [T x d] x [d x N] on 16x16x32 bf16 MFMAs, N the
//                      concatenated output columns (q, then w, then k).  A
//                      workgroup takes TM tokens x 64 or 128 columns (16 or 32 per wave)
//                      over one slice of the hidden dims: the h tile is staged
//                      in LDS (shared by the four waves), each wave streams
//                      its own weight rows straight into B fragments.  The
//                      hidden dims are split over gridDim.z slices when the
//                      grid would otherwise not fill the chip (decode: 16
//                      tokens stream 120 MB of weights), each slice writing
//                      fp32 partial sums to the workspace.
//   proj_finish_kernel one workgroup per token: the partial sums are added in
//                      slice order, the query's amax gives its scale, and its
//                      H_I * D_I values are encoded to FP8; w and k are written
//                      as float32.
#include "fp8_encode.h"
#include "launch.h"

namespace dsa {

constexpr int PJ_NT = 256;                  // threads per workgroup (4 waves)
constexpr int PJ_BK = 64;                   // hidden dims per stage
constexpr int PJ_ASTRIDE = PJ_BK * 2 + 16;  // bytes per staged h row (padded: rotates LDS banks)
constexpr int PJ_MAX_SPLITS = 8;

#ifndef LDS_AS
#define LDS_AS __attribute__((address_space(3)))
#endif

template <int TM, int JC>
__global__ __launch_bounds__(PJ_NT) void proj_gemm_kernel(const uint16_t* __restrict__ h,
                                                          const uint16_t* __restrict__ wq,
                                                          const uint16_t* __restrict__ ww,
                                                          const uint16_t* __restrict__ wk, int T, int d, int Nq,
                                                          int Nw, int N, int kchunk, float* __restrict__ part) {
  constexpr int MT = TM / 16;                         // 16-token tiles
  constexpr int BN = 4 * 16 * JC;                     // output columns per workgroup (16 JC per wave)
  constexpr int ACH = TM * (PJ_BK / 8);               // 16-byte chunks of one staged h tile
  constexpr int APER = (ACH + PJ_NT - 1) / PJ_NT;     // chunks per thread
  __shared__ __align__(16) uint8_t a_lds[2][TM * PJ_ASTRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int t0 = blockIdx.y * TM;
  const int k_begin = blockIdx.z * kchunk;
  const int nsteps = kchunk / PJ_BK;

  // the weight rows of this lane's JC output columns (columns past N read
  // the last one; their results are not stored)
  const int c0 = blockIdx.x * BN + wid * 16 * JC;
  const uint16_t* wrow[JC];
#pragma unroll
  for (int j = 0; j < JC; ++j) {
    const int col = min(c0 + 16 * j + n, N - 1);
    const uint16_t* base = col < Nq ? wq + (int64_t)col * d
                                    : (col < Nq + Nw ? ww + (int64_t)(col - Nq) * d : wk + (int64_t)(col - Nq - Nw) * d);
    wrow[j] = base + k_begin + 8 * g;
  }

  // h tile: row r = chunk / 8 (token t0 + r, rows past T read the last
  // token), 16-byte chunk c = chunk % 8 of the stage's 64 dims
  v4i areg[APER];
  auto a_load = [&](int step) {
#pragma unroll
    for (int r = 0; r < APER; ++r) {
      const int c = tid + PJ_NT * r;
      if (ACH % PJ_NT == 0 || c < ACH) {
        const int tok = min(t0 + (c >> 3), T - 1);
        areg[r] = *reinterpret_cast<const v4i*>(h + (int64_t)tok * d + k_begin + step * PJ_BK + 8 * (c & 7));
      }
    }
  };
  auto a_store = [&](int buf) {
#pragma unroll
    for (int r = 0; r < APER; ++r) {
      const int c = tid + PJ_NT * r;
      if (ACH % PJ_NT == 0 || c < ACH)
        *reinterpret_cast<LDS_AS v4i*>((LDS_AS uint8_t*)a_lds[buf] + (c >> 3) * PJ_ASTRIDE + 16 * (c & 7)) = areg[r];
    }
  };
  // B fragments of one stage: [column tile][half of the 64 dims]
  v4i breg[JC][2];
  auto b_load = [&](int step) {
#pragma unroll
    for (int j = 0; j < JC; ++j)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        breg[j][hh] = *reinterpret_cast<const v4i*>(wrow[j] + step * PJ_BK + 32 * hh);
  };

  v4f acc[MT][JC];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < JC; ++j) acc[mt][j] = v4f{0.f, 0.f, 0.f, 0.f};

  a_load(0);
  b_load(0);
  a_store(0);
  __syncthreads();
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    v4i bcur[JC][2];
#pragma unroll
    for (int j = 0; j < JC; ++j)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) bcur[j][hh] = breg[j][hh];
    const bool more = step + 1 < nsteps;
    if (more) {
      a_load(step + 1);
      b_load(step + 1);
    }
    const LDS_AS uint8_t* abuf = (const LDS_AS uint8_t*)a_lds[buf];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        // A fragment: token 16mt + n, dims 32hh + 8g .. +8 of the stage
        const v8bf a = *reinterpret_cast<const LDS_AS v8bf*>(abuf + (16 * mt + n) * PJ_ASTRIDE + 64 * hh + 16 * g);
#pragma unroll
        for (int j = 0; j < JC; ++j)
          acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(v8bf, bcur[j][hh]), acc[mt][j],
                                                               0, 0, 0);
      }
    if (more) a_store(buf ^ 1);
    __syncthreads();
  }

  // lane holds column c0 + 16j + n for tokens t0 + 16mt + 4g + i
  float* __restrict__ out = part + (int64_t)blockIdx.z * T * N;
#pragma unroll
  for (int j = 0; j < JC; ++j) {
    const int col = c0 + 16 * j + n;
    if (col >= N) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + 16 * mt + 4 * g + i;
        if (tok < T) out[(int64_t)tok * N + col] = acc[mt][j][i];
      }
  }
}

// V = Nq / NT query values per thread: from V = 4 on, groups of four
// consecutive values at 4 tid + 4 NT c (16-byte loads, consecutive threads
// on consecutive bytes), else single values at tid + NT e.  A wide query
// (8192 values) takes 1024 threads, so that all of a token's partial sums are
// in flight at once.  The split partial sums are added in split order, so
// the result does not depend on the launch.
template <int V, int NT>
__global__ __launch_bounds__(NT) void proj_finish_kernel(const float* __restrict__ part, int T, int N, int Nq,
                                                            int Nw, int Nk, int splits, uint8_t* __restrict__ q8,
                                                            float* __restrict__ qs, float* __restrict__ w,
                                                            float* __restrict__ k_new) {
  __shared__ float red[NT / 64];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const float* __restrict__ row = part + (int64_t)t * N;
  const int64_t zs = (int64_t)T * N;
  auto at = [&](int e) { return V >= 4 ? 4 * tid + 4 * NT * (e >> 2) + (e & 3) : tid + NT * e; };

  float v[V];
  if constexpr (V >= 4) {
#pragma unroll
    for (int c = 0; c < V / 4; ++c) {
      const float4 a = *reinterpret_cast<const float4*>(row + 4 * tid + 4 * NT * c);
      v[4 * c + 0] = a.x;
      v[4 * c + 1] = a.y;
      v[4 * c + 2] = a.z;
      v[4 * c + 3] = a.w;
    }
    for (int z = 1; z < splits; ++z)
#pragma unroll
      for (int c = 0; c < V / 4; ++c) {
        const float4 a = *reinterpret_cast<const float4*>(row + z * zs + 4 * tid + 4 * NT * c);
        v[4 * c + 0] += a.x;
        v[4 * c + 1] += a.y;
        v[4 * c + 2] += a.z;
        v[4 * c + 3] += a.w;
      }
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) v[e] = row[at(e)];
    for (int z = 1; z < splits; ++z)
#pragma unroll
      for (int e = 0; e < V; ++e) v[e] += row[z * zs + at(e)];
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < V; ++e) amax = fmaxf(amax, fabsf(v[e]));
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 64));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) amax = fmaxf(amax, red[i]);
  const float scale = e4m3fn_scale(amax);

  uint8_t* __restrict__ dst = q8 + (int64_t)t * Nq;
  if constexpr (V >= 4) {
#pragma unroll
    for (int c = 0; c < V / 4; ++c) {
      u32 word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) word |= e4m3fn_quantise(v[4 * c + e], scale) << (8 * e);
      *reinterpret_cast<u32*>(dst + 4 * tid + 4 * NT * c) = word;
    }
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) dst[at(e)] = (uint8_t)e4m3fn_quantise(v[e], scale);
  }
  if (tid == 0) qs[t] = scale;

  for (int j = tid; j < Nw + Nk; j += NT) {
    float s = row[Nq + j];
    for (int z = 1; z < splits; ++z) s += row[z * zs + Nq + j];
    if (j < Nw)
      w[(int64_t)t * Nw + j] = s;
    else
      k_new[(int64_t)t * Nk + (j - Nw)] = s;
  }
}

bool proj_supported(int H_I, int D_I, int d) {
  return indexer_supported(H_I, D_I) && d >= PJ_BK && d % PJ_BK == 0 && d <= (1 << 16);
}

static int proj_tm(int T) { return T <= 32 ? 16 : 64; }
// output columns per workgroup: with 16-token tiles (decode) one 16-column
// tile per wave, so that the weight stream is spread over twice as many
// workgroups (a read of this size reaches about 3.5 TB/s from 528 workgroups
// and 5.5 from 1024); two per wave otherwise
static int proj_bn(int T) { return proj_tm(T) == 16 ? 64 : 128; }

// splits of the hidden dims: enough workgroups to fill the chip (about 1024),
// each slice at least 256 dims and a whole number of stages
static int proj_splits(int T, int d, int H_I, int D_I) {
  const int N = H_I * D_I + H_I + D_I;
  const int base = ((N + proj_bn(T) - 1) / proj_bn(T)) * ((T + proj_tm(T) - 1) / proj_tm(T));
  int s = 1;
  while (base * s < 1024 && 2 * s <= PJ_MAX_SPLITS && d % (2 * s * PJ_BK) == 0 && d / (2 * s) >= 256) s *= 2;
  return s;
}

// fp32 partial sums per hidden-dim slice (N = H_I D_I + H_I + D_I columns;
// the key columns are carved whether or not the call asks for the key)
WsLayout proj_layout(int T, int d, int H_I, int D_I) {
  WsLayout L;
  const size_t N = (size_t)H_I * D_I + H_I + D_I;
  L.add("part", (size_t)proj_splits(T, d, H_I, D_I) * T * N * 4);
  return L;
}

size_t proj_workspace_bytes(int T, int d, int H_I, int D_I) { return proj_layout(T, d, H_I, D_I).total; }

hipError_t launch_indexer_project(int T, int d, int H_I, int D_I, const uint16_t* h, const uint16_t* wq,
                                  const uint16_t* ww, const uint16_t* wk, uint8_t* q8, float* qs, float* w,
                                  float* k_new, void* ws, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int Nq = H_I * D_I, Nw = H_I, Nk = wk != nullptr ? D_I : 0;
  const int N = Nq + Nw + Nk;
  const int splits = proj_splits(T, d, H_I, D_I);
  const int kchunk = d / splits;
  const int tm = proj_tm(T);
  float* part = static_cast<float*>(proj_layout(T, d, H_I, D_I).at(ws, 0));
  const int bn = proj_bn(T);
  const dim3 grid((N + bn - 1) / bn, (T + tm - 1) / tm, splits);
  if (tm == 16)
    hipLaunchKernelGGL((proj_gemm_kernel<16, 1>), grid, dim3(PJ_NT), 0, stream, h, wq, ww, wk, T, d, Nq, Nw, N, kchunk,
                       part);
  else
    hipLaunchKernelGGL((proj_gemm_kernel<64, 2>), grid, dim3(PJ_NT), 0, stream, h, wq, ww, wk, T, d, Nq, Nw, N, kchunk,
                       part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
#define DSA_PJ_FINISH(VV, NTT)                                                                                  \
  hipLaunchKernelGGL((proj_finish_kernel<VV, NTT>), dim3(T), dim3(NTT), 0, stream, part, T, N, Nq, Nw, Nk, splits, q8, \
                     qs, w, k_new)
  switch (Nq) {
    case 8192: DSA_PJ_FINISH(8, 1024); break;
    case 4096: DSA_PJ_FINISH(4, 1024); break;
    case 512: DSA_PJ_FINISH(2, 256); break;
    case 256: DSA_PJ_FINISH(1, 256); break;
    default: return hipErrorInvalidValue;
  }
#undef DSA_PJ_FINISH
  return hipGetLastError();
}

}  // namespace dsa
