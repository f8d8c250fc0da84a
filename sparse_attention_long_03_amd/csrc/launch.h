// Internal launchers of the gfx950 kernels (called by the C ABI layer after
// validation).  Every launcher enqueues on `stream` and returns the launch
// status; none allocates memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace dsa {

// (1) indexer logits; returns false if (H_I, D_I) has no built kernel.
bool indexer_supported(int H_I, int D_I);
hipError_t launch_indexer(int T, int max_len, int H_I, int D_I, const uint8_t* q8, const float* qs, const float* w,
                          const uint8_t* k8, const float* ks, const int32_t* seq_id, const int32_t* pos,
                          const Layout& lay, float* logits, int64_t ld, hipStream_t stream);

// (2) top-k; valid length of row t is valid_len[t] + len_add.
size_t topk_workspace_bytes(int T, int64_t ld);
hipError_t launch_topk(const float* logits, int64_t ld, const int32_t* valid_len, int len_add, int T, int k,
                       int32_t* idx, void* ws, hipStream_t stream);

// (3) sparse MLA attention (+ split combine)
bool attn_supported(int H);
int attn_splits(int T, int H, int k);
size_t attn_workspace_bytes(int T, int H, int k);
hipError_t launch_attn(int T, int H, const uint16_t* q, const uint16_t* kv, const int32_t* idx, const int32_t* seq_id,
                       const Layout& lay, int k, float sm_scale, uint16_t* out, float* lse, void* ws,
                       hipStream_t stream);

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace dsa
