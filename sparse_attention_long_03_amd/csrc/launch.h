// Internal launchers of the gfx950 kernels (called by the C ABI layer after
// validation).  Every launcher enqueues on `stream` and returns the launch
// status; none allocates memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace dsa {

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// A workspace layout: named regions, each starting on a 256-byte boundary at
// an offset from the workspace base.  Every call that takes a workspace
// computes both its stated size (total) and its pointers from one of these,
// so the two cannot disagree; dsa_workspace_layout reports them.  A region
// may hold a sub-step's own layout (add_sub); `flat` lists the leaf regions
// with offsets from this layout's base and the name of the region they sit in.
struct WsRegion {
  const char* parent;  // null for a region of this layout itself
  const char* name;
  size_t off, bytes;
};

struct WsLayout {
  static constexpr int MAX = 8, MAX_FLAT = 16;
  const char* name[MAX] = {};
  size_t off[MAX] = {};
  size_t bytes[MAX] = {};
  int n = 0;
  size_t total = 0;
  WsRegion flat[MAX_FLAT] = {};
  int nflat = 0;

  int add(const char* nm, size_t b) {
    name[n] = nm;
    off[n] = total;
    bytes[n] = b;
    total += align256(b);
    flat[nflat++] = WsRegion{nullptr, nm, off[n], b};
    return n++;
  }
  int add_sub(const char* nm, const WsLayout& sub) {
    const int i = add(nm, sub.total);
    --nflat;  // the container is reported through its regions
    for (int j = 0; j < sub.nflat; ++j) flat[nflat++] = WsRegion{nm, sub.flat[j].name, off[i] + sub.flat[j].off, sub.flat[j].bytes};
    return i;
  }
  int index(const char* nm) const {
    for (int i = 0; i < n; ++i) {
      const char *a = name[i], *b = nm;
      while (*a && *a == *b) ++a, ++b;
      if (*a == *b) return i;
    }
    return -1;
  }
  void* at(void* base, int i) const { return static_cast<char*>(base) + off[i]; }
};

// Layouts of the workspaces, one per operation (T == 0 gives an empty one)
WsLayout topk_layout(int T, int64_t max_len, int k);          // hist, counts, above, ckey, cpos
WsLayout fused_topk_layout(int T, int cap);                    // ckey, cpos
WsLayout attn_layout(int T, int H, int k);                     // o, ml (none with one split)
WsLayout dense_attn_layout(int T, int H, int max_len);         // o, ml (none with one split)
WsLayout scatter_layout(int64_t N);                            // keys_b, vals_a, vals_b, hist, totals
WsLayout attn_bwd_layout(int T, int H, int k);                 // dsp, slot_grad, rows, cnt, scatter
WsLayout kl_layout(int T, int k);                              // slot_dk, rows, scatter
WsLayout kl_target_dense_layout(int T, int H, int max_len);    // ml
WsLayout proj_layout(int T, int d, int H_I, int D_I);          // part


// (1) indexer logits; `hist` (nullable) receives the per-row 2048-bin
// histogram of the top 11 key bits (must be zeroed first).
bool indexer_supported(int H_I, int D_I);
hipError_t launch_indexer(int T, int max_len, int H_I, int D_I, const uint8_t* q8, const float* qs, const float* w,
                          const uint8_t* k8, const float* ks, const int32_t* seq_id, const int32_t* pos,
                          const Layout& lay, float* logits, int64_t ld, u32* hist, hipStream_t stream);

// (1+2) indexer fused with top-k (many query tokens): candidate lists of
// `cap` slots per token in the workspace (8 * T * cap bytes).
int fused_topk_cap(int max_len, int k);              // preferred capacity
int fused_topk_cap_from_bytes(int T, size_t bytes);  // capacity a workspace holds
size_t fused_topk_workspace_bytes(int T, int cap);
bool fused_topk_cap_ok(int cap, int k);
hipError_t launch_indexer_topk(int T, int max_len, int H_I, int D_I, const uint8_t* q8, const float* qs, const float* w,
                               const uint8_t* k8, const float* ks, const int32_t* seq_id, const int32_t* pos,
                               const Layout& lay, int k, int cap, int32_t* idx, void* ws, hipStream_t stream);

// (2) top-k; valid length of row t is valid_len[t] + len_add.  The histogram
// lives at the start of the top-k workspace (topk_hist_buffer); with
// hist_ready the caller has already filled it (fused indexer epilogue).
constexpr int64_t kTopkMaxLen = 4 * 1024 * 1024;  // longest row the selection handles
size_t topk_workspace_bytes(int T, int64_t max_len, int k);
u32* topk_hist_buffer(void* ws);
hipError_t launch_topk_zero_hist(void* ws, int T, hipStream_t stream);
hipError_t launch_topk(const float* logits, int64_t ld, const int32_t* valid_len, int len_add, int T, int max_len,
                       int k, int32_t* idx, void* ws, bool hist_ready, hipStream_t stream);

// (3) sparse MLA attention (+ split combine)
bool attn_supported(int H);
int attn_splits(int T, int H, int k);
size_t attn_workspace_bytes(int T, int H, int k);
hipError_t launch_attn(int T, int H, const uint16_t* q, const uint16_t* kv, const int32_t* idx, const int32_t* seq_id,
                       const Layout& lay, int k, float sm_scale, uint16_t* out, float* lse, void* ws,
                       hipStream_t stream);

// cache write: quantise new index keys to FP8 and store them (+ latent rows)
hipError_t launch_cache_write(int T, int D_I, const int32_t* seq_id, const int32_t* pos, const Layout& lay,
                              const float* k_new, const uint16_t* kv_new, uint8_t* k8, float* ks, uint16_t* kv,
                              hipStream_t stream);

// the indexer's inputs from hidden states: q (FP8 + per-token scale), w and
// optionally k, from bf16 h [T, d] and weights Wq [H_I*D_I, d], Ww [H_I, d],
// Wk [D_I, d]; fp32 partial sums in the workspace
bool proj_supported(int H_I, int D_I, int d);
size_t proj_workspace_bytes(int T, int d, int H_I, int D_I);
hipError_t launch_indexer_project(int T, int d, int H_I, int D_I, const uint16_t* h, const uint16_t* wq,
                                  const uint16_t* ww, const uint16_t* wk, uint8_t* q8, float* qs, float* w,
                                  float* k_new, void* ws, hipStream_t stream);

// (3') masked dense variant of (3): all positions 0..pos[t], unselected masked
bool dense_attn_supported(int max_len);
size_t dense_attn_workspace_bytes(int T, int H, int max_len);
hipError_t launch_dense_attn(int T, int H, const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                             const int32_t* seq_id, const int32_t* pos, const Layout& lay, int k, int max_len,
                             float sm_scale, uint16_t* out, float* lse, void* ws, hipStream_t stream);

// scatter-add of bf16 rows (W = 576 or 128 values) into an fp32 table:
// dst[rows[i]] += src_rows[i] for every i with rows[i] != 0xFFFFFFFF; rows is
// overwritten (it is the first buffer of the sort); num_rows bounds the ids.
size_t row_scatter_workspace_bytes(int64_t N);
hipError_t launch_row_scatter_add(u32* rows, int N, int64_t num_rows, const uint16_t* src_rows, int W, float* dst,
                                  void* ws, hipStream_t stream);

// (3) backward: dq, and the gradients of the selected rows added into dkv
// (fp32, 576 per cache row; num_rows = rows of the cache)
bool attn_bwd_supported(int H);
bool attn_bwd_size_ok(int T, int k);
size_t attn_bwd_workspace_bytes(int T, int H, int k);
hipError_t launch_attn_bwd_dq(int T, int H, const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                              const int32_t* seq_id, const Layout& lay, int k, float sm_scale, const uint16_t* out,
                              const float* lse, const uint16_t* dout, float* dq, void* ws, hipStream_t stream);
hipError_t launch_attn_bwd_dkv(int T, int H, const uint16_t* q, const uint16_t* dout, int64_t num_rows, int k,
                               float* dkv, void* ws, hipStream_t stream);

// indexer KL training signal: target (head-mean attention probabilities of
// the selected entries) and the loss with its gradients (H_I = 64, D_I = 128)
bool kl_supported(int H_I, int D_I);
bool kl_size_ok(int T, int k);
size_t kl_workspace_bytes(int T, int k);
hipError_t launch_kl_target(int T, int H, const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                            const int32_t* seq_id, const Layout& lay, int k, float sm_scale, const float* lse,
                            float* target, hipStream_t stream);
// the dense warm-up's target over every position 0..pos[t] (T x ld fp32),
// with the dense attention's lse computed on the way (workspace: per chunk of
// 2048 positions and head, a running max and sum)
size_t kl_target_dense_workspace_bytes(int T, int H, int max_len);
hipError_t launch_kl_target_dense(int T, int H, int max_len, const uint16_t* q, const uint16_t* kv,
                                  const int32_t* seq_id, const int32_t* pos, const Layout& lay, float sm_scale,
                                  float* target, int64_t ld, float* lse_out, void* ws, hipStream_t stream);
hipError_t launch_kl_target_dense_lse(int T, int H, int max_len, const uint16_t* q, const uint16_t* kv,
                                      const int32_t* seq_id, const int32_t* pos, const Layout& lay, float sm_scale,
                                      const float* lse, float* target, int64_t ld, hipStream_t stream);
hipError_t launch_kl(int T, const uint8_t* q8, const float* qs, const float* w, const uint8_t* k8, const float* ks,
                     const int32_t* idx, const int32_t* seq_id, const Layout& lay, int64_t num_rows, int k,
                     const float* target, float* loss, float* dq, float* dw, float* dk, void* ws,
                     hipStream_t stream);

}  // namespace dsa
