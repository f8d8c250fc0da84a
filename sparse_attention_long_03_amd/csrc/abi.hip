// C ABI of the DSA path: host-side validation, workspace carving, dispatch.
// Validation runs before any HIP call, so every error path can be exercised
// without a GPU.  Nothing here allocates memory.
//
// dsa_forward chains the method's steps in the order of "DeepSeek V3.2-Exp
// Cuts Prolonged-Context Costs With DeepSeek Sparse Consideration (DSA)":
// (1) the lightning indexer's logits, (2) the top-k selection and the
// attention over the selected entries, under MLA in MQA mode
// ("Instantiation").
#include <mutex>

#include "dsa.h"
#include "launch.h"

using namespace dsa;

namespace {

constexpr int kMaxK = 2048;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_queries(const dsa_queries* q) {
  if (q == nullptr) return DSA_ERR_INVALID_ARG;
  if (q->T < 0 || q->B < 1 || q->max_len < 0) return DSA_ERR_INVALID_ARG;
  if (q->max_len > kTopkMaxLen) return DSA_ERR_UNSUPPORTED;
  if (q->T > 0 && (q->seq_id == nullptr || q->pos == nullptr || q->max_len < 1)) return DSA_ERR_INVALID_ARG;
  return DSA_OK;
}

int check_layout(const dsa_kv_layout* l, const dsa_queries* q, Layout* out) {
  if (l == nullptr) return DSA_ERR_INVALID_ARG;
  if (l->paged != 0 && l->paged != 1) return DSA_ERR_INVALID_ARG;
  if (l->paged) {
    if (l->block_table == nullptr || l->max_pages < 1 || l->num_pages < 1) return DSA_ERR_INVALID_ARG;
    if (l->page_size != 64) return DSA_ERR_UNSUPPORTED;
    if ((int64_t)l->max_pages * 64 < q->max_len) return DSA_ERR_INVALID_ARG;
  } else {
    if (l->seq_capacity < q->max_len || l->seq_capacity < 1) return DSA_ERR_INVALID_ARG;
  }
  out->block_table = l->block_table;
  out->seq_capacity = l->seq_capacity;
  out->max_pages = l->max_pages;
  out->paged = l->paged;
  return DSA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

// dsa_forward selects from the logits as they are produced (no logits
// buffer) once the batch has this many query tokens: enough workgroups of 8
// tokens to fill the chip, and the row-per-token logits would be large.
constexpr int32_t kFusedMinT = 2048;

bool forward_fused(int32_t T) { return T >= kFusedMinT; }

// dsa_forward's workspace: the selection (when the caller passes no idx_out),
// then either the fused selection's candidate lists (from kFusedMinT query
// tokens) or the logits and the top-k workspace, then the attention's split
// partials.
WsLayout forward_layout(int32_t T, int32_t max_len, int32_t H, int32_t k, bool with_idx) {
  const int64_t ld = ((int64_t)max_len + 3) & ~int64_t(3);
  WsLayout L;
  if (with_idx) L.add("sel", (size_t)T * k * 4);
  if (forward_fused(T)) {
    L.add_sub("fused", fused_topk_layout(T, fused_topk_cap(max_len, k)));
  } else {
    L.add("logits", (size_t)T * ld * 4);
    L.add_sub("topk", topk_layout(T, max_len, k));
  }
  L.add_sub("attn", attn_layout(T, H, k));
  return L;
}

size_t forward_ws(int32_t T, int32_t max_len, int32_t H, int32_t k, bool with_idx) {
  return forward_layout(T, max_len, H, k, with_idx).total;
}

// the indexer's inputs (shared by the logits and the fused selection calls)
int validate_indexer_inputs(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H_I, int32_t D_I,
                            const uint8_t* q_fp8, const float* q_scale, const float* w, const uint8_t* k_fp8,
                            const float* k_scale, Layout* lay) {
  int st = check_queries(q);
  if (st) return st;
  if ((st = check_layout(layout, q, lay))) return st;
  if (H_I < 1 || D_I < 1) return DSA_ERR_INVALID_ARG;
  if (!indexer_supported(H_I, D_I)) return DSA_ERR_UNSUPPORTED;
  if (q->T == 0) return DSA_OK;
  if (!q_fp8 || !q_scale || !w || !k_fp8 || !k_scale) return DSA_ERR_INVALID_ARG;
  if (!aligned(q_fp8, 16) || !aligned(k_fp8, 16)) return DSA_ERR_INVALID_ARG;
  return DSA_OK;
}

int validate_indexer(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H_I, int32_t D_I,
                     const uint8_t* q_fp8, const float* q_scale, const float* w, const uint8_t* k_fp8,
                     const float* k_scale, const float* logits, int64_t ld, Layout* lay) {
  int st = validate_indexer_inputs(q, layout, H_I, D_I, q_fp8, q_scale, w, k_fp8, k_scale, lay);
  if (st || q->T == 0) return st;
  if (!logits || !aligned(logits, 16)) return DSA_ERR_INVALID_ARG;
  if (ld < q->max_len || (ld & 3)) return DSA_ERR_INVALID_ARG;
  return DSA_OK;
}

int validate_attn(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H, const void* q_bf16,
                  const void* kv_bf16, const int32_t* idx, int32_t k, float sm_scale, const void* out, Layout* lay) {
  int st = check_queries(q);
  if (st) return st;
  if ((st = check_layout(layout, q, lay))) return st;
  if (H < 1 || k < 1) return DSA_ERR_INVALID_ARG;
  if (!(sm_scale > 0.f) || sm_scale != sm_scale) return DSA_ERR_INVALID_ARG;
  if (k > kMaxK || !attn_supported(H)) return DSA_ERR_UNSUPPORTED;
  if (q->T == 0) return DSA_OK;
  if (!q_bf16 || !kv_bf16 || !idx || !out) return DSA_ERR_INVALID_ARG;
  if (!aligned(q_bf16, 16) || !aligned(kv_bf16, 16) || !aligned(out, 16)) return DSA_ERR_INVALID_ARG;
  return DSA_OK;
}

}  // namespace

extern "C" {

int32_t dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_status_str(int32_t status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARG: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported shape or option";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_HIP: return "HIP launch error";
    case DSA_ERR_SCRATCH_LIMIT: return "request exceeds the no-allocation entry point's static scratch (64 MiB per GPU)";
    default: return "unknown status";
  }
}

size_t dsa_workspace_bytes(int32_t op, int32_t T, int32_t max_len, int32_t H, int32_t k) {
  if (T < 0 || max_len < 0 || H < 0 || k < 0) return 0;
  const int64_t ld = ((int64_t)max_len + 3) & ~int64_t(3);
  switch (op) {
    case DSA_OP_TOPK: return (k > 0) ? topk_workspace_bytes(T, max_len, k) : 0;
    case DSA_OP_ATTN: return (H > 0 && k > 0) ? attn_workspace_bytes(T, H, k) : 0;
    case DSA_OP_FORWARD: return (H > 0 && k > 0) ? forward_ws(T, max_len, H, k, true) : 0;
    case DSA_OP_INDEXER_TOPK: return (k > 0) ? fused_topk_workspace_bytes(T, fused_topk_cap(max_len, k)) : 0;
    case DSA_OP_DENSE_ATTN: return (H > 0) ? dense_attn_workspace_bytes(T, H, max_len) : 0;
    case DSA_OP_ATTN_BWD: return (H > 0 && k > 0 && attn_bwd_size_ok(T, k)) ? attn_bwd_workspace_bytes(T, H, k) : 0;
    case DSA_OP_INDEXER_KL: return (k > 0 && kl_size_ok(T, k)) ? kl_workspace_bytes(T, k) : 0;
    case DSA_OP_KL_TARGET_DENSE: return (H > 0 && max_len > 0) ? kl_target_dense_workspace_bytes(T, H, max_len) : 0;
    case DSA_OP_INDEXER_PROJ:  // (T, d, H_I, D_I)
      return proj_supported(H, k, max_len) ? proj_workspace_bytes(T, max_len, H, k) : 0;
    default: return 0;
  }
}

int32_t dsa_workspace_layout(int32_t op, int32_t T, int32_t max_len, int32_t H, int32_t k, dsa_ws_region* regions,
                             int32_t max_regions) {
  if (T < 0 || max_len < 0 || H < 0 || k < 0 || max_regions < 0 || (max_regions > 0 && regions == nullptr))
    return DSA_ERR_INVALID_ARG;
  if (dsa_workspace_bytes(op, T, max_len, H, k) == 0) return 0;  // none needed, or not supported
  WsLayout L;
  switch (op) {
    case DSA_OP_TOPK: L = topk_layout(T, max_len, k); break;
    case DSA_OP_ATTN: L = attn_layout(T, H, k); break;
    case DSA_OP_FORWARD: L = forward_layout(T, max_len, H, k, true); break;
    case DSA_OP_INDEXER_TOPK: L = fused_topk_layout(T, fused_topk_cap(max_len, k)); break;
    case DSA_OP_DENSE_ATTN: L = dense_attn_layout(T, H, max_len); break;
    case DSA_OP_ATTN_BWD: L = attn_bwd_layout(T, H, k); break;
    case DSA_OP_INDEXER_KL: L = kl_layout(T, k); break;
    case DSA_OP_KL_TARGET_DENSE: L = kl_target_dense_layout(T, H, max_len); break;
    case DSA_OP_INDEXER_PROJ: L = proj_layout(T, max_len, H, k); break;  // (T, d, H_I, D_I)
    default: return DSA_ERR_INVALID_ARG;
  }
  for (int i = 0; i < L.nflat && i < max_regions; ++i)
    regions[i] = dsa_ws_region{L.flat[i].parent, L.flat[i].name, (uint64_t)L.flat[i].off, (uint64_t)L.flat[i].bytes};
  return L.nflat;
}

int dsa_indexer_logits(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H_I, int32_t D_I,
                       const uint8_t* q_fp8, const float* q_scale, const float* w, const uint8_t* k_fp8,
                       const float* k_scale, float* logits, int64_t ld_logits, hipStream_t stream) {
  Layout lay;
  int st = validate_indexer(q, layout, H_I, D_I, q_fp8, q_scale, w, k_fp8, k_scale, logits, ld_logits, &lay);
  if (st || q->T == 0) return st;
  return hip_status(launch_indexer(q->T, q->max_len, H_I, D_I, q_fp8, q_scale, w, k_fp8, k_scale, q->seq_id, q->pos,
                                   lay, logits, ld_logits, nullptr, stream));
}

int dsa_indexer_topk(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H_I, int32_t D_I,
                     const uint8_t* q_fp8, const float* q_scale, const float* w, const uint8_t* k_fp8,
                     const float* k_scale, int32_t k, int32_t* idx, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  Layout lay;
  int st = validate_indexer_inputs(q, layout, H_I, D_I, q_fp8, q_scale, w, k_fp8, k_scale, &lay);
  if (st) return st;
  if (k < 1) return DSA_ERR_INVALID_ARG;
  if (k > kMaxK) return DSA_ERR_UNSUPPORTED;
  if (q->T == 0) return DSA_OK;
  if (idx == nullptr) return DSA_ERR_INVALID_ARG;
  const int cap = fused_topk_cap_from_bytes(q->T, workspace_bytes);
  if (workspace == nullptr || !aligned(workspace, 256) || !fused_topk_cap_ok(cap, k)) return DSA_ERR_WORKSPACE;
  return hip_status(launch_indexer_topk(q->T, q->max_len, H_I, D_I, q_fp8, q_scale, w, k_fp8, k_scale, q->seq_id, q->pos, lay, k,
                                        cap, idx, workspace, stream));
}

int dsa_cache_write(const dsa_queries* q, const dsa_kv_layout* layout, int32_t D_I, const float* k_new,
                    const void* kv_new_bf16, uint8_t* k_fp8, float* k_scale, void* kv_bf16, hipStream_t stream) {
  Layout lay;
  int st = check_queries(q);
  if (st) return st;
  if ((st = check_layout(layout, q, &lay))) return st;
  if (D_I < 1) return DSA_ERR_INVALID_ARG;
  if (D_I != 64 && D_I != 128) return DSA_ERR_UNSUPPORTED;
  if ((kv_new_bf16 == nullptr) != (kv_bf16 == nullptr)) return DSA_ERR_INVALID_ARG;
  if (q->T == 0) return DSA_OK;
  if (!k_new || !k_fp8 || !k_scale) return DSA_ERR_INVALID_ARG;
  if (!aligned(k_fp8, 16) || (kv_bf16 && (!aligned(kv_bf16, 16) || !aligned(kv_new_bf16, 16))))
    return DSA_ERR_INVALID_ARG;
  return hip_status(launch_cache_write(q->T, D_I, q->seq_id, q->pos, lay, k_new,
                                      static_cast<const uint16_t*>(kv_new_bf16), k_fp8, k_scale,
                                      static_cast<uint16_t*>(kv_bf16), stream));
}

int dsa_indexer_project(int32_t T, int32_t d, int32_t H_I, int32_t D_I, const void* h_bf16, const void* wq_bf16,
                        const void* ww_bf16, const void* wk_bf16, uint8_t* q_fp8, float* q_scale, float* w,
                        float* k_new, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (T < 0 || d < 1 || H_I < 1 || D_I < 1) return DSA_ERR_INVALID_ARG;
  if (!proj_supported(H_I, D_I, d)) return DSA_ERR_UNSUPPORTED;
  if ((wk_bf16 == nullptr) != (k_new == nullptr)) return DSA_ERR_INVALID_ARG;
  if (T == 0) return DSA_OK;
  if (!h_bf16 || !wq_bf16 || !ww_bf16 || !q_fp8 || !q_scale || !w) return DSA_ERR_INVALID_ARG;
  if (!aligned(h_bf16, 16) || !aligned(wq_bf16, 16) || !aligned(ww_bf16, 16) || !aligned(q_fp8, 16) ||
      (wk_bf16 && !aligned(wk_bf16, 16)))
    return DSA_ERR_INVALID_ARG;
  const size_t need = proj_workspace_bytes(T, d, H_I, D_I);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256)) return DSA_ERR_WORKSPACE;
  return hip_status(launch_indexer_project(T, d, H_I, D_I, static_cast<const uint16_t*>(h_bf16),
                                           static_cast<const uint16_t*>(wq_bf16), static_cast<const uint16_t*>(ww_bf16),
                                           static_cast<const uint16_t*>(wk_bf16), q_fp8, q_scale, w, k_new, workspace,
                                           stream));
}

int dsa_topk(const float* logits, int64_t ld_logits, const int32_t* valid_len, int32_t T, int32_t max_len,
             int32_t k, int32_t* idx, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (T < 0 || max_len < 0 || k < 1) return DSA_ERR_INVALID_ARG;
  if (k > kMaxK || max_len > kTopkMaxLen) return DSA_ERR_UNSUPPORTED;
  if (T == 0) return DSA_OK;
  if (!logits || !valid_len || !idx) return DSA_ERR_INVALID_ARG;
  if (ld_logits < max_len || (ld_logits & 3) || !aligned(logits, 16)) return DSA_ERR_INVALID_ARG;
  const size_t need = topk_workspace_bytes(T, max_len, k);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256)) return DSA_ERR_WORKSPACE;
  return hip_status(launch_topk(logits, ld_logits, valid_len, 0, T, max_len, k, idx, workspace, false, stream));
}

int dsa_sparse_mla_attn(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H, const void* q_bf16,
                        const void* kv_bf16, const int32_t* idx, int32_t k, float sm_scale, void* out_bf16,
                        float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Layout lay;
  int st = validate_attn(q, layout, H, q_bf16, kv_bf16, idx, k, sm_scale, out_bf16, &lay);
  if (st || q->T == 0) return st;
  const size_t need = attn_workspace_bytes(q->T, H, k);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256)))
    return DSA_ERR_WORKSPACE;
  return hip_status(launch_attn(q->T, H, static_cast<const uint16_t*>(q_bf16), static_cast<const uint16_t*>(kv_bf16),
                                idx, q->seq_id, lay, k, sm_scale, static_cast<uint16_t*>(out_bf16), lse, workspace,
                                stream));
}

int dsa_masked_dense_attn(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H, const void* q_bf16,
                          const void* kv_bf16, const int32_t* idx, int32_t k, float sm_scale, void* out_bf16,
                          float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Layout lay;
  int st = validate_attn(q, layout, H, q_bf16, kv_bf16, idx, k, sm_scale, out_bf16, &lay);
  if (st) return st;
  if (!dense_attn_supported(q->max_len)) return DSA_ERR_UNSUPPORTED;
  if (q->T == 0) return DSA_OK;
  const size_t need = dense_attn_workspace_bytes(q->T, H, q->max_len);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256)))
    return DSA_ERR_WORKSPACE;
  return hip_status(launch_dense_attn(q->T, H, static_cast<const uint16_t*>(q_bf16),
                                      static_cast<const uint16_t*>(kv_bf16), idx, q->seq_id, q->pos, lay, k,
                                      q->max_len, sm_scale, static_cast<uint16_t*>(out_bf16), lse, workspace, stream));
}

namespace {

// Validation shared by the backward entry points.  `need_fwd` covers the
// arguments of the dq step (kv, idx, out, lse, dq), `need_dkv` those of the
// dkv step (dkv).  Fills lay and num_rows.
int validate_bwd(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H, const void* q_bf16,
                 const void* kv_bf16, const int32_t* idx, int32_t k, float sm_scale, const void* out_bf16,
                 const float* lse, const void* d_out_bf16, const float* dq, const float* dkv, const void* workspace,
                 size_t workspace_bytes, bool need_fwd, bool need_dkv, Layout* lay, int64_t* num_rows) {
  int st = check_queries(q);
  if (st) return st;
  if ((st = check_layout(layout, q, lay))) return st;
  if (H < 1 || k < 1) return DSA_ERR_INVALID_ARG;
  if (!(sm_scale > 0.f) || sm_scale != sm_scale) return DSA_ERR_INVALID_ARG;
  if (k > kMaxK || !attn_bwd_supported(H)) return DSA_ERR_UNSUPPORTED;
  *num_rows = layout->paged ? (int64_t)layout->num_pages * 64 : (int64_t)q->B * layout->seq_capacity;
  if (*num_rows >= (int64_t(1) << 31) || !attn_bwd_size_ok(q->T, k)) return DSA_ERR_UNSUPPORTED;
  if (q->T == 0) return DSA_OK;
  if (!q_bf16 || !d_out_bf16 || !aligned(q_bf16, 16) || !aligned(d_out_bf16, 16)) return DSA_ERR_INVALID_ARG;
  if (need_fwd) {
    if (!kv_bf16 || !idx || !out_bf16 || !lse || !dq) return DSA_ERR_INVALID_ARG;
    if (!aligned(kv_bf16, 16) || !aligned(out_bf16, 16) || !aligned(dq, 16)) return DSA_ERR_INVALID_ARG;
  }
  if (need_dkv && (!dkv || !aligned(dkv, 16))) return DSA_ERR_INVALID_ARG;
  const size_t need = attn_bwd_workspace_bytes(q->T, H, k);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256)) return DSA_ERR_WORKSPACE;
  return DSA_OK;
}

}  // namespace

int dsa_sparse_mla_attn_bwd(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H, const void* q_bf16,
                            const void* kv_bf16, const int32_t* idx, int32_t k, float sm_scale, const void* out_bf16,
                            const float* lse, const void* d_out_bf16, float* dq, float* dkv, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  Layout lay;
  int64_t num_rows;
  int st = validate_bwd(q, layout, H, q_bf16, kv_bf16, idx, k, sm_scale, out_bf16, lse, d_out_bf16, dq, dkv,
                        workspace, workspace_bytes, true, true, &lay, &num_rows);
  if (st || q->T == 0) return st;
  const uint16_t* qb = static_cast<const uint16_t*>(q_bf16);
  const uint16_t* dob = static_cast<const uint16_t*>(d_out_bf16);
  hipError_t e = launch_attn_bwd_dq(q->T, H, qb, static_cast<const uint16_t*>(kv_bf16), idx, q->seq_id, lay, k,
                                    sm_scale, static_cast<const uint16_t*>(out_bf16), lse, dob, dq, workspace, stream);
  if (e != hipSuccess) return DSA_ERR_HIP;
  return hip_status(launch_attn_bwd_dkv(q->T, H, qb, dob, num_rows, k, dkv, workspace, stream));
}

int dsa_sparse_mla_attn_bwd_dq(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H, const void* q_bf16,
                               const void* kv_bf16, const int32_t* idx, int32_t k, float sm_scale,
                               const void* out_bf16, const float* lse, const void* d_out_bf16, float* dq,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Layout lay;
  int64_t num_rows;
  int st = validate_bwd(q, layout, H, q_bf16, kv_bf16, idx, k, sm_scale, out_bf16, lse, d_out_bf16, dq, nullptr,
                        workspace, workspace_bytes, true, false, &lay, &num_rows);
  if (st || q->T == 0) return st;
  return hip_status(launch_attn_bwd_dq(q->T, H, static_cast<const uint16_t*>(q_bf16),
                                       static_cast<const uint16_t*>(kv_bf16), idx, q->seq_id, lay, k, sm_scale,
                                       static_cast<const uint16_t*>(out_bf16), lse,
                                       static_cast<const uint16_t*>(d_out_bf16), dq, workspace, stream));
}

int dsa_sparse_mla_attn_bwd_dkv(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H, const void* q_bf16,
                                int32_t k, const void* d_out_bf16, float* dkv, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  Layout lay;
  int64_t num_rows;
  int st = validate_bwd(q, layout, H, q_bf16, nullptr, nullptr, k, 1.f, nullptr, nullptr, d_out_bf16, nullptr, dkv,
                        workspace, workspace_bytes, false, true, &lay, &num_rows);
  if (st || q->T == 0) return st;
  return hip_status(launch_attn_bwd_dkv(q->T, H, static_cast<const uint16_t*>(q_bf16),
                                        static_cast<const uint16_t*>(d_out_bf16), num_rows, k, dkv, workspace,
                                        stream));
}

int dsa_indexer_kl_target(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H, const void* q_bf16,
                          const void* kv_bf16, const int32_t* idx, int32_t k, float sm_scale, const float* lse,
                          float* target, hipStream_t stream) {
  Layout lay;
  int st = validate_attn(q, layout, H, q_bf16, kv_bf16, idx, k, sm_scale, target, &lay);
  if (st || q->T == 0) return st;
  if (!lse || !aligned(target, 4)) return DSA_ERR_INVALID_ARG;
  return hip_status(launch_kl_target(q->T, H, static_cast<const uint16_t*>(q_bf16),
                                     static_cast<const uint16_t*>(kv_bf16), idx, q->seq_id, lay, k, sm_scale, lse,
                                     target, stream));
}

int dsa_indexer_kl_target_dense(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H, const void* q_bf16,
                                const void* kv_bf16, float sm_scale, float* target, int64_t ld_target, float* lse_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Layout lay;
  int st = check_queries(q);
  if (st) return st;
  if ((st = check_layout(layout, q, &lay))) return st;
  if (H < 1 || !(sm_scale > 0.f)) return DSA_ERR_INVALID_ARG;
  if (!attn_supported(H)) return DSA_ERR_UNSUPPORTED;
  if (q->T == 0) return DSA_OK;
  if (!q_bf16 || !kv_bf16 || !target || !aligned(q_bf16, 16) || !aligned(kv_bf16, 16) || !aligned(target, 4))
    return DSA_ERR_INVALID_ARG;
  if (ld_target < q->max_len) return DSA_ERR_INVALID_ARG;
  const size_t need = kl_target_dense_workspace_bytes(q->T, H, q->max_len);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256)) return DSA_ERR_WORKSPACE;
  return hip_status(launch_kl_target_dense(q->T, H, q->max_len, static_cast<const uint16_t*>(q_bf16),
                                           static_cast<const uint16_t*>(kv_bf16), q->seq_id, q->pos, lay, sm_scale,
                                           target, ld_target, lse_out, workspace, stream));
}

int dsa_indexer_kl_target_dense_lse(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H,
                                    const void* q_bf16, const void* kv_bf16, float sm_scale, const float* lse,
                                    float* target, int64_t ld_target, hipStream_t stream) {
  Layout lay;
  int st = check_queries(q);
  if (st) return st;
  if ((st = check_layout(layout, q, &lay))) return st;
  if (H < 1 || !(sm_scale > 0.f)) return DSA_ERR_INVALID_ARG;
  if (!attn_supported(H)) return DSA_ERR_UNSUPPORTED;
  if (q->T == 0) return DSA_OK;
  if (!q_bf16 || !kv_bf16 || !lse || !target || !aligned(q_bf16, 16) || !aligned(kv_bf16, 16) || !aligned(lse, 4) ||
      !aligned(target, 4))
    return DSA_ERR_INVALID_ARG;
  if (ld_target < q->max_len) return DSA_ERR_INVALID_ARG;
  return hip_status(launch_kl_target_dense_lse(q->T, H, q->max_len, static_cast<const uint16_t*>(q_bf16),
                                               static_cast<const uint16_t*>(kv_bf16), q->seq_id, q->pos, lay,
                                               sm_scale, lse, target, ld_target, stream));
}

int dsa_indexer_kl(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H_I, int32_t D_I,
                   const uint8_t* q_fp8, const float* q_scale, const float* w, const uint8_t* k_fp8,
                   const float* k_scale, const int32_t* idx, int32_t k, const float* target, float* loss, float* dq,
                   float* dw, float* dk, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Layout lay;
  int st = validate_indexer_inputs(q, layout, H_I, D_I, q_fp8, q_scale, w, k_fp8, k_scale, &lay);
  if (st) return st;
  if (!kl_supported(H_I, D_I)) return DSA_ERR_UNSUPPORTED;
  if (k < 1) return DSA_ERR_INVALID_ARG;
  const int64_t num_rows = layout->paged ? (int64_t)layout->num_pages * 64 : (int64_t)q->B * layout->seq_capacity;
  if (k > kMaxK || num_rows >= (int64_t(1) << 31) || !kl_size_ok(q->T, k)) return DSA_ERR_UNSUPPORTED;
  if (q->T == 0) return DSA_OK;
  if (!idx || !target || !loss || !dq || !dw || !dk) return DSA_ERR_INVALID_ARG;
  if (!aligned(dk, 16) || !aligned(dq, 16)) return DSA_ERR_INVALID_ARG;
  const size_t need = kl_workspace_bytes(q->T, k);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256)) return DSA_ERR_WORKSPACE;
  return hip_status(launch_kl(q->T, q_fp8, q_scale, w, k_fp8, k_scale, idx, q->seq_id, lay, num_rows, k, target, loss,
                              dq, dw, dk, workspace, stream));
}

}  // extern "C"

// The static scratch of dsa_forward_noalloc: one copy per GPU, held until the
// process ends.  Host code never uses the symbol's name as an address: the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken once
// per device with that device current, and kept per device below.
static __device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace {

// dsa_forward's argument checks, shared with dsa_forward_noalloc.  Fills lay.
int validate_forward(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H_I, int32_t D_I,
                     const uint8_t* iq_fp8, const float* iq_scale, const float* iw, const uint8_t* ik_fp8,
                     const float* ik_scale, int32_t H, const void* q_bf16, const void* kv_bf16, int32_t k,
                     float sm_scale, const void* out_bf16, Layout* lay) {
  int st = check_queries(q);
  if (st) return st;
  if ((st = check_layout(layout, q, lay))) return st;
  if (H_I < 1 || D_I < 1 || H < 1 || k < 1) return DSA_ERR_INVALID_ARG;
  if (!(sm_scale > 0.f)) return DSA_ERR_INVALID_ARG;
  if (!indexer_supported(H_I, D_I) || !attn_supported(H) || k > kMaxK) return DSA_ERR_UNSUPPORTED;
  if (q->T == 0) return DSA_OK;
  if (!iq_fp8 || !iq_scale || !iw || !ik_fp8 || !ik_scale || !q_bf16 || !kv_bf16 || !out_bf16)
    return DSA_ERR_INVALID_ARG;
  if (!aligned(iq_fp8, 16) || !aligned(ik_fp8, 16) || !aligned(q_bf16, 16) || !aligned(kv_bf16, 16) ||
      !aligned(out_bf16, 16))
    return DSA_ERR_INVALID_ARG;
  return DSA_OK;
}

// (1) -> (2) -> (3) over a workspace of at least forward_ws(...) bytes
// (validated arguments).
int run_forward(const dsa_queries* q, const Layout& lay, int32_t H_I, int32_t D_I, const uint8_t* iq_fp8,
                const float* iq_scale, const float* iw, const uint8_t* ik_fp8, const float* ik_scale, int32_t H,
                const void* q_bf16, const void* kv_bf16, int32_t k, float sm_scale, void* out_bf16, float* lse,
                int32_t* idx_out, void* workspace, hipStream_t stream) {
  const int64_t ld = ((int64_t)q->max_len + 3) & ~int64_t(3);
  const WsLayout L = forward_layout(q->T, q->max_len, H, k, idx_out == nullptr);
  int32_t* idx = idx_out != nullptr ? idx_out : static_cast<int32_t*>(L.at(workspace, L.index("sel")));
  hipError_t e;
  if (forward_fused(q->T)) {
    // many query tokens: indexer and selection in one pass, no logits stored
    const int cap = fused_topk_cap(q->max_len, k);
    void* ws_sel = L.at(workspace, L.index("fused"));
    e = launch_indexer_topk(q->T, q->max_len, H_I, D_I, iq_fp8, iq_scale, iw, ik_fp8, ik_scale, q->seq_id, q->pos,
                            lay, k, cap, idx, ws_sel, stream);
    if (e != hipSuccess) return DSA_ERR_HIP;
  } else {
    float* logits = static_cast<float*>(L.at(workspace, L.index("logits")));
    void* ws_topk = L.at(workspace, L.index("topk"));
    e = launch_topk_zero_hist(ws_topk, q->T, stream);
    if (e != hipSuccess) return DSA_ERR_HIP;
    e = launch_indexer(q->T, q->max_len, H_I, D_I, iq_fp8, iq_scale, iw, ik_fp8, ik_scale, q->seq_id, q->pos, lay,
                       logits, ld, topk_hist_buffer(ws_topk), stream);
    if (e != hipSuccess) return DSA_ERR_HIP;
    e = launch_topk(logits, ld, q->pos, 1, q->T, q->max_len, k, idx, ws_topk, true, stream);
    if (e != hipSuccess) return DSA_ERR_HIP;
  }
  void* ws_attn = L.at(workspace, L.index("attn"));
  e = launch_attn(q->T, H, static_cast<const uint16_t*>(q_bf16), static_cast<const uint16_t*>(kv_bf16), idx, q->seq_id,
                  lay, k, sm_scale, static_cast<uint16_t*>(out_bf16), lse, ws_attn, stream);
  return hip_status(e);
}

constexpr size_t kScratchBytes = DSA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return DSA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" {

int dsa_forward(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H_I, int32_t D_I,
                const uint8_t* iq_fp8, const float* iq_scale, const float* iw, const uint8_t* ik_fp8,
                const float* ik_scale, int32_t H, const void* q_bf16, const void* kv_bf16, int32_t k,
                float sm_scale, void* out_bf16, float* lse, int32_t* idx_out, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  Layout lay;
  int st = validate_forward(q, layout, H_I, D_I, iq_fp8, iq_scale, iw, ik_fp8, ik_scale, H, q_bf16, kv_bf16, k,
                            sm_scale, out_bf16, &lay);
  if (st || q->T == 0) return st;
  const size_t need = forward_ws(q->T, q->max_len, H, k, idx_out == nullptr);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256)) return DSA_ERR_WORKSPACE;
  return run_forward(q, lay, H_I, D_I, iq_fp8, iq_scale, iw, ik_fp8, ik_scale, H, q_bf16, kv_bf16, k, sm_scale,
                     out_bf16, lse, idx_out, workspace, stream);
}

int dsa_forward_noalloc(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H_I, int32_t D_I,
                        const uint8_t* iq_fp8, const float* iq_scale, const float* iw, const uint8_t* ik_fp8,
                        const float* ik_scale, int32_t H, const void* q_bf16, const void* kv_bf16, int32_t k,
                        float sm_scale, void* out_bf16, float* lse, int32_t* idx_out, hipStream_t stream) {
  Layout lay;
  int st = validate_forward(q, layout, H_I, D_I, iq_fp8, iq_scale, iw, ik_fp8, ik_scale, H, q_bf16, kv_bf16, k,
                            sm_scale, out_bf16, &lay);
  if (st || q->T == 0) return st;
  if (forward_ws(q->T, q->max_len, H, k, idx_out == nullptr) > kScratchBytes) return DSA_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if ((st = scratch_for_current_device(&ws))) return st;
  return run_forward(q, lay, H_I, D_I, iq_fp8, iq_scale, iw, ik_fp8, ik_scale, H, q_bf16, kv_bf16, k, sm_scale,
                     out_bf16, lse, idx_out, ws, stream);
}

}  // extern "C"
