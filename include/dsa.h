/*
 * dsa.h — C ABI of the MI355X (gfx950) DeepSeek Sparse Attention hot path.
 *
 * The path, as the DeepSeek-V3.2-Exp articles describe it ("DeepSeek V3.2-Exp
 * Cuts Prolonged-Context Costs With DeepSeek Sparse Consideration (DSA)",
 * nextbusiness24.com, parts (1), (2) and "Instantiation"):
 *
 *   (1) a lightning indexer scores, for each query token, every earlier token
 *       of its sequence with a few small FP8 heads and a ReLU;
 *   (2) each query keeps only its top-k (k = 2048) tokens;
 *   (3) standard softmax attention runs over that subset, under MLA in MQA
 *       mode: one latent KV row per token is shared by all query heads.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers documented "device" must point to GPU memory (hipMalloc or
 *   torch CUDA tensors); descriptor structs are host memory and are read
 *   before the call returns.
 * - The caller owns every buffer, including workspaces.  The library
 *   allocates no memory and keeps no state between calls, so it is
 *   re-entrant; calls on one stream run in order.  The one exception is
 *   dsa_forward_noalloc, whose workspace is a static array of the library
 *   (one per GPU; see there).
 * - Every call only enqueues work on `stream` and returns; nothing waits.
 * - Errors: each call returns DSA_OK (0) or a negative DSA_ERR_* code and
 *   enqueues nothing when it fails validation.  Validation covers host-side
 *   scalars, null pointers, alignment and workspace size.  The contents of
 *   device index arrays (seq_id, pos, valid_len, idx, block_table) are
 *   trusted: out-of-range values there are undefined behaviour (the indexer
 *   and the selection clamp pos[t] and valid lengths to max_len, so those
 *   never write past their rows).
 * - All tensors are dense, row-major, with the strides stated per argument.
 * - Key positions are logical token positions within a sequence (0-based),
 *   so results do not depend on whether the caches are paged.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 1

/* status codes */
#define DSA_OK 0
#define DSA_ERR_INVALID_ARG (-1) /* null pointer, bad size, misaligned buffer   */
#define DSA_ERR_UNSUPPORTED (-2) /* valid request outside the built shapes       */
#define DSA_ERR_WORKSPACE (-3)   /* workspace missing or smaller than required    */
#define DSA_ERR_HIP (-4)         /* a HIP launch reported an error                */
#define DSA_ERR_SCRATCH_LIMIT (-5) /* dsa_forward_noalloc: request larger than its static scratch */

/* Query tokens.  Query t belongs to sequence seq_id[t] and sits at logical
 * position pos[t]; it sees the tokens 0..pos[t] of its sequence (its own
 * position included: the causal rule).  Decode has one or a few trailing
 * tokens per sequence; prefill has pos[t] = t for one sequence.           */
typedef struct dsa_queries {
  int32_t T;              /* number of query tokens, >= 0                       */
  int32_t B;              /* number of sequences, >= 1                          */
  const int32_t* seq_id;  /* device int32[T], each in [0, B)                    */
  const int32_t* pos;     /* device int32[T], each in [0, max_len)              */
  int32_t max_len;        /* host: an upper bound of pos[t] + 1 over all t      */
} dsa_queries;

/* Cache layout, shared by the indexer key cache and the latent KV cache.
 * Contiguous: tensors are [B, seq_capacity, ...] and token s of sequence b is
 *   row b * seq_capacity + s.
 * Paged (the serving layout with 64-token pages, "DeepSeek V3.2-Exp: Sparse
 *   Attention, Long Context, and Cheaper API", mundobytes.com, "Quick guide to
 *   run it locally" and "Open kernels and ecosystem support"): tensors are
 *   [num_pages, page_size, ...]; token s of sequence b lives in physical page
 *   block_table[b * max_pages + s / page_size], row s % page_size.          */
typedef struct dsa_kv_layout {
  int32_t paged;              /* 0 = contiguous, 1 = paged                       */
  int32_t page_size;          /* paged: must be 64                               */
  const int32_t* block_table; /* paged: device int32[B, max_pages]               */
  int32_t max_pages;          /* paged: row stride of block_table                */
  int32_t num_pages;          /* paged: number of physical pages (>= 1)          */
  int64_t seq_capacity;       /* contiguous: tokens per sequence (>= max_len)    */
} dsa_kv_layout;

/* ---------------------------------------------------------------------------
 * (0) Cache write: store new tokens into the caches that (1) and (3) read.
 * The indexer scores in FP8 ("... Sparse Consideration (DSA)", part (1)), so
 * each new token's float32 index key is quantised with one float32 scale per
 * token:
 *     scale  = max(amax / 448, 2^-126),   amax = max_i |k_new[t, i]|
 *     code_i = e4m3fn(clamp(k_new[t, i] / scale, -448, 448))
 * rounding to the nearest e4m3fn value, ties to the even code (float32
 * division, exactly rounded).  Token t is written at logical position pos[t]
 * of sequence seq_id[t]: codes to k_fp8, scale to k_scale and, when given,
 * its 576-value latent row to kv_bf16 (copied bit for bit).  Positions must
 * be distinct within a call; other rows are not touched.
 *
 *   q           : seq_id / pos of the new tokens (pos[t] < max_len)
 *   D_I         : 64 or 128
 *   k_new       : device float[T, D_I], finite
 *   kv_new_bf16 : device bf16[T, 576] or NULL (then kv_bf16 must be NULL)
 *   k_fp8, k_scale, kv_bf16 : the caches, in the layout above
 * ------------------------------------------------------------------------- */
int dsa_cache_write(const dsa_queries* q, const dsa_kv_layout* layout, int32_t D_I, const float* k_new,
                    const void* kv_new_bf16, uint8_t* k_fp8, float* k_scale, void* kv_bf16, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * (0b) The indexer's inputs from the tokens' hidden states ("... Sparse
 * Consideration (DSA)", part (1): for each query token h_t the indexer forms
 * a few small heads and one weight per head; each token also has its own
 * index key).  The pages give no formula; the reading is plain linear maps
 * without bias, accumulated in fp32 on the matrix cores from bf16 inputs:
 *     q[t, j, c] = sum_i Wq[j * D_I + c, i] * h[t, i]     (head-major rows)
 *     w[t, j]    = sum_i Ww[j, i] * h[t, i]
 *     k[t, c]    = sum_i Wk[c, i] * h[t, i]                (optional)
 * The query is then quantised per token exactly as dsa_cache_write quantises
 * a key, over all of its H_I * D_I values: q_scale[t] = max(amax / 448,
 * 2^-126), q_fp8 = e4m3fn(clamp(q / q_scale, +-448)), ties to even -- the
 * q_fp8 / q_scale that dsa_indexer_logits takes.  k is the float32 key that
 * dsa_cache_write stores.
 *
 *   T, d      : tokens >= 0; hidden width d, a multiple of 64, <= 65536
 *   H_I, D_I  : as for dsa_indexer_logits
 *   h_bf16    : device bf16[T, d]                 (16-byte aligned)
 *   wq_bf16   : device bf16[H_I * D_I, d]         (16-byte aligned)
 *   ww_bf16   : device bf16[H_I, d]               (16-byte aligned)
 *   wk_bf16   : device bf16[D_I, d] or NULL       (16-byte aligned)
 *   q_fp8     : device uint8[T, H_I, D_I] (16-byte aligned); q_scale : device float[T]
 *   w         : device float[T, H_I];  k_new : device float[T, D_I], NULL iff wk_bf16 is
 *   workspace : device, >= dsa_workspace_bytes(DSA_OP_INDEXER_PROJ, T, d, H_I, D_I),
 *               256-byte aligned (fp32 partial sums of the projection)
 * ------------------------------------------------------------------------- */
int dsa_indexer_project(int32_t T, int32_t d, int32_t H_I, int32_t D_I, const void* h_bf16, const void* wq_bf16,
                        const void* ww_bf16, const void* wk_bf16, uint8_t* q_fp8, float* q_scale, float* w,
                        float* k_new, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * (1) Lightning indexer logits.
 *   logits[t * ld_logits + s] =
 *       q_scale[t] * k_scale[s] * sum_j w[t,j] * ReLU( sum_d q[t,j,d] * k[s,d] )
 * for s in 0..pos[t], where q and k are OCP e4m3fn FP8 codes (the FP8 of
 * gfx950) and the dot products accumulate in fp32 on the matrix cores.
 * Entries s > pos[t] of a row are left unwritten.
 *
 *   H_I, D_I  : indexer heads and head dim; built: (H_I, D_I) in
 *               {(64,128), (64,64), (4,128), (4,64)}.
 *   q_fp8     : device uint8[T, H_I, D_I]       (16-byte aligned)
 *   q_scale   : device float[T]                 per-token dequantisation scale
 *   w         : device float[T, H_I]            per-head weights (any sign)
 *   k_fp8     : device uint8 cache, [*, D_I] per token (layout above; 16-byte aligned)
 *   k_scale   : device float cache, one per token (layout above)
 *   logits    : device float[T, ld_logits], ld_logits >= max_len, multiple of 4
 * ------------------------------------------------------------------------- */
int dsa_indexer_logits(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H_I, int32_t D_I,
                       const uint8_t* q_fp8, const float* q_scale, const float* w, const uint8_t* k_fp8,
                       const float* k_scale, float* logits, int64_t ld_logits, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * (2) Top-k selection ("DeepSeek V3.2-Exp Cuts Prolonged-Context Costs ...",
 * part (2)).  Row t holds valid_len[t] values logits[t*ld_logits + s],
 * s < valid_len[t].  idx[t, :] receives the positions of the k largest values,
 * equal values ordered by the lower position first and -0 equal to +0; when
 * valid_len[t] <= k every position is kept and the row is padded with -1.
 * The positions are written in a deterministic order that is not sorted by
 * value.  NaN values give an unspecified (but in-range) selection.
 *
 *   logits    : device float[T, ld_logits]
 *   valid_len : device int32[T], each in [0, max_len]
 *   max_len   : host upper bound of valid_len, <= ld_logits
 *   k         : 1 <= k <= 2048
 *   idx       : device int32[T, k]
 *   workspace : device, >= dsa_workspace_bytes(DSA_OP_TOPK, T, max_len, 0, k), 256-byte aligned
 * ------------------------------------------------------------------------- */
int dsa_topk(const float* logits, int64_t ld_logits, const int32_t* valid_len, int32_t T, int32_t max_len,
             int32_t k, int32_t* idx, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * (1) + (2) fused, for batches with many query tokens (prefill): idx[t, :]
 * receives exactly what dsa_indexer_logits followed by dsa_topk (valid length
 * pos[t] + 1) would give, but the logits are consumed as they are produced
 * and never stored.  Query tokens are taken 8 at a time; consecutive tokens
 * of one sequence share their key reads, so the call suits prefill-like
 * batches (a few thousand tokens or more); a decode batch is better served by
 * the two separate calls.
 *
 *   arguments : as for dsa_indexer_logits; k as for dsa_topk;
 *   idx       : device int32[T, k], positions in a deterministic order that
 *               is not sorted by value (rows with pos[t] + 1 <= k: all
 *               positions ascending, then -1)
 *   workspace : device, 256-byte aligned; it holds a candidate list of `cap`
 *               slots (8 bytes each) per query token, with cap = the largest
 *               multiple of 64 not above 12288 that fits workspace_bytes / T;
 *               cap >= k + 320 is required (DSA_ERR_WORKSPACE otherwise).
 *               A smaller cap gives the same result with more work;
 *               dsa_workspace_bytes(DSA_OP_INDEXER_TOPK, T, max_len, 0, k) is
 *               the size at which no list ever needs compacting for rows up
 *               to about 7.9K positions.
 * ------------------------------------------------------------------------- */
int dsa_indexer_topk(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H_I, int32_t D_I,
                     const uint8_t* q_fp8, const float* q_scale, const float* w, const uint8_t* k_fp8,
                     const float* k_scale, int32_t k, int32_t* idx, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* ---------------------------------------------------------------------------
 * (3) Sparse attention under MLA in MQA mode ("... Sparse Consideration
 * (DSA)", parts (2) and "Instantiation").  For query t, head h and the
 * selected positions i = idx[t, j] != -1 of sequence seq_id[t]:
 *     z_i = sm_scale * <q[t,h,0:576], kv_row_i[0:576]>
 *     out[t,h,c] = sum_i softmax(z)_i * kv_row_i[c],   c < 512
 *     lse[t,h]   = ln sum_i exp(z_i)
 * An all-padding row gives out = 0 and lse = -inf.
 *
 *   H         : query heads; built: 16, 32, 64 or 128
 *   q_bf16    : device bf16[T, H, 576]          (16-byte aligned)
 *   kv_bf16   : device bf16 latent cache, 576 per token (layout above; 16-byte aligned)
 *   idx       : device int32[T, k], entries in [0, pos[t]] or -1
 *   k         : 1 <= k <= 2048
 *   out_bf16  : device bf16[T, H, 512]
 *   lse       : device float[T, H] or NULL
 *   workspace : device, >= dsa_workspace_bytes(DSA_OP_ATTN, T, 0, H, k), 256-byte aligned
 * ------------------------------------------------------------------------- */
int dsa_sparse_mla_attn(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H, const void* q_bf16,
                        const void* kv_bf16, const int32_t* idx, int32_t k, float sm_scale, void* out_bf16,
                        float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * (3b) Backward of (3) ("... Sparse Consideration (DSA)", opening paragraph
 * and "Teaching signal": the sparse path is trained).  Given the forward's
 * out and lse for the same q, kv and idx, and the output gradient d_out, with
 * P_i = exp(z_i - lse), dP_i = <d_out[t,h], kv_row_i[0:512]>,
 * D = <d_out[t,h], out[t,h]> and dS_i = P_i (dP_i - D):
 *     dq[t,h,:]       = sm_scale * sum_i dS_i * kv_row_i[0:576]
 *     dkv[row_i, :]  += sm_scale * sum_h dS_hi * q[t,h,:]
 *     dkv[row_i, c]  += sum_h P_hi * d_out[t,h,c],   c < 512
 * summed over every query t and selected entry i (a row selected twice by one
 * query, or by several queries, receives every contribution).  P and dS are
 * rounded to bf16 for the products, as are the per-entry row gradients before
 * they are summed in fp32; the order of the fp32 sums into dkv is not fixed.
 *
 *   arguments : q, layout, H, q_bf16, kv_bf16, idx, k, sm_scale as for
 *               dsa_sparse_mla_attn (the same values as the forward call)
 *   out_bf16  : device bf16[T, H, 512]  the forward's output (16-byte aligned)
 *   lse       : device float[T, H]      the forward's log-sum-exp
 *   d_out_bf16: device bf16[T, H, 512]  gradient of the output (16-byte aligned)
 *   dq        : device float[T, H, 576] written (16-byte aligned)
 *   dkv       : device float cache, 576 per token in the layout of kv_bf16
 *               (B * seq_capacity rows, or num_pages * 64); the gradients are
 *               ADDED to it (zero it first for a plain gradient); rows no
 *               query selected are not touched.  16-byte aligned.
 *   workspace : device, >= dsa_workspace_bytes(DSA_OP_ATTN_BWD, T, 0, H, k),
 *               256-byte aligned; about k * (4H + 1168) bytes per query token.
 *   limits    : T * roundup(k, 32) < 2^31; fewer than 2^31 cache rows.
 * ------------------------------------------------------------------------- */
int dsa_sparse_mla_attn_bwd(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H, const void* q_bf16,
                            const void* kv_bf16, const int32_t* idx, int32_t k, float sm_scale, const void* out_bf16,
                            const float* lse, const void* d_out_bf16, float* dq, float* dkv, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* The two steps of dsa_sparse_mla_attn_bwd, for callers that want dq first
 * (it is on the critical path of the layers below) and dkv later or on
 * another stream.  dsa_sparse_mla_attn_bwd_dq computes dq and leaves P, dS and
 * the selected rows in the workspace; dsa_sparse_mla_attn_bwd_dkv then adds
 * the dkv gradient.  The dkv step must be enqueued after the dq step (same
 * stream, or ordered by an event) with the same q, layout, H, k, q_bf16,
 * d_out_bf16 and workspace, and nothing may write the workspace in between.
 * Arguments and errors as for dsa_sparse_mla_attn_bwd.                     */
int dsa_sparse_mla_attn_bwd_dq(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H, const void* q_bf16,
                               const void* kv_bf16, const int32_t* idx, int32_t k, float sm_scale,
                               const void* out_bf16, const float* lse, const void* d_out_bf16, float* dq,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);
int dsa_sparse_mla_attn_bwd_dkv(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H, const void* q_bf16,
                                int32_t k, const void* d_out_bf16, float* dkv, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * (1b) The indexer's training signal ("... Sparse Consideration (DSA)",
 * "Teaching signal": the indexer learns the main attention's head-summed
 * distribution through a KL divergence; the target takes no gradient).
 *
 * dsa_indexer_kl_target: for the entries j of idx[t, :] (the sparse stage's
 * selection; for the dense warm-up see dsa_indexer_kl_target_dense),
 *     target[t, j] = (1/H) sum_h exp(z[t,h,j] - lse[t,h]),
 *     z = sm_scale * <q[t,h,:], kv_row_j>,
 * the head-summed attention probabilities normalised to total 1; 0 for
 * padding entries (-1).  q, kv, idx, k, sm_scale and lse are those of the
 * forward (dsa_sparse_mla_attn); the rows sum to 1 up to rounding.
 *   target    : device float[T, k] (16-byte aligned)
 *   built     : H in {16, 32, 64, 128}, k <= 2048; no workspace
 * ------------------------------------------------------------------------- */
int dsa_indexer_kl_target(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H, const void* q_bf16,
                          const void* kv_bf16, const int32_t* idx, int32_t k, float sm_scale, const float* lse,
                          float* target, hipStream_t stream);

/* dsa_indexer_kl_target_dense: the dense warm-up's target ("Teaching signal":
 * first a short dense warm-up, the main model frozen), over every position
 * s = 0..pos[t] of the query's sequence at any context length:
 *     target[t * ld_target + s] = (1/H) sum_h exp(z[t,h,s] - lse[t,h]),
 *     lse[t,h] = ln sum_{s <= pos[t]} exp(z[t,h,s])   (the dense attention's),
 * with z as above.  The lse is computed here from every position (two passes
 * over the rows) and written to lse_out when it is not NULL.  Entries past
 * pos[t] of a row are left unwritten.  The rows sum to 1 up to rounding.
 *   arguments : q, layout, H, q_bf16, kv_bf16, sm_scale as for dsa_sparse_mla_attn
 *   target    : device float[T, ld_target], ld_target >= max_len
 *   lse_out   : device float[T, H] or NULL
 *   workspace : device, >= dsa_workspace_bytes(DSA_OP_KL_TARGET_DENSE, T, max_len, H, 0),
 *               256-byte aligned (8 bytes per query, head and 2048 positions)
 * ------------------------------------------------------------------------- */
int dsa_indexer_kl_target_dense(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H, const void* q_bf16,
                                const void* kv_bf16, float sm_scale, float* target, int64_t ld_target, float* lse_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* dsa_indexer_kl_target_dense_lse: the same dense warm-up target as
 * dsa_indexer_kl_target_dense, given the dense attention's lse:
 *     target[t * ld_target + s] = (1/H) sum_h exp(z[t,h,s] - lse[t,h])
 * for s = 0..pos[t].  During the warm-up the main model runs dense attention
 * over every position, and its forward returns exactly this lse ("Teaching
 * signal": the target is the main attention's head-summed distribution), so
 * the target needs one pass over the rows instead of two and no workspace.
 * Entries past pos[t] are left unwritten.
 *   arguments : q, layout, H, q_bf16, kv_bf16, sm_scale as for dsa_sparse_mla_attn
 *   lse       : device float[T, H], natural log, over positions 0..pos[t]
 *               (the rows sum to 1 only when it is that lse)
 *   target    : device float[T, ld_target], ld_target >= max_len
 * ------------------------------------------------------------------------- */
int dsa_indexer_kl_target_dense_lse(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H, const void* q_bf16,
                                    const void* kv_bf16, float sm_scale, const float* lse, float* target,
                                    int64_t ld_target, hipStream_t stream);

/* dsa_indexer_kl: with the indexer logits I (as dsa_indexer_logits) at the
 * selected entries, q[t, j] = softmax_j I[t, idx[t, j]] over the entries != -1:
 *     loss[t] = sum_j target[t,j] (log target[t,j] - log q[t,j])
 * (entries with target 0 contribute 0; the target rows should sum to 1), and
 * the gradients of sum_t loss[t] through I = sum_h w_h ReLU(qd_h . kd_s),
 * qd = q_scale * q_fp8 and kd = k_scale * k_fp8 (the FP8 quantisation taken
 * as the identity), with dI = q - target:
 *     dw[t,h]   = sum_j dI_j ReLU(qd_h . kd_j)
 *     dq[t,h,:] = w_h sum_j dI_j [qd_h . kd_j > 0] kd_j
 *     dk[row_j] += dI_j sum_h w_h [qd_h . kd_j > 0] qd_h
 *   indexer arguments as for dsa_indexer_logits; built: H_I = 64, D_I = 128
 *   idx, k    : the selection (k <= 2048)
 *   target    : device float[T, k], e.g. from dsa_indexer_kl_target
 *   loss      : device float[T];  dq : device float[T, H_I, D_I];  dw : device float[T, H_I]
 *   dk        : device float cache, D_I per token in the layout of k_fp8; the
 *               gradients are ADDED (zero it first); 16-byte aligned
 *   workspace : device, >= dsa_workspace_bytes(DSA_OP_INDEXER_KL, T, 0, 0, k),
 *               256-byte aligned (about 17.5 * k bytes per query token)
 * The per-entry key gradients are rounded to bf16 before their sum per cache
 * row, as are the ReLU-masked products inside the dq and dk contractions.
 * ------------------------------------------------------------------------- */
int dsa_indexer_kl(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H_I, int32_t D_I,
                   const uint8_t* q_fp8, const float* q_scale, const float* w, const uint8_t* k_fp8,
                   const float* k_scale, const int32_t* idx, int32_t k, const float* target, float* loss, float* dq,
                   float* dw, float* dk, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * (3') Masked dense variant of (3) ("... Sparse Consideration (DSA)", "Lets
 * Discuss it's effectivity and accuracy": at short lengths the prefill runs
 * as a masked dense attention).  For query t every position s <= pos[t] of
 * its sequence is read in order and scored; positions absent from idx[t, :]
 * are masked out.  The result is that of dsa_sparse_mla_attn on the same
 * idx (up to floating-point summation order); the rows are read contiguously
 * instead of gathered.  Entries of idx outside 0..pos[t] are ignored, and a
 * position listed twice counts once.
 *
 *   arguments : as for dsa_sparse_mla_attn; max_len <= 16384
 *   workspace : device, >= dsa_workspace_bytes(DSA_OP_DENSE_ATTN, T, max_len, H, k)
 * ------------------------------------------------------------------------- */
int dsa_masked_dense_attn(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H, const void* q_bf16,
                          const void* kv_bf16, const int32_t* idx, int32_t k, float sm_scale, void* out_bf16,
                          float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * (1) -> (2) -> (3) on one stream ("FP8 index -> top-k selection -> sparse
 * core attention").  Arguments as above; idx_out (device int32[T, k]) receives
 * the selection, or may be NULL to keep it inside the workspace.  With
 * T >= 2048 query tokens, (1) and (2) run fused as in dsa_indexer_topk (no
 * logits in memory); below that they run as dsa_indexer_logits + dsa_topk.
 * The selection is the same either way.
 *   workspace : device, >= dsa_workspace_bytes(DSA_OP_FORWARD, T, max_len, H, k)
 * ------------------------------------------------------------------------- */
int dsa_forward(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H_I, int32_t D_I,
                const uint8_t* iq_fp8, const float* iq_scale, const float* iw, const uint8_t* ik_fp8,
                const float* ik_scale, int32_t H, const void* q_bf16, const void* kv_bf16, int32_t k,
                float sm_scale, void* out_bf16, float* lse, int32_t* idx_out, void* workspace,
                size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * dsa_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Arguments, results and errors as for dsa_forward;
 * the workspace is a static device array inside the library, one copy per GPU
 * of DSA_NOALLOC_SCRATCH_BYTES (64 MiB), held from the first call on that GPU
 * until the process ends.  The call allocates nothing; it returns
 * DSA_ERR_SCRATCH_LIMIT, enqueuing nothing, when the request needs more than
 * the scratch holds (dsa_workspace_bytes(DSA_OP_FORWARD, ...) bytes, less
 * T * k * 4 when idx_out is given) -- in practice decode batches below 2048
 * query tokens, e.g. 16 queries of 128K positions (about 45 MB).  Every call
 * on a GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other host threads) race and must be serialised by the caller.
 * The current device must be the one the stream and buffers belong to.
 * ------------------------------------------------------------------------- */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int dsa_forward_noalloc(const dsa_queries* q, const dsa_kv_layout* layout, int32_t H_I, int32_t D_I,
                        const uint8_t* iq_fp8, const float* iq_scale, const float* iw, const uint8_t* ik_fp8,
                        const float* ik_scale, int32_t H, const void* q_bf16, const void* kv_bf16, int32_t k,
                        float sm_scale, void* out_bf16, float* lse, int32_t* idx_out, hipStream_t stream);

/* Workspace sizes (bytes) for an operation; 0 when none is needed. */
#define DSA_OP_TOPK 1
#define DSA_OP_ATTN 2
#define DSA_OP_FORWARD 3
#define DSA_OP_INDEXER_TOPK 4
#define DSA_OP_DENSE_ATTN 5
#define DSA_OP_ATTN_BWD 6
#define DSA_OP_INDEXER_KL 7
#define DSA_OP_INDEXER_PROJ 8 /* arguments (T, d, H_I, D_I) in place of (T, max_len, H, k) */
#define DSA_OP_KL_TARGET_DENSE 9
size_t dsa_workspace_bytes(int32_t op, int32_t T, int32_t max_len, int32_t H, int32_t k);

/* ---------------------------------------------------------------------------
 * dsa_workspace_layout: the regions a call with these sizes carves out of its
 * workspace, for checking and debugging.  Same arguments as
 * dsa_workspace_bytes.  Each region starts on a 256-byte boundary at `offset`
 * bytes from the workspace base; regions a sub-step keeps inside its own part
 * of the workspace are listed one by one, with that part's name in `parent`
 * (NULL for a region of the call itself); names are static strings.  The
 * regions are disjoint and, with each size rounded up to 256 bytes, tile
 * [0, dsa_workspace_bytes(...)).  The call writes at most max_regions entries
 * and returns the number of regions (0 when the operation needs no
 * workspace), or DSA_ERR_INVALID_ARG (negative sizes or max_regions, regions
 * NULL with max_regions > 0, unknown op).  Host only: no device is touched.
 * ------------------------------------------------------------------------- */
typedef struct {
  const char* parent;
  const char* name;
  uint64_t offset;
  uint64_t bytes;
} dsa_ws_region;
int32_t dsa_workspace_layout(int32_t op, int32_t T, int32_t max_len, int32_t H, int32_t k, dsa_ws_region* regions,
                             int32_t max_regions);

/* Static string for a status code (never NULL). */
const char* dsa_status_str(int32_t status);

/* DSA_ABI_VERSION of the built library. */
int32_t dsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
