"""Plain float64 reference of the DSA hot path: indexer -> top-k -> sparse MLA attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests, the
smoke check and the benchmark's CPU-baseline leg, never by the product path.

Sources.  The pages describe the method in prose only:

* [DSA-article] "DeepSeek V3.2-Exp Cuts Prolonged-Context Costs With DeepSeek
  Sparse Consideration (DSA) Whereas Sustaining Benchmark Parity"
  (nextbusiness24.com), parts "(1) Lightning indexer (FP8, few heads)",
  "(2) Fine-grained token selection (top-k)" and "Instantiation".
* [mundobytes] "DeepSeek V3.2-Exp: Sparse Attention, Long Context, and Cheaper
  API" (mundobytes.com), sections "How it works: Lightning Indexer and Token
  Selection", "Quick guide to run it locally" (the serving command with
  `--page-size 64`) and "Open kernels and ecosystem support" (paged
  indexer-logit kernels).

Where the pages leave a step open, the reading taken here is stated at the
function.  Every floating-point step runs in float64 on exactly decoded
inputs, so the only rounding is float64 rounding.
"""

from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------


def _e4m3fn_value(code: int) -> float:
    """Value of one OCP 8-bit floating-point E4M3 ("e4m3fn") code.

    [DSA-article] (1) says the indexer runs in FP8; the FP8 of the target GPU
    is the OCP E4M3 format: bit 7 sign, bits 6..3 exponent with bias 7,
    bits 2..0 mantissa; exponent field 0 encodes subnormals
    (-1)^s * 2^-6 * m/8; the all-ones exponent with mantissa 7 is NaN; there
    is no infinity, so exponent 15 with mantissa 0..6 is an ordinary normal
    number (largest 448).
    """
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = math.ldexp(m / 8.0, -6)
    else:
        mag = math.ldexp(1.0 + m / 8.0, e - 7)
    return -mag if s else mag


_E4M3FN_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3fn(codes) -> np.ndarray:
    """Decode an array of e4m3fn byte codes (uint8) to float64, exactly.

    [DSA-article] (1): the indexer computes in FP8, read here as the OCP E4M3
    ("e4m3fn") format of gfx950 (see _e4m3fn_value).
    """
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        raise TypeError("e4m3fn codes must be uint8")
    return _E4M3FN_TABLE[c]


def decode_bf16(bits) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to float64, exactly.

    [DSA-article] "Instantiation": the attention runs on MLA latent rows shared
    by all query heads; the pages fix no width for them or for the queries, and
    bfloat16 is the reading taken for both.

    bfloat16 is the upper half of an IEEE-754 binary32: the value is the
    binary32 whose bits are ``bits << 16``.
    """
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("bf16 values must be passed as uint16 bit patterns")
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Cache addressing (contiguous or 64-token pages)
# ---------------------------------------------------------------------------


def logical_rows(cache: np.ndarray, b: int, n: int, block_table=None, page_size: int = 64) -> np.ndarray:
    """First ``n`` logical token rows of sequence ``b`` of a cache.

    Contiguous caches are laid out ``[B, L_max, ...]``.  Paged caches follow
    the serving layout [mundobytes] names (pages of 64 tokens, with the
    indexer-logit kernels also offered in paged form): ``[P, page_size, ...]``
    physical pages, and ``block_table[b, j]`` is the physical page holding
    logical tokens ``j*page_size .. j*page_size+page_size-1`` of sequence b.
    """
    if block_table is None:
        return cache[b, :n]
    npages = -(-n // page_size)
    pages = np.asarray(block_table)[b, :npages]
    rows = cache[pages].reshape((npages * page_size,) + cache.shape[2:])
    return rows[:n]


# ---------------------------------------------------------------------------
# (a1) Lightning indexer
# ---------------------------------------------------------------------------


def indexer_logits_row(q8_t, qs_t, w_t, k8_rows, ks_rows) -> np.ndarray:
    """Index logits of one query token against ``n`` key tokens, float64.

    [DSA-article] (1): for a query token, a light scoring function computes an
    index logit I[t,s] against each earlier token, using a few small indexer
    heads with a ReLU, in FP8.  The pages print no formula; the reading taken
    here is

        I[t,s] = qs[t] * ks[s] * sum_j w[t,j] * ReLU( sum_d q[t,j,d] * k[s,d] )

    with q (``[H_I, D_I]``) and k (``[n, D_I]``) the decoded FP8 codes,
    one key vector per token shared by all indexer heads, a per-head weight
    w[t,j], and positive per-token dequantisation scales qs, ks (positive
    scales commute with the ReLU, so applying them outside is exact).
    """
    q = decode_e4m3fn(np.asarray(q8_t))                 # [H_I, D_I]
    k = decode_e4m3fn(np.asarray(k8_rows))              # [n, D_I]
    w = np.asarray(w_t, dtype=np.float64)               # [H_I]
    dots = k @ q.T                                      # [n, H_I]   q[t,j] . k[s]
    relu = np.maximum(dots, 0.0)
    acc = relu @ w                                      # sum over heads
    return float(qs_t) * np.asarray(ks_rows, dtype=np.float64) * acc


def indexer_logits(q8, qs, w, k8, ks, seq_id, pos, block_table=None, page_size: int = 64) -> np.ndarray:
    """Index logits for every query token, ``[T, max(pos)+1]`` float64.

    Query t belongs to sequence ``seq_id[t]`` and sits at position ``pos[t]``;
    it scores the tokens s = 0 .. pos[t] of its sequence.  [DSA-article] (1)
    says "earlier tokens"; the reading taken here includes the query's own
    position (s <= t), the causal rule of prefill.  Entries past pos[t] are
    NaN (they are not defined).
    """
    seq_id = np.asarray(seq_id)
    pos = np.asarray(pos)
    T = len(pos)
    width = int(pos.max()) + 1 if T else 0
    out = np.full((T, width), np.nan)
    for t in range(T):
        n = int(pos[t]) + 1
        b = int(seq_id[t])
        krows = logical_rows(k8, b, n, block_table, page_size)
        srows = logical_rows(ks, b, n, block_table, page_size)
        out[t, :n] = indexer_logits_row(q8[t], qs[t], w[t], krows, srows)
    return out


# ---------------------------------------------------------------------------
# (a2) Fine-grained token selection
# ---------------------------------------------------------------------------


def topk_select(values, n_valid: int, k: int) -> np.ndarray:
    """Positions of the top-k entries of one row; ``int32[k]`` in rank order.

    [DSA-article] (2): each query keeps only its top-k key-value entries.  A
    plain definition: order the valid positions s = 0 .. n_valid-1 by value,
    largest first, and take the first min(k, n_valid).  Readings where the
    pages are silent: equal values are ordered by the lower position first;
    -0 and +0 are equal (IEEE comparison); when fewer than k positions are
    valid, all of them are kept and the rest of the row is padded with -1.
    The values are compared exactly as given (the library stores logits in
    float32, and so are the values passed here).
    """
    v = np.asarray(values)[:n_valid]
    v = np.where(v == 0, np.zeros((), v.dtype), v)      # -0 == +0
    s = np.arange(n_valid)
    order = np.lexsort((s, -v))                          # value desc, then position asc
    take = order[: min(k, n_valid)]
    out = np.full(k, -1, dtype=np.int32)
    out[: len(take)] = take
    return out


# ---------------------------------------------------------------------------
# (a3) Sparse attention under MLA in MQA mode
# ---------------------------------------------------------------------------


def sparse_mla_attention(q_bits, kv_bits, idx, seq_id, scale: float, d_v: int = 512,
                         block_table=None, page_size: int = 64):
    """Softmax attention of every query head over its selected latent rows.

    [DSA-article] (2): standard attention runs only over the selected subset.
    "Instantiation": DSA runs under MLA in MQA mode, so each latent KV entry
    is shared by all query heads.  Reading: a latent row holds D = 576 values
    (512 without rope followed by 64 rope); the key is the whole row and the
    value is its first ``d_v`` = 512 entries; entries of ``idx`` equal to -1
    are padding and are skipped.

    For query t and head h over the selected rows i:
        z_i = scale * <q[t,h,:], row_i[:D]>
        o[t,h,:] = sum_i softmax(z)_i * row_i[:d_v]
        lse[t,h] = log sum_i exp(z_i)          (natural log)
    An empty selection gives o = 0 and lse = -inf.

    ``q_bits`` is ``uint16[T, H, D]`` and ``kv_bits`` the bf16 cache as uint16
    (contiguous ``[B, L_max, D]`` or paged ``[P, page, D]``).  Returns float64
    ``o[T, H, d_v]`` and ``lse[T, H]``.
    """
    q_bits = np.asarray(q_bits)
    idx = np.asarray(idx)
    seq_id = np.asarray(seq_id)
    T, H, D = q_bits.shape
    out = np.zeros((T, H, d_v))
    lse = np.full((T, H), -np.inf)
    for t in range(T):
        sel = idx[t][idx[t] >= 0].astype(np.int64)
        if sel.size == 0:
            continue
        b = int(seq_id[t])
        n = int(sel.max()) + 1
        rows = decode_bf16(logical_rows(kv_bits, b, n, block_table, page_size)[sel])   # [m, D]
        q = decode_bf16(q_bits[t])                                                    # [H, D]
        z = scale * (q @ rows.T)                                                      # [H, m]
        m = z.max(axis=1, keepdims=True)
        p = np.exp(z - m)
        l = p.sum(axis=1, keepdims=True)
        out[t] = (p @ rows[:, :d_v]) / l
        lse[t] = m[:, 0] + np.log(l[:, 0])
    return out, lse


# ---------------------------------------------------------------------------
# (a4) The whole path
# ---------------------------------------------------------------------------


def dsa_forward(iq8, iqs, iw, ik8, iks, q_bits, kv_bits, seq_id, pos, k: int, scale: float,
                d_v: int = 512, block_table=None, page_size: int = 64):
    """Indexer -> top-k -> sparse attention, as [DSA-article] chains them
    ("FP8 index -> top-k selection -> sparse core attention").

    The selection decides integers from floating values, so it takes its
    decision on the logits rounded to float32, the precision in which the
    library stores them.  Returns ``(logits_f64, idx, out, lse)``.
    """
    logits = indexer_logits(iq8, iqs, iw, ik8, iks, seq_id, pos, block_table, page_size)
    T = len(pos)
    idx = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        n = int(pos[t]) + 1
        idx[t] = topk_select(logits[t, :n].astype(np.float32), n, k)
    out, lse = sparse_mla_attention(q_bits, kv_bits, idx, seq_id, scale, d_v, block_table, page_size)
    return logits, idx, out, lse


# ---------------------------------------------------------------------------
# (f4) Cache write: quantise a new token's index key, store it and its latent row
# ---------------------------------------------------------------------------
#
# [DSA-article] (1): the indexer runs in FP8, so each token's index key is
# stored as FP8 before it is scored.  Reading taken (the pages give no
# quantisation recipe): one float32 scale per token, scale = max(amax / 448,
# 2^-126) where amax is the largest |x| of the key and 448 the largest e4m3fn
# value; each element is x / scale (float32 division), clamped to +-448, then
# rounded to the nearest e4m3fn value, ties to the even code.

E4M3FN_MAX = 448.0
SCALE_FLOOR = 2.0 ** -126

# non-negative finite e4m3fn values: codes 0x00..0x7E, strictly increasing
_E4M3FN_POS = _E4M3FN_TABLE[:0x7F]


def encode_e4m3fn(y) -> np.ndarray:
    """Nearest e4m3fn code of each value (|y| <= 448), ties to the even code.

    [DSA-article] (1): the index keys are FP8; the pages give no rounding rule,
    and round to nearest, ties to even, is the reading.

    The magnitude is rounded among the 127 non-negative finite values; the
    sign bit is the sign of y (so -0.0, and negative values that round to
    zero, give 0x80).
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    if np.any(a > E4M3FN_MAX) or np.any(np.isnan(a)):
        raise ValueError("encode_e4m3fn expects finite values with |y| <= 448")
    hi = np.searchsorted(_E4M3FN_POS, a, side="left")          # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3FN_POS[lo]
    d_hi = _E4M3FN_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(a == _E4M3FN_POS[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    return (mag | (np.signbit(y).astype(np.uint8) << 7)).astype(np.uint8)


def quantize_index_key(x) -> tuple:
    """(codes uint8[D], scale float32) of one token's float32 index key.

    [DSA-article] (1): index keys are FP8 with one float32 scale per token.  The
    pages give no recipe; this is the plain one: scale = max(amax / 448,
    2^-126), x / scale as a float32 division, clamped to +-448, then
    encode_e4m3fn."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x)) if x.size else np.float32(0)
    scale = np.float32(max(np.float32(amax) / np.float32(E4M3FN_MAX), np.float32(SCALE_FLOOR)))
    y = np.clip(x / scale, np.float32(-E4M3FN_MAX), np.float32(E4M3FN_MAX)).astype(np.float32)
    return encode_e4m3fn(y), scale


def cache_write(k8_cache, ks_cache, kv_cache, seq_id, pos, k_new, kv_new_bits=None, block_table=None,
                page_size: int = 64):
    """Store new tokens into the caches (returns updated copies).

    [DSA-article] (1) (FP8 index keys) and [mundobytes] "Quick guide to run it
    locally" (caches in 64-token pages): the step before the indexer, which
    stores each new token's key and latent row where later queries read them.

    Token t goes to logical position pos[t] of sequence seq_id[t] (contiguous
    ``[B, L, ...]`` caches, or physical page ``block_table[b, pos // 64]`` row
    ``pos % 64``): its index key quantised by quantize_index_key, its scale,
    and (if given) its 576-value latent row, copied bit for bit.
    """
    k8_cache, ks_cache = np.array(k8_cache, copy=True), np.array(ks_cache, copy=True)
    kv_cache = None if kv_cache is None else np.array(kv_cache, copy=True)
    for t in range(len(seq_id)):
        b, s = int(seq_id[t]), int(pos[t])
        if block_table is None:
            where = (b, s)
        else:
            where = (int(np.asarray(block_table)[b, s // page_size]), s % page_size)
        codes, scale = quantize_index_key(np.asarray(k_new)[t])
        k8_cache[where] = codes
        ks_cache[where] = scale
        if kv_new_bits is not None:
            kv_cache[where] = np.asarray(kv_new_bits)[t]
    return k8_cache, ks_cache, kv_cache


# ---------------------------------------------------------------------------
# (f4b) The indexer's inputs from a token's hidden state
# ---------------------------------------------------------------------------
#
# [DSA-article] (1): for each query token h_t in R^d the indexer forms a few
# small heads q[t, j] and one weight w[t, j] per head, and every earlier token
# contributes its own index key.  The pages give no formula for these.
# Reading taken: plain linear maps of the hidden state, without bias,
#   q[t] = Wq h_t   (H_I * D_I values, head j = rows j*D_I .. j*D_I + D_I - 1)
#   w[t] = Ww h_t   (H_I values)
#   k[t] = Wk h_t   (D_I values, the token's own index key)
# with the query then stored like an index key: FP8 e4m3fn with one float32
# scale per token over all of its H_I * D_I values (quantize_index_key).  The
# products are taken exactly (float64 over bf16 inputs, whose products and
# sums are exact to float64 rounding) and rounded once to float32, the
# precision from which the query is quantised.


def indexer_projection(h_bits, wq_bits, ww_bits, H_I: int, D_I: int, wk_bits=None):
    """(q8 uint8[T, H_I, D_I], qs float32[T], w float32[T, H_I], k float32[T, D_I]
    or None) from hidden states h (bf16 bits [T, d]) and bf16 weight bits
    Wq [H_I*D_I, d], Ww [H_I, d], Wk [D_I, d] (optional)."""
    h = decode_bf16(h_bits)
    q = (h @ decode_bf16(wq_bits).T).astype(np.float32)
    w = (h @ decode_bf16(ww_bits).T).astype(np.float32)
    T = h.shape[0]
    q8 = np.zeros((T, H_I, D_I), dtype=np.uint8)
    qs = np.zeros(T, dtype=np.float32)
    for t in range(T):
        codes, scale = quantize_index_key(q[t])
        q8[t] = codes.reshape(H_I, D_I)
        qs[t] = scale
    k = None if wk_bits is None else (h @ decode_bf16(wk_bits).T).astype(np.float32)
    return q8, qs, w, k


# ---------------------------------------------------------------------------
# (f1) Masked dense variant of the sparse attention (short prefill lengths)
# ---------------------------------------------------------------------------
#
# [DSA-article] "Lets Discuss it's effectivity and accuracy", first point:
# at short lengths the prefill is run as a masked dense attention rather than
# as a gather of the selected rows.  Reading taken: for query t, every
# position s <= pos[t] of its sequence is scored and the positions not in the
# query's selection are masked out (score -inf) before the softmax -- the
# same set, hence the same result, as sparse_mla_attention, reached over
# contiguous rows.


def masked_dense_attention(q_bits, kv_bits, idx, seq_id, pos, scale: float, d_v: int = 512, block_table=None,
                           page_size: int = 64):
    """out float64[T, H, d_v], lse float64[T, H] over all s <= pos[t] with the
    positions absent from idx[t] masked out (empty selection: out 0, lse -inf).

    [DSA-article] "Lets Discuss it's effectivity and accuracy": at short
    lengths prefill runs as a masked dense attention.  Over the same selection
    it equals sparse_mla_attention; only the order of the rows differs."""
    q = decode_bf16(q_bits)
    T, H, D = q.shape
    out = np.zeros((T, H, d_v))
    lse = np.full((T, H), -np.inf)
    for t in range(T):
        n = int(pos[t]) + 1
        rows = decode_bf16(logical_rows(kv_bits, int(seq_id[t]), n, block_table, page_size))  # [n, D]
        sel = np.asarray(idx[t])
        sel = sel[sel >= 0]
        mask = np.zeros(n, dtype=bool)
        mask[sel] = True
        if not mask.any():
            continue
        z = scale * (q[t] @ rows.T)                  # [H, n]
        z = np.where(mask[None, :], z, -np.inf)
        m = z.max(axis=1, keepdims=True)
        p = np.exp(z - m)
        l = p.sum(axis=1, keepdims=True)
        out[t] = (p @ rows[:, :d_v]) / l
        lse[t] = m[:, 0] + np.log(l[:, 0])
    return out, lse


# ---------------------------------------------------------------------------
# (f3) Backward of the sparse MLA-MQA attention
# ---------------------------------------------------------------------------
#
# [DSA-article] opening paragraph and "Teaching signal": DSA is a trainable
# sparsification, the sparse stage training the main model through the
# selected set.  With o = softmax(z) V over the selected rows i, z_i =
# scale <q, kv_i>, V = kv[:, :512], and an output gradient dO, the gradients
# follow from the chain rule:
#   P_i = exp(z_i - lse),  dP_i = <dO, kv_i[:512]>,  D = <dO, o>,
#   dZ_i = P_i (dP_i - D),
#   dq = scale sum_i dZ_i kv_i[:576],
#   dkv_i[:576] += scale sum_h dZ_hi q_h,   dkv_i[:512] += sum_h P_hi dO_h.
# Several queries may select one row; their contributions add up.


def sparse_mla_attention_backward(q_bits, kv_bits, idx, seq_id, scale: float, d_out, d_v: int = 512,
                                  block_table=None, page_size: int = 64):
    """(dq float64[T, H, D], dkv_sel float64[T, k, D], dkv float64[cache shape]).

    [DSA-article] opening paragraph and "Teaching signal": DSA is trained, so
    the attention of (2) over the selected rows needs its gradient; this is
    the derivative of sparse_mla_attention.

    dkv_sel[t, j] is the gradient reaching the row idx[t, j] from query t
    (zero for padding); dkv adds them up per cache row.
    """
    q = decode_bf16(q_bits)
    kv = decode_bf16(kv_bits)
    d_out = np.asarray(d_out, dtype=np.float64)
    T, H, D = q.shape
    k = np.asarray(idx).shape[1]
    dq = np.zeros((T, H, D))
    dkv_sel = np.zeros((T, k, D))
    dkv = np.zeros(kv.shape)
    bt = None if block_table is None else np.asarray(block_table)
    for t in range(T):
        b = int(seq_id[t])
        sel = np.asarray(idx[t])
        js = np.nonzero(sel >= 0)[0]
        if len(js) == 0:
            continue
        pos = sel[js]
        if bt is None:
            where = [(b, int(s)) for s in pos]
        else:
            where = [(int(bt[b, int(s) // page_size]), int(s) % page_size) for s in pos]
        rows = np.stack([kv[w] for w in where])              # [n, D]
        z = scale * (q[t] @ rows.T)                           # [H, n]
        m = z.max(axis=1, keepdims=True)
        p = np.exp(z - m)
        p /= p.sum(axis=1, keepdims=True)                     # P_i = exp(z_i - lse)
        o = p @ rows[:, :d_v]                                 # [H, d_v]
        dP = d_out[t] @ rows[:, :d_v].T                       # [H, n]
        Dh = np.sum(d_out[t] * o, axis=1, keepdims=True)      # [H, 1]
        dZ = p * (dP - Dh)                                    # [H, n]
        dq[t] = scale * (dZ @ rows)
        g = scale * (dZ.T @ q[t])                             # [n, D]
        g[:, :d_v] += p.T @ d_out[t]
        dkv_sel[t, js] = g
        for r, w in enumerate(where):
            dkv[w] += g[r]
    return dq, dkv_sel, dkv


# ---------------------------------------------------------------------------
# (f2) Indexer training signal: KL divergence to the attention distribution
# ---------------------------------------------------------------------------
#
# [DSA-article] "Teaching signal": the indexer learns to imitate the main
# attention's distribution summed over heads, through a KL divergence; the
# target takes no gradient (the indexer's gradients stay apart from the
# language loss).  Reading, for the sparse stage (the selected set of each
# query; the dense warm-up is the same with every position 0..pos[t]
# selected):
#   target   p_t[j] = (1/H) sum_h softmax_h(z_t)[j]   over the selected entries
#            (the head sum, normalised to total 1)
#   indexer  q_t[j] = softmax_j(I[t, idx[t, j]])      over the same entries
#   loss     L_t = sum_j p_t[j] (log p_t[j] - log q_t[j])  (terms with p = 0 are 0)
#   dL/dI[t, idx[t, j]] = q_t[j] - p_t[j]
# and through I = sum_h w_h ReLU(qd_h . kd_s), with qd = qs * q8 and
# kd = ks * k8 the dequantised FP8 query and key (quantisation taken as the
# identity in the backward):
#   dL/dw_h  = sum_j dI_j ReLU(qd_h . kd_j)
#   dL/dqd_h = w_h sum_j dI_j [qd_h . kd_j > 0] kd_j
#   dL/dkd_j = dI_j sum_h w_h [qd_h . kd_j > 0] qd_h     (added per cache row)


def indexer_kl_target(q_bits, kv_bits, idx, seq_id, scale: float, block_table=None, page_size: int = 64):
    """float64 [T, k]: the head-mean attention probability of each selected
    entry (0 for padding entries).

    [DSA-article] "Teaching signal": the indexer learns to imitate the main
    attention's head-summed distribution; divided by the number of heads it
    sums to 1 over the selected entries."""
    q = decode_bf16(q_bits)
    kv = decode_bf16(kv_bits)
    T, H, D = q.shape
    idx = np.asarray(idx)
    out = np.zeros(idx.shape)
    bt = None if block_table is None else np.asarray(block_table)
    for t in range(T):
        js = np.nonzero(idx[t] >= 0)[0]
        if len(js) == 0:
            continue
        b = int(seq_id[t])
        if bt is None:
            rows = kv[b, idx[t, js]]
        else:
            rows = np.stack([kv[int(bt[b, int(s) // page_size]), int(s) % page_size] for s in idx[t, js]])
        z = scale * (q[t] @ rows.T)                            # [H, n]
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        out[t, js] = p.mean(axis=0)
    return out


def indexer_kl(q8, qs, w, k8, ks, idx, seq_id, target, block_table=None, page_size: int = 64):
    """KL loss of the indexer against `target` and its gradients.

    [DSA-article] "Teaching signal": the indexer is trained through a KL
    divergence toward the target distribution, its gradients kept apart from
    the main model's loss.

    Returns (loss [T], dI [T, k], dq [T, H_I, D_I], dw [T, H_I], dk in the
    key cache's shape [..., D_I]), float64; padding entries of idx get dI = 0.
    """
    qd = decode_e4m3fn(np.asarray(q8)) * np.asarray(qs, dtype=np.float64)[:, None, None]   # [T, H_I, D_I]
    w = np.asarray(w, dtype=np.float64)
    k8 = np.asarray(k8)
    kscale = np.asarray(ks, dtype=np.float64)
    target = np.asarray(target, dtype=np.float64)
    idx = np.asarray(idx)
    T = qd.shape[0]
    loss = np.zeros(T)
    dI = np.zeros(idx.shape)
    dq = np.zeros(qd.shape)
    dw = np.zeros(w.shape)
    dk = np.zeros(k8.shape)
    bt = None if block_table is None else np.asarray(block_table)
    for t in range(T):
        js = np.nonzero(idx[t] >= 0)[0]
        if len(js) == 0:
            continue
        b = int(seq_id[t])
        if bt is None:
            where = [(b, int(s)) for s in idx[t, js]]
        else:
            where = [(int(bt[b, int(s) // page_size]), int(s) % page_size) for s in idx[t, js]]
        kd = np.stack([decode_e4m3fn(k8[wh]) * kscale[wh] for wh in where])   # [n, D_I]
        r = qd[t] @ kd.T                                                     # [H_I, n]
        logit = w[t] @ np.maximum(r, 0.0)                                    # [n]
        qdist = np.exp(logit - logit.max())
        qdist /= qdist.sum()
        p = target[t, js]
        pos = p > 0
        loss[t] = np.sum(p[pos] * (np.log(p[pos]) - np.log(qdist[pos])))
        g = qdist - p                                                        # dL/dI
        dI[t, js] = g
        m = (r > 0).astype(np.float64)
        dw[t] = np.maximum(r, 0.0) @ g
        dq[t] = w[t][:, None] * ((m * g[None, :]) @ kd)
        gk = g[:, None] * ((m * w[t][:, None]).T @ qd[t])                    # [n, D_I]
        for i, wh in enumerate(where):
            dk[wh] += gk[i]
    return loss, dI, dq, dw, dk
