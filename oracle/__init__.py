"""CPU oracle for the DeepSeek Sparse Attention (DSA) decode/prefill hot path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 NumPy
reference that the GPU library is checked against.  Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it; the product
path (the HIP library and its Python binding) never does, and this package
imports nothing from the product package.

Every function states the passage of the source pages it follows.  The pages
are web articles about DeepSeek-V3.2-Exp; the primary one is
"DeepSeek V3.2-Exp Cuts Prolonged-Context Costs With DeepSeek Sparse
Consideration (DSA) Whereas Sustaining Benchmark Parity" (nextbusiness24.com,
a MarkTechPost repost whose English is synonym-spun: "Consideration" means
attention).  It is cited below as [DSA-article] with its part name.
"""

from .dsa_oracle import (  # noqa: F401
    decode_e4m3fn,
    decode_bf16,
    logical_rows,
    indexer_logits,
    indexer_logits_row,
    topk_select,
    sparse_mla_attention,
    dsa_forward,
    encode_e4m3fn,
    quantize_index_key,
    cache_write,
    indexer_projection,
    masked_dense_attention,
    sparse_mla_attention_backward,
    indexer_kl_target,
    indexer_kl,
)
