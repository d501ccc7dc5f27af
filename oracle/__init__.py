"""CPU fp64 oracle for MLA decode over a paged latent KV cache.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call anything in this package; the product
path (the HIP library and its Python binding) never does, and this package
imports nothing from it.

What it computes is the plain definition of the method: scaled dot-product
attention of every query row over the visible latent rows of its sequence,
with the full score matrix materialised, in float64. The kernel described on
the pages (PaddleNLP issue #10157, "Multi-head Latent Attention (MLA) operator",
overview) splits one MLA pass into data load, QK GEMM, online-softmax update
and PV GEMM; the online softmax reaches the same result as the plain softmax up
to rounding order, so the oracle is the plain softmax written out.

It also holds the cache append (each sequence's newest latent rows stored in
their pages, quantised per token to E4M3FN for the 8-bit cache), the step
just before attention in a decode step.

Every function is pinned by tests that do not reuse it (closed forms,
invariants, a pure-Python brute force, library cross-checks); see tests/.
"""
from .mla_oracle import (  # noqa: F401
    PAGE_TOKENS, D_QK, D_V,
    bf16_bits_to_f64, e4m3fn_value, E4M3FN_TABLE, decode_e4m3fn,
    sequence_rows, visible_counts, attend, attend_partials, lse_merge,
    mla_decode, mla_decode_sequence, mla_decode_varlen,
    E4M3FN_MAX, encode_e4m3fn, quantize_token_e4m3, append_kv, quantize_query_rows_e4m3, query_row_exponent,
    D_NOPE, D_ROPE, D_QK_PREFILL, D_V_PREFILL, mla_prefill,
)
from . import prefill_quant  # noqa: F401,E402
