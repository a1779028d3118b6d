"""CPU oracle for DSA sparse-MLA prefill attention (float64, numpy).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the library.
"""

from .dsa_oracle import (  # noqa: F401
    UNION_BLOCK,
    bf16_to_f64,
    convert_req_index_to_global,
    dense_causal_mha,
    dequant_latent_fp8,
    fp8_e4m3_to_f64,
    group_union_mask,
    group_union_mask_varlen,
    grouped_sparse_mqa,
    grouped_sparse_mqa_varlen,
    masked_mha,
    pertoken_sparse_mqa,
    pertoken_sparse_mqa_fp8,
    pertoken_sparse_mqa_varlen,
    pertoken_sparse_mqa_varlen_fp8,
    physical_row,
    request_of_tokens,
    selected_positions,
    softmax_attention,
    union_pad,
    varlen_groups,
)
