"""CPU oracle for DSA sparse-MLA prefill attention (float64, numpy).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the library.
"""

from .dsa_oracle import (  # noqa: F401
    UNION_BLOCK,
    bf16_to_f64,
    group_union_mask,
    grouped_sparse_mqa,
    masked_mha,
    pertoken_sparse_mqa,
    selected_positions,
    softmax_attention,
    union_pad,
)
