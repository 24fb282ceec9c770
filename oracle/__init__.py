"""Plain CPU fp64 oracle of the KV-cache correction hot path (test infrastructure).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may import
this package.  The product path (the HIP library and its Python binding) never does.
"""
from .kvc_oracle import (  # noqa: F401
    chain,
    correct,
    correct_pooled,
    correct_rank,
    cosine_scores,
    effective_rank,
    fanout,
    fit_anchor,
    fit_from_gram,
    gram,
    layer_error,
    pool,
    pool_insert,
    project,
    rank_descriptor,
    rank_error_curve,
    rank_scores,
    reliability,
    rel_frobenius,
    round_to_bf16,
    round_to_dtype,
    select_anchors,
    segment_error,
    softmax_weights,
)
