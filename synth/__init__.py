"""Seeded synthetic workloads for the shared-context KV-cache correction path.

This package only draws inputs: base caches, planted low-rank deltas, exact caches,
anchor factors and descriptor targets.  It performs none of the correction or fit
arithmetic (no pooling, no cosine, no softmax, no truncation); both the fp64 oracle
and the HIP library consume the tensors it returns, bit for bit.
"""
from .workloads import (  # noqa: F401
    CONFIGS,
    Config,
    Case,
    Edge,
    build_descriptors,
    fit_input,
    generate,
    generate_fanout,
    generate_pool,
    planted_spectrum,
    pool_descriptors,
    to_f64,
)
