"""Seeded synthetic inputs for the five paged-KV workloads.

This module only draws numbers: normal K/V/q tensors with the outlier
structure described on the page "Half the Cache, Twice the Context"
(section "What the cache loses when you round it": persistent key-channel
outliers scaled by 4 on every 16th channel, value-token outliers scaled by 6
on every 64th token), rounded to bf16, plus seeded page permutations and
context lengths.  It holds none of the quantize / attend arithmetic, so the
oracle and the HIP path can both consume its output without sharing code.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    seed_for,
    kv_rows,
    queries,
    page_permutation,
    q8_batch_lengths,
    planted_position,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
)
