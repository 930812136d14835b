"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

Holds no arithmetic of the method: only shapes, seeded lengths, shuffled
page allocation, seeded values and byte/flop bookkeeping.
"""

from .synth import (  # noqa: F401
    PRESETS,
    Workload,
    make_workload,
    build_single_level,
    build_two_level,
    build_tree,
    permute_groups,
    share_leading_pages,
    build_family_case,
    build_token_batch,
    build_mixed,
    make_values,
    fill_stale,
    algorithmic_cost,
    subset_for_queries,
)
