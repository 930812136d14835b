"""Prefix-shared decode attention for MI355X (gfx950): Python binding of libpsa.so.

The entry points keep the C names (include/psa.h): ``psa_build_plan``,
``psa_plan_upload``, ``psa_decode_attention``, ``psa_merge``,
``psa_flatten_prefix_tree``, ``psa_identify_prefix_groups``, ``psa_plan_get_info``.  The library is loaded on
first use and its absence is an error.
"""

from ._lib import (  # noqa: F401
    DEBUG_POISON,
    DISTINCT_ONLY,
    EXPORTS,
    ISSUE_PATTERNS,
    FORCE_MATVEC,
    LIB_PATH,
    NO_TILE_PAIRS,
    NO_PAGE_SHARING,
    NO_XCD_ORDER,
    PREFIX_ONLY,
    PSA_BF16,
    PSA_F32,
    Plan,
    PsaError,
    lib,
    make_config,
    psa_build_plan,
    psa_debug_issue_probe,
    psa_debug_mfma_peak,
    psa_debug_read_peak,
    psa_decode_attention,
    psa_decode_attention_noalloc,
    psa_flatten_prefix_tree,
    psa_identify_prefix_groups,
    psa_merge,
    psa_plan_get_info,
    psa_plan_upload,
)
from .runner import DecodeStep  # noqa: F401
