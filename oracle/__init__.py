"""Plain, slow, fp64 CPU oracle for prefix-shared decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or link anything in this package; only
the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP path: it reads the same
host copies of the KV pools and page tables and computes the definitions
written out on the pages, one query at a time.

Sources (the pages this oracle restates; no listing is copied):

* "BatchLLM: Optimizing Large Batched LLM Inference with Global Prefix
  Sharing and Throughput-oriented Token Batching", summary page on
  papercache.org (cited below as *BatchLLM*), §2.2 Eq. 1 (prefix / distinct
  partial attention merged by online softmax), §3.2 Eq. 2 (token-saving
  rate), §4.2 + Fig. 4 (maximising first-level prefix reuse on a compact
  prefix tree by dynamic programming), §5 (prefix identification from
  nested input ids).
* The continuous-batching post on guijiagi.com (cited as *CB blog*),
  "block management" and "attention computation" sections: paged KV
  blocks, block tables, gather-by-table, truncate to the sequence length,
  softmax(q K^T / sqrt(d)) V.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
something other than itself (closed forms, hand-computed cases, a library
routine on special cases, invariants, brute force on tiny inputs).
"""

from .attention import (  # noqa: F401
    EMPTY_M,
    gather_segment,
    query_context,
    partial_attention,
    merge_partials,
    merge_many,
    decode_attention,
    decode_attention_rows,
)
from .flatten import (  # noqa: F401
    maximize_reuse,
    grouping_saving,
    flatten_tree,
    saving_rate,
    prefix_tree_from_tokens,
    identify_groups,
)
