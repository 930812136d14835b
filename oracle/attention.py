"""fp64 oracle of prefix-shared decode attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY: imported by tests, ``__graft_entry__.smoke()`` and
``bench.py``'s cpu_baseline leg, never by the product path.

What is computed (plain definitions, no blocking or fusion):

* Paged KV (CB blog, "block management"): the KV of a sequence lives in
  fixed-size physical blocks named by a block table; logically contiguous
  tokens are scattered over physical pages (BatchLLM §2.2, KV cache).  Our
  pools are laid out ``[num_pages, num_kv_heads, page_size, head_dim]``;
  token ``t`` of a segment sits in page ``pages[t // page_size]`` at slot
  ``t % page_size``.
* Decode attention for one query (CB blog, "attention computation"): gather
  the blocks named by the table, keep the first ``num_tokens`` tokens, then
  ``softmax(q K^T * scale) V`` with ``scale = 1/sqrt(head_dim)``.
* Prefix sharing (BatchLLM §2.2, Eq. 1): a query of a prefix-sharing group
  attends to the group's prefix KV followed by its own distinct KV.  The
  oracle computes this as ONE softmax over the concatenated context, which is
  the result Eq. 1's split-then-merge has to reproduce.
* ``partial_attention`` / ``merge_partials``: Eq. 1's two operations.  The
  page writes ``online_softmax(O_prefix, O_distinct)`` without the statistics
  it needs; following the online-normaliser reference the page cites, a
  partial result carries (O, m, l): O normalised by its own l, m the maximum
  scaled score (natural-log units), l = sum(exp(s - m)).  The empty partial
  is (0, -inf, 0).

GQA: query head ``h`` reads kv head ``h // (Hq // Hkv)`` (contiguous mapping;
the pages do not state one).
"""

from __future__ import annotations

import math

import numpy as np

EMPTY_M = -math.inf


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def gather_segment(pool, pages, length, kvh, page_size):
    """Tokens ``0..length-1`` of one paged segment for kv head ``kvh``.

    CB blog, "attention computation": collect the blocks of the block table in
    order, concatenate them, truncate to the sequence's token count.
    Returns float64 ``[length, head_dim]``.
    """
    length = int(length)
    head_dim = pool.shape[-1]
    if length == 0:
        return np.zeros((0, head_dim), dtype=np.float64)
    npages = -(-length // page_size)
    pages = np.asarray(pages, dtype=np.int64)[:npages]
    blocks = [_f64(pool[int(p), kvh]) for p in pages]  # each [page_size, d]
    return np.concatenate(blocks, axis=0)[:length]


def query_context(batch, i):
    """The (pages, length) segments query ``i`` attends to, in context order.

    BatchLLM §2.2 Eq. 1 / §5: a query of group g sees the group's prefix then
    its own distinct part; a query with no group (``query_group == -1``)
    sees only its distinct part.  With ``query_prefix_len`` (optional) query
    i sees only the first ``query_prefix_len[i]`` prefix tokens: a token of a
    prefill chunk batched with decode queries (BatchLLM §4.3, Fig. 10c)
    attends causally, to its context up to and including itself.
    """
    segs = []
    g = int(batch["query_group"][i])
    if g >= 0:
        a, b = int(batch["group_page_off"][g]), int(batch["group_page_off"][g + 1])
        lp = int(batch["group_prefix_len"][g])
        lim = batch.get("query_prefix_len")
        if lim is not None:
            lp = min(lp, int(lim[i]))
        segs.append((batch["group_pages"][a:b], lp))
    a, b = int(batch["query_page_off"][i]), int(batch["query_page_off"][i + 1])
    segs.append((batch["query_pages"][a:b], int(batch["query_distinct_len"][i])))
    return segs


def partial_attention(q_rows, K, V, scale):
    """Eq. 1's ``partial_attention`` for query rows ``q_rows [r, d]``.

    Returns (O [r, d] normalised, m [r], l [r]) in float64.  An empty token
    range gives the empty partial (0, -inf, 0).
    """
    q_rows = _f64(q_rows)
    K = _f64(K)
    V = _f64(V)
    r, d = q_rows.shape
    if K.shape[0] == 0:
        return np.zeros((r, V.shape[1] if V.ndim == 2 else d)), np.full(r, EMPTY_M), np.zeros(r)
    s = scale * (q_rows @ K.T)  # [r, L] scaled scores
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    O = (p @ V) / l[:, None]
    return O, m, l


def merge_partials(a, b):
    """Eq. 1's ``online_softmax``: merge two partial results of the same rows.

    m = max(m_a, m_b); w_x = l_x * exp(m_x - m); l = w_a + w_b;
    O = (w_a O_a + w_b O_b) / l.  Merging with an empty partial is the
    identity; merging two empty partials gives the empty partial.
    """
    Oa, ma, la = (_f64(x) for x in a)
    Ob, mb, lb = (_f64(x) for x in b)
    m = np.maximum(ma, mb)
    with np.errstate(invalid="ignore"):
        wa = np.where(la > 0, la * np.exp(ma - m), 0.0)
        wb = np.where(lb > 0, lb * np.exp(mb - m), 0.0)
    l = wa + wb
    safe = np.where(l > 0, l, 1.0)
    O = (wa[..., None] * Oa + wb[..., None] * Ob) / safe[..., None]
    O = np.where((l > 0)[..., None], O, 0.0)
    m = np.where(l > 0, m, EMPTY_M)
    return O, m, l


def merge_many(parts):
    """Left fold of ``merge_partials`` over a list of partials."""
    acc = parts[0]
    for p in parts[1:]:
        acc = merge_partials(acc, p)
    return acc


def _scale_for(head_dim, scale):
    return 1.0 / math.sqrt(head_dim) if scale is None or scale <= 0 else float(scale)


def decode_attention(q, k_pool, v_pool, batch, scale=None, queries=None):
    """Plain decode attention of every query over prefix ++ distinct context.

    ``q [N, Hq, d]``; ``k_pool, v_pool [num_pages, Hkv, page_size, d]``;
    ``batch`` holds the page tables (see ``query_context``).  Returns
    (O [n, Hq, d], m [n, Hq], l [n, Hq]) in float64 for the queries listed in
    ``queries`` (default: all, in order).  Scale 1/sqrt(d) unless given
    (CB blog, "attention computation").
    """
    q = np.asarray(q)
    n_all, hq, d = q.shape
    hkv = k_pool.shape[1]
    page_size = k_pool.shape[2]
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    r = hq // hkv
    sc = _scale_for(d, scale)
    qs = range(n_all) if queries is None else list(queries)
    O = np.zeros((len(qs), hq, d))
    M = np.zeros((len(qs), hq))
    L = np.zeros((len(qs), hq))
    for oi, i in enumerate(qs):
        segs = query_context(batch, i)
        if sum(length for _, length in segs) == 0:
            raise ValueError(f"query {i} has an empty context")
        for kvh in range(hkv):
            K = np.concatenate([gather_segment(k_pool, p, n, kvh, page_size) for p, n in segs])
            V = np.concatenate([gather_segment(v_pool, p, n, kvh, page_size) for p, n in segs])
            rows = slice(kvh * r, (kvh + 1) * r)
            O[oi, rows], M[oi, rows], L[oi, rows] = partial_attention(q[i, rows], K, V, sc)
    return O, M, L


def decode_attention_rows(q, k_pool, v_pool, batch, pairs, scale=None):
    """Like ``decode_attention`` but only for listed (query, q_head) pairs.

    Used for sampled checks at full size.  Returns O [len(pairs), d], m, l.
    """
    q = np.asarray(q)
    _, hq, d = q.shape
    hkv = k_pool.shape[1]
    page_size = k_pool.shape[2]
    r = hq // hkv
    sc = _scale_for(d, scale)
    O = np.zeros((len(pairs), d))
    M = np.zeros(len(pairs))
    L = np.zeros(len(pairs))
    for j, (i, h) in enumerate(pairs):
        kvh = h // r
        segs = query_context(batch, i)
        K = np.concatenate([gather_segment(k_pool, p, n, kvh, page_size) for p, n in segs])
        V = np.concatenate([gather_segment(v_pool, p, n, kvh, page_size) for p, n in segs])
        o, m, l = partial_attention(q[i, h][None, :], K, V, sc)
        O[j], M[j], L[j] = o[0], m[0], l[0]
    return O, M, L
