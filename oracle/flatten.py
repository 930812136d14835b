"""Oracle for flattening a multi-level prefix tree to single-level groups.

TEST INFRASTRUCTURE ONLY (see the package docstring).

BatchLLM §4.2 and Fig. 4: prompts are organised in a compact prefix tree
(each node is a run of tokens shared by everything below it).  Only one
prefix level is kept: every request ends up in at most one prefix-sharing
group whose prefix is a common prefix of all its members (the root-to-node
token path of a tree node), and deeper levels are unfolded into the
request's distinct part.  The grouping is chosen to maximise first-level
token reuse, solved bottom-up on the tree by dynamic programming.

Objective (pinned by the Fig. 4 discussion: sharing a 1-token node among 5
prompts saves 4 tokens, sharing an 8-token prefix between 2 prompts saves
8): a group of n requests with prefix length a saves a * (n - 1) tokens;
maximise the sum over groups.  This is also the saved-token count of the
token-saving rate, BatchLLM §3.2 Eq. 2.

DP (plain reading; the algorithm body is not on the page).  For node D with
path length a(D), h_D[k] is the best saving inside D's subtree when k of its
requests are handed up to D's parent still ungrouped.  Children (and requests
attached directly at D, each handing up itself) combine by max-plus
convolution; then D may form one group from j >= 2 of the k handed-up
requests: h'_D[k - j] = max(h_D[k] + a(D) * (j - 1)).  The answer is
max_k h_root[k] at a virtual root of path length 0.  Ties prefer fewer
groups.

Tree format (plain dict of arrays):
  node_parent[M]   parent node id, -1 = child of the virtual root
  node_len[M]      tokens in the node
  query_node[N]    deepest tree node whose tokens the query shares, -1 = none
For ``flatten_tree`` also node_page_off[M+1], node_pages, query_distinct_len,
query_page_off[N+1], query_pages and page_size.
"""

from __future__ import annotations

import numpy as np

NEG = -(1 << 62)


def path_lengths(node_parent, node_len):
    """a(D): tokens on the path from the (virtual) root through D."""
    m = len(node_parent)
    a = [None] * m
    for d in range(m):
        chain = []
        x = d
        while x >= 0 and a[x] is None:
            chain.append(x)
            x = int(node_parent[x])
            if len(chain) > m:
                raise ValueError("cycle in node_parent")
        base = 0 if x < 0 else a[x]
        for y in reversed(chain):
            base += int(node_len[y])
            a[y] = base
    return a


def _maxplus(h, t):
    """Max-plus convolution; returns (result, split) with split[k] = k taken from t."""
    n = len(h) + len(t) - 1
    out = [NEG] * n
    split = [0] * n
    for i, hv in enumerate(h):
        if hv == NEG:
            continue
        for j, tv in enumerate(t):
            if tv == NEG:
                continue
            v = hv + tv
            if v > out[i + j]:
                out[i + j] = v
                split[i + j] = j
    return out, split


def maximize_reuse(node_parent, node_len, query_node):
    """Best total saving and one optimal grouping.

    Returns (saving, group_node) with group_node[i] = node at which query i's
    group is formed, or -1 when it stays ungrouped.
    """
    node_parent = [int(x) for x in node_parent]
    query_node = [int(x) for x in query_node]
    m = len(node_parent)
    a = path_lengths(node_parent, node_len)
    kids = [[] for _ in range(m + 1)]  # index m = virtual root
    direct = [[] for _ in range(m + 1)]
    for d, p in enumerate(node_parent):
        kids[m if p < 0 else p].append(d)
    for i, d in enumerate(query_node):
        direct[m if d < 0 else d].append(i)
    path = a + [0]

    memo = {}

    # post-order without recursion limits
    order = []
    stack = [(m, False)]
    while stack:
        x, done = stack.pop()
        if done:
            order.append(x)
            continue
        stack.append((x, True))
        for c in kids[x]:
            stack.append((c, False))

    for x in order:
        # items: children tables then direct queries (each a table [NEG, 0])
        h = [0]
        splits = []
        items = [("node", c) for c in kids[x]] + [("query", i) for i in direct[x]]
        for kind, v in items:
            t = memo[v]["out"] if kind == "node" else [NEG, 0]
            h, sp = _maxplus(h, t)
            splits.append(sp)
        # optional group at x from j >= 2 handed-up queries
        out = list(h)
        choice = [(k, 0) for k in range(len(h))]
        for k in range(2, len(h) if x != m else 0):
            if h[k] == NEG:
                continue
            for j in range(2, k + 1):
                v = h[k] + path[x] * (j - 1)
                if v > out[k - j]:
                    out[k - j] = v
                    choice[k - j] = (k, j)
        memo[x] = {"out": out, "in": h, "choice": choice, "items": items, "splits": splits}

    root = memo[m]
    best_k = max(range(len(root["out"])), key=lambda k: (root["out"][k], -k))
    best = root["out"][best_k]

    group_node = [-1] * len(query_node)

    def backtrack(x, k_out):
        """Returns the ids of the k_out queries handed up from x's subtree."""
        e = memo[x]
        k_in, j = e["choice"][k_out]
        # undo the convolution chain to find each item's handed-up count
        counts = []
        k = k_in
        for sp in reversed(e["splits"]):
            counts.append(sp[k])
            k -= sp[k]
        counts.reverse()
        ids = []
        for (kind, v), c in zip(e["items"], counts):
            if kind == "node":
                ids.extend(backtrack(v, c))
            elif c == 1:
                ids.append(v)
        if j and x != m:
            for i in ids[:j]:
                group_node[i] = x
            ids = ids[j:]
        return ids

    backtrack(m, best_k)
    return int(best), group_node


def grouping_saving(node_parent, node_len, query_node, group_node):
    """Saving of a given grouping: sum over groups of a(D) * (n - 1).

    Raises ValueError if a query is grouped at a node that is not on its path.
    """
    a = path_lengths(node_parent, node_len)
    counts = {}
    for i, g in enumerate(group_node):
        g = int(g)
        if g < 0:
            continue
        x = int(query_node[i])
        while x >= 0 and x != g:
            x = int(node_parent[x])
        if x != g:
            raise ValueError(f"query {i} grouped at node {g}, which is not on its path")
        counts[g] = counts.get(g, 0) + 1
    return sum(a[g] * (n - 1) for g, n in counts.items())


def flatten_tree(tree, group_node):
    """Single-level batch (page tables) from a tree and a grouping.

    A group formed at node D gets the pages of the root-to-D path as its
    prefix; every query keeps the pages of the nodes below its group (or the
    whole path when ungrouped) followed by its own distinct pages (BatchLLM
    §4.2: deeper levels are unfolded into the distinct part).  Nodes must
    hold whole pages.  Groups of one query are dissolved.
    """
    P = int(tree["page_size"])
    parent = [int(x) for x in tree["node_parent"]]
    nlen = [int(x) for x in tree["node_len"]]
    if any(x % P for x in nlen):
        raise ValueError("tree nodes must hold whole pages")
    noff = tree["node_page_off"]
    npg = tree["node_pages"]

    def node_pages(d):
        return list(npg[int(noff[d]):int(noff[d + 1])])

    def path(d):
        out = []
        while d >= 0:
            out.append(d)
            d = parent[d]
        return out[::-1]

    counts = {}
    for g in group_node:
        if g >= 0:
            counts[g] = counts.get(g, 0) + 1
    gids = sorted(g for g, c in counts.items() if c >= 2)
    gidx = {g: i for i, g in enumerate(gids)}
    group_prefix_len, group_page_off, group_pages = [], [0], []
    for g in gids:
        pages = [p for d in path(g) for p in node_pages(d)]
        group_pages.extend(pages)
        group_page_off.append(len(group_pages))
        group_prefix_len.append(sum(nlen[d] for d in path(g)))
    qn = tree["query_node"]
    qoff = tree["query_page_off"]
    qpg = tree["query_pages"]
    query_group, dlen, qpoff, qpages = [], [], [0], []
    for i in range(len(qn)):
        g = int(group_node[i])
        g = g if g in gidx else -1
        nodes = path(int(qn[i])) if int(qn[i]) >= 0 else []
        if g >= 0:
            nodes = nodes[nodes.index(g) + 1:]
        pages = [p for d in nodes for p in node_pages(d)]
        own = list(qpg[int(qoff[i]):int(qoff[i + 1])])
        qpages.extend(pages + own)
        qpoff.append(len(qpages))
        query_group.append(gidx[g] if g >= 0 else -1)
        dlen.append(sum(nlen[d] for d in nodes) + int(tree["query_distinct_len"][i]))
    return {
        "page_size": P,
        "group_prefix_len": np.asarray(group_prefix_len, dtype=np.int32),
        "group_page_off": np.asarray(group_page_off, dtype=np.int64),
        "group_pages": np.asarray(group_pages, dtype=np.int32),
        "query_group": np.asarray(query_group, dtype=np.int32),
        "query_distinct_len": np.asarray(dlen, dtype=np.int32),
        "query_page_off": np.asarray(qpoff, dtype=np.int64),
        "query_pages": np.asarray(qpages, dtype=np.int32),
    }


def saving_rate(logical_tokens, saved_tokens):
    """BatchLLM §3.2 Eq. 2: (1 - processed / logical) * 100, processed = logical - saved."""
    logical_tokens = float(logical_tokens)
    if logical_tokens <= 0:
        return 0.0
    return (1.0 - (logical_tokens - float(saved_tokens)) / logical_tokens) * 100.0


def prefix_tree_from_tokens(requests):
    """Compact prefix tree of token sequences (BatchLLM §4.2: prompts in a
    compact prefix tree, each node a run of tokens shared by everything below
    it; the identification step of §5 takes nested input ids).

    Plain construction: a character trie with one node per token position,
    each trie node counting the requests that pass through it; a trie node
    is kept as a tree node when at least two requests pass through it and it
    is the deepest such node before the requests passing through it change
    (a child with fewer passing requests, or a request ending there).  The
    kept nodes, linked to their nearest kept ancestor, are the compact tree;
    a request hangs at the deepest kept node on its path (-1 = none).

    Returns (node_parent, node_len, query_node) in the tree format above.
    """
    root = {"kids": {}, "count": 0, "ends": 0, "depth": 0}
    paths = []
    for seq in requests:
        node = root
        node["count"] += 1
        path = [node]
        for t in seq:
            t = int(t)
            if t not in node["kids"]:
                node["kids"][t] = {"kids": {}, "count": 0, "ends": 0, "depth": node["depth"] + 1}
            node = node["kids"][t]
            node["count"] += 1
            path.append(node)
        node["ends"] += 1
        paths.append(path)

    def kept(nd):
        if nd is root or nd["count"] < 2:
            return False
        if nd["ends"] > 0:
            return True
        return all(c["count"] < nd["count"] for c in nd["kids"].values())

    ids = {}
    node_parent, node_depth = [], []
    for path in paths:
        last = -1
        for nd in path:
            if not kept(nd):
                continue
            key = id(nd)
            if key not in ids:
                ids[key] = len(node_parent)
                node_parent.append(last)
                node_depth.append(nd["depth"])
            last = ids[key]
    query_node = []
    for path in paths:
        q = -1
        for nd in path:
            if kept(nd):
                q = ids[id(nd)]
        query_node.append(q)
    node_len = [node_depth[d] - (node_depth[p] if p >= 0 else 0) for d, p in enumerate(node_parent)]
    return node_parent, node_len, query_node


def identify_groups(requests):
    """Prefix-sharing groups of token sequences: the compact prefix tree,
    then ``maximize_reuse`` on it.  Returns (saving, group_prefix_len per
    request, -1 when ungrouped; group node per request)."""
    node_parent, node_len, query_node = prefix_tree_from_tokens(requests)
    saving, group_node = maximize_reuse(node_parent, node_len, query_node)
    a = path_lengths(node_parent, node_len)
    prefix = [a[g] if g >= 0 else -1 for g in group_node]
    return saving, prefix, group_node
