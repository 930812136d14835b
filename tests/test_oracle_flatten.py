"""Pins for the prefix-tree flattening oracle and the saving rate (CPU only).

* Brute force: the DP optimum equals the best grouping over all set
  partitions of the requests on random trees of up to 8 requests.
* Printed values: Fig. 4's two savings (4 and 8 tokens) and §6.3.1's saving
  rates (85.2 %, 92.6 %) of the BatchLLM summary page (tests/golden).
* Closed form: the two-level 4 x 16 x 16 workload saves 64 * 3072 * 15
  tokens when every sub-prefix forms its own group.
* Flattening keeps every query's token sequence.
* Token-level identification (compact tree from token ids + the DP): the
  Fig. 4 reading written as token sequences gives the golden tree and its
  savings; on tiny random token sets the result equals the best partition
  of the requests with each group saving LCP(group) * (size - 1).
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import flatten as F
from workloads import build_two_level, make_values

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def set_partitions(items):
    if not items:
        yield []
        return
    first, rest = items[0], items[1:]
    for part in set_partitions(rest):
        for i in range(len(part)):
            yield part[:i] + [[first] + part[i]] + part[i + 1:]
        yield [[first]] + part


def brute_force(node_parent, node_len, query_node):
    """Best saving over all partitions; a block's prefix is its members' deepest common node."""
    a = F.path_lengths(node_parent, node_len)

    def ancestors(x):
        out = []
        while x >= 0:
            out.append(x)
            x = int(node_parent[x])
        return out

    best = 0
    n = len(query_node)
    for part in set_partitions(list(range(n))):
        tot = 0
        for block in part:
            if len(block) < 2:
                continue
            common = set(ancestors(int(query_node[block[0]])))
            for i in block[1:]:
                common &= set(ancestors(int(query_node[i])))
            if common:
                tot += max(a[x] for x in common) * (len(block) - 1)
        best = max(best, tot)
    return best


def random_tree(rng, n_nodes, n_queries, max_len=9):
    parent = [-1]
    for d in range(1, n_nodes):
        parent.append(int(rng.integers(-1, d)))
    lens = [int(x) for x in rng.integers(1, max_len + 1, size=n_nodes)]
    qn = [int(x) for x in rng.integers(-1, n_nodes, size=n_queries)]
    return parent, lens, qn


@pytest.mark.parametrize("seed", range(40))
def test_dp_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    n_nodes = int(rng.integers(1, 7))
    n_q = int(rng.integers(1, 9))
    parent, lens, qn = random_tree(rng, n_nodes, n_q)
    best, grouping = oracle.maximize_reuse(parent, lens, qn)
    assert best == brute_force(parent, lens, qn)
    assert oracle.grouping_saving(parent, lens, qn, grouping) == best


def test_greedy_deepest_is_not_always_optimal():
    """A small deep node can be worth less than leaving its prompts in a big shallow group."""
    # node 0 (10 tokens) has child node 1 (1 token); 2 queries under node 1, 1 query at node 0
    parent, lens, qn = [-1, 0], [10, 1], [1, 1, 0]
    best, g = oracle.maximize_reuse(parent, lens, qn)
    assert best == 20 == brute_force(parent, lens, qn)  # all three at node 0: 10 * 2
    assert oracle.grouping_saving(parent, lens, qn, [1, 1, -1]) == 11


def test_fig4_printed_savings():
    with open(os.path.join(GOLDEN, "fig4_reuse.json")) as f:
        g = json.load(f)
    for p in g["printed"]:
        assert oracle.grouping_saving(g["node_parent"], g["node_len"], g["query_node"], p["grouping"]) == p["saving"]
    best, grouping = oracle.maximize_reuse(g["node_parent"], g["node_len"], g["query_node"])
    assert best >= max(p["saving"] for p in g["printed"])
    assert best == g["derived_optimum"]["saving"] == brute_force(g["node_parent"], g["node_len"], g["query_node"])


def test_saving_rate_printed_values():
    with open(os.path.join(GOLDEN, "saving_rate.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        n = c["sharing_degree"]
        logical = n * (c["prefix"] + c["distinct"])
        # the best single-level grouping: one group of n at the prefix node
        parent, lens, qn = [-1], [c["prefix"]], [0] * n
        saved, _ = oracle.maximize_reuse(parent, lens, qn)
        assert round(oracle.saving_rate(logical, saved), 1) == c["rate_percent_printed"]


def test_two_level_closed_form():
    wl = build_two_level("t", 32, 8, 128, "bf16", 4, 1024, 16, 2048, 16, (32, 256))
    t = wl.tree
    best, grouping = oracle.maximize_reuse(t["node_parent"], t["node_len"], t["query_node"])
    assert best == 64 * 3072 * 15 == 2_949_120
    # every sub-prefix node is a group of its 16 requests
    assert all(grouping[i] == t["query_node"][i] for i in range(len(grouping)))
    # the root-level alternative is worse, as the closed form says
    root_group = [int(t["node_parent"][x]) for x in t["query_node"]]
    assert oracle.grouping_saving(t["node_parent"], t["node_len"], t["query_node"], root_group) == 4 * 1024 * 255


def test_flatten_keeps_each_query_context():
    wl = build_two_level("t", 2, 1, 8, "f32", 2, 32, 3, 16, 2, (0, 20), seed=3)
    t = wl.tree
    best, grouping = oracle.maximize_reuse(t["node_parent"], t["node_len"], t["query_node"])
    batch = oracle.flatten_tree(t, grouping)
    q, k, v = (x.double().numpy() for x in make_values(wl, "cpu", 3))

    def tree_context(i):
        nodes = []
        x = int(t["query_node"][i])
        while x >= 0:
            nodes.append(x)
            x = int(t["node_parent"][x])
        pages = [p for d in reversed(nodes) for p in t["node_pages"][t["node_page_off"][d]:t["node_page_off"][d + 1]]]
        pages += list(t["query_pages"][t["query_page_off"][i]:t["query_page_off"][i + 1]])
        n = sum(int(t["node_len"][d]) for d in nodes) + int(t["query_distinct_len"][i])
        return pages, n

    for i in range(len(t["query_node"])):
        pages, n = tree_context(i)
        want = oracle.gather_segment(k, pages, n, 0, 16)
        got = np.concatenate([oracle.gather_segment(k, p, m, 0, 16) for p, m in oracle.query_context(batch, i)])
        np.testing.assert_array_equal(got, want)
    # saved tokens of the flattened batch = DP optimum
    qg = batch["query_group"]
    saved = sum(int(batch["group_prefix_len"][g]) * (int((qg == g).sum()) - 1) for g in range(len(batch["group_prefix_len"])))
    assert saved == best


def test_flatten_rejects_unaligned_nodes():
    t = {"page_size": 16, "node_parent": [-1], "node_len": [10], "node_page_off": [0, 1], "node_pages": [0],
         "query_node": [0, 0], "query_distinct_len": [1, 1], "query_page_off": [0, 1, 2], "query_pages": [1, 2]}
    with pytest.raises(ValueError):
        oracle.flatten_tree(t, [0, 0])


def test_dp_pin_catches_planted_mistake(monkeypatch):
    """Planting a wrong objective (a * n instead of a * (n - 1)) breaks the printed Fig. 4 savings."""
    def bad(node_parent, node_len, query_node, group_node):
        a = F.path_lengths(node_parent, node_len)
        counts = {}
        for g in group_node:
            if g >= 0:
                counts[g] = counts.get(g, 0) + 1
        return sum(a[g] * n for g, n in counts.items())

    monkeypatch.setattr(oracle, "grouping_saving", bad)
    with pytest.raises(AssertionError):
        test_fig4_printed_savings()


# ---------------- prefix identification from token ids ----------------

FIG4_TOKENS = [[1, 50], [2, 60, 61], [2, 70], [2, 3, 4, 5, 6, 7, 8, 9, 80], [2, 3, 4, 5, 6, 7, 8, 9, 90, 91], [2, 99]]


def test_tokens_fig4_reading():
    """Prompt 1 starts with 'a', prompts 2-6 with 'b'; prompts 4 and 5 share
    8 tokens.  The tree keeps the nodes shared by two or more prompts: 'b'
    (depth 1) and the 8-token run (depth 8, under 'b')."""
    with open(os.path.join(GOLDEN, "fig4_reuse.json")) as f:
        g = json.load(f)
    parent, length, qnode = oracle.prefix_tree_from_tokens(FIG4_TOKENS)
    assert parent == [-1, 0] and length == [1, 7] and qnode == [-1, 0, 0, 1, 1, 0]
    printed = {p["saving"] for p in g["printed"]}
    assert F.grouping_saving(parent, length, qnode, [-1, 0, 0, 0, 0, 0]) in printed  # all five under 'b'
    assert F.grouping_saving(parent, length, qnode, [-1, -1, -1, 1, 1, -1]) in printed  # prompts 4 and 5
    saving, prefix, _ = oracle.identify_groups(FIG4_TOKENS)
    assert saving == g["derived_optimum"]["saving"] and prefix == [-1, 1, 1, 8, 8, 1]


def lcp(a, b):
    k = 0
    while k < min(len(a), len(b)) and a[k] == b[k]:
        k += 1
    return k


def brute_force_tokens(seqs):
    best = 0
    for part in set_partitions(list(range(len(seqs)))):
        tot = 0
        for grp in part:
            if len(grp) >= 2:
                common = min(lcp(seqs[grp[0]], seqs[j]) for j in grp[1:])
                tot += common * (len(grp) - 1)
        best = max(best, tot)
    return best


@pytest.mark.parametrize("seed", range(40))
def test_tokens_identification_matches_brute_force(seed):
    rng = np.random.default_rng(500 + seed)
    n = int(rng.integers(1, 8))
    alphabet = int(rng.integers(1, 4))
    seqs = [list(rng.integers(0, alphabet, size=int(rng.integers(0, 7)))) for _ in range(n)]
    if rng.random() < 0.3 and n >= 2:  # duplicates and prefixes of other requests
        seqs[1] = list(seqs[0])
        if n >= 3:
            seqs[2] = list(seqs[0][: len(seqs[0]) // 2])
    saving, prefix, _ = oracle.identify_groups(seqs)
    assert saving == brute_force_tokens(seqs)
    # the grouping itself is valid and worth what it claims
    groups = {}
    for i, p in enumerate(prefix):
        if p >= 0:
            groups.setdefault(p, []).append(i)
    claimed = 0
    _, _, gnode = oracle.identify_groups(seqs)
    by_node = {}
    for i, gn in enumerate(gnode):
        if gn >= 0:
            by_node.setdefault(gn, []).append(i)
    for members in by_node.values():
        p = prefix[members[0]]
        assert len(members) >= 2 and all(prefix[j] == p for j in members)
        assert all(len(seqs[j]) >= p and list(seqs[j][:p]) == list(seqs[members[0]][:p]) for j in members)
        claimed += p * (len(members) - 1)
    assert claimed == saving


def test_tokens_tree_pin_catches_planted_mistake(monkeypatch):
    """Keeping a node where all requests continue together (no branch)
    would split a run; the Fig. 4 pin must notice."""
    orig = F.prefix_tree_from_tokens

    def wrong(requests):
        parent, length, qnode = orig(requests)
        return parent, [x + 1 for x in length], qnode  # off by one token per node

    monkeypatch.setattr(F, "prefix_tree_from_tokens", wrong)
    monkeypatch.setattr(oracle, "prefix_tree_from_tokens", wrong)
    with pytest.raises(AssertionError):
        test_tokens_fig4_reading()
