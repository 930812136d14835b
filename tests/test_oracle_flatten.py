"""Pins for the prefix-tree flattening oracle and the saving rate (CPU only).

* Brute force: the DP optimum equals the best grouping over all set
  partitions of the requests on random trees of up to 8 requests.
* Printed values: Fig. 4's two savings (4 and 8 tokens) and §6.3.1's saving
  rates (85.2 %, 92.6 %) of the BatchLLM summary page (tests/golden).
* Closed form: the two-level 4 x 16 x 16 workload saves 64 * 3072 * 15
  tokens when every sub-prefix forms its own group.
* Flattening keeps every query's token sequence.
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
