"""Host-side tests of the C ABI (CPU only; no kernel is launched).

* the library loads and exports every function include/*.h declares;
* the plan covers every (query, q head, context token) exactly once and its
  partial-slot bookkeeping is consistent;
* every validation error is reachable and reported with its status;
* plan statistics equal the workload bookkeeping;
* the C++ prefix-tree flattening reaches the oracle's (brute-force pinned)
  optimum and keeps every query's token sequence.
"""

import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import prefix_shared_decode_amd as P
from workloads import algorithmic_cost, build_single_level, build_two_level, make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in ("psa.h", "psa_debug.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(psa_[a-z_]+)\s*\(", text):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    declared = _declared_functions()
    assert {"psa_build_plan", "psa_decode_attention", "psa_merge"} <= declared
    out = subprocess.run(["nm", "-D", "--defined-only", P.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    assert declared <= exported, declared - exported
    L = P.lib()
    for name in declared:
        assert hasattr(L, name)
    assert set(P.EXPORTS) == declared
    assert L.psa_version() == 1


def _cfg(wl, **kw):
    return P.make_config(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages, wl.dtype, **kw)


def _coverage(wl, plan):
    """Expand the work list to (query, kv head) -> list of (segment, tok_begin, tok_end, slot j)."""
    b = wl.batch
    r = wl.num_q_heads // wl.num_kv_heads
    n_gpages = len(b["group_pages"])
    _, slot_off = plan.queries()
    cov = {}
    members = {}
    for i, g in enumerate(b["query_group"]):
        if g >= 0:
            members.setdefault(int(g), []).append(i)
    member_list = [int(x) for x in plan.members()]  # the plan's member array
    # it lists each group's members in query order, every group with members once, contiguously
    assert sorted(member_list) == sorted(i for g in members for i in members[g])
    first_row = {}
    for mi, qi in enumerate(member_list):
        g = int(b["query_group"][qi])
        first_row.setdefault(g, mi)
    for g, qs in members.items():
        assert member_list[first_row[g]: first_row[g] + len(qs)] == qs
    lim = b.get("query_prefix_len")
    items = plan.items()
    assert len(items) % 4 == 0
    for u in range(len(items) // 4):
        unit = items[4 * u: 4 * u + 4]
        if unit[0][0] & 0xFF == 2:
            assert all(x[0] == 0 for x in unit[1:]), "an MFMA tile fills its unit"
    for kind_full, kvh, ident, tb, te, pbase, a, bb in items:
        kind = kind_full & 0xFF
        if kind == 1:
            seg = "p" if pbase < n_gpages else "d"
            if seg == "p":
                g = int(b["query_group"][ident])
                assert pbase == b["group_page_off"][g] + tb // 16
            else:
                assert pbase == n_gpages + b["query_page_off"][ident] + tb // 16
            j = bb // wl.num_kv_heads - slot_off[ident] if bb >= 0 else 0
            if bb >= 0:
                assert bb % wl.num_kv_heads == kvh
            cov.setdefault((ident, kvh), []).append((seg, tb, te, j, a))
        elif kind == 2:
            assert a % r == 0 and bb % r == 0 and 0 < bb <= 128
            assert pbase == b["group_page_off"][ident] + tb // 16
            # rows of other groups than `ident` (a shared-node tile) must hold
            # the same pages for these tokens
            own = b["group_pages"][b["group_page_off"][ident] + tb // 16: b["group_page_off"][ident] + (te + 15) // 16]
            for mi in range(a // r, (a + bb) // r):
                qi = member_list[mi]
                vis = int(lim[qi]) if lim is not None else None
                if vis is not None and vis <= tb:
                    continue  # this row's prefix limit ends before the tile: no piece
                g2 = int(b["query_group"][qi])
                if g2 != ident:
                    assert te <= b["group_prefix_len"][g2]
                    other = b["group_pages"][b["group_page_off"][g2] + tb // 16: b["group_page_off"][g2] + (te + 15) // 16]
                    assert list(other) == list(own), (ident, g2, tb, te)
                cov.setdefault((qi, kvh), []).append(("p", tb, te if vis is None else min(te, vis),
                                                      kind_full >> 8, None))
        elif kind == 3:
            for kvh2 in range(wl.num_kv_heads):
                cov.setdefault((ident, kvh2), []).append(("e", 0, 0, 0, None))
        else:
            assert kind == 0
    return cov


def _check_coverage(wl, plan, prefix=True, distinct=True):
    b = wl.batch
    cov = _coverage(wl, plan)
    expected, slot_off = plan.queries()
    for i in range(wl.num_queries):
        g = int(b["query_group"][i])
        lp = int(b["group_prefix_len"][g]) if g >= 0 else 0
        if g >= 0 and b.get("query_prefix_len") is not None:
            lp = int(b["query_prefix_len"][i])
        ld = int(b["query_distinct_len"][i])
        for kvh in range(wl.num_kv_heads):
            parts = cov.get((i, kvh), [])
            want_p = set(range(lp)) if prefix else set()
            want_d = set(range(ld)) if distinct else set()
            got_p, got_d = [], []
            for seg, tb, te, _, _ in parts:
                assert tb % 16 == 0
                (got_p if seg == "p" else got_d if seg == "d" else []).extend(range(tb, te))
            assert sorted(got_p) == sorted(want_p)
            assert sorted(got_d) == sorted(want_d)
            real = [x for x in parts if x[0] != "e"]
            assert expected[i] == len(real)
            if not real:
                assert any(x[0] == "e" for x in parts)
            assert sorted(x[3] for x in real) == list(range(len(real)))
            assert all(x[4] is None or x[4] == expected[i] for x in real)
            # prefix partials come first
            assert all(x[3] < sum(1 for y in real if y[0] == "p") for x in real if x[0] == "p")
            assert (slot_off[i] >= 0) == (expected[i] >= 2)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_plan_covers_every_token_once(seed, dtype):
    rng = np.random.default_rng(seed)
    hkv = int(rng.choice([1, 2, 4]))
    r = int(rng.choice([1, 2, 4, 8]))
    groups = [(int(rng.integers(0, 200)), int(rng.integers(1, 40)), (0, int(rng.integers(1, 300)))) for _ in range(3)]
    wl = build_single_level("t", hkv * r, hkv, 64, dtype, groups, (4, (1, 700)), seed=seed)
    # make sure no query has an empty context
    for i in range(wl.num_queries):
        g = wl.batch["query_group"][i]
        if (wl.batch["group_prefix_len"][g] if g >= 0 else 0) + wl.batch["query_distinct_len"][i] == 0:
            pytest.skip("drew an empty context")
    for kw in ({}, {"prefix_chunk_tokens": 48, "distinct_chunk_tokens": 32, "mfma_tile_rows": 32},
               {"flags": P.FORCE_MATVEC}, {"flags": P.NO_XCD_ORDER, "mfma_min_rows": 1}):
        plan = P.psa_build_plan(_cfg(wl), wl.batch, **kw)
        _check_coverage(wl, plan)
    plan = P.psa_build_plan(_cfg(wl), wl.batch, flags=P.PREFIX_ONLY)
    _check_coverage(wl, plan, distinct=False)
    plan = P.psa_build_plan(_cfg(wl), wl.batch, flags=P.DISTINCT_ONLY)
    _check_coverage(wl, plan, prefix=False)


def test_mfma_tiles_only_for_bf16_groups_with_enough_rows():
    wl = build_single_level("t", 4, 2, 128, "bf16", [(64, 3, (1, 5)), (64, 5, (1, 5))], [], seed=1)
    plan = P.psa_build_plan(_cfg(wl), wl.batch)  # rows 6 and 10 < 16
    assert plan.info()["num_prefix_items"] == 0
    plan = P.psa_build_plan(_cfg(wl), wl.batch, mfma_min_rows=8)
    it = plan.items()
    assert set(it[(it[:, 0] & 0xFF) == 2][:, 2]) == {1}
    wl32 = build_single_level("t", 4, 2, 128, "f32", [(64, 30, (1, 5))], [], seed=1)
    assert P.psa_build_plan(_cfg(wl32), wl32.batch).info()["num_prefix_items"] == 0


def test_xcd_order_keeps_prefix_sets_on_one_xcd():
    wl = make_workload("llama3_8b_8x100")
    plan = P.psa_build_plan(_cfg(wl), wl.batch)
    it = plan.items()
    pos = {}
    for idx in range(0, len(it), 4):
        row = it[idx]
        if row[0] & 0xFF == 2:
            pos.setdefault((row[2], row[1], row[0] >> 8), []).append(idx // 4)
    # 8 groups x 8 kv heads x 1 prefix chunk, each set = 4 row tiles
    assert len(pos) == 64 and all(len(v) == 4 for v in pos.values())
    for v in pos.values():
        assert len({x % 8 for x in v}) == 1
    # longest first (without tile pairs): all MFMA units come before the mat-vec units
    kinds = P.psa_build_plan(_cfg(wl), wl.batch, flags=P.NO_TILE_PAIRS).items()[::4, 0] & 0xFF
    assert kinds[:256].tolist() == [2] * 256 and set(kinds[256:].tolist()) == {1}
    # a smaller explicit chunk splits each set's prefix
    it = P.psa_build_plan(_cfg(wl), wl.batch, prefix_chunk_tokens=1024).items()
    assert ((it[::4, 0] & 0xFF) == 2).sum() == 512


@pytest.mark.parametrize("name", ["tiny_fp32_1x4", "llama3_8b_8x100", "longchat13b_1x256", "no_sharing_512"])
def test_plan_statistics_match_bookkeeping(name):
    wl = make_workload(name)
    plan = P.psa_build_plan(_cfg(wl), wl.batch)
    info = plan.info()
    cost = algorithmic_cost(wl)
    assert info["algorithmic_bytes"] == cost["bytes"]
    assert info["algorithmic_flops"] == cost["flops"]
    assert info["prefix_flops"] == cost["flops_prefix"]
    assert info["logical_tokens"] == cost["logical_tokens"]
    assert info["processed_tokens"] == cost["processed_tokens"]
    assert info["saved_tokens"] == cost["logical_tokens"] - cost["processed_tokens"]


def _tiny():
    return build_single_level("t", 4, 2, 64, "bf16", [(40, 2, (1, 9))], [5], seed=0)


def _status(fn):
    with pytest.raises(P.PsaError) as e:
        fn()
    return e.value.status_name


def test_error_paths():
    wl = _tiny()
    b = wl.batch
    c = _cfg(wl)
    mk = lambda cfg=c, batch=b, **kw: P.psa_build_plan(cfg, batch, **kw)  # noqa: E731
    cfg = lambda **kw: P.make_config(**{**dict(num_q_heads=4, num_kv_heads=2, head_dim=64,  # noqa: E731
                                               num_pages=wl.num_pages, kv_dtype="bf16"), **kw})
    assert _status(lambda: mk(cfg(num_q_heads=5))) == "PSA_ERR_INVALID_ARGUMENT"
    assert _status(lambda: mk(cfg(num_q_heads=32, num_kv_heads=2))) == "PSA_ERR_UNSUPPORTED"  # r = 16
    assert _status(lambda: mk(cfg(head_dim=96))) == "PSA_ERR_UNSUPPORTED"
    assert _status(lambda: mk(cfg(page_size=32))) == "PSA_ERR_UNSUPPORTED"
    assert _status(lambda: mk(cfg(num_pages=0))) == "PSA_ERR_INVALID_ARGUMENT"
    bad = dict(b, query_pages=np.where(np.arange(len(b["query_pages"])) == 0, wl.num_pages, b["query_pages"]))
    assert _status(lambda: mk(batch=bad)) == "PSA_ERR_OUT_OF_RANGE"
    bad = dict(b, query_distinct_len=b["query_distinct_len"] + 16)
    assert _status(lambda: mk(batch=bad)) == "PSA_ERR_OUT_OF_RANGE"
    bad = dict(b, query_distinct_len=-b["query_distinct_len"])
    assert _status(lambda: mk(batch=bad)) == "PSA_ERR_INVALID_ARGUMENT"
    bad = dict(b, query_page_off=b["query_page_off"][::-1].copy())
    assert _status(lambda: mk(batch=bad)) == "PSA_ERR_INVALID_ARGUMENT"
    bad = dict(b, query_group=np.full_like(b["query_group"], 7))
    assert _status(lambda: mk(batch=bad)) == "PSA_ERR_INVALID_ARGUMENT"
    # empty context: an ungrouped query with no distinct tokens
    bad = dict(b, query_distinct_len=np.where(b["query_group"] < 0, 0, b["query_distinct_len"]).astype(np.int32))
    assert _status(lambda: mk(batch=bad)) == "PSA_ERR_INVALID_ARGUMENT"
    P.psa_build_plan(c, bad, flags=P.PREFIX_ONLY)  # allowed when only the prefix is covered
    assert _status(lambda: mk(flags=P.PREFIX_ONLY | P.DISTINCT_ONLY)) == "PSA_ERR_INVALID_ARGUMENT"
    assert _status(lambda: mk(prefix_chunk_tokens=20)) == "PSA_ERR_INVALID_ARGUMENT"
    assert _status(lambda: mk(mfma_tile_rows=256)) == "PSA_ERR_INVALID_ARGUMENT"
    assert _status(lambda: mk(prefix_chunk_tokens=4096)) == "PSA_ERR_INVALID_ARGUMENT"
    assert _status(lambda: mk(distinct_chunk_tokens=2048)) == "PSA_ERR_INVALID_ARGUMENT"
    assert _status(lambda: mk(flags=0x400)) == "PSA_ERR_INVALID_ARGUMENT"
    # messages name the problem
    with pytest.raises(P.PsaError, match="page id"):
        mk(batch=dict(b, group_pages=np.full_like(b["group_pages"], -3)))


def test_decode_rejects_host_pointers_and_small_workspace_without_launching():
    """Calls that must fail before any kernel: they touch only host-side checks."""
    import ctypes as C

    L = P.lib()
    wl = _tiny()
    plan = P.psa_build_plan(_cfg(wl), wl.batch)
    ws_bytes = plan.info()["workspace_bytes"]
    host = (C.c_uint8 * 4096)()
    st = L.psa_decode_attention(plan.handle, C.addressof(host), C.addressof(host), C.addressof(host),
                                C.addressof(host), None, None, C.addressof(host), ws_bytes - 1, None)
    assert P._lib.STATUS[st] == "PSA_ERR_WORKSPACE_TOO_SMALL"
    st = L.psa_plan_upload(plan.handle, C.addressof(host), plan.info()["image_bytes"] - 1, None)
    assert P._lib.STATUS[st] == "PSA_ERR_WORKSPACE_TOO_SMALL"
    st = L.psa_decode_attention(plan.handle, C.addressof(host), C.addressof(host), C.addressof(host),
                                C.addressof(host), None, None, C.addressof(host), ws_bytes, None)
    assert P._lib.STATUS[st] == "PSA_ERR_INVALID_ARGUMENT"  # workspace never uploaded
    st = L.psa_merge(4, 96, *([None] * 9), None)
    assert P._lib.STATUS[st] == "PSA_ERR_UNSUPPORTED"
    st = L.psa_merge(4, 64, *([None] * 9), None)
    assert P._lib.STATUS[st] == "PSA_ERR_INVALID_ARGUMENT"
    assert L.psa_merge(0, 64, *([None] * 9), None) == 0


def test_empty_batch_plans_no_work():
    wl = build_single_level("t", 2, 1, 64, "bf16", [], [], seed=0)
    plan = P.psa_build_plan(_cfg(wl), wl.batch)
    assert plan.info()["num_items"] == 0


# ---------------- flattening ----------------

def _random_tree(seed, page=16):
    rng = np.random.default_rng(seed)
    m = int(rng.integers(1, 7))
    parent = [-1] + [int(rng.integers(-1, d)) for d in range(1, m)]
    lens = [page * int(x) for x in rng.integers(1, 6, size=m)]
    n = int(rng.integers(1, 9))
    qn = [int(x) for x in rng.integers(-1, m, size=n)]
    dl = [int(x) for x in rng.integers(0, 40, size=n)]
    perm = rng.permutation(10_000)
    pos = 0
    node_pages, noff = [], [0]
    for ln in lens:
        node_pages += [int(x) for x in perm[pos:pos + ln // page]]
        pos += ln // page
        noff.append(len(node_pages))
    qpages, qoff = [], [0]
    for x in dl:
        k = -(-x // page)
        qpages += [int(y) for y in perm[pos:pos + k]]
        pos += k
        qoff.append(len(qpages))
    return {"page_size": page, "node_parent": parent, "node_len": lens, "node_page_off": noff,
            "node_pages": node_pages, "query_node": qn, "query_distinct_len": dl, "query_page_off": qoff,
            "query_pages": qpages}


def _tree_context(t, i):
    nodes = []
    x = int(t["query_node"][i])
    while x >= 0:
        nodes.append(x)
        x = int(t["node_parent"][x])
    pages = [p for d in reversed(nodes) for p in t["node_pages"][t["node_page_off"][d]:t["node_page_off"][d + 1]]]
    pages += list(t["query_pages"][t["query_page_off"][i]:t["query_page_off"][i + 1]])
    return pages, sum(int(t["node_len"][d]) for d in nodes) + int(t["query_distinct_len"][i])


@pytest.mark.parametrize("seed", range(40))
def test_flatten_matches_oracle_optimum(seed):
    t = _random_tree(seed)
    batch, saved = P.psa_flatten_prefix_tree(t)
    best, _ = oracle.maximize_reuse(t["node_parent"], t["node_len"], t["query_node"])
    assert saved == best
    # the returned groups realise that saving and keep every query's tokens
    qg = batch["query_group"]
    got = sum(int(batch["group_prefix_len"][g]) * (int((qg == g).sum()) - 1) for g in range(len(batch["group_prefix_len"])))
    assert got == best
    assert all((qg == g).sum() >= 2 for g in range(len(batch["group_prefix_len"])))
    for i in range(len(t["query_node"])):
        pages, n = _tree_context(t, i)
        segs = oracle.query_context(batch, i)
        flat = []
        total = 0
        for p, ln in segs:
            assert ln % 16 == 0 or (p is segs[-1][0])
            flat += list(p[: -(-ln // 16)])
            total += ln
        assert total == n
        assert flat == pages[: -(-n // 16)]


@pytest.mark.parametrize("seed", range(30))
def test_flatten_matches_brute_force_directly(seed):
    """The C++ flattening's saving equals the best over every set partition
    of the queries (a block saves its deepest common node's path length times
    its size minus one), computed by brute force, not through the oracle's
    dynamic program."""
    from test_oracle_flatten import brute_force

    t = _random_tree(1000 + seed)
    _, saved = P.psa_flatten_prefix_tree(t)
    assert saved == brute_force(t["node_parent"], t["node_len"], t["query_node"])


@pytest.mark.parametrize("seed", range(30))
def test_identification_matches_brute_force_directly(seed):
    """psa_identify_prefix_groups on small random token sets (duplicates and
    prompts that are prefixes of others included) saves exactly the best over
    every set partition, each block saving its longest common prefix times its
    size minus one (brute force, not the oracle's trie and DP)."""
    from test_oracle_flatten import brute_force_tokens

    rng = np.random.default_rng(2000 + seed)
    n = int(rng.integers(1, 8))
    seqs = [[int(x) for x in rng.integers(0, int(rng.integers(1, 4)), size=int(rng.integers(0, 7)))] for _ in range(n)]
    if n >= 3 and rng.random() < 0.4:
        seqs[1] = list(seqs[0])
        seqs[2] = list(seqs[0][: len(seqs[0]) // 2])
    res = P.psa_identify_prefix_groups(seqs)
    assert res["saved_tokens"] == brute_force_tokens(seqs)


def test_flatten_two_level_workload_closed_form():
    wl = build_two_level("t", 32, 8, 128, "bf16", 4, 1024, 16, 2048, 16, (32, 256))
    batch, saved = P.psa_flatten_prefix_tree(wl.tree)
    assert saved == 64 * 3072 * 15
    assert len(batch["group_prefix_len"]) == 64 and set(batch["group_prefix_len"]) == {3072}
    cfg = P.make_config(32, 8, 128, wl.num_pages, "bf16")
    info = P.psa_build_plan(cfg, batch).info()
    assert info["saved_tokens"] == saved


def test_flatten_two_level_workload_keeps_every_context():
    """The library's flattening of the full two-level workload (the batch the
    kernel runs at full size) keeps each query's tokens: group prefix pages ++
    own pages name the tree's root-to-query pages in order, with the same
    token count."""
    from workloads import make_workload

    wl = make_workload("two_level_4x16x16")
    t = wl.tree
    batch, _ = P.psa_flatten_prefix_tree(t)
    for i in range(len(t["query_node"])):
        pages, n = _tree_context(t, i)
        flat, total = [], 0
        for p, ln in oracle.query_context(batch, i):
            flat += [int(x) for x in p[: -(-ln // 16)]]
            total += ln
        assert total == n
        assert flat == [int(x) for x in pages[: -(-n // 16)]]


def test_unique_kv_bytes_count_shared_pages_once():
    """plan_info.unique_kv_bytes: KV over distinct (page, slot) places.  On the
    flattened two-level workload the 4 root prefixes (1024 tokens) count once,
    not once per sub-group: 4 * 1024 + 64 * 2048 tokens plus every distinct
    part; with no shared pages (8x100) it equals prefix + distinct KV bytes;
    a page two segments share counts the slots of the longer one."""
    from workloads import make_workload

    wl = make_workload("two_level_4x16x16")
    batch, _ = P.psa_flatten_prefix_tree(wl.tree)
    info = P.psa_build_plan(P.make_config(32, 8, 128, wl.num_pages, "bf16"), batch).info()
    tok = 4 * 1024 + 64 * 2048 + int(np.sum(batch["query_distinct_len"]))
    assert info["unique_kv_bytes"] == tok * 8 * 128 * 2 * 2
    assert info["prefix_kv_bytes"] == 64 * 3072 * 8 * 128 * 2 * 2
    wl = make_workload("llama3_8b_8x100")
    info = P.psa_build_plan(P.make_config(32, 8, 128, wl.num_pages, "bf16"), wl.batch).info()
    assert info["unique_kv_bytes"] == info["prefix_kv_bytes"] + info["distinct_kv_bytes"]
    # two groups naming the same two pages, with 20 and 30 tokens: 30 tokens once; a query of 5 tokens
    batch = {"page_size": 16, "group_prefix_len": [20, 30], "group_page_off": [0, 2, 4], "group_pages": [3, 4, 3, 4],
             "query_group": [0, 0, 1, 1, -1], "query_distinct_len": [0, 0, 0, 0, 5],
             "query_page_off": [0, 0, 0, 0, 0, 1], "query_pages": [7]}
    info = P.psa_build_plan(P.make_config(4, 2, 64, 8, "bf16"), batch).info()
    assert info["unique_kv_bytes"] == (30 + 5) * 2 * 64 * 2 * 2


def test_flatten_error_paths():
    t = _random_tree(3)
    assert _status(lambda: P.psa_flatten_prefix_tree(dict(t, node_len=[x + 1 for x in t["node_len"]]))) == \
        "PSA_ERR_INVALID_ARGUMENT"
    bad = dict(t, node_parent=[len(t["node_parent"])] + list(t["node_parent"][1:]))
    assert _status(lambda: P.psa_flatten_prefix_tree(bad)) == "PSA_ERR_INVALID_ARGUMENT"
    if len(t["node_parent"]) >= 2:
        cyc = dict(t, node_parent=[1, 0] + list(t["node_parent"][2:]))
        assert _status(lambda: P.psa_flatten_prefix_tree(cyc)) == "PSA_ERR_INVALID_ARGUMENT"
    assert _status(lambda: P.psa_flatten_prefix_tree(t, page_size=8)) == "PSA_ERR_UNSUPPORTED"


def test_mfma_tiles_start_two_to_a_cu():
    """On the 8x100 shape, each XCD queue (units i with i % 8 == x) holds its
    32 MFMA tiles at local positions [0, 16) and [32, 48): positions k and
    k + 32 start on the same CU.  Without pairing they lead the queue.  Both
    orders cover every (query, kv head) exactly."""
    from workloads import make_workload

    wl = make_workload("llama3_8b_8x100")
    for flags, want in ((0, list(range(16)) + list(range(32, 48))), (P.NO_TILE_PAIRS, list(range(32)))):
        plan = P.psa_build_plan(_cfg(wl), wl.batch, flags=flags)
        items = plan.items()
        kinds = items[::4, 0] & 0xFF
        for x in range(8):
            local = kinds[x::8]
            assert list(np.nonzero(local == 2)[0]) == want, (flags, x)
        _check_coverage(wl, plan)


def test_mfma_tiles_beyond_a_round_of_pairs():
    """More than two MFMA tiles per CU in an XCD queue.  Tiles that share
    their prefix chunk with other row tiles (the prefill chunks of the mixed
    preset: compute bound, read from L2) are spread evenly over the first
    three quarters of each queue, interleaved with the mat-vec units; tiles
    that are their chunk's only row tile (the flattened two-level shape
    without shared pages: each streams its own pages) lead the queue, longest
    first.  NO_TILE_PAIRS keeps every tile first.  Every order covers every
    (query, kv head) exactly."""
    from workloads import make_workload

    wl = make_workload("mixed_7prefill_256decode")
    plan = P.psa_build_plan(_cfg(wl), wl.batch)
    kinds = plan.items()[::4, 0] & 0xFF
    for x in range(8):
        local = kinds[x::8]
        pos = np.nonzero(local == 2)[0]
        n, npx = len(local), len(pos)
        span = int(0.75 * n)
        assert npx > 64 and pos[0] == 0 and pos[-1] < span
        # tile k sits where k / npx of the span is reached: never two in a row
        # for long, never far from its even place
        want = np.ceil(np.arange(npx) * span / npx)
        assert np.abs(pos - want).max() <= 1, x
    _check_coverage(wl, plan)

    wl = make_workload("two_level_4x16x16")
    batch, _ = P.psa_flatten_prefix_tree(wl.tree)

    class W:  # the flattened batch with the workload's shape
        pass

    fw = W()
    fw.__dict__.update(wl.__dict__)
    fw.batch = batch
    fw.num_queries = len(batch["query_group"])
    for flags in (P.NO_PAGE_SHARING, P.NO_TILE_PAIRS | P.NO_PAGE_SHARING):
        plan = P.psa_build_plan(_cfg(wl), batch, flags=flags)
        kinds = plan.items()[::4, 0] & 0xFF
        for x in range(8):
            assert list(np.nonzero(kinds[x::8] == 2)[0]) == list(range(128)), (flags, x)
        _check_coverage(fw, plan)


def test_tile_pairs_leave_mat_vec_room_at_the_start():
    """Pairs are kept while they leave at least 4 of an XCD's 32 CUs to the
    mat-vec units when the launch starts: 14 groups of the 8x100 shape (56
    tiles an XCD, 28 CUs of pairs) keep pairs at [0, 28) and [32, 60); 15
    groups (60 tiles, 2 CUs left) are spread like the compute-bound tiles
    of the mixed preset."""
    from workloads import make_workload

    for g, paired in ((14, True), (15, False)):
        wl = make_workload(f"llama3_8b_{g}x100")
        plan = P.psa_build_plan(_cfg(wl), wl.batch)
        kinds = plan.items()[::4, 0] & 0xFF
        for x in range(8):
            pos = np.nonzero(kinds[x::8] == 2)[0]
            assert len(pos) == 4 * g, (g, x)
            if paired:
                assert list(pos) == list(range(28)) + list(range(32, 60)), x
            else:
                span = int(0.75 * len(kinds[x::8]))
                want = np.ceil(np.arange(len(pos)) * span / len(pos))
                assert np.abs(pos - want).max() <= 1, x
        _check_coverage(wl, plan)


def _flat(wl):
    batch, _ = P.psa_flatten_prefix_tree(wl.tree)

    class W:  # the flattened batch with the workload's shape
        pass

    fw = W()
    fw.__dict__.update(wl.__dict__)
    fw.batch = batch
    fw.num_queries = len(batch["query_group"])
    return fw


def test_family_tiles_cover_a_shared_root_once():
    """Flattened 4x16x16: the 16 groups of a root begin with the root's 64
    pages, so its 1024 tokens are tiled once over all 256 members (8 tiles of
    128 rows per kv head), and each group keeps one 2048-token chunk of its
    own: 4*8*8 + 64*8 = 768 MFMA tiles, 3 pieces per query as before."""
    from workloads import make_workload

    fw = _flat(make_workload("two_level_4x16x16"))
    b = fw.batch
    plan = P.psa_build_plan(_cfg(fw), b)
    it = plan.items()
    mf = it[(it[:, 0] & 0xFF) == 2]
    assert len(mf) == 768 and plan.info()["num_prefix_items"] == 768
    fam = mf[mf[:, 4] == 1024]
    assert len(fam) == 256 and (fam[:, 3] == 0).all() and (fam[:, 7] == 128).all()
    assert ((fam[:, 0] >> 8) == 0).all()
    own = mf[mf[:, 3] == 1024]
    assert len(own) == 512 and (own[:, 4] == 3072).all() and ((own[:, 0] >> 8) == 1).all()
    expected, _ = plan.queries()
    assert (expected == 3).all()
    _check_coverage(fw, plan)
    plain = P.psa_build_plan(_cfg(fw), b, flags=P.NO_PAGE_SHARING)
    assert plain.info()["num_prefix_items"] == 1024
    _check_coverage(fw, plain)


@pytest.mark.parametrize("seed", range(3))
def test_shared_nodes_do_not_need_consecutive_group_numbers(seed):
    """The flattened 4x16x16 batch with its 64 groups renumbered at random (a
    root's 16 groups scattered over the numbering): the plan still tiles each
    root's 1024 tokens once over all of its members (the same 768 MFMA tiles,
    3 pieces per query), and covers every token once."""
    from workloads import make_workload, permute_groups

    fw = _flat(make_workload("two_level_4x16x16"))
    perm = np.random.default_rng(seed).permutation(len(fw.batch["group_prefix_len"]))
    fw.batch = permute_groups(fw.batch, perm)
    plan = P.psa_build_plan(_cfg(fw), fw.batch)
    it = plan.items()
    mf = it[(it[:, 0] & 0xFF) == 2]
    assert len(mf) == 768
    assert len(mf[mf[:, 4] == 1024]) == 256 and (mf[mf[:, 4] == 1024][:, 7] == 128).all()
    expected, _ = plan.queries()
    assert (expected == 3).all()
    _check_coverage(fw, plan)


@pytest.mark.parametrize("r", [1, 4])
def test_nested_shared_nodes_three_levels(r):
    """A three-level tree (2 roots of 512 tokens, 2 children of 256 each, 2
    leaves of 128 each, 8 requests per leaf) flattens to 8 leaf groups of 896
    tokens.  The plan covers each root's 512 tokens once over its 4 groups,
    each middle node's 256 tokens once over its 2 groups, and each group's
    own 128 tokens (MFMA tiles at r 4, mat-vec at r 1, below 16 rows): at r
    4 per kv head 2 + 4 + 8 tiles, and 3 prefix pieces per query.  Without page sharing, 8 tiles per
    kv head over 896 tokens."""
    from workloads import build_tree

    wl = build_tree("t3", 4 * r, 4, 64, "bf16", [(2, 512), (2, 256), (2, 128)], 8, (1, 40), seed=3)
    fw = _flat(wl)
    assert set(fw.batch["group_prefix_len"].tolist()) == {896}
    plan = P.psa_build_plan(_cfg(fw), fw.batch)
    it = plan.items()
    mf = it[((it[:, 0] & 0xFF) == 2) & (it[:, 1] == 0)]
    spans = sorted(set((int(a), int(b)) for a, b in mf[:, 3:5]))
    own_mfma = 8 * r >= 16  # a group's own rows (at r 1 its own tokens go to mat-vec tiles)
    assert spans == [(0, 512), (512, 768)] + ([(768, 896)] if own_mfma else [])
    rows = {sp: int(mf[(mf[:, 3] == sp[0]) & (mf[:, 4] == sp[1])][:, 7].sum()) for sp in spans}
    assert rows == {sp: 64 * r for sp in spans}
    if r == 4:
        assert len(mf) == 2 + 4 + 8
    expected, _ = plan.queries()
    dl = np.asarray(fw.batch["query_distinct_len"])
    assert (expected == 3 + (dl > 0)).all()
    _check_coverage(fw, plan)
    plain = P.psa_build_plan(_cfg(fw), fw.batch, flags=P.NO_PAGE_SHARING)
    pm = plain.items()
    pm = pm[((pm[:, 0] & 0xFF) == 2) & (pm[:, 1] == 0)]
    assert sorted(set((int(a), int(b)) for a, b in pm[:, 3:5])) == ([(0, 896)] if own_mfma else [])
    _check_coverage(fw, plain)


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("r", [1, 4, 8])
def test_family_tiles_edge_shapes(seed, r):
    """Family tiles next to empty and mat-vec own parts, several chunks of the
    shared part, small tiles, and the PREFIX_ONLY / DISTINCT_ONLY plans: every
    token is covered once and the partial counts match."""
    from workloads import build_family_case

    wl = build_family_case(seed, r=r)
    plan = P.psa_build_plan(_cfg(wl), wl.batch)
    it = plan.items()
    mf = it[(it[:, 0] & 0xFF) == 2]
    rows = (3 + 2 + 1 + 1) * r  # the family's members
    fam = mf[np.isin(mf[:, 2], [0, 1, 2, 3]) & (mf[:, 4] <= 64)]  # tiles may read any family group's pages
    if rows >= 16:
        assert len(fam) > 0 and fam[fam[:, 1] == 0][:, 7].sum() == rows
    for kw in ({}, {"prefix_chunk_tokens": 32}, {"prefix_chunk_tokens": 48, "mfma_tile_rows": 16},
               {"flags": P.PREFIX_ONLY}, {"flags": P.DISTINCT_ONLY}, {"flags": P.NO_PAGE_SHARING},
               {"mfma_min_rows": 1}):
        plan = P.psa_build_plan(_cfg(wl), wl.batch, **kw)
        fl = kw.get("flags", 0)
        _check_coverage(wl, plan, prefix=not fl & P.DISTINCT_ONLY, distinct=not fl & P.PREFIX_ONLY)


def test_peak_entry_points_reject_bad_arguments():
    """Argument checks of psa_debug_read_peak / psa_debug_mfma_peak / psa_debug_issue_probe come before
    any device access (no GPU needed): NULL pointers, sizes out of range, and
    too-small sinks are errors with a message."""
    import ctypes as C

    L = P.lib()
    fake = C.c_void_p(0x1000)
    cases = [
        (L.psa_debug_read_peak, (None, 1 << 20, fake, 2048 * 256, None), "NULL"),
        (L.psa_debug_read_peak, (fake, 1000, fake, 2048 * 256, None), "multiple of 16"),
        (L.psa_debug_read_peak, (fake, 3 << 30, fake, 2048 * 256, None), "multiple of 16"),
        (L.psa_debug_read_peak, (fake, 1 << 20, fake, 100, None), "sink needs"),
        (L.psa_debug_mfma_peak, (None, 2048 * 256, 64, None), "NULL"),
        (L.psa_debug_mfma_peak, (fake, 2048 * 256, 12, None), "multiple of 8"),
        (L.psa_debug_mfma_peak, (fake, 10, 64, None), "out needs"),
        (L.psa_debug_issue_probe, (0, None, 1024, 16, None), "NULL"),
        (L.psa_debug_issue_probe, (8, fake, 1024, 16, None), "pattern"),
        (L.psa_debug_issue_probe, (0, fake, 1024, 0, None), "iters"),
        (L.psa_debug_issue_probe, (0, fake, 1000, 16, None), "cycles needs"),
    ]
    for fn, args, msg in cases:
        assert fn(*args) != 0
        assert msg in L.psa_last_error().decode()



@pytest.mark.parametrize("seed", range(4))
def test_prefill_chunks_with_decode_cover_causal_contexts(seed):
    """Prefill chunks batched with decode queries: every chunk token's
    prefix pieces cover exactly its causal context [0, cached + t + 1), MFMA
    tiles stop at their rows' last key, and the mat-vec path clips its items
    to each query's limit."""
    from workloads import build_mixed

    rng = np.random.default_rng(seed)
    prefill = [(int(rng.integers(0, 5)) * 16, int(rng.integers(1, 90))) for _ in range(3)]
    wl = build_mixed("m", 8, 2, 64, "bf16", [(int(rng.integers(1, 300)), 9, (0, 50))], prefill, seed=seed)
    b = wl.batch
    for kw in ({}, {"prefix_chunk_tokens": 32, "mfma_tile_rows": 16}, {"flags": P.FORCE_MATVEC},
               {"flags": P.PREFIX_ONLY}, {"mfma_min_rows": 1}):
        plan = P.psa_build_plan(_cfg(wl), b, **kw)
        _check_coverage(wl, plan, distinct=not kw.get("flags", 0) & P.PREFIX_ONLY)
        it = plan.items()
        for row in it[(it[:, 0] & 0xFF) == 2]:
            assert row[4] <= b["group_prefix_len"][row[2]]
    bad = dict(b, query_prefix_len=b["query_prefix_len"] + 1)  # past the group prefix
    with pytest.raises(P.PsaError):
        P.psa_build_plan(_cfg(wl), bad)
