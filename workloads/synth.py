"""Synthetic workloads for prefix-shared decode attention.

Shapes follow the workloads the pages discuss (BatchLLM §6 micro-benchmarks
and industrial summary task; the Feather explainer's 8 groups x 100
requests and its no-sharing control); the values are seeded i.i.d. N(0, 1),
so no dataset item is involved.

Recipe (fixed draw order): lengths -> page permutation (numpy PCG64 seeded
with ``seed``) -> Q -> K pool -> V pool (torch generator on the target
device seeded with ``seed``).  bf16 inputs are N(0, 1) float32 draws rounded
to bf16 (round-to-nearest-even, torch's cast); fp32 inputs are float64
draws rounded to float32.  "Uniform a-b" lengths are i.i.d. integers with
both ends included.  Page ids are a random permutation of the pool, so block
tables are non-contiguous.  Every pool slot, including the unused tail of a
segment's last page, holds a draw (stale but finite values).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import re

import numpy as np

PAGE = 16


@dataclass
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str  # "bf16" or "f32"
    num_pages: int
    batch: dict  # single-level page tables (see oracle.attention.query_context)
    tree: dict | None = None  # two-level input, if the workload has one
    seed: int = 0
    page_size: int = PAGE
    meta: dict = field(default_factory=dict)

    @property
    def num_queries(self) -> int:
        return len(self.batch["query_group"])


def _alloc(rng_perm, lengths, P):
    """Assign consecutive ids of a shuffled page list to each segment."""
    offs = [0]
    pages = []
    pos = 0
    for n in lengths:
        k = -(-int(n) // P)
        pages.extend(int(x) for x in rng_perm[pos:pos + k])
        pos += k
        offs.append(len(pages))
    return np.asarray(offs, dtype=np.int64), np.asarray(pages, dtype=np.int32), pos


def build_single_level(name, hq, hkv, d, dtype, groups, ungrouped_lens, seed=0,
                       spare_pages=0, P=PAGE, lens_fn=None):
    """Workload from explicit groups.

    ``groups``: list of (prefix_len, n_requests, (lo, hi)) or
    (prefix_len, [distinct lengths]); ``ungrouped_lens``: (count, (lo, hi)) or
    a list of lengths for queries with no shared prefix.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    # 1. lengths
    g_prefix, g_members = [], []
    for g in groups:
        if isinstance(g[1], (list, tuple, np.ndarray)) and len(g) == 2:
            lp, dl = g
            dl = [int(x) for x in dl]
        else:
            lp, n, (lo, hi) = g
            dl = [int(x) for x in rng.integers(lo, hi, size=n, endpoint=True)]
        g_prefix.append(int(lp))
        g_members.append(dl)
    if isinstance(ungrouped_lens, tuple) and len(ungrouped_lens) == 2 and isinstance(ungrouped_lens[1], tuple):
        cnt, (lo, hi) = ungrouped_lens
        u = [int(x) for x in rng.integers(lo, hi, size=cnt, endpoint=True)]
    else:
        u = [int(x) for x in ungrouped_lens]
    qgroup = [gi for gi, dl in enumerate(g_members) for _ in dl] + [-1] * len(u)
    dlen = [x for dl in g_members for x in dl] + u
    # 2. page permutation
    need = sum(-(-x // P) for x in g_prefix) + sum(-(-x // P) for x in dlen)
    num_pages = max(1, need + spare_pages)
    perm = rng.permutation(num_pages)
    goff, gpages, used = _alloc(perm, g_prefix, P)
    qoff, qpages, _ = _alloc(perm[used:], dlen, P)
    batch = {
        "page_size": P,
        "group_prefix_len": np.asarray(g_prefix, dtype=np.int32),
        "group_page_off": goff,
        "group_pages": gpages,
        "query_group": np.asarray(qgroup, dtype=np.int32),
        "query_distinct_len": np.asarray(dlen, dtype=np.int32),
        "query_page_off": qoff,
        "query_pages": qpages,
    }
    return Workload(name, hq, hkv, d, dtype, num_pages, batch, None, seed, P)


def share_leading_pages(wl, first, last, pages):
    """Make groups first+1..last begin with the first `pages` page ids of
    group `first` (in place): the shape a flattened tree gives the groups
    below one shared node.  Their own pages there become unused."""
    b = wl.batch
    off, gp = b["group_page_off"], b["group_pages"]
    for g in range(first + 1, last + 1):
        n = min(pages, int(off[g + 1] - off[g]), int(off[first + 1] - off[first]))
        gp[off[g]: off[g] + n] = gp[off[first]: off[first] + n]
    return wl


def build_mixed(name, hq, hkv, d, dtype, decode_groups, prefill, seed=0):
    """Decode queries and chunks of prefill tokens in one batch.

    ``decode_groups``: as in ``build_single_level``.  ``prefill``: list of
    (cached, chunk) token counts: a request whose first ``cached`` tokens are
    already in the KV cache and whose next ``chunk`` tokens (their K/V written
    too) are being prefilled.  It becomes a group whose prefix is its context
    [0, cached + chunk) and whose members are the chunk's tokens, token t of
    the chunk seeing the context up to and including itself
    (``query_prefix_len`` = cached + t + 1) with no distinct part.
    """
    groups = list(decode_groups) + [(c + n, [0] * n) for c, n in prefill]
    wl = build_single_level(name, hq, hkv, d, dtype, groups, [], seed)
    b = wl.batch
    lim = np.asarray(b["group_prefix_len"], dtype=np.int32)[b["query_group"]].copy()
    base = len(decode_groups)
    for j, (c, n) in enumerate(prefill):
        members = np.nonzero(b["query_group"] == base + j)[0]
        lim[members] = c + 1 + np.arange(n, dtype=np.int32)
    b["query_prefix_len"] = lim
    return wl


def build_token_batch(n_requests=8000, sharing=3, prefix=(1000, 2100), distinct=(1, 60), system=50, seed=0):
    """Token-id prompts shaped like the pages' industrial summary workload
    (about 3 requests per document, documents of about 1570 tokens, a few
    dozen distinct tokens each), behind a common system prompt: a two-level
    tree whose best single level is the documents.  Returns a list of int32
    arrays."""
    rng = np.random.Generator(np.random.PCG64(seed))
    sys_prompt = rng.integers(0, 32000, size=system, dtype=np.int32)
    out = []
    while len(out) < n_requests:
        doc = rng.integers(0, 32000, size=int(rng.integers(prefix[0], prefix[1] + 1)), dtype=np.int32)
        for _ in range(min(sharing, n_requests - len(out))):
            tail = rng.integers(0, 32000, size=int(rng.integers(distinct[0], distinct[1] + 1)), dtype=np.int32)
            out.append(np.concatenate([sys_prompt, doc, tail]))
    return out


def build_family_case(seed, r=4, hkv=2, d=64):
    """Groups 0..3 begin with the same 4 pages (64 tokens): group 1's prefix
    is exactly those pages, group 0 has a ragged rest, groups 2 and 3 have
    one request each; group 4 shares nothing with them and group 5 shares 3
    pages with group 4.  Plus two requests without a group."""
    wl = build_single_level("family_case", hkv * r, hkv, d, "bf16",
                            [(100, 3, (0, 30)), (64, 2, (1, 20)), (200, 1, (0, 50)), (70, 1, (1, 9)),
                             (90, 5, (0, 40)), (48, 4, (1, 30))], (2, (1, 60)), seed=seed)
    share_leading_pages(wl, 0, 3, 4)
    share_leading_pages(wl, 4, 5, 3)
    return wl


def build_two_level(name, hq, hkv, d, dtype, n_roots, root_len, n_subs, sub_len,
                    n_req, dist_range, seed=0, P=PAGE):
    """Two-level prefix tree: roots -> sub-prefixes -> requests.

    The tree (node_parent, node_len, node pages, query_node, distinct pages)
    is the workload's input; flattening it to single-level groups is the
    library's job.  ``batch`` is left empty until flattened.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    n_q = n_roots * n_subs * n_req
    lo, hi = dist_range
    dlen = [int(x) for x in rng.integers(lo, hi, size=n_q, endpoint=True)]
    node_parent, node_len = [], []
    for r in range(n_roots):
        node_parent.append(-1)
        node_len.append(root_len)
    for r in range(n_roots):
        for s in range(n_subs):
            node_parent.append(r)
            node_len.append(sub_len)
    query_node = [n_roots + r * n_subs + s for r in range(n_roots) for s in range(n_subs) for _ in range(n_req)]
    need = sum(-(-x // P) for x in node_len) + sum(-(-x // P) for x in dlen)
    perm = rng.permutation(need)
    noff, npages, used = _alloc(perm, node_len, P)
    qoff, qpages, _ = _alloc(perm[used:], dlen, P)
    tree = {
        "page_size": P,
        "node_parent": np.asarray(node_parent, dtype=np.int32),
        "node_len": np.asarray(node_len, dtype=np.int32),
        "node_page_off": noff,
        "node_pages": npages,
        "query_node": np.asarray(query_node, dtype=np.int32),
        "query_distinct_len": np.asarray(dlen, dtype=np.int32),
        "query_page_off": qoff,
        "query_pages": qpages,
    }
    wl = Workload(name, hq, hkv, d, dtype, need, {}, tree, seed, P)
    return wl


def build_tree(name, hq, hkv, d, dtype, levels, n_req, dist_range, seed=0, P=PAGE):
    """Prefix tree of any depth: ``levels`` = [(branching, tokens), ...] from
    the roots down (level 0 has ``branching`` roots; every node of level k has
    ``branching_{k+1}`` children); ``n_req`` requests hang under each node of
    the last level, each with its own distinct tokens drawn from
    ``dist_range``.  Node lengths must be page multiples.  Like
    ``build_two_level``, ``batch`` is left empty until flattened."""
    rng = np.random.Generator(np.random.PCG64(seed))
    node_parent, node_len, frontier = [], [], [-1]
    for branching, tokens in levels:
        nxt = []
        for parent in frontier:
            for _ in range(branching):
                nxt.append(len(node_parent))
                node_parent.append(parent)
                node_len.append(int(tokens))
        frontier = nxt
    query_node = [leaf for leaf in frontier for _ in range(n_req)]
    lo, hi = dist_range
    dlen = [int(x) for x in rng.integers(lo, hi, size=len(query_node), endpoint=True)]
    need = sum(-(-x // P) for x in node_len) + sum(-(-x // P) for x in dlen)
    perm = rng.permutation(need)
    noff, npages, used = _alloc(perm, node_len, P)
    qoff, qpages, _ = _alloc(perm[used:], dlen, P)
    tree = {
        "page_size": P,
        "node_parent": np.asarray(node_parent, dtype=np.int32),
        "node_len": np.asarray(node_len, dtype=np.int32),
        "node_page_off": noff,
        "node_pages": npages,
        "query_node": np.asarray(query_node, dtype=np.int32),
        "query_distinct_len": np.asarray(dlen, dtype=np.int32),
        "query_page_off": qoff,
        "query_pages": qpages,
    }
    return Workload(name, hq, hkv, d, dtype, need, {}, tree, seed, P)


def permute_groups(batch, perm):
    """The same batch with group g renumbered perm[g] (page tables moved with
    it); queries keep their order.  Groups that share leading pages are then
    no longer numbered consecutively."""
    perm = np.asarray(perm, dtype=np.int64)
    G = len(batch["group_prefix_len"])
    inv = np.empty(G, dtype=np.int64)
    inv[perm] = np.arange(G)
    lens, pages, off = [], [], [0]
    for new in range(G):
        g = int(inv[new])
        a, b = int(batch["group_page_off"][g]), int(batch["group_page_off"][g + 1])
        lens.append(int(batch["group_prefix_len"][g]))
        pages.extend(int(x) for x in batch["group_pages"][a:b])
        off.append(len(pages))
    out = dict(batch)
    out["group_prefix_len"] = np.asarray(lens, dtype=np.int32)
    out["group_page_off"] = np.asarray(off, dtype=np.int64)
    out["group_pages"] = np.asarray(pages, dtype=np.int32)
    qg = np.asarray(batch["query_group"], dtype=np.int64)
    out["query_group"] = np.where(qg >= 0, perm[np.maximum(qg, 0)], -1).astype(np.int32)
    return out


def _mixed(seed):
    return build_mixed("mixed_7prefill_256decode", 32, 8, 128, "bf16", [(2048, 128, (64, 512))] * 2,
                       [(1024, 512)] * 7, seed)


def _tiny_fp32(seed):
    return build_single_level("tiny_fp32_1x4", 2, 1, 64, "f32", [(128, 4, (8, 32))], [], seed)


def _llama8b(seed):
    return build_single_level("llama3_8b_8x100", 32, 8, 128, "bf16",
                              [(2048, 100, (64, 512))] * 8, [], seed)


def _longchat(seed):
    return build_single_level("longchat13b_1x256", 40, 40, 128, "bf16",
                              [(10240, 256, (128, 1024))], [], seed)


def _nosharing(seed):
    return build_single_level("no_sharing_512", 32, 8, 128, "bf16", [], (512, (1024, 4096)), seed)


def _twolevel(seed):
    return build_two_level("two_level_4x16x16", 32, 8, 128, "bf16", 4, 1024, 16, 2048, 16,
                           (32, 256), seed)


PRESETS = {
    "tiny_fp32_1x4": _tiny_fp32,
    "llama3_8b_8x100": _llama8b,
    "longchat13b_1x256": _longchat,
    "no_sharing_512": _nosharing,
    "two_level_4x16x16": _twolevel,
    "mixed_7prefill_256decode": _mixed,
}


def make_workload(name, seed=0):
    """A preset by name; also "llama3_8b_<G>x100" for any group count G (the
    8 x 100 shape with more or fewer prefix groups, for occupancy studies;
    not part of PRESETS)."""
    if name not in PRESETS:
        m = re.fullmatch(r"llama3_8b_(\d+)x100", name)
        if m and int(m.group(1)) > 0:
            return build_single_level(name, 32, 8, 128, "bf16", [(2048, 100, (64, 512))] * int(m.group(1)), [], seed)
    return PRESETS[name](seed)


def make_values(wl, device="cpu", seed=None):
    """Seeded Q, K pool and V pool as torch tensors on ``device``.

    q [N, Hq, d]; pools [num_pages, Hkv, page_size, d]; dtype bf16 or fp32.
    """
    import torch

    seed = wl.seed if seed is None else seed
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    n = _num_queries(wl)
    qshape = (n, wl.num_q_heads, wl.head_dim)
    pshape = (wl.num_pages, wl.num_kv_heads, wl.page_size, wl.head_dim)
    out = []
    for shape in (qshape, pshape, pshape):
        if wl.dtype == "bf16":
            x = torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
        else:
            x = torch.randn(shape, generator=g, device=device, dtype=torch.float64).to(torch.float32)
        out.append(x)
    return tuple(out)


def _num_queries(wl):
    if wl.tree is not None:
        return len(wl.tree["query_node"])
    return len(wl.batch["query_group"])


def _segments(wl):
    """(pages, length) of every stored KV segment (tree nodes or groups, then queries)."""
    src = wl.tree if wl.tree is not None else wl.batch
    segs = []
    if wl.tree is not None:
        for i in range(len(src["node_len"])):
            segs.append((src["node_pages"][src["node_page_off"][i]:src["node_page_off"][i + 1]], int(src["node_len"][i])))
    else:
        for gi in range(len(src["group_prefix_len"])):
            segs.append((src["group_pages"][src["group_page_off"][gi]:src["group_page_off"][gi + 1]], int(src["group_prefix_len"][gi])))
    for i in range(len(src["query_distinct_len"])):
        segs.append((src["query_pages"][src["query_page_off"][i]:src["query_page_off"][i + 1]], int(src["query_distinct_len"][i])))
    return segs


def fill_stale(wl, k_pool, v_pool, value=1.0e4):
    """Overwrite the unused tail slots of every segment's last page with +-value.

    Used by an edge test: a kernel that lets a slot beyond a segment's length
    into its softmax shows up as a gross error.
    """
    P = wl.page_size
    for pages, n in _segments(wl):
        if n % P == 0 or len(pages) == 0:
            continue
        last = int(pages[(n - 1) // P])
        k_pool[last, :, n % P:, :] = value
        v_pool[last, :, n % P:, :] = -value


def algorithmic_cost(wl, batch=None):
    """Algorithmic bytes and flops of one decode step (bookkeeping only).

    KV bytes: prefix once per group + distinct once per query, page padding
    excluded; plus Q read and O (fp32) written.  Flops: 4 * d * Hq per
    attended token per query (2 for q.k, 2 for p.v).
    """
    b = wl.batch if batch is None else batch
    e = 2 if wl.dtype == "bf16" else 4
    hkv, hq, d = wl.num_kv_heads, wl.num_q_heads, wl.head_dim
    lp = np.asarray(b["group_prefix_len"], dtype=np.int64)
    ld = np.asarray(b["query_distinct_len"], dtype=np.int64)
    qg = np.asarray(b["query_group"], dtype=np.int64)
    prefix_tok = int(lp.sum())
    distinct_tok = int(ld.sum())
    n = len(qg)
    kv_prefix = prefix_tok * hkv * d * 2 * e
    kv_distinct = distinct_tok * hkv * d * 2 * e
    q_bytes = n * hq * d * e
    o_bytes = n * hq * d * 4
    seen = np.where(qg >= 0, lp[np.maximum(qg, 0)] if len(lp) else 0, 0)
    if b.get("query_prefix_len") is not None:
        seen = np.where(qg >= 0, np.minimum(seen, np.asarray(b["query_prefix_len"], dtype=np.int64)), 0)
    attended = ld + seen
    flops_total = 4 * d * hq * int(attended.sum())
    flops_prefix = 4 * d * hq * int(seen.sum())
    return {
        "kv_prefix_bytes": kv_prefix,
        "kv_distinct_bytes": kv_distinct,
        "kv_bytes": kv_prefix + kv_distinct,
        "q_bytes": q_bytes,
        "o_bytes": o_bytes,
        "bytes": kv_prefix + kv_distinct + q_bytes + o_bytes,
        "flops": flops_total,
        "flops_prefix": flops_prefix,
        "flops_distinct": flops_total - flops_prefix,
        "logical_tokens": int(attended.sum()),
        "processed_tokens": prefix_tok + distinct_tok,
    }


def subset_for_queries(batch, queries):
    """Page tables restricted to ``queries`` with page ids renumbered densely.

    Returns (sub_batch, page_ids) where ``page_ids[j]`` is the original id of
    new page j; the caller copies exactly those pages out of the pools.  Used
    for sampled oracle checks at full size.
    """
    queries = [int(i) for i in queries]
    groups = sorted({int(batch["query_group"][i]) for i in queries if int(batch["query_group"][i]) >= 0})
    gmap = {g: j for j, g in enumerate(groups)}
    ids = {}

    def remap(pages):
        out = []
        for p in pages:
            p = int(p)
            if p not in ids:
                ids[p] = len(ids)
            out.append(ids[p])
        return out

    gpages, goff, glen = [], [0], []
    for g in groups:
        a, b = int(batch["group_page_off"][g]), int(batch["group_page_off"][g + 1])
        gpages.extend(remap(batch["group_pages"][a:b]))
        goff.append(len(gpages))
        glen.append(int(batch["group_prefix_len"][g]))
    qpages, qoff, qg, dl = [], [0], [], []
    for i in queries:
        a, b = int(batch["query_page_off"][i]), int(batch["query_page_off"][i + 1])
        qpages.extend(remap(batch["query_pages"][a:b]))
        qoff.append(len(qpages))
        g = int(batch["query_group"][i])
        qg.append(gmap[g] if g >= 0 else -1)
        dl.append(int(batch["query_distinct_len"][i]))
    lim = batch.get("query_prefix_len")
    sub = {
        "page_size": batch["page_size"],
        "group_prefix_len": np.asarray(glen, dtype=np.int32),
        "group_page_off": np.asarray(goff, dtype=np.int64),
        "group_pages": np.asarray(gpages, dtype=np.int32),
        "query_group": np.asarray(qg, dtype=np.int32),
        "query_distinct_len": np.asarray(dl, dtype=np.int32),
        "query_page_off": np.asarray(qoff, dtype=np.int64),
        "query_pages": np.asarray(qpages, dtype=np.int32),
    }
    if lim is not None:
        sub["query_prefix_len"] = np.asarray([int(lim[i]) for i in queries], dtype=np.int32)
    order = np.empty(len(ids), dtype=np.int64)
    for p, j in ids.items():
        order[j] = p
    return sub, order
