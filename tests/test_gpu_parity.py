"""GPU parity: the fused HIP path (through the C ABI) against the fp64 oracle.

Every case is compared element by element on the whole output: the small
shapes directly, the full-size workloads in the bench's launch configuration
with the oracle spread over worker processes (tests/oracle_pool.py).  Tolerances: bf16 inputs max |err|
<= 1e-2 and relative L2 <= 5e-3; fp32 inputs 1e-5 for both.
"""

import numpy as np
import pytest

import oracle
import prefix_shared_decode_amd as P
from workloads import build_single_level, build_two_level, fill_stale, make_workload

from gpu_helpers import (assert_close, assert_lse_close, log, oracle_all, run, to_host64,
                         values)

pytestmark = pytest.mark.gpu


def _check_full(wl, batch, q, k, v, what, out_dtype="f32", lse=True, **kw):
    log(f"case {what}: queries={len(batch['query_group'])} plan={kw}")
    step, out, m, l = run(wl, batch, q, k, v, out_dtype=out_dtype, **kw)
    O, M, L = oracle_all(wl, batch, q, k, v)
    assert_close(to_host64(out), O, wl.dtype if out_dtype == "f32" else "bf16", what)
    if lse:
        assert_lse_close(m, l, M, L, 1e-5 if wl.dtype == "f32" else 2e-4)
    return step, out, m, l


# ---------------- the tiny fp32 workload, exactly ----------------

def test_tiny_fp32_exact_config():
    wl = make_workload("tiny_fp32_1x4")
    q, k, v = values(wl)
    _check_full(wl, wl.batch, q, k, v, "tiny_fp32_1x4")


# ---------------- reduced shapes of the bf16 workloads ----------------

SMALL = {
    # Llama-3-8B heads (32/8, d128): 2 groups x 20 requests, ragged prefix, multi-chunk
    "gqa4_groups": dict(hq=32, hkv=8, d=128, groups=[(300, 20, (0, 200)), (77, 9, (1, 90))], ung=(3, (1, 300))),
    # LongChat-like MHA (40/40 heads): one group, prefix spans several chunks
    "mha_group": dict(hq=40, hkv=40, d=128, groups=[(700, 24, (5, 100))], ung=(0, (1, 2))),
    # no sharing: pure paged decode with several distinct chunks
    "no_sharing": dict(hq=32, hkv=8, d=128, groups=[], ung=(12, (1, 1500))),
    # head_dim 64 and GQA ratio 8
    "d64_r8": dict(hq=16, hkv=2, d=64, groups=[(130, 6, (0, 70))], ung=(2, (1, 40))),
    # GQA ratio 2 with a group just above the MFMA threshold
    "r2_tail_rows": dict(hq=8, hkv=4, d=128, groups=[(33, 9, (0, 20))], ung=(1, (1, 17))),
    # GQA ratio 8 at head_dim 128 (64 query heads over 8 kv heads)
    "gqa8_d128": dict(hq=64, hkv=8, d=128, groups=[(260, 10, (0, 120)), (40, 3, (1, 30))], ung=(2, (1, 200))),
}


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("opts", [dict(), dict(prefix_chunk_tokens=128, distinct_chunk_tokens=64, mfma_tile_rows=32),
                                  dict(flags=P.FORCE_MATVEC)], ids=["default", "small_chunks", "matvec_only"])
def test_small_bf16(name, opts):
    s = SMALL[name]
    wl = build_single_level(name, s["hq"], s["hkv"], s["d"], "bf16", s["groups"], s["ung"], seed=11, spare_pages=5)
    q, k, v = values(wl)
    _check_full(wl, wl.batch, q, k, v, f"{name}/{opts}", **opts)


def test_two_level_small_flattened():
    wl = build_two_level("two_level_small", 32, 8, 128, "bf16", 2, 64, 3, 128, 4, (0, 60), seed=5)
    batch, saved = P.psa_flatten_prefix_tree(wl.tree)
    assert saved == 6 * 192 * 3
    q, k, v = values(wl)
    log("case two_level_small")
    _, out, m, l = run(wl, batch, q, k, v)
    # the oracle reads each query's context straight from the tree
    O, M, L = oracle.decode_attention(to_host64(q), to_host64(k), to_host64(v),
                                      oracle.flatten_tree(wl.tree, [-1] * len(wl.tree["query_node"])))
    assert_close(to_host64(out), O, "bf16", "two_level_small")


def test_library_loaded_before_torch_initialises_the_gpu():
    """A fresh process whose first call into the library is host-only (the
    tree flattening) and only then touches the GPU through torch: the binding
    loads torch's HIP runtime before the library, so both use one runtime."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import numpy as np, oracle, prefix_shared_decode_amd as P\n"
        "from workloads import build_two_level, make_values\n"
        "wl = build_two_level('t', 32, 8, 128, 'bf16', 2, 64, 3, 128, 4, (0, 60), seed=5)\n"
        "batch, _ = P.psa_flatten_prefix_tree(wl.tree)\n"
        "import torch\n"
        "q, k, v = make_values(wl, 'cuda')\n"
        "cfg = P.make_config(32, 8, 128, wl.num_pages, 'bf16', 'f32')\n"
        "step = P.DecodeStep(cfg, batch)\n"
        "out = torch.empty((len(batch['query_group']), 32, 128), dtype=torch.float32, device='cuda')\n"
        "step(q, k, v, out)\n"
        "torch.cuda.synchronize()\n"
        "f = lambda t: t.float().cpu().numpy().astype(np.float64)\n"
        "O, _, _ = oracle.decode_attention(f(q), f(k), f(v), batch)\n"
        "print('maxerr', float(np.abs(f(out) - O).max()))\n")
    log("case library loaded before torch initialises the GPU (child process)")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    err = float(r.stdout.split("maxerr")[-1])
    assert err <= 1e-2, r.stdout


@pytest.mark.parametrize("r,d", [(1, 128), (4, 64), (4, 128), (8, 128)])
@pytest.mark.parametrize("opts", [dict(), dict(prefix_chunk_tokens=32, mfma_tile_rows=16),
                                  dict(flags=P.NO_PAGE_SHARING), dict(mfma_min_rows=1)],
                         ids=["default", "small_chunks", "no_sharing", "min_rows_1"])
def test_family_tiles(r, d, opts):
    """Consecutive groups that begin with the same pages: one set of MFMA
    tiles over all their members covers those pages, next to empty and
    mat-vec sized rests of each group."""
    from workloads import build_family_case

    wl = build_family_case(7, r=r, d=d)
    q, k, v = values(wl)
    _check_full(wl, wl.batch, q, k, v, f"family r{r} d{d} {opts}", **opts)


@pytest.mark.parametrize("seed", range(8))
def test_random_small_workloads(seed):
    """Seeded random shapes: GQA ratio, head dim, group sizes and prefix
    lengths (ragged, some groups sharing their leading pages), distinct
    lengths including empty ones, and random chunk / tile options."""
    from workloads import share_leading_pages

    rng = np.random.default_rng(100 + seed)
    r = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 4])) if r > 1 else int(rng.choice([2, 8]))
    d = int(rng.choice([64, 128]))
    groups = []
    for _ in range(int(rng.integers(1, 6))):
        n = int(rng.integers(1, 30))
        groups.append((int(rng.integers(1, 700)), n, (0, int(rng.integers(1, 400)))))
    wl = build_single_level(f"rand{seed}", hkv * r, hkv, d, "bf16", groups, (int(rng.integers(0, 5)), (1, 500)),
                            seed=seed, spare_pages=3)
    if len(groups) >= 2 and rng.random() < 0.7:  # the first groups begin with the same pages
        share_leading_pages(wl, 0, int(rng.integers(1, len(groups))), int(rng.integers(1, 20)))
    opts = {}
    if rng.random() < 0.5:
        opts = dict(prefix_chunk_tokens=int(rng.choice([64, 256, 1024, 2048])),
                    distinct_chunk_tokens=int(rng.choice([32, 128, 1024])),
                    mfma_tile_rows=int(rng.choice([16, 64, 128])), mfma_min_rows=int(rng.choice([1, 16, 48])))
    q, k, v = values(wl)
    _check_full(wl, wl.batch, q, k, v, f"random seed {seed} r{r} hkv{hkv} d{d} {opts}", **opts)


@pytest.mark.parametrize("r,d", [(4, 128), (8, 128), (4, 64), (1, 128)])
@pytest.mark.parametrize("opts", [dict(), dict(prefix_chunk_tokens=64, mfma_tile_rows=32),
                                  dict(flags=P.FORCE_MATVEC), dict(mfma_min_rows=1)],
                         ids=["default", "small_chunks", "matvec_only", "min_rows_1"])
def test_prefill_chunks_with_decode(r, d, opts):
    """Prefill chunks (causal: each token sees its context up to itself)
    in the same launch as decode queries; chunk starts and lengths ragged
    against the 64-token blocks and the tiles' rows."""
    from workloads import build_mixed

    wl = build_mixed(f"mixed r{r} d{d}", 2 * r, 2, d, "bf16", [(150, 11, (0, 90)), (70, 3, (1, 40))],
                     [(0, 37), (64, 70), (112, 5), (16, 129)], seed=13)
    q, k, v = values(wl)
    _check_full(wl, wl.batch, q, k, v, f"prefill+decode r{r} d{d} {opts}", **opts)


@pytest.mark.parametrize("seed", range(3))
def test_random_prefix_limits(seed):
    """Decode queries that see only part of their group's prefix: random
    limits, including 0 (distinct part only), exact chunk and block
    boundaries and the whole prefix, with default and small chunks."""
    rng = np.random.default_rng(70 + seed)
    wl = build_single_level(f"lim{seed}", 32, 8, 128, "bf16", [(700, 24, (1, 80)), (130, 6, (1, 30))], (2, (1, 50)),
                            seed=seed)
    b = wl.batch
    lp = np.asarray(b["group_prefix_len"])[np.maximum(b["query_group"], 0)]
    lim = rng.integers(0, lp + 1)
    picks = [0, 64, 63, 65, 128, 256, 512]
    for j, v in enumerate(picks):
        lim[j] = min(v, lp[j])
    lim[len(picks)] = lp[len(picks)]
    b["query_prefix_len"] = lim.astype(np.int32)
    q, k, v = values(wl)
    for opts in (dict(), dict(prefix_chunk_tokens=128, mfma_tile_rows=32), dict(flags=P.FORCE_MATVEC)):
        _check_full(wl, b, q, k, v, f"random limits seed {seed} {opts}", **opts)


# ---------------- edge cases ----------------

@pytest.mark.parametrize("seed", [0, 1])
def test_shared_nodes_with_scattered_group_numbers(seed):
    """A flattened two-level tree whose groups are renumbered at random: the
    groups of one root are no longer consecutive, the plan still shares the
    root's tokens across them; the output equals the oracle's (contexts read
    from the tree), and the plan without page sharing's."""
    from workloads import permute_groups

    wl = build_two_level("two_level_perm", 32, 8, 128, "bf16", 3, 128, 4, 96, 5, (0, 70), seed=40 + seed)
    batch, _ = P.psa_flatten_prefix_tree(wl.tree)
    batch = permute_groups(batch, np.random.default_rng(seed).permutation(len(batch["group_prefix_len"])))
    q, k, v = values(wl)
    O, M, L = oracle.decode_attention(to_host64(q), to_host64(k), to_host64(v),
                                      oracle.flatten_tree(wl.tree, [-1] * len(wl.tree["query_node"])))
    for kw in ({}, {"prefix_chunk_tokens": 64, "mfma_tile_rows": 32}, {"flags": P.NO_PAGE_SHARING}):
        log(f"case scattered groups seed {seed} {kw}")
        _, out, m, l = run(wl, batch, q, k, v, **kw)
        assert_close(to_host64(out), O, "bf16", f"scattered groups {kw}")
        assert_lse_close(m, l, M, L, 2e-4)


@pytest.mark.parametrize("r", [1, 4])
def test_nested_shared_nodes(r):
    """Three-level tree (roots 512, children 256, leaves 128, 8 requests per
    leaf), flattened to leaf groups: root and middle tokens are each tiled
    once over all the groups below them (nested shared nodes).  Output equals
    the oracle's, read from the tree, with default and small chunks."""
    from workloads import build_tree

    wl = build_tree("nested", 8 * r, 8, 128, "bf16", [(2, 512), (2, 256), (2, 128)], 8, (0, 50), seed=7 + r)
    batch, _ = P.psa_flatten_prefix_tree(wl.tree)
    q, k, v = values(wl)
    O, M, L = oracle.decode_attention(to_host64(q), to_host64(k), to_host64(v),
                                      oracle.flatten_tree(wl.tree, [-1] * len(wl.tree["query_node"])))
    for kw in ({}, {"prefix_chunk_tokens": 128, "distinct_chunk_tokens": 32}):
        log(f"case nested r {r} {kw}")
        _, out, m, l = run(wl, batch, q, k, v, **kw)
        assert_close(to_host64(out), O, "bf16", f"nested r {r} {kw}")
        assert_lse_close(m, l, M, L, 2e-4)


def test_stale_padding_is_masked():
    wl = build_single_level("stale", 32, 8, 128, "bf16", [(37, 17, (0, 35))], (3, (1, 20)), seed=3)
    q, k, v = values(wl)
    fill_stale(wl, k, v, 1.0e4)
    _check_full(wl, wl.batch, q, k, v, "stale+-1e4")
    _check_full(wl, wl.batch, q, k, v, "stale+-1e4 matvec", flags=P.FORCE_MATVEC)


@pytest.mark.parametrize("fill", ["nan", "inf"])
def test_nonfinite_padding_is_never_read(fill):
    """Slots past a segment's length hold NaN (K and V) or +Inf in K and -Inf
    in V.  The context ends before them, so no weight (not even a zero) may
    meet them: the output is the oracle's, on MFMA, small-chunk and mat-vec
    plans, bf16 and fp32."""
    wl = build_single_level("nonfinite", 32, 8, 128, "bf16", [(37, 17, (0, 35)), (300, 5, (1, 40))],
                            (3, (1, 20)), seed=3)
    q, k, v = values(wl)
    fill_stale(wl, k, v, float(fill))
    _check_full(wl, wl.batch, q, k, v, f"padding {fill}")
    _check_full(wl, wl.batch, q, k, v, f"padding {fill}, small chunks", prefix_chunk_tokens=64,
                distinct_chunk_tokens=32, mfma_tile_rows=32)
    _check_full(wl, wl.batch, q, k, v, f"padding {fill}, mat-vec only", flags=P.FORCE_MATVEC)
    wl32 = build_single_level("nonfinite32", 8, 4, 128, "f32", [(45, 6, (1, 30))], (2, (1, 40)), seed=9)
    q, k, v = values(wl32)
    fill_stale(wl32, k, v, float(fill))
    _check_full(wl32, wl32.batch, q, k, v, f"padding {fill}, fp32")


def test_single_token_and_empty_distinct():
    # prefix of one token with empty distinct parts; distinct of one token without prefix
    wl = build_single_level("tiny_ctx", 8, 2, 128, "bf16", [(1, [0, 0, 0, 0, 1, 0, 0, 0]), (16, [0] * 5)],
                            [1, 1, 16, 17], seed=4)
    q, k, v = values(wl)
    _check_full(wl, wl.batch, q, k, v, "single-token", mfma_min_rows=4)


def test_fp32_larger_and_scale():
    wl = build_single_level("f32_mix", 8, 4, 128, "f32", [(200, 10, (0, 90))], (4, (1, 600)), seed=8)
    q, k, v = values(wl)
    _check_full(wl, wl.batch, q, k, v, "f32 d128")
    log("case f32 custom scale")
    _, out, m, l = run(wl, wl.batch, q, k, v, sm_scale=0.3)
    O, M, L = oracle_all(wl, wl.batch, q, k, v, sm_scale=0.3)
    assert_close(to_host64(out), O, "f32", "f32 scale 0.3")


@pytest.mark.parametrize("r,d", [(1, 64), (4, 64), (8, 64), (1, 128), (4, 128), (8, 128)])
def test_fp32_every_head_shape(r, d):
    """fp32 K/V (mat-vec tiles only: the MFMA tile is bf16) at every GQA ratio
    and head dim the library instantiates besides r 2, which the other fp32
    cases cover; d 128 with r 8 keeps one page in flight."""
    wl = build_single_level(f"f32_r{r}_d{d}", 2 * r, 2, d, "f32", [(150, 5, (0, 70)), (33, 2, (1, 20))],
                            (2, (1, 300)), seed=30 + r + d)
    q, k, v = values(wl)
    _check_full(wl, wl.batch, q, k, v, f"f32 r{r} d{d}")
    _check_full(wl, wl.batch, q, k, v, f"f32 r{r} d{d} small chunks", prefix_chunk_tokens=64,
                distinct_chunk_tokens=32)


def test_bf16_r2_d64():
    """bf16 at GQA ratio 2 and head dim 64 (the one bf16 instantiation no other
    case reaches): MFMA tiles, small chunks, mat-vec only."""
    wl = build_single_level("bf16_r2_d64", 8, 4, 64, "bf16", [(300, 20, (0, 80)), (70, 3, (1, 30))],
                            (2, (1, 200)), seed=44)
    q, k, v = values(wl)
    _check_full(wl, wl.batch, q, k, v, "bf16 r2 d64")
    _check_full(wl, wl.batch, q, k, v, "bf16 r2 d64 small chunks", prefix_chunk_tokens=64, distinct_chunk_tokens=32,
                mfma_tile_rows=32)
    _check_full(wl, wl.batch, q, k, v, "bf16 r2 d64 mat-vec only", flags=P.FORCE_MATVEC)


def test_bf16_output():
    wl = build_single_level("bf16_out", 32, 8, 128, "bf16", [(256, 12, (4, 64))], (2, (1, 99)), seed=9)
    q, k, v = values(wl)
    log("case bf16 output")
    _, out, _, _ = run(wl, wl.batch, q, k, v, out_dtype="bf16")
    O, _, _ = oracle_all(wl, wl.batch, q, k, v)
    assert_close(to_host64(out), O, "bf16", "bf16 out")


def test_empty_batch_is_a_no_op():
    import torch

    wl = build_single_level("empty", 32, 8, 128, "bf16", [], [], seed=0)
    step = P.DecodeStep(P.make_config(32, 8, 128, 1, "bf16"), wl.batch)
    z = torch.zeros((0, 32, 128), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((1, 8, 16, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((0, 32, 128), dtype=torch.float32, device="cuda")
    step(z, pool, pool, out)
    torch.cuda.synchronize()


# ---------------- partials, merge, determinism ----------------

def test_prefix_and_distinct_partials_merge_to_fused():
    import torch

    wl = build_single_level("split", 32, 8, 128, "bf16", [(160, 12, (0, 80)), (48, 3, (3, 9))], (3, (1, 50)), seed=2)
    q, k, v = values(wl)
    log("case PREFIX_ONLY / DISTINCT_ONLY / psa_merge")
    _, op, mp, lp = run(wl, wl.batch, q, k, v, flags=P.PREFIX_ONLY)
    _, od, md, ld = run(wl, wl.batch, q, k, v, flags=P.DISTINCT_ONLY)
    _, of, mf, lf = run(wl, wl.batch, q, k, v)
    # each partial against the oracle's partial over the same token range
    b = wl.batch
    prefix_only = dict(b, query_distinct_len=np.zeros_like(b["query_distinct_len"]))
    distinct_only = dict(b, query_group=np.full_like(b["query_group"], -1))
    qh, kh, vh = to_host64(q), to_host64(k), to_host64(v)
    has_p = b["query_group"] >= 0
    has_d = b["query_distinct_len"] > 0
    Op, Mp, Lp = oracle.decode_attention(qh[has_p], kh, vh, {**prefix_only, **_rows(prefix_only, has_p)})
    assert_close(to_host64(op)[has_p], Op, "bf16", "prefix partial")
    assert np.all(to_host64(lp)[~has_p] == 0) and np.all(to_host64(mp)[~has_p] == -np.inf)
    assert np.all(to_host64(op)[~has_p] == 0)
    Od, Md, Ld = oracle.decode_attention(qh[has_d], kh, vh, {**distinct_only, **_rows(distinct_only, has_d)})
    assert_close(to_host64(od)[has_d], Od, "bf16", "distinct partial")
    # psa_merge of the two partials equals the fused result
    n, hq, d = op.shape
    o = torch.empty_like(op)
    m = torch.empty_like(mp)
    l = torch.empty_like(lp)
    P.psa_merge(op.view(-1, d), mp.view(-1), lp.view(-1), od.view(-1, d), md.view(-1), ld.view(-1),
                o.view(-1, d), m.view(-1), l.view(-1))
    torch.cuda.synchronize()
    mx = float((o - of).abs().max())
    log(f"  merge vs fused max diff {mx:.3e}")
    assert mx <= 2e-6
    # in-place merge (outputs alias the a inputs)
    P.psa_merge(op.view(-1, d), mp.view(-1), lp.view(-1), od.view(-1, d), md.view(-1), ld.view(-1),
                op.view(-1, d), mp.view(-1), lp.view(-1))
    torch.cuda.synchronize()
    assert torch.equal(op, o) and torch.equal(mp, m) and torch.equal(lp, l)


def _rows(batch, mask):
    """Restrict a batch's query arrays to the queries in ``mask``."""
    idx = np.nonzero(mask)[0]
    qoff = batch["query_page_off"]
    pages, off = [], [0]
    for i in idx:
        pages.extend(batch["query_pages"][qoff[i]:qoff[i + 1]])
        off.append(len(pages))
    return {"query_group": batch["query_group"][idx], "query_distinct_len": batch["query_distinct_len"][idx],
            "query_page_off": np.asarray(off, np.int64), "query_pages": np.asarray(pages, np.int32)}


def test_psa_merge_against_oracle():
    import torch

    rng = np.random.default_rng(0)
    rows, d = 300, 128
    Oa, Ob = rng.standard_normal((rows, d)), rng.standard_normal((rows, d))
    ma, mb = rng.standard_normal(rows) * 3, rng.standard_normal(rows) * 3
    la, lb = rng.uniform(0.5, 40, rows), rng.uniform(0.5, 40, rows)
    # empty partials on some rows (identity), both empty on one
    ma[:5], la[:5], Oa[:5] = -np.inf, 0, 0
    mb[3:8], lb[3:8], Ob[3:8] = -np.inf, 0, 0
    Oe, Me, Le = oracle.merge_partials((Oa, ma, la), (Ob, mb, lb))
    t = lambda x: torch.tensor(x, dtype=torch.float32, device="cuda")  # noqa: E731
    o, m, l = t(np.zeros((rows, d))), t(np.zeros(rows)), t(np.zeros(rows))
    log("case psa_merge vs oracle")
    P.psa_merge(t(Oa), t(ma), t(la), t(Ob), t(mb), t(lb), o, m, l)
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_host64(o), Oe, atol=2e-6, rtol=0)
    np.testing.assert_allclose(to_host64(l), Le, rtol=2e-6)
    assert np.all(to_host64(m)[3:5] == -np.inf)


def test_deterministic_and_reusable_workspace():
    import torch

    wl = build_single_level("det", 32, 8, 128, "bf16", [(400, 30, (0, 300))], (4, (1, 900)), seed=6)
    q, k, v = values(wl)
    log("case determinism x20 (same workspace: queues and counters reset themselves), poisoned slots")
    step, out, m, l = run(wl, wl.batch, q, k, v, prefix_chunk_tokens=128, distinct_chunk_tokens=128)
    ref, mref, lref = out.clone(), m.clone(), l.clone()
    for _ in range(20):
        for t in (out, m, l):
            t.fill_(float("nan"))
        step(q, k, v, out, m, l)
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(m, mref) and torch.equal(l, lref)
    _, out2, _, _ = run(wl, wl.batch, q, k, v, prefix_chunk_tokens=128, distinct_chunk_tokens=128,
                        flags=P.NO_XCD_ORDER)
    assert torch.equal(out2, ref)
    _, out3, _, _ = run(wl, wl.batch, q, k, v, prefix_chunk_tokens=128, distinct_chunk_tokens=128,
                        flags=P.DEBUG_POISON)
    assert torch.equal(out3, ref)


def test_traced_launch_records_every_unit():
    """The traced entry point (per-unit timing for the bench's timelines)
    gives the untraced launch's bits and one valid record per unit: start
    <= end, an XCD id below 8, and the unit's kind from the plan."""
    import torch

    wl = build_single_level("trace", 32, 8, 128, "bf16", [(400, 30, (0, 300))], (4, (1, 900)), seed=7)
    q, k, v = values(wl)
    log("case traced launch: records and bits")
    plan = P.psa_build_plan(P.make_config(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages, wl.dtype),
                            wl.batch, prefix_chunk_tokens=128, distinct_chunk_tokens=128)
    info = plan.info()
    ws = torch.empty(max(int(info["workspace_bytes"]), 256), dtype=torch.uint8, device="cuda")
    P.psa_plan_upload(plan, ws)
    n = len(wl.batch["query_group"])
    outs = []
    units = int(info["num_items"])
    tr = torch.zeros(units * 4, dtype=torch.int64, device="cuda")
    for traced in (False, True):
        o = torch.full((n, wl.num_q_heads, wl.head_dim), float("nan"), dtype=torch.float32, device="cuda")
        P.psa_decode_attention(plan, q, k, v, o, ws, trace=tr if traced else None)
        torch.cuda.synchronize()
        outs.append(o)
    assert torch.equal(outs[0], outs[1])
    t = tr.view(units, 4).cpu().numpy()
    kinds = np.asarray(plan.items()).reshape(units, 4, 8)[:, 0, 0] & 0xFF
    assert (t[:, 0] > 0).all() and (t[:, 1] >= t[:, 0]).all()
    assert (((t[:, 2] >> 32) & 0xF) < 8).all()
    assert np.array_equal(t[:, 3], kinds)


@pytest.mark.parametrize("case", ["two_level_three_pieces", "many_prefix_chunks"])
def test_merge_paths_give_the_same_bits(case):
    """Queries of three pieces (root tile, own tile, distinct part) and of
    five to twelve (1024- and 2048-token prefixes in 256-token chunks plus
    distinct parts in 128-token chunks):
    whichever piece arrives last merges, in registers or from memory, in one
    batch of loads or piece by piece, so repeated launches and plans that
    reorder the work must give the same bits, and match the oracle."""
    import torch

    if case == "two_level_three_pieces":
        wl = build_two_level("merge3", 32, 8, 128, "bf16", 2, 256, 3, 512, 6, (16, 200), seed=9)
        batch, _ = P.psa_flatten_prefix_tree(wl.tree)
        kw = {}
        ctx = oracle.flatten_tree(wl.tree, [-1] * len(wl.tree["query_node"]))
    else:
        wl = build_single_level("merge10", 32, 8, 128, "bf16", [(1024, 6, (100, 400)), (2048, 6, (100, 400))],
                                (2, (50, 300)), seed=10)
        batch = wl.batch
        kw = dict(prefix_chunk_tokens=256, distinct_chunk_tokens=128)
        ctx = None
    q, k, v = values(wl)
    log(f"case {case}: repeats and reordered plans, bit for bit")
    step, out, m, l = run(wl, batch, q, k, v, **kw)
    ref, mref, lref = out.clone(), m.clone(), l.clone()
    if ctx is not None:
        O, M, L = oracle.decode_attention(to_host64(q), to_host64(k), to_host64(v), ctx)
    else:
        O, M, L = oracle_all(wl, batch, q, k, v)
    assert_close(to_host64(out), O, "bf16", case)
    assert_lse_close(m, l, M, L, 2e-4)
    for _ in range(10):
        for t in (out, m, l):
            t.fill_(float("nan"))
        step(q, k, v, out, m, l)
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(m, mref) and torch.equal(l, lref)
    for flags in (P.NO_XCD_ORDER, P.NO_TILE_PAIRS, P.DEBUG_POISON):
        _, o2, m2, l2 = run(wl, batch, q, k, v, flags=flags, **kw)
        assert torch.equal(o2, ref) and torch.equal(m2, mref) and torch.equal(l2, lref), flags


# ---------------- full-size workloads, whole output ----------------

FULL = ["llama3_8b_8x100", "longchat13b_1x256", "no_sharing_512", "two_level_4x16x16", "mixed_7prefill_256decode",
        # the 8x100 shape with 15 groups: 60 MFMA tiles an XCD, spread through
        # the queue between the mat-vec units instead of paired at its start
        "llama3_8b_15x100"]
# queries per oracle worker batch (the LongChat-like contexts are 10.8K tokens x 40 heads)
FULL_CHUNK = {"longchat13b_1x256": 4}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size_whole_output(name):
    """Every query and head of a full-size workload, in the bench's launch
    configuration (default plan), against the fp64 oracle; max |err| and
    relative L2 over the whole output tensor, log-sum-exp on every row.

    The two-level workload runs on the library's flattening of its tree; the
    oracle reads each query's context straight from the tree (root pages ++
    sub-prefix pages ++ distinct pages), so a flattening that dropped or
    repeated pages would fail here."""
    import torch

    from oracle_pool import oracle_full

    wl = make_workload(name)
    batch = wl.batch
    ref_batch = wl.batch
    if wl.tree is not None:
        batch, _ = P.psa_flatten_prefix_tree(wl.tree)
        ref_batch = oracle.flatten_tree(wl.tree, [-1] * len(wl.tree["query_node"]))
    log(f"case full {name}: generating values")
    q, k, v = values(wl)
    log(f"case full {name}: launching")
    _, out, m, l = run(wl, batch, q, k, v)
    assert torch.isfinite(out).all()
    got, gm, gl = to_host64(out), to_host64(m), to_host64(l)
    O, M, L = oracle_full(ref_batch, q, k, v, FULL_CHUNK.get(name, 16), log=log, what=name)
    assert_close(got, O, "bf16", f"full {name}, whole output {got.shape}")
    lse = np.abs((gm + np.log(gl)) - (M + np.log(L)))
    log(f"  lse max err {lse.max():.3e} over {lse.size} rows")
    assert lse.max() <= 2e-4


def test_late_dominant_key_triggers_exact_rescaling():
    """A key far above everything before it, late in a chunk: the mat-vec tile's
    fixed reference max is exceeded and the tile redoes the chunk; the MFMA
    tile rescales its accumulators.  Either way the result is the plain softmax."""
    import torch

    wl = build_single_level("late_key", 32, 8, 128, "bf16", [(400, 6, (0, 30))], (3, (200, 300)), seed=13)
    q, k, v = values(wl)
    b = wl.batch
    r = 4
    # ungrouped query 6: dominant key at its distinct token 250 for kv head 1
    i = 6
    pages = b["query_pages"][b["query_page_off"][i]:b["query_page_off"][i + 1]]
    t = 250 if b["query_distinct_len"][i] > 250 else int(b["query_distinct_len"][i]) - 1
    k[int(pages[t // 16]), 1, t % 16, :] = (12.0 * q[i, 1 * r, :].float()).to(torch.bfloat16)
    # group 0: dominant key at prefix token 380 for kv head 2
    gp = b["group_pages"][b["group_page_off"][0]:b["group_page_off"][1]]
    k[int(gp[380 // 16]), 2, 380 % 16, :] = (12.0 * q[0, 2 * r, :].float()).to(torch.bfloat16)
    _check_full(wl, b, q, k, v, "late dominant key")
    _check_full(wl, b, q, k, v, "late dominant key, mat-vec only", flags=P.FORCE_MATVEC)


def test_measured_peak_kernels_run():
    """The two ceiling kernels run, write every sink entry, and report sane
    rates (a read well below 8 TB/s is still above 1 TB/s; the MFMA run is
    above 0.5 PFLOP/s)."""
    import torch

    buf = torch.ones(64 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.full((2048 * 256,), -1, dtype=torch.int32, device="cuda")
    out = torch.full((2048 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    log("case measured peak kernels")
    P.psa_debug_read_peak(buf, sink)
    flops = P.psa_debug_mfma_peak(out, 256)
    torch.cuda.synchronize()
    # bytes of value 1: the xor of an even number of 16-byte chunks per thread
    assert int((sink == -1).sum()) == 0
    assert bool(torch.isfinite(out).all())
    def best_ms(fn, reps=5):  # one launch can be slowed by clocks ramping or a neighbour: take the best
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return min(ts)

    assert buf.numel() / (best_ms(lambda: P.psa_debug_read_peak(buf, sink)) / 1e3) > 1e12
    assert flops * 4 / (best_ms(lambda: P.psa_debug_mfma_peak(out, 1024)) / 1e3) > 5e14



def test_issue_probe_runs():
    """Every issue-probe pattern runs, writes a positive cycle count for every
    wave, and the counts scale with the work (after a warm-up launch, four
    times the iterations take more than three times the cycles)."""
    import torch

    cyc = torch.full((1024,), -1, dtype=torch.int64, device="cuda")
    for pat in P.ISSUE_PATTERNS:
        log(f"case issue probe pattern {pat}")
        P.psa_debug_issue_probe(pat, cyc, 64)
        P.psa_debug_issue_probe(pat, cyc, 64)
        torch.cuda.synchronize()
        short = cyc.clone()
        P.psa_debug_issue_probe(pat, cyc, 256)
        torch.cuda.synchronize()
        assert bool((short > 0).all()) and bool((cyc > 0).all())
        assert float(cyc.double().median()) > 3 * float(short.double().median())


def test_workspace_must_hold_the_launching_plans_image():
    """A workspace overwritten by another plan's upload is refused before the
    launch; one overwritten outside the library (its image header no longer
    names the plan) makes the kernel write NaN into every output instead of
    reading a stale work list.  A fresh upload makes it valid again."""
    import torch

    wl = build_single_level("ws_id", 32, 8, 128, "bf16", [(200, 20, (0, 60))], (3, (1, 90)), seed=21)
    q, k, v = values(wl)
    cfg = P.make_config(32, 8, 128, wl.num_pages, "bf16")
    plan_a = P.psa_build_plan(cfg, wl.batch)
    plan_b = P.psa_build_plan(cfg, wl.batch, prefix_chunk_tokens=64)
    nbytes = max(plan_a.info()["workspace_bytes"], plan_b.info()["workspace_bytes"])
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    n = len(wl.batch["query_group"])
    out = torch.zeros(n, 32, 128, dtype=torch.float32, device="cuda")
    m = torch.zeros(n, 32, dtype=torch.float32, device="cuda")
    l = torch.zeros(n, 32, dtype=torch.float32, device="cuda")
    O, M, L = oracle_all(wl, wl.batch, q, k, v)
    log("case workspace identity: plan a, then plan b uploaded over it")
    P.psa_plan_upload(plan_a, ws)
    P.psa_decode_attention(plan_a, q, k, v, out, ws, m, l)
    torch.cuda.synchronize()
    assert_close(to_host64(out), O, "bf16", "plan a")
    P.psa_plan_upload(plan_b, ws)
    torch.cuda.synchronize()
    with pytest.raises(P.PsaError) as e:
        P.psa_decode_attention(plan_a, q, k, v, out, ws, m, l)
    assert "another plan" in str(e.value)
    log("case workspace identity: header overwritten outside the library")
    P.psa_plan_upload(plan_a, ws)
    torch.cuda.synchronize()
    ws[:8].zero_()
    P.psa_decode_attention(plan_a, q, k, v, out, ws, m, l)
    torch.cuda.synchronize()
    assert bool(torch.isnan(out).all()) and bool(torch.isnan(m).all()) and bool(torch.isnan(l).all())
    P.psa_plan_upload(plan_a, ws)
    P.psa_decode_attention(plan_a, q, k, v, out, ws, m, l)
    torch.cuda.synchronize()
    assert_close(to_host64(out), O, "bf16", "plan a after a fresh upload")
