"""Pins for the fp64 attention oracle (CPU only).

Each check ties the oracle to something other than itself: hand-computed
closed forms (tests/golden), a library routine on special cases (torch's
scaled_dot_product_attention in float64), and invariants of the mathematics
(Eq. 1 split-and-merge, permutation and shift invariance, GQA = MHA with
repeated KV).  The mutation tests at the end plant plausible mistakes in a
copy of the oracle and check that the pins catch each one.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from workloads import build_single_level, make_values

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hand_cases():
    with open(os.path.join(GOLDEN, "attention_hand_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _hand_cases(), ids=lambda c: c["name"])
def test_hand_cases(case):
    O, m, l = oracle.partial_attention(np.array(case["q"]), np.array(case["K"]), np.array(case["V"]), case["scale"])
    np.testing.assert_allclose(O, case["O"], atol=1e-9)
    np.testing.assert_allclose(m, case["m"], atol=1e-9)
    np.testing.assert_allclose(l, case["l"], atol=1e-9)
    if "split_at" in case:
        s = case["split_at"]
        K, V = np.array(case["K"]), np.array(case["V"])
        a = oracle.partial_attention(np.array(case["q"]), K[:s], V[:s], case["scale"])
        b = oracle.partial_attention(np.array(case["q"]), K[s:], V[s:], case["scale"])
        for part, exp in ((a, case["prefix_partial"]), (b, case["distinct_partial"])):
            np.testing.assert_allclose(part[0], exp["O"], atol=1e-12)
            np.testing.assert_allclose(part[1], exp["m"], atol=1e-12)
            np.testing.assert_allclose(part[2], exp["l"], atol=1e-12)
        merged = oracle.merge_partials(a, b)
        np.testing.assert_allclose(merged[0], case["O"], atol=1e-9)
        np.testing.assert_allclose(merged[2], case["l"], atol=1e-9)


def _random_workload(seed, hq=4, hkv=2, d=16, groups=((37, 3, (0, 40)), (16, 2, (5, 20))), ungrouped=(2, (1, 50))):
    wl = build_single_level("t", hq, hkv, d, "f32", list(groups), ungrouped, seed=seed, spare_pages=3)
    q, k, v = make_values(wl, "cpu", seed)
    return wl, q.double().numpy(), k.double().numpy(), v.double().numpy()


def _dense_context(wl, k, v, i, kvh):
    segs = oracle.query_context(wl.batch, i)
    K = np.concatenate([A.gather_segment(k, p, n, kvh, wl.page_size) for p, n in segs])
    V = np.concatenate([A.gather_segment(v, p, n, kvh, wl.page_size) for p, n in segs])
    return K, V


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_against_torch_sdpa_gqa(seed):
    """Special case reducing to a library routine: float64 SDPA with KV repeated r times."""
    wl, q, k, v = _random_workload(seed)
    O, M, L = oracle.decode_attention(q, k, v, wl.batch)
    r = wl.num_q_heads // wl.num_kv_heads
    for i in range(wl.num_queries):
        Ks, Vs = zip(*[_dense_context(wl, k, v, i, h) for h in range(wl.num_kv_heads)])
        Kt = torch.from_numpy(np.stack(Ks)).repeat_interleave(r, dim=0)  # [Hq, L, d]
        Vt = torch.from_numpy(np.stack(Vs)).repeat_interleave(r, dim=0)
        qt = torch.from_numpy(q[i])[:, None, :]  # [Hq, 1, d]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=1 / math.sqrt(wl.head_dim))
        np.testing.assert_allclose(O[i], ref[:, 0].numpy(), rtol=0, atol=1e-12)
        # m and l against their definitions via logsumexp from torch
        s = (Kt @ qt.transpose(1, 2))[:, :, 0] / math.sqrt(wl.head_dim)
        np.testing.assert_allclose(M[i], s.max(dim=1).values.numpy(), atol=1e-12)
        np.testing.assert_allclose(np.log(L[i]) + M[i], torch.logsumexp(s, dim=1).numpy(), atol=1e-12)


def test_paged_gather_matches_dense_scatter():
    """Scatter a dense context into shuffled pages and gather it back."""
    rng = np.random.default_rng(5)
    P, hkv, d = 16, 3, 8
    n = 53
    dense = rng.standard_normal((n, d))
    pages = rng.permutation(10)[:4]
    pool = rng.standard_normal((10, hkv, P, d))
    for t in range(n):
        pool[pages[t // P], 1, t % P] = dense[t]
    np.testing.assert_array_equal(A.gather_segment(pool, pages, n, 1, P), dense)
    assert A.gather_segment(pool, pages, 0, 1, P).shape == (0, d)


@pytest.mark.parametrize("seed", [0, 3])
def test_split_and_merge_equals_unsplit(seed):
    """BatchLLM §2.2 Eq. 1 at every split point, including mid-page, and in 3+ pieces."""
    rng = np.random.default_rng(seed)
    L, d, r = 45, 8, 3
    q = rng.standard_normal((r, d))
    K = rng.standard_normal((L, d))
    V = rng.standard_normal((L, d))
    sc = 0.37
    ref = oracle.partial_attention(q, K, V, sc)
    for s in range(1, L):
        a = oracle.partial_attention(q, K[:s], V[:s], sc)
        b = oracle.partial_attention(q, K[s:], V[s:], sc)
        got = oracle.merge_partials(a, b)
        for x, y in zip(got, ref):
            np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-12)
    cuts = [0, 7, 16, 17, 31, L]
    parts = [oracle.partial_attention(q, K[a:b], V[a:b], sc) for a, b in zip(cuts[:-1], cuts[1:])]
    got = oracle.merge_many(parts)
    for x, y in zip(got, ref):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-12)


def test_merge_commutative_associative_identity():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((2, 4))
    K = rng.standard_normal((30, 4)) * 3
    V = rng.standard_normal((30, 4))
    a, b, c = (oracle.partial_attention(q, K[s], V[s], 1.0) for s in (slice(0, 9), slice(9, 20), slice(20, 30)))
    ab, ba = oracle.merge_partials(a, b), oracle.merge_partials(b, a)
    for x, y in zip(ab, ba):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-13)
    l1 = oracle.merge_partials(oracle.merge_partials(a, b), c)
    l2 = oracle.merge_partials(a, oracle.merge_partials(b, c))
    for x, y in zip(l1, l2):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-12)
    empty = oracle.partial_attention(q, K[:0], V[:0], 1.0)
    assert np.all(empty[1] == -np.inf) and np.all(empty[2] == 0) and np.all(empty[0] == 0)
    for x, y in zip(oracle.merge_partials(a, empty), a):
        np.testing.assert_array_equal(x, y)
    for x, y in zip(oracle.merge_partials(empty, a), a):
        np.testing.assert_array_equal(x, y)
    ee = oracle.merge_partials(empty, empty)
    assert np.all(ee[2] == 0) and np.all(ee[1] == -np.inf) and np.all(ee[0] == 0)


def test_permutation_and_shift_invariance():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((3, 6))
    K = rng.standard_normal((25, 6))
    V = rng.standard_normal((25, 6))
    ref = oracle.partial_attention(q, K, V, 0.5)
    perm = rng.permutation(25)
    got = oracle.partial_attention(q, K[perm], V[perm], 0.5)
    for x, y in zip(got, ref):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-12)
    # adding the same vector to every key shifts each row's scores by a constant
    delta = rng.standard_normal(6)
    got = oracle.partial_attention(q, K + delta, V, 0.5)
    np.testing.assert_allclose(got[0], ref[0], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(got[1] - ref[1], 0.5 * (q @ delta), atol=1e-12)


def test_dominant_key_and_convexity():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((1, 8))
    K = rng.standard_normal((20, 8))
    V = rng.standard_normal((20, 8))
    K[13] = 60.0 * q[0]
    O, m, l = oracle.partial_attention(q, K, V, 1.0)
    np.testing.assert_allclose(O[0], V[13], atol=1e-12)
    np.testing.assert_allclose(l, 1.0, atol=1e-12)
    K = rng.standard_normal((20, 8))
    O, _, _ = oracle.partial_attention(q, K, V, 1.0)
    assert np.all(O[0] <= V.max(axis=0) + 1e-15) and np.all(O[0] >= V.min(axis=0) - 1e-15)


def test_gqa_equals_mha_with_repeated_kv():
    wl, q, k, v = _random_workload(4, hq=6, hkv=2)
    O, M, L = oracle.decode_attention(q, k, v, wl.batch)
    k3 = np.repeat(k, 3, axis=1)
    v3 = np.repeat(v, 3, axis=1)
    O2, M2, L2 = oracle.decode_attention(q, k3, v3, wl.batch)
    np.testing.assert_allclose(O, O2, atol=1e-13)
    np.testing.assert_allclose(M, M2, atol=1e-13)


def test_group_query_equals_concatenated_unshared_query():
    """A grouped query attends to prefix ++ distinct; writing its context as one
    unshared page table (CB blog's per-request paged_attention) gives the same
    result when the prefix ends on a page boundary."""
    wl, q, k, v = _random_workload(6, groups=((32, 3, (0, 40)),), ungrouped=(0, (1, 2)))
    b = wl.batch
    O, M, L = oracle.decode_attention(q, k, v, b)
    gp = list(b["group_pages"])
    qpages, qoff = [], [0]
    for i in range(wl.num_queries):
        qpages += gp + list(b["query_pages"][b["query_page_off"][i]:b["query_page_off"][i + 1]])
        qoff.append(len(qpages))
    flat = dict(b, query_group=np.full(wl.num_queries, -1, np.int32),
                query_distinct_len=b["query_distinct_len"] + 32,
                query_page_off=np.array(qoff), query_pages=np.array(qpages))
    O2, M2, L2 = oracle.decode_attention(q, k, v, flat)
    np.testing.assert_allclose(O, O2, atol=1e-13)
    np.testing.assert_allclose(L, L2, rtol=1e-13)


def test_rows_api_matches_full():
    wl, q, k, v = _random_workload(7)
    O, M, L = oracle.decode_attention(q, k, v, wl.batch)
    pairs = [(0, 0), (2, 3), (wl.num_queries - 1, 1)]
    O2, M2, L2 = oracle.decode_attention_rows(q, k, v, wl.batch, pairs)
    for j, (i, h) in enumerate(pairs):
        np.testing.assert_allclose(O2[j], O[i, h], rtol=0, atol=1e-14)
        np.testing.assert_allclose([M2[j], L2[j]], [M[i, h], L[i, h]], rtol=1e-14)


def test_empty_context_rejected():
    wl = build_single_level("t", 2, 1, 8, "f32", [], [0, 3])
    q, k, v = make_values(wl, "cpu", 0)
    with pytest.raises(ValueError):
        oracle.decode_attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), wl.batch)


# ---- planted mistakes: each must be caught by the pins above -------------

_ORIG_PARTIAL = A.partial_attention
_ORIG_MERGE = A.merge_partials


def _mutants():
    def no_scale(q, K, V, scale):
        return _ORIG_PARTIAL(q, K, V, 1.0)

    def no_max_shift(q, K, V, scale):
        O, m, l = _ORIG_PARTIAL(q, K, V, scale)
        return O, np.zeros_like(m), l * np.exp(m)

    def unnormalised(q, K, V, scale):
        O, m, l = _ORIG_PARTIAL(q, K, V, scale)
        return O * l[:, None], m, l

    def transposed_weights(q, K, V, scale):
        s = scale * (np.asarray(q, float) @ np.asarray(K, float).T)
        m = s.max(axis=1)
        p = np.exp(s - m[:, None])
        l = p.sum(axis=1)
        return (p @ np.asarray(V, float)) / l.sum(), m, l

    def drops_last_token(q, K, V, scale):
        return _ORIG_PARTIAL(q, K[:-1], V[:-1], scale) if len(K) > 1 else _ORIG_PARTIAL(q, K, V, scale)

    return [no_scale, no_max_shift, unnormalised, transposed_weights, drops_last_token]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_pins_catch_planted_mistakes(mutant, monkeypatch):
    monkeypatch.setattr(oracle, "partial_attention", mutant)
    monkeypatch.setattr(A, "partial_attention", mutant)
    failures = 0
    for case in _hand_cases():
        try:
            test_hand_cases(case)
        except AssertionError:
            failures += 1
    try:
        test_against_torch_sdpa_gqa(0)
    except AssertionError:
        failures += 1
    assert failures > 0, f"no pin caught mutant {mutant.__name__}"


def _merge_mutants():
    def no_l_weight(a, b):
        Oa, ma, la = a
        Ob, mb, lb = b
        m = np.maximum(ma, mb)
        wa, wb = np.exp(ma - m), np.exp(mb - m)
        l = la * wa + lb * wb
        return (wa[:, None] * Oa + wb[:, None] * Ob) / (wa + wb)[:, None], m, l

    def wrong_sign(a, b):
        Oa, ma, la = a
        Ob, mb, lb = b
        m = np.maximum(ma, mb)
        wa, wb = la * np.exp(m - ma), lb * np.exp(m - mb)
        l = wa + wb
        return (wa[:, None] * Oa + wb[:, None] * Ob) / l[:, None], m, l

    return [no_l_weight, wrong_sign]


@pytest.mark.parametrize("mutant", _merge_mutants(), ids=lambda f: f.__name__)
def test_merge_pins_catch_planted_mistakes(mutant, monkeypatch):
    monkeypatch.setattr(oracle, "merge_partials", mutant)
    monkeypatch.setattr(A, "merge_partials", mutant)
    caught = False
    try:
        test_split_and_merge_equals_unsplit(0)
    except AssertionError:
        caught = True
    assert caught


@pytest.mark.parametrize("seed", [0, 1])
def test_prefill_chunk_equals_causal_sdpa(seed):
    """A prefill chunk batched as a group with per-token prefix limits
    (query_prefix_len) equals the chunk rows of causal attention over the
    request's whole context: float64 SDPA with is_causal on the full token
    sequence (library routine), cut to the chunk's rows."""
    from workloads import build_mixed

    cached, chunk = 32 * (seed + 1), 21 + 7 * seed
    wl = build_mixed("pf", 8, 2, 64, "f32", [], [(cached, chunk)], seed=seed)
    q, k, v = make_values(wl, "cpu")
    q, k, v = q.double().numpy(), k.double().numpy(), v.double().numpy()
    O, _, _ = oracle.decode_attention(q, k, v, wl.batch)
    b = wl.batch
    total = cached + chunk
    pages = b["group_pages"][b["group_page_off"][0]: b["group_page_off"][1]]
    r = wl.num_q_heads // wl.num_kv_heads
    K = np.stack([A.gather_segment(k, pages, total, h, wl.page_size) for h in range(wl.num_kv_heads)])
    V = np.stack([A.gather_segment(v, pages, total, h, wl.page_size) for h in range(wl.num_kv_heads)])
    Kt = torch.from_numpy(K).repeat_interleave(r, dim=0)  # [Hq, total, d]
    Vt = torch.from_numpy(V).repeat_interleave(r, dim=0)
    # queries for the cached positions do not exist; give them zeros and keep only the chunk rows
    Q = np.zeros((wl.num_q_heads, total, wl.head_dim))
    Q[:, cached:] = q.transpose(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(Q), Kt, Vt, is_causal=True,
                                                           scale=1 / math.sqrt(wl.head_dim))
    np.testing.assert_allclose(O, ref[:, cached:].numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)
