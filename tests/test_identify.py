"""Prefix identification from token ids through the C ABI (host code, CPU):
against the oracle (a plain trie and the same DP objective) on seeded random
batches, a validity check of every returned group, and the error paths."""

import ctypes as C

import numpy as np
import pytest

import oracle
import prefix_shared_decode_amd as P
from prefix_shared_decode_amd import _lib as L


def check_groups(seqs, res):
    """Every group's members share its prefix; the saving is what it claims."""
    rg, gl, gf = res["request_group"], res["group_prefix_len"], res["group_first_request"]
    assert len(rg) == len(seqs) and len(gl) == len(gf)
    claimed = 0
    for g in range(len(gl)):
        members = np.nonzero(rg == g)[0]
        assert len(members) >= 2 and members[0] == gf[g]
        p = int(gl[g])
        assert p > 0
        ref = list(seqs[gf[g]][:p])
        for j in members:
            assert len(seqs[j]) >= p and list(seqs[j][:p]) == ref
        claimed += p * (len(members) - 1)
    assert claimed == res["saved_tokens"]


def random_batch(rng, n, alphabet, max_len, n_roots=0):
    seqs = []
    roots = [list(rng.integers(0, alphabet, size=int(rng.integers(1, max_len + 1)))) for _ in range(n_roots)]
    for _ in range(n):
        head = list(roots[int(rng.integers(0, n_roots))]) if n_roots else []
        seqs.append(head + list(rng.integers(0, alphabet, size=int(rng.integers(0, max_len + 1)))))
    if n >= 3 and rng.random() < 0.5:
        seqs[1] = list(seqs[0])
        seqs[2] = list(seqs[0][: len(seqs[0]) // 2])
    return seqs


@pytest.mark.parametrize("seed", range(60))
def test_identification_matches_oracle(seed):
    rng = np.random.default_rng(900 + seed)
    n = int(rng.integers(0, 60))
    seqs = random_batch(rng, n, int(rng.integers(1, 5)), int(rng.integers(1, 12)), int(rng.integers(0, 4)))
    res = P.psa_identify_prefix_groups(seqs)
    saving, _, _ = oracle.identify_groups(seqs)
    assert res["saved_tokens"] == saving
    check_groups(seqs, res)


def test_identification_two_level_shape():
    """4 roots x 16 sub-prefixes x 16 requests (the two-level workload's
    shape at 1/32 of its token counts): the best single level is each
    sub-prefix with its root, 64 groups of 16 saving (32 + 64) * 15 each."""
    rng = np.random.default_rng(3)
    seqs = []
    for r in range(4):
        root = [1000 + r] + list(rng.integers(0, 50, size=31))
        for s in range(16):
            sub = [2000 + s] + list(rng.integers(0, 50, size=63))
            for q in range(16):
                seqs.append(root + sub + [3000 + q] + list(rng.integers(0, 50, size=int(rng.integers(0, 8)))))
    res = P.psa_identify_prefix_groups(seqs)
    assert res["saved_tokens"] == 64 * 96 * 15 == oracle.identify_groups(seqs)[0]
    assert len(res["group_prefix_len"]) == 64 and set(res["group_prefix_len"].tolist()) == {96}
    check_groups(seqs, res)


def test_identification_error_paths():
    lib = L.lib()
    h = C.c_void_p()
    off = np.array([0, 2, 1], dtype=np.int64)
    tok = np.array([1, 2], dtype=np.int32)
    i64, i32 = C.POINTER(C.c_int64), C.POINTER(C.c_int32)
    assert lib.psa_identify_prefix_groups(2, off.ctypes.data_as(i64), tok.ctypes.data_as(i32), C.byref(h)) != 0
    assert b"non-decreasing" in lib.psa_last_error()
    off = np.array([1, 2], dtype=np.int64)
    assert lib.psa_identify_prefix_groups(1, off.ctypes.data_as(i64), tok.ctypes.data_as(i32), C.byref(h)) != 0
    assert lib.psa_identify_prefix_groups(-1, off.ctypes.data_as(i64), tok.ctypes.data_as(i32), C.byref(h)) != 0
    assert lib.psa_identify_prefix_groups(1, None, tok.ctypes.data_as(i32), C.byref(h)) != 0
    off = np.array([0, 2], dtype=np.int64)
    assert lib.psa_identify_prefix_groups(1, off.ctypes.data_as(i64), None, C.byref(h)) != 0
    assert lib.psa_identify_prefix_groups(1, off.ctypes.data_as(i64), tok.ctypes.data_as(i32), None) != 0
    assert lib.psa_prefix_groups_view(None, None, None, None, None, None) != 0
    lib.psa_free_prefix_groups(None)


def test_identification_industrial_shape_closed_form():
    """8000 prompts: a common 50-token system prompt, documents shared by 3
    requests.  The best single level is the documents (with the system
    prompt): saving = sum over documents of (common prefix) * (requests - 1),
    the common prefix being the documents' requests' shortest pairwise
    common prefix."""
    from workloads import build_token_batch

    seqs = build_token_batch()
    res = P.psa_identify_prefix_groups(seqs)

    def lcp(a, b):
        m = min(len(a), len(b))
        d = np.nonzero(a[:m] != b[:m])[0]
        return int(d[0]) if len(d) else m

    want = 0
    for i in range(0, len(seqs), 3):
        grp = seqs[i:i + 3]
        if len(grp) >= 2:
            want += min(lcp(grp[0], x) for x in grp[1:]) * (len(grp) - 1)
    assert res["saved_tokens"] == want
    assert len(res["group_prefix_len"]) == -(-len(seqs) // 3)
