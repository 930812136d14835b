"""The worker-process runner of the oracle (tests/oracle_pool.py) returns
exactly what one direct oracle call returns: it only splits the queries into
batches, renumbers their pages and widens the raw inputs exactly."""

import numpy as np

import oracle
from workloads import build_mixed, build_single_level, make_values

from oracle_pool import oracle_full


def test_pool_equals_direct_oracle_bf16():
    wl = build_single_level("pool", 8, 2, 64, "bf16", [(100, 6, (0, 40)), (37, 3, (1, 20))], (3, (1, 50)), seed=4)
    q, k, v = make_values(wl, "cpu")
    O, M, L = oracle_full(wl.batch, q, k, v, 4, workers=2, what="pool bf16")
    O2, M2, L2 = oracle.decode_attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), wl.batch)
    assert np.array_equal(O, O2) and np.array_equal(M, M2) and np.array_equal(L, L2)


def test_pool_equals_direct_oracle_fp32_limits_scale():
    wl = build_mixed("pool_mixed", 8, 2, 64, "f32", [(64, 3, (1, 30))], [(32, 16)], seed=2)
    q, k, v = make_values(wl, "cpu")
    O, M, L = oracle_full(wl.batch, q, k, v, 5, scale=0.3, workers=2, what="pool fp32")
    O2, M2, L2 = oracle.decode_attention(q.numpy(), k.numpy(), v.numpy(), wl.batch, scale=0.3)
    assert np.array_equal(O, O2) and np.array_equal(M, M2) and np.array_equal(L, L2)
