"""The structural work counts used by the benchmark's roofline figures equal the
per-level candidate and scored counts the oracle records while routing."""
import numpy as np
import pytest

import oracle
from hierarchical_top_amd import workcount


@pytest.mark.parametrize("N,C,g,K_top", [(1024, 16, 2, 4), (1000, 16, 4, 8), (4096, 16, 4, 8), (3000, 32, 2, 6),
                                         (1024, 16, 2, 32), (700, 16, 8, 5)])
def test_walk_equals_oracle_trace(N, C, g, K_top):
    rng = np.random.default_rng(N + C + g + K_top)
    d = 8
    K = rng.standard_normal((1, N, 1, d)).astype(np.float32)
    Q = rng.standard_normal((N, 1, d)).astype(np.float32)
    t = np.arange(N)
    pyr = oracle.Pyramid(K, N, C, g)
    r = oracle.route(pyr, Q, [0] * N, t, K_top, causal=True, trace=True)
    s = workcount.walk(t, N, C, g, K_top)
    assert workcount.levels(N, C, g) == pyr.M
    for l in range(1, pyr.L + 1):
        np.testing.assert_array_equal(s[l], r["trace"][:, 0, l, 1], err_msg="level %d" % l)


def test_totals_at_the_large_shapes():
    # 256K: 16 query heads on 4 KV heads, d=128, C=64, g=4, K_top=8
    r = workcount.route_work(1, 262144, 4, 4, 128, 64, 4, 8)
    assert r["upper_mac"] == 173577076736 and r["leaf_mac"] == 941034045440
    b = workcount.bsa_work(1, 262144, 4, 4, 128, 64, 8)
    assert abs(b["mac"] / 1e12 - 1.098) < 1e-3
    a = workcount.attn_work(1, 65536, 32, 128, 64, 8)
    assert abs(a["mac"] / 1e12 - 0.257) < 1e-3


def test_decode_walk_matches_oracle_at_the_level_boundary():
    rng = np.random.default_rng(3)
    C, g, K_top, d = 16, 4, 8, 8
    for n in (1024, 1025, 1040, 1041, 3000):
        K = rng.standard_normal((1, n, 1, d)).astype(np.float32)
        q = rng.standard_normal((1, 1, d)).astype(np.float32)
        pyr = oracle.Pyramid(K, n, C, g)
        r = oracle.route(pyr, q, [0], [n - 1], K_top, trace=True)
        s = workcount.walk([n - 1], n, C, g, K_top)
        for l in range(1, pyr.L + 1):
            assert s[l][0] == r["trace"][0, 0, l, 1]
