"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks the oracle (oracle/pisa_oracle.c) against one of:
  * closed forms worked by hand from the definitions (tests/golden/hand_examples.json);
  * special cases that reduce to a library routine (scipy logsumexp / softmax,
    torch scaled_dot_product_attention, numpy means over raw keys);
  * invariants the method guarantees (bounds of eq 19-20, forced set of
    appendix B, the Jensen sandwich of appendix A.1, causality).
All citations refer to "Block Sparse Attention with Log-Linear Complexity".
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))
e = math.e


def ev(expr):
    return float(eval(expr, {"math": math, "e": e}))


def _w1_pyr():
    w = GOLD["w1"]
    K = np.array(w["keys"], np.float32).reshape(1, w["N"], 1, w["d"])
    return oracle.Pyramid(K, w["N"], w["C"], w["g"]), np.array(w["q"], np.float32)


# --------------------------------------------------------------------------
# Hand-worked closed forms (section 3.2, section 3.1, appendix B, appendix A.1)
# --------------------------------------------------------------------------

def test_w1_levels_and_summaries():
    w = GOLD["w1"]
    pyr, _ = _w1_pyr()
    assert pyr.M == w["levels"]
    for l, vals in w["summaries"].items():
        got = pyr.level(int(l)).ravel()
        np.testing.assert_allclose(got, [ev(v) for v in vals], rtol=0, atol=1e-15)


def test_w1_scores():
    pyr, q = _w1_pyr()
    for s in GOLD["w1"]["scores"]:
        got = oracle.score(pyr, q, 0, 0, s["level"], s["node"])
        assert got == pytest.approx(ev(s["value"]), abs=1e-13)


def test_w1_noncausal_routes_and_exhaustive_miss():
    pyr, q = _w1_pyr()
    for case in GOLD["w1"]["noncausal_routes"]:
        r = oracle.route(pyr, q.reshape(1, 1, 1), [0], [case["t"]], case["K_top"], causal=False)
        assert r["idx"][0, 0].tolist() == case["idx"]
        np.testing.assert_allclose(r["score"][0, 0], [ev(x) for x in case["score"]], atol=1e-13)
    b = oracle.bsa(pyr, q.reshape(1, 1, 1), [0], [7], 1, causal=False)
    assert b["idx"][0, 0].tolist() == GOLD["w1"]["exhaustive_k1"]


def test_w2_forced_policy():
    w = GOLD["w2"]
    K = np.array(w["keys"], np.float32).reshape(1, w["N"], 1, w["d"])
    pyr = oracle.Pyramid(K, w["N"], w["C"], w["g"])
    q = np.array(w["q"], np.float32).reshape(1, 1, 1)
    for case in w["causal_routes"]:
        r = oracle.route(pyr, q, [0], [case["t"]], case["K_top"], causal=True)
        assert r["idx"][0, 0].tolist() == case["idx"], case["note"]
        kept = [s for i, s in zip(r["idx"][0, 0], r["score"][0, 0]) if i >= 0]
        assert all(math.isinf(s) and s > 0 for s in kept)


def test_w3_jensen_equality_case():
    pyr, q = _w1_pyr()
    for n in GOLD["w3"]["nodes"]:
        s = oracle.score(pyr, q, 0, 0, n["level"], n["node"])
        F_hat = s - math.log(2)
        assert F_hat == pytest.approx(ev(n["F_hat"]), abs=1e-13)
        assert ev(n["mean_logit"]) <= F_hat + 1e-13 <= ev(n["F_q"]) + 2e-13


@pytest.mark.parametrize("case", GOLD["walks"]["cases"], ids=lambda c: "N%d" % c["N"])
def test_structural_walk(case):
    rng = np.random.default_rng(7)
    N, C, g, Kt = case["N"], case["C"], case["g"], case["K_top"]
    d, H = 16, 1
    K = rng.standard_normal((1, N, H, d)).astype(np.float32)
    Q = rng.standard_normal((1, H, d)).astype(np.float32)
    pyr = oracle.Pyramid(K, N, C, g)
    r = oracle.route(pyr, Q, [0], [case["t"]], Kt, causal=True, trace=True)
    for l, (nA, ns) in case["per_level"].items():
        assert r["trace"][0, 0, int(l)].tolist() == [nA, ns], "level %s" % l


# --------------------------------------------------------------------------
# Pyramid: closed forms on perfect trees, the unweighted tail rule (eq 15)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("C,g,k", [(4, 2, 5), (16, 4, 3), (8, 3, 3)])
def test_perfect_tree_summaries_are_raw_means(C, g, k):
    rng = np.random.default_rng(1)
    N, H, d = C * g ** k, 2, 5
    K = rng.standard_normal((2, N, H, d)).astype(np.float32)
    pyr = oracle.Pyramid(K, N, C, g)
    assert pyr.L == k + 1
    for l in range(1, pyr.L + 1):
        span = C * g ** (l - 1)
        lev = pyr.level(l)
        for i in range(pyr.M[l]):
            want = K[:, i * span:(i + 1) * span].astype(np.float64).mean(axis=1)  # [B][H][d]
            np.testing.assert_allclose(lev[:, :, i], want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("g", [2, 4])
def test_imperfect_tree_tail_is_unweighted(g):
    rng = np.random.default_rng(2)
    N, C, d = 1000, 16, 3
    K = rng.standard_normal((1, N, 1, d)).astype(np.float32)
    Kd = K[0, :, 0].astype(np.float64)
    pyr = oracle.Pyramid(K, N, C, g)
    M = pyr.M
    assert M[1] == 63  # leaf 62 holds tokens 992..999
    leaf = lambda i: Kd[i * C:min(i * C + C, N)].mean(axis=0)
    np.testing.assert_allclose(pyr.level(1)[0, 0, 62], leaf(62), atol=1e-14)
    # the last level-2 node: unweighted mean of its existing children
    last2 = M[2] - 1
    kids = [leaf(r) for r in range(last2 * g, min(last2 * g + g, M[1]))]
    np.testing.assert_allclose(pyr.level(2)[0, 0, last2], np.mean(kids, axis=0), atol=1e-14)
    # ... which is not the token-weighted mean of its span when children differ in size
    tok_mean = Kd[last2 * g * C:N].mean(axis=0)
    if len(kids) > 1:
        assert np.abs(pyr.level(2)[0, 0, last2] - tok_mean).max() > 1e-3
    # the level-3 tail node: mean of level-2 children, each already a mean of leaves
    last3 = M[3] - 1
    l2 = [pyr.level(2)[0, 0, r] for r in range(last3 * g, min(last3 * g + g, M[2]))]
    full2 = [np.mean([leaf(x) for x in range(r * g, min(r * g + g, M[1]))], axis=0)
             for r in range(last3 * g, min(last3 * g + g, M[2]))]
    np.testing.assert_allclose(l2, full2, atol=1e-14)
    np.testing.assert_allclose(pyr.level(3)[0, 0, last3], np.mean(full2, axis=0), atol=1e-14)


def test_level_sizes():
    for N, C, g in [(1, 16, 2), (16, 16, 2), (17, 16, 2), (1000, 16, 4), (262144, 64, 4),
                    (262145, 64, 4), (5, 2, 3)]:
        M = oracle.levels(N, C, g)
        assert M[0] == N and M[1] == -(-N // C) and M[-1] == 1
        for l in range(1, len(M) - 1):
            assert M[l + 1] == -(-M[l] // g) and M[l] > 1
    assert oracle.levels(262144, 64, 4) == [262144, 4096, 1024, 256, 64, 16, 4, 1]
    assert len(oracle.levels(262145, 64, 4)) - 1 == 8


# --------------------------------------------------------------------------
# Scores reduce to scipy's logsumexp (eq 21) and sum over heads (eq 22)
# --------------------------------------------------------------------------

def test_scores_match_library_logsumexp():
    rng = np.random.default_rng(3)
    N, C, g, d, H = 300, 16, 4, 8, 2
    K = rng.standard_normal((1, N, H, d)).astype(np.float32)
    q = rng.standard_normal(d).astype(np.float32)
    pyr = oracle.Pyramid(K, N, C, g)
    for h in range(H):
        Kh = K[0, :, h].astype(np.float64)
        for i in range(pyr.M[1]):
            z = Kh[i * C:min(i * C + C, N)] @ q.astype(np.float64) / math.sqrt(d)
            assert oracle.score(pyr, q, 0, h, 1, i) == pytest.approx(logsumexp(z), abs=1e-12)
        for l in range(2, pyr.L + 1):
            for i in range(pyr.M[l]):
                kids = pyr.level(l - 1)[0, h, i * g:min(i * g + g, pyr.M[l - 1])]
                z = kids @ q.astype(np.float64) / math.sqrt(d)
                assert oracle.score(pyr, q, 0, h, l, i) == pytest.approx(logsumexp(z), abs=1e-12)


def test_group_scores_are_sums_of_head_scores():
    rng = np.random.default_rng(4)
    N, C, g, d, Hq = 512, 16, 2, 8, 3
    K = rng.standard_normal((1, N, 1, d)).astype(np.float32)
    Q = rng.standard_normal((5, Hq, d)).astype(np.float32)
    t = np.array([511, 400, 300, 200, 100])
    pyr = oracle.Pyramid(K, N, C, g)
    r = oracle.route(pyr, Q, [0] * 5, t, 4, causal=True)
    checked = 0
    for n in range(5):
        for i, s in zip(r["idx"][n, 0], r["score"][n, 0]):
            if i >= 0 and np.isfinite(s):
                want = sum(oracle.score(pyr, Q[n, j], 0, 0, 1, int(i)) for j in range(Hq))
                assert s == pytest.approx(want, abs=1e-12)
                checked += 1
    assert checked > 0


# --------------------------------------------------------------------------
# Reductions to brute force (section 3.2: a level with at most K candidates is
# kept whole, so K_top >= M_2 turns PISA into exhaustive leaf LSE selection)
# --------------------------------------------------------------------------

# numpy's routines for the three block scores of section 4.4 (eq 50-52): np.var is the
# population variance (ddof=0), as eq 44 defines it
REDUCERS = {"lse": logsumexp, "mean": np.mean, "mean_var": lambda z: np.mean(z) + 0.5 * np.var(z)}


def exhaustive_lse(K, Q, t, C, Kt, causal=True, kind="lse"):
    """Brute force: score every eligible non-forced leaf by the summed raw-key score
    (LSE, or the PISA-1 / PISA-2 reductions of the same logits)."""
    red = REDUCERS[kind]
    N, H, d = K.shape[1], K.shape[2], K.shape[3]
    Hq = Q.shape[1]
    G = Hq // H
    M1 = -(-N // C)
    out = []
    for n, tt in enumerate(t):
        c = tt // C
        row = []
        for h in range(H):
            elig = list(range(c + 1)) if causal else list(range(M1))
            F = sorted({0, c} | ({c - 1} if c >= 1 else set())) if causal else []
            if len(elig) <= Kt:
                row.append(sorted(elig))
                continue
            S = [i for i in elig if i not in F]
            u = []
            for i in S:
                Kb = K[0, i * C:min(i * C + C, N), h].astype(np.float64)
                u.append(sum(red(Kb @ Q[n, h * G + j].astype(np.float64) / math.sqrt(d))
                             for j in range(G)))
            order = sorted(range(len(S)), key=lambda k: (-u[k], S[k]))
            row.append(sorted(F + [S[k] for k in order[:Kt - len(F)]]))
        out.append(row)
    return out


@pytest.mark.parametrize("Kt", [32, 64])
def test_reduction_to_exhaustive_on_tiny(Kt):
    rng = np.random.default_rng(5)
    N, C, g, d = 1024, 16, 2, 64
    K = rng.standard_normal((1, N, 1, d)).astype(np.float32)
    Q = rng.standard_normal((N, 1, d)).astype(np.float32)
    pyr = oracle.Pyramid(K, N, C, g)
    t = np.arange(0, N, 7)
    r = oracle.route(pyr, Q[t], [0] * len(t), t, Kt, causal=True, trace=True)
    want = exhaustive_lse(K, Q[t], t, C, Kt)
    for n in range(len(t)):
        got = [int(x) for x in r["idx"][n, 0] if x >= 0]
        assert got == want[n][0], "t=%d" % t[n]
        assert len(got) == min(Kt, t[n] // C + 1)
    if Kt == 64:
        assert r["trace"][..., 1].sum() == 0  # nothing is ever scored
    else:
        assert r["trace"][:, 0, 2:, 1].sum() == 0 and r["trace"][-1, 0, 1].tolist() == [64, 61]


@pytest.mark.parametrize("kind", ["lse", "mean", "mean_var"])
def test_reduction_to_exhaustive_grouped_noncausal(kind):
    rng = np.random.default_rng(6)
    N, C, g, d, H, Hq = 200, 8, 4, 8, 2, 4
    K = rng.standard_normal((1, N, H, d)).astype(np.float32)
    Q = rng.standard_normal((10, Hq, d)).astype(np.float32)
    pyr = oracle.Pyramid(K, N, C, g)
    Kt = pyr.M[2]  # every level above the leaves is kept whole
    t = np.arange(10) * 19
    r = oracle.route(pyr, Q, [0] * 10, t, Kt, causal=False, score_kind=kind)
    want = exhaustive_lse(K, Q, t, C, Kt, causal=False, kind=kind)
    for n in range(10):
        for h in range(H):
            assert [int(x) for x in r["idx"][n, h] if x >= 0] == want[n][h]


# --------------------------------------------------------------------------
# Invariants: budget and candidate bounds (eq 19-20), forced set and causality
# (appendix B), the Jensen sandwich (appendix A.1 eq 39)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("N,C,g,Kt", [(1000, 16, 2, 4), (1000, 16, 4, 4), (4096, 16, 4, 8)])
def test_budget_forced_and_causal(N, C, g, Kt):
    rng = np.random.default_rng(8)
    d = 16
    K = rng.standard_normal((1, N, 1, d)).astype(np.float32)
    t = np.arange(N)
    Q = rng.standard_normal((N, 1, d)).astype(np.float32)
    pyr = oracle.Pyramid(K, N, C, g)
    r = oracle.route(pyr, Q, [0] * N, t, Kt, causal=True, trace=True)
    for n in range(N):
        c = t[n] // C
        got = [int(x) for x in r["idx"][n, 0] if x >= 0]
        assert len(got) == min(Kt, c + 1) and len(set(got)) == len(got)
        assert got == sorted(got) and all(x <= c for x in got)
        assert {0, c} | ({c - 1} if c >= 1 else set()) <= set(got)
        assert (r["idx"][n, 0][len(got):] == -1).all()
    assert (r["trace"][..., 0] <= g * Kt).all()


def test_jensen_sandwich_on_random_perfect_tree():
    rng = np.random.default_rng(9)
    C, g, k, d = 4, 2, 6, 8
    N = C * g ** k
    K = rng.standard_normal((1, N, 1, d)).astype(np.float32)
    Kd = K[0, :, 0].astype(np.float64)
    pyr = oracle.Pyramid(K, N, C, g)
    for trial in range(4):
        q = rng.standard_normal(d).astype(np.float32)
        qd = q.astype(np.float64)
        for l in range(2, pyr.L + 1):
            span, cspan = C * g ** (l - 1), C * g ** (l - 2)
            for i in range(pyr.M[l]):
                m = [Kd[(i * g + j) * cspan:(i * g + j + 1) * cspan].mean(0) @ qd / math.sqrt(d)
                     for j in range(g)]
                F_hat = oracle.score(pyr, q, 0, 0, l, i) - math.log(g)
                F_q = logsumexp(Kd[i * span:(i + 1) * span] @ qd / math.sqrt(d)) - math.log(span)
                assert np.mean(m) <= F_hat + 1e-12
                assert F_hat <= F_q + 1e-12
                assert F_hat == pytest.approx(logsumexp(m) - math.log(g), abs=1e-12)


def test_planted_block_is_found():
    """A past leaf whose keys all equal beta * q / |q| with beta |q| / sqrt(d) = 40 wins
    at every level (its share of each ancestor summary stays far above the noise)."""
    rng = np.random.default_rng(10)
    N, C, g, d, Kt = 1024, 16, 2, 64, 4
    for t, j in [(1023, 5), (900, 30), (700, 1), (500, 17)]:
        K = rng.standard_normal((1, N, 1, d)).astype(np.float32)
        q = rng.standard_normal(d).astype(np.float32)
        for sign in (+1, -1):
            Kp = K.copy()
            beta = 40 * math.sqrt(d) / np.linalg.norm(q)
            Kp[0, j * C:(j + 1) * C, 0] = sign * beta * q / np.linalg.norm(q)
            pyr = oracle.Pyramid(Kp, N, C, g)
            r = oracle.route(pyr, q.reshape(1, 1, d), [0], [t], Kt, causal=True)
            assert (j in r["idx"][0, 0]) == (sign > 0 or j == 0)


def test_decode_route_equals_prefix_route():
    """Routing the last token of a length-n prefix equals routing position n-1 inside a
    longer sequence: every node the query ranks lies in its past (appendix B)."""
    rng = np.random.default_rng(11)
    N, C, g, d, Hq = 2048, 16, 4, 16, 2
    K = rng.standard_normal((1, N, 1, d)).astype(np.float32)
    Q = rng.standard_normal((N, Hq, d)).astype(np.float32)
    full = oracle.Pyramid(K, N, C, g)
    ns = [1, 2, 16, 17, 63, 64, 65, 255, 256, 257, 1024, 1025, 2000, 2048]
    r_full = oracle.route(full, Q[np.array(ns) - 1], [0] * len(ns), np.array(ns) - 1, 8, causal=True)
    for k, n in enumerate(ns):
        pre = oracle.Pyramid(K[:, :n].copy(), n, C, g)
        r = oracle.route(pre, Q[n - 1:n], [0], [n - 1], 8, causal=True)
        assert r["idx"][0].tolist() == r_full["idx"][k].tolist(), "n=%d" % n


def test_head_permutation_symmetry():
    rng = np.random.default_rng(12)
    N, C, g, d = 1024, 16, 2, 16
    K = rng.standard_normal((1, N, 1, d)).astype(np.float32)
    Q = rng.standard_normal((64, 4, d)).astype(np.float32)
    t = np.arange(64) * 16
    pyr = oracle.Pyramid(K, N, C, g)
    a = oracle.route(pyr, Q, [0] * 64, t, 4)
    b = oracle.route(pyr, Q[:, [2, 0, 3, 1]], [0] * 64, t, 4)
    assert (a["idx"] == b["idx"]).all()
    np.testing.assert_allclose(a["score"], b["score"], atol=1e-12)


def test_single_head_groups_route_independently():
    rng = np.random.default_rng(13)
    N, C, g, d = 512, 16, 2, 16
    K = rng.standard_normal((1, N, 2, d)).astype(np.float32)
    Q = rng.standard_normal((32, 2, d)).astype(np.float32)
    t = np.arange(32) * 16 + 3
    both = oracle.route(oracle.Pyramid(K, N, C, g), Q, [0] * 32, t, 4)
    for h in range(2):
        one = oracle.route(oracle.Pyramid(K[:, :, h:h + 1].copy(), N, C, g), Q[:, h:h + 1],
                           [0] * 32, t, 4)
        assert (one["idx"][:, 0] == both["idx"][:, h]).all()


# --------------------------------------------------------------------------
# Exhaustive selector against scipy softmax (section 3.1, appendix C's per-head
# normalisation), attention against torch SDPA (eq 6)
# --------------------------------------------------------------------------

def test_bsa_matches_library_softmax():
    rng = np.random.default_rng(14)
    N, C, g, d, H, Hq, Kt = 640, 16, 2, 16, 2, 4, 5
    K = rng.standard_normal((1, N, H, d)).astype(np.float32)
    Q = rng.standard_normal((40, Hq, d)).astype(np.float32)
    t = np.arange(40) * 16 + 5
    pyr = oracle.Pyramid(K, N, C, g)
    r = oracle.bsa(pyr, Q, [0] * 40, t, Kt)
    G = Hq // H
    for n in range(40):
        c = t[n] // C
        for h in range(H):
            means = np.stack([K[0, i * C:(i + 1) * C, h].astype(np.float64).mean(0)
                              for i in range(c + 1)])
            F = sorted({0, c} | ({c - 1} if c >= 1 else set()))
            if c + 1 <= Kt:
                want = list(range(c + 1))
            else:
                S = [i for i in range(c + 1) if i not in F]
                u = sum(softmax(means[S] @ Q[n, h * G + j].astype(np.float64) / math.sqrt(d))
                        for j in range(G))
                order = sorted(range(len(S)), key=lambda k: (-u[k], S[k]))
                want = sorted(F + [S[k] for k in order[:Kt - len(F)]])
                np.testing.assert_allclose(np.sort(u)[::-1][:Kt - len(F)],
                                           np.sort(r["score"][n, h][np.isfinite(r["score"][n, h])])[::-1],
                                           atol=1e-12)
            assert [int(x) for x in r["idx"][n, h] if x >= 0] == want


def test_bsa_two_heads_per_head_normalisation():
    """Two query heads whose unnormalised scores favour leaf 1 while the per-head softmax,
    summed, favours leaf 0 (closed form in tests/golden): the normalisation is per head."""
    w = GOLD["bsa_two_heads"]
    K = np.array(w["keys"], np.float32).reshape(1, w["N"], 1, w["d"])
    pyr = oracle.Pyramid(K, w["N"], w["C"], w["g"])
    q = np.array(w["q"], np.float32).reshape(1, 2, w["d"])
    u = oracle.bsa_scores(pyr, q, [0], [w["N"] - 1], 1, causal=False)[0, 0]
    np.testing.assert_allclose(u, [ev(x) for x in w["u"]], rtol=0, atol=1e-14)
    for pick in w["picks"]:
        r = oracle.bsa(pyr, q, [0], [w["N"] - 1], pick["K_top"], causal=False)
        assert [int(x) for x in r["idx"][0, 0] if x >= 0] == pick["idx"]
        kept = r["score"][0, 0][:len(pick["idx"])]
        np.testing.assert_allclose(kept, [ev(w["u"][i]) for i in pick["idx"]], rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_bsa_probabilities_sum_to_group_size(causal):
    """Each head's softmax over the scored leaves sums to one, so the grouped scores of one
    (query, KV head) sum to G_Q over the scored set; forced leaves carry +inf, future -inf."""
    rng = np.random.default_rng(16)
    N, C, g, d, H, Hq, Kt = 700, 16, 4, 16, 2, 6, 5
    K = rng.standard_normal((1, N, H, d)).astype(np.float32)
    Q = (2.0 * rng.standard_normal((30, Hq, d))).astype(np.float32)
    t = np.linspace(0, N - 1, 30).astype(np.int64)
    pyr = oracle.Pyramid(K, N, C, g)
    u = oracle.bsa_scores(pyr, Q, [0] * 30, t, Kt, causal=causal)
    M1 = pyr.M[1]
    for n in range(30):
        c = t[n] // C if causal else M1 - 1
        E = c + 1
        for h in range(H):
            row = u[n, h]
            assert np.isneginf(row[E:]).all()
            if E <= Kt:
                assert np.isposinf(row[:E]).all()
                continue
            F = sorted({0, c, c - 1}) if causal else []
            assert np.isposinf(row[F]).all() and np.isfinite(np.delete(row[:E], F)).all()
            assert np.delete(row[:E], F).sum() == pytest.approx(Hq // H, abs=1e-12)


# --------------------------------------------------------------------------
# Tie-resolution reachability (the checker behind the near-tie parity protocol)
# --------------------------------------------------------------------------

def test_w1_tie_resolution_costs():
    w = GOLD["w1_tie_resolutions"]
    pyr, q = _w1_pyr()
    qi = q.reshape(1, 1, 1)
    for tgt in w["targets"]:
        eps = oracle.route_reach(pyr, qi, [0], [w["t"]], [0], np.array([tgt["idx"]]), w["K_top"],
                                 causal=False, cap=10.0)
        assert eps[0] == pytest.approx(ev(tgt["cost"]), abs=1e-13), tgt["note"]
        cost = ev(tgt["cost"])
        if cost > 0:  # a cap below the cost rules the resolution out
            eps = oracle.route_reach(pyr, qi, [0], [w["t"]], [0], np.array([tgt["idx"]]), w["K_top"],
                                     causal=False, cap=cost * 0.99)
            assert np.isposinf(eps[0])
    for bad in w["unreachable"]:
        eps = oracle.route_reach(pyr, qi, [0], [w["t"]], [0], np.array([bad]), w["K_top"], causal=False,
                                 cap=10.0)
        assert np.isposinf(eps[0]), w["unreachable_note"]


def _brute_force_paths(pyr, q_heads, h, t, Kt, causal):
    """Every kept leaf set reachable by keeping ANY K_top - |F| of the non-forced candidates
    at each ranked level (no pruning), with the smallest path cost: the largest, over the
    ranked levels, of max(0, best dropped score - worst kept score)."""
    C, g, M = pyr.C, pyr.g, pyr.M
    c = t // C
    memo = {}

    def u(l, i):
        if (l, i) not in memo:
            memo[(l, i)] = sum(oracle.score(pyr, q, 0, h, l, i) for q in q_heads)
        return memo[(l, i)]

    out = {}

    def rec(l, A, cost):
        span = C * g ** (l - 1)
        if causal:
            A = [i for i in A if i * span <= t]
        if len(A) <= Kt:
            choices = [(list(A), 0.0)]
        else:
            den = span // C
            F = sorted({0, c // den} | ({(c - 1) // den} if c >= 1 else set())) if causal else []
            R = [i for i in A if i not in F]
            choices = []
            for S in itertools.combinations(R, Kt - len(F)):
                dropped = [u(l, i) for i in R if i not in S]
                cl = max(0.0, max(dropped) - min(u(l, i) for i in S)) if S else 0.0
                choices.append((F + list(S), cl))
        for I, cl in choices:
            nc = max(cost, cl)
            if l == 1:
                key = tuple(sorted(I))
                out[key] = min(out.get(key, math.inf), nc)
            else:
                rec(l - 1, sorted(r for i in I for r in range(i * g, min(i * g + g, M[l - 1]))), nc)

    rec(pyr.L, [0], 0.0)
    return out


@pytest.mark.parametrize("N,C,g,Kt,causal", [(64, 8, 2, 2, False), (128, 8, 2, 4, True), (100, 4, 3, 4, True)])
def test_reach_matches_brute_force(N, C, g, Kt, causal):
    """On trees small enough to enumerate every path, the checker's smallest cost for each
    reachable leaf set equals the brute-force minimum, a cap just below it rules the set
    out, and sets that no path reaches get +inf."""
    rng = np.random.default_rng(17 + N)
    d, H, Hq = 8, 1, 2
    K = (0.5 * rng.standard_normal((1, N, H, d))).astype(np.float32)
    pyr = oracle.Pyramid(K, N, C, g)
    M1 = pyr.M[1]
    checked = 0
    for t in ([N - 1, N // 2, 3 * C + 1] if causal else [N - 1]):
        q = rng.standard_normal((1, Hq, d)).astype(np.float32)
        paths = _brute_force_paths(pyr, list(q[0]), 0, t, Kt, causal)
        sets = list(paths)
        tg = np.full((len(sets), Kt), -1, np.int32)
        for k, s in enumerate(sets):
            tg[k, :len(s)] = s
        eps = oracle.route_reach(pyr, np.repeat(q, len(sets), 0), [0] * len(sets), [t] * len(sets),
                                 [0] * len(sets), tg, Kt, causal=causal, cap=1e9)
        np.testing.assert_allclose(eps, [paths[s] for s in sets], rtol=0, atol=1e-12)
        r = oracle.route(pyr, q, [0], [t], Kt, causal=causal)
        assert paths[tuple(int(x) for x in r["idx"][0, 0] if x >= 0)] == 0.0
        pos = [k for k, s in enumerate(sets) if paths[s] > 0]
        if pos:
            sub = tg[pos]
            eps2 = oracle.route_reach(pyr, np.repeat(q, len(pos), 0), [0] * len(pos), [t] * len(pos),
                                      [0] * len(pos), sub, Kt, causal=causal,
                                      cap=0.999 * min(paths[sets[k]] for k in pos))
            assert np.isposinf(eps2).all()
        # leaf sets of the right size that no path reaches
        E = min(M1, t // C + 1) if causal else M1
        extra = [s for s in itertools.combinations(range(E), min(Kt, E)) if s not in paths][:40]
        if extra:
            tg3 = np.array([list(s) + [-1] * (Kt - len(s)) for s in extra], np.int32)
            eps3 = oracle.route_reach(pyr, np.repeat(q, len(extra), 0), [0] * len(extra), [t] * len(extra),
                                      [0] * len(extra), tg3, Kt, causal=causal, cap=1e9)
            assert np.isposinf(eps3).all()
        checked += len(sets)
    assert checked > 10


def test_reach_reports_undecided_on_budget():
    """With a budget of one kept set per item the search cannot reach a set that needs a
    resolution below the top level: NaN (undecided), never a false +inf or a false cost."""
    pyr, q = _w1_pyr()
    eps = oracle.route_reach(pyr, q.reshape(1, 1, 1), [0], [7], [0], np.array([[3]]), 1, causal=False,
                             cap=10.0, budget=1)
    assert np.isnan(eps[0])


@pytest.mark.parametrize("causal", [True, False])
def test_attention_matches_sdpa(causal):
    rng = np.random.default_rng(15)
    N, C, d, H, Hq = 200, 16, 32, 2, 4
    K = rng.standard_normal((1, N, H, d)).astype(np.float32)
    V = rng.standard_normal((1, N, H, d)).astype(np.float32)
    Q = rng.standard_normal((N, Hq, d)).astype(np.float32)
    M1 = -(-N // C)
    t = np.arange(N)
    for sel_kind in ("all", "subset"):
        if sel_kind == "all":
            sel = np.tile(np.arange(M1, dtype=np.int32), (N, H, 1))
        else:
            sel = np.full((N, H, 4), -1, np.int32)
            for n in range(N):
                for h in range(H):
                    pick = rng.choice(M1, size=3, replace=False)
                    sel[n, h, :3] = np.sort(pick)
        r = oracle.sparse_attn(Q, [0] * N, t, K, V, N, C, sel, causal=causal)
        mask = torch.zeros(Hq, N, N, dtype=torch.bool)
        for n in range(N):
            for hq in range(Hq):
                for i in sel[n, hq // (Hq // H)]:
                    if i >= 0:
                        mask[hq, n, i * C:min(i * C + C, N)] = True
        if causal:
            mask &= torch.ones(N, N, dtype=torch.bool).tril()
        empty = ~mask.any(-1)
        mask[empty] = True  # keep SDPA finite; such rows are checked separately
        q = torch.from_numpy(Q).double().permute(1, 0, 2)
        k = torch.from_numpy(K[0]).double().permute(1, 0, 2).repeat_interleave(Hq // H, 0)
        v = torch.from_numpy(V[0]).double().permute(1, 0, 2).repeat_interleave(Hq // H, 0)
        want = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
        want = want.permute(1, 0, 2).numpy()
        emp = empty.permute(1, 0).numpy()
        np.testing.assert_allclose(r["out"][~emp], want[~emp], atol=1e-10)
        assert (r["out"][emp] == 0).all() and np.isneginf(r["lse"][emp]).all()


# --------------------------------------------------------------------------
# PISA-1 / PISA-2 block scores (section 4.4 eq 32-34, appendix A.2 eq 43-52)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("N", [64, 56])
def test_pisa12_closed_forms_on_arithmetic_logits(N):
    """Keys whose first coordinate is the token index r and a query (8, 0, ..) with
    d = 64 give the logits z_r = 8 r / sqrt(64) = r. A run of n consecutive integers
    has mean (first + last) / 2 and population variance (n^2 - 1) / 12; two values a < b
    have variance (b - a)^2 / 4. Leaves hold C = 16 tokens (the last one 8 when N = 56),
    g = 2."""
    d, C, g = 64, 16, 2
    K = np.zeros((1, N, 1, d), np.float32)
    K[0, :, 0, 0] = np.arange(N)
    q = np.zeros(d, np.float32)
    q[0] = 8.0
    pyr = oracle.Pyramid(K, N, C, g)
    leaf_mean = []
    for i in range(pyr.M[1]):
        lo, hi = i * C, min(i * C + C, N)
        n = hi - lo
        mean, var = (lo + hi - 1) / 2, (n * n - 1) / 12
        leaf_mean.append(mean)
        assert oracle.score(pyr, q, 0, 0, 1, i, kind="mean") == pytest.approx(mean, abs=1e-12)
        assert oracle.score(pyr, q, 0, 0, 1, i, kind="mean_var") == pytest.approx(mean + var / 2, abs=1e-12)
    # level 2: the logits are the two leaf means (unweighted, eq 14-15)
    node_mean = []
    for j in range(pyr.M[2]):
        a, b = leaf_mean[2 * j], leaf_mean[2 * j + 1]
        node_mean.append((a + b) / 2)
        assert oracle.score(pyr, q, 0, 0, 2, j, kind="mean") == pytest.approx((a + b) / 2, abs=1e-12)
        assert oracle.score(pyr, q, 0, 0, 2, j, kind="mean_var") == pytest.approx(
            (a + b) / 2 + (b - a) ** 2 / 8, abs=1e-12)
    a, b = node_mean
    assert oracle.score(pyr, q, 0, 0, 3, 0, kind="mean_var") == pytest.approx((a + b) / 2 + (b - a) ** 2 / 8,
                                                                              abs=1e-12)


def test_pisa12_are_the_taylor_truncations_of_normalised_lse():
    """Appendix A.2 eq 45-49: with phi(lam) = LSE(lam z) - log m, phi(0) = 0,
    phi'(0) = mean and phi''(0) = variance. Scaling the query by lam scales every logit
    by lam, so PISA-1(lam q) = lam mean and PISA-2(lam q) = lam mean + lam^2 var / 2 must
    approach phi(lam) to second and third order as lam -> 0."""
    rng = np.random.default_rng(31)
    N, C, g, d = 256, 16, 4, 16
    K = rng.standard_normal((1, N, 1, d)).astype(np.float32)
    pyr = oracle.Pyramid(K, N, C, g)
    q = rng.standard_normal(d).astype(np.float32)
    for l, i, m in ((1, 3, C), (2, 1, g), (3, 0, g)):
        err1, err2 = [], []
        for lam in (1 / 16, 1 / 32, 1 / 64):
            ql = (q * np.float32(lam)).astype(np.float32)  # exact: power-of-two scaling
            phi = oracle.score(pyr, ql, 0, 0, l, i) - math.log(m)
            err1.append(phi - oracle.score(pyr, ql, 0, 0, l, i, kind="mean"))
            err2.append(phi - oracle.score(pyr, ql, 0, 0, l, i, kind="mean_var"))
        # second order: halving lam quarters the gap (to within its own O(lam) correction)
        assert err1[0] > 0 and 3.5 < err1[0] / err1[1] < 4.5 and 3.7 < err1[1] / err1[2] < 4.3
        # third order: halving lam divides the remaining gap by about 8
        assert abs(err2[1]) < abs(err1[1]) / 10
        assert 6.5 < err2[0] / err2[1] < 9.5 and 7.2 < err2[1] / err2[2] < 8.8


def test_pisa12_jensen_and_variance_bounds():
    """Eq 40: the mean logit is at most the normalised LSE (equality when the logits are
    equal); the variance is non-negative, so PISA-2 >= PISA-1."""
    rng = np.random.default_rng(32)
    N, C, g, d = 200, 8, 2, 8
    K = rng.standard_normal((1, N, 1, d)).astype(np.float32)
    K[0, 0:C, 0] = K[0, 0, 0]  # leaf 0: identical keys, so identical logits
    pyr = oracle.Pyramid(K, N, C, g)
    q = rng.standard_normal(d).astype(np.float32)
    for l in range(1, pyr.L + 1):
        for i in range(pyr.M[l]):
            m = min(C, N - i * C) if l == 1 else min(g, pyr.M[l - 1] - i * g)
            s0 = oracle.score(pyr, q, 0, 0, l, i) - math.log(m)
            s1 = oracle.score(pyr, q, 0, 0, l, i, kind="mean")
            s2 = oracle.score(pyr, q, 0, 0, l, i, kind="mean_var")
            assert s1 <= s0 + 1e-12 and s1 <= s2
    assert oracle.score(pyr, q, 0, 0, 1, 0, kind="mean") == pytest.approx(
        oracle.score(pyr, q, 0, 0, 1, 0) - math.log(C), abs=1e-12)
    assert oracle.score(pyr, q, 0, 0, 1, 0, kind="mean_var") == oracle.score(pyr, q, 0, 0, 1, 0, kind="mean")


@pytest.mark.parametrize("kind", ["mean", "mean_var"])
def test_pisa12_route_reduces_to_exhaustive_on_tiny(kind):
    """K_top = 32 at N = 1024, C = 16: every level above the leaves is kept whole, so
    the route is the exhaustive leaf selection by the summed PISA-1 / PISA-2 scores."""
    rng = np.random.default_rng(33)
    N, C, g, d = 1024, 16, 2, 64
    K = rng.standard_normal((1, N, 1, d)).astype(np.float32)
    Q = rng.standard_normal((N, 2, d)).astype(np.float32)
    pyr = oracle.Pyramid(K, N, C, g)
    t = np.arange(0, N, 11)
    r = oracle.route(pyr, Q[t], [0] * len(t), t, 32, causal=True, score_kind=kind)
    want = exhaustive_lse(K, Q[t], t, C, 32, kind=kind)
    for n in range(len(t)):
        assert [int(x) for x in r["idx"][n, 0] if x >= 0] == want[n][0], "t=%d" % t[n]


# --------------------------------------------------------------------------
# Backward of block-sparse attention (section 3.1 eq 6; section 3.3: gradients
# flow through attention on the selected entries)
# --------------------------------------------------------------------------
def _grid(rng, shape, lim=2.0):
    """Values on the 2^-10 grid: x and x +- 2^-10 are exact in float32."""
    return (np.round(rng.uniform(-lim, lim, shape) * 1024) / 1024).astype(np.float32)


def _random_selection(rng, N, H, C, K_top, causal):
    M1 = -(-N // C)
    sel = np.full((N, H, K_top), -1, np.int32)
    for n in range(N):
        hi = (n // C + 1) if causal else M1
        for h in range(H):
            k = int(rng.integers(0, min(K_top, hi) + 1))
            sel[n, h, :k] = np.sort(rng.choice(hi, size=k, replace=False))
    return sel


@pytest.mark.parametrize("causal", [True, False])
def test_attn_bwd_matches_central_differences(causal):
    """Every gradient entry against (L(x + eps) - L(x - eps)) / (2 eps) of the forward oracle's
    loss L = sum dO . o, eps = 2^-10 (error O(eps^2)); rows with no visible key included."""
    rng = np.random.default_rng(41 + causal)
    N, C, H, Hq, d, Kt = 14, 4, 2, 4, 4, 3
    Q, K, V = _grid(rng, (N, Hq, d)), _grid(rng, (1, N, H, d)), _grid(rng, (1, N, H, d))
    dO = _grid(rng, (N, Hq, d))
    sel = _random_selection(rng, N, H, C, Kt, causal)
    t = np.arange(N)
    g = oracle.sparse_attn_bwd(Q, [0] * N, t, K, V, dO, N, C, sel, causal=causal, threads=1)

    def loss(Qx, Kx, Vx):
        o = oracle.sparse_attn(Qx, [0] * N, t, Kx, Vx, N, C, sel, causal=causal, threads=1)["out"]
        return float((o * dO.astype(np.float64)).sum())

    eps = 2.0 ** -10
    for name, arr, grad in (("Q", Q, g["dQ"]), ("K", K, g["dK"]), ("V", V, g["dV"])):
        fd = np.zeros(arr.size)
        for k in range(arr.size):
            hi, lo = arr.copy(), arr.copy()
            hi.reshape(-1)[k] += eps
            lo.reshape(-1)[k] -= eps
            args_hi = {"Q": (hi, K, V), "K": (Q, hi, V), "V": (Q, K, hi)}[name]
            args_lo = {"Q": (lo, K, V), "K": (Q, lo, V), "V": (Q, K, lo)}[name]
            fd[k] = (loss(*args_hi) - loss(*args_lo)) / (2 * eps)
        np.testing.assert_allclose(grad.reshape(-1), fd, rtol=0, atol=2e-5, err_msg=name)
    assert np.abs(g["dK"]).max() > 0.05 and np.abs(g["dQ"]).max() > 0.05


def test_attn_bwd_dense_equals_torch_autograd():
    """Selecting every block makes eq 6 dense causal softmax attention: the gradients equal
    torch autograd (float64) of softmax(Q K^T / sqrt(d) + causal mask) V with grouped heads."""
    rng = np.random.default_rng(43)
    N, C, H, Hq, d = 90, 16, 2, 6, 8
    Q = rng.standard_normal((N, Hq, d)).astype(np.float32)
    K = rng.standard_normal((1, N, H, d)).astype(np.float32)
    V = rng.standard_normal((1, N, H, d)).astype(np.float32)
    dO = rng.standard_normal((N, Hq, d)).astype(np.float32)
    M1 = -(-N // C)
    sel = np.tile(np.arange(M1, dtype=np.int32), (N, H, 1))
    g = oracle.sparse_attn_bwd(Q, [0] * N, np.arange(N), K, V, dO, N, C, sel, causal=True)
    q = torch.from_numpy(Q).double().permute(1, 0, 2).requires_grad_()
    k = torch.from_numpy(K[0]).double().permute(1, 0, 2).requires_grad_()
    v = torch.from_numpy(V[0]).double().permute(1, 0, 2).requires_grad_()
    G = Hq // H
    s = q @ k.repeat_interleave(G, 0).transpose(1, 2) / math.sqrt(d)
    s = s.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), float("-inf"))
    o = torch.softmax(s, -1) @ v.repeat_interleave(G, 0)
    o.backward(torch.from_numpy(dO).double().permute(1, 0, 2))
    np.testing.assert_allclose(g["dQ"], q.grad.permute(1, 0, 2).numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(g["dK"][0], k.grad.permute(1, 0, 2).numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(g["dV"][0], v.grad.permute(1, 0, 2).numpy(), rtol=0, atol=1e-10)


def test_attn_bwd_sum_identities():
    """Softmax rows sum to one, so per (sequence, KV head) the key gradients sum to zero and
    the value gradients sum to the upstream gradients of the rows that see a key."""
    rng = np.random.default_rng(44)
    B, N, C, H, Hq, d, Kt = 2, 150, 8, 2, 4, 16, 5
    K = rng.standard_normal((B, N, H, d)).astype(np.float32)
    V = rng.standard_normal((B, N, H, d)).astype(np.float32)
    Q = rng.standard_normal((B * N, Hq, d)).astype(np.float32)
    dO = rng.standard_normal((B * N, Hq, d)).astype(np.float32)
    sel = np.concatenate([_random_selection(rng, N, H, C, Kt, True) for _ in range(B)])
    ib = np.repeat(np.arange(B), N)
    it = np.tile(np.arange(N), B)
    g = oracle.sparse_attn_bwd(Q, ib, it, K, V, dO, N, C, sel, causal=True)
    seen = (sel >= 0).any(-1)  # [items][H]: every selected block starts at or before t
    G = Hq // H
    for b in range(B):
        for h in range(H):
            np.testing.assert_allclose(g["dK"][b, :, h].sum(0), 0.0, atol=1e-9)
            rows = (ib == b) & seen[:, h]
            want = dO[rows][:, h * G:(h + 1) * G].astype(np.float64).sum((0, 1))
            np.testing.assert_allclose(g["dV"][b, :, h].sum(0), want, atol=1e-9)


def test_attn_bwd_saved_output_form():
    """sum_j p_j dp_j = dO . o: handed the (float32-rounded) exact forward output, the
    saved-output form of the backward gives the same gradients; handed a perturbed
    output O + e, dQ moves by -dO.e * sum_j p_j k_j / sqrt(d), the attention output
    with values k (the oracle forward with V replaced by K)."""
    rng = np.random.default_rng(45)
    N, C, H, Hq, d, Kt = 120, 8, 2, 4, 16, 5
    K = rng.standard_normal((1, N, H, d)).astype(np.float32)
    V = rng.standard_normal((1, N, H, d)).astype(np.float32)
    Q = rng.standard_normal((N, Hq, d)).astype(np.float32)
    dO = rng.standard_normal((N, Hq, d)).astype(np.float32)
    sel = _random_selection(rng, N, H, C, Kt, True)
    t = np.arange(N)
    O = oracle.sparse_attn(Q, [0] * N, t, K, V, N, C, sel)["out"].astype(np.float32)
    g0 = oracle.sparse_attn_bwd(Q, [0] * N, t, K, V, dO, N, C, sel)
    g1 = oracle.sparse_attn_bwd(Q, [0] * N, t, K, V, dO, N, C, sel, O=O)
    for k in ("dQ", "dK", "dV"):
        np.testing.assert_allclose(g1[k], g0[k], rtol=0, atol=1e-5 * np.abs(g0[k]).max())
    e = (rng.standard_normal(O.shape) * 0.01).astype(np.float32)
    g2 = oracle.sparse_attn_bwd(Q, [0] * N, t, K, V, dO, N, C, sel, O=O + e)
    kbar = oracle.sparse_attn(Q, [0] * N, t, K, K, N, C, sel)["out"]  # sum_j p_j k_j
    dD = ((O + e).astype(np.float64) * dO).sum(-1) - (O.astype(np.float64) * dO).sum(-1)
    want = g1["dQ"] - dD[..., None] * kbar / math.sqrt(d)
    np.testing.assert_allclose(g2["dQ"], want, rtol=0, atol=1e-9)
    np.testing.assert_allclose(g2["dV"], g1["dV"], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# Block-selection quality against full attention (section 4.4 eq 35-36,
# appendix D.2 eq 55-57)
# --------------------------------------------------------------------------
def _quality_problem(seed, N=160, C=8, H=2, Hq=4, d=8, Kt=5):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((1, N, H, d)).astype(np.float32)
    Q = (1.5 * rng.standard_normal((N, Hq, d))).astype(np.float32)
    sel = _random_selection(rng, N, H, C, Kt, True)
    return rng, Q, K, sel, N, C, H, Hq, d, Kt


def test_block_mass_is_dense_softmax_summed_per_block():
    """P(B) (eq 56) = the head average of each head's full causal softmax summed over the
    block's tokens: torch float64 softmax over the whole causal prefix as the reference."""
    _, Q, K, sel, N, C, H, Hq, d, Kt = _quality_problem(46)
    t = np.arange(N)
    r = oracle.selection_quality(Q, [0] * N, t, K, N, C, sel, with_mass=True)
    G = Hq // H
    q = torch.from_numpy(Q).double().permute(1, 0, 2)
    k = torch.from_numpy(K[0]).double().permute(1, 0, 2).repeat_interleave(G, 0)
    s = q @ k.transpose(1, 2) / math.sqrt(d)
    s = s.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), float("-inf"))
    p = torch.softmax(s, -1).reshape(Hq, N, N // C, C).sum(-1)   # [Hq][N][M1]
    want = p.reshape(H, G, N, N // C).mean(1).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(r["mass"], want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["mass"].sum(-1), 1.0, atol=1e-12)


def test_reference_set_maximises_captured_mass():
    """The reference set (forced blocks plus the highest-mass others) captures the most
    mass of any set of K_top blocks holding the forced ones (brute force over subsets),
    and is the lower-index choice among equal masses; a selection equal to it has
    Recall@K = MassRatio = 1, and known overlaps give Recall@K = overlap / K_top."""
    import itertools
    _, Q, K, sel, N, C, H, Hq, d, Kt = _quality_problem(47, N=88, C=8)
    t = np.arange(N)
    r = oracle.selection_quality(Q, [0] * N, t, K, N, C, sel, with_mass=True)
    for n in range(0, N, 7):
        c = n // C
        for h in range(H):
            ref = [x for x in r["ref"][n, h] if x >= 0]
            if c + 1 <= Kt:
                assert ref == list(range(c + 1))
                continue
            F = {0, c - 1, c}
            others = [B for B in range(c + 1) if B not in F]
            m = r["mass"][n, h]
            best = max(itertools.combinations(others, Kt - 3), key=lambda S: (sum(m[list(S)]), [-x for x in S]))
            assert ref == sorted(F | set(best))
    r2 = oracle.selection_quality(Q, [0] * N, t, K, N, C, r["ref"])
    np.testing.assert_allclose(r2["ratio"], 1.0, atol=1e-12)
    full = np.array([[c + 1 > Kt for _ in range(H)] for c in t // C])
    assert (r2["recall"][full] == 1.0).all()
    # swap one non-forced reference block for an eligible block outside it: recall drops by 1/K
    alt = r["ref"].copy()
    for n in range(N):
        c = n // C
        if c + 1 <= Kt:
            continue
        for h in range(H):
            out = [B for B in range(c + 1) if B not in alt[n, h]]
            row = sorted([x for x in alt[n, h] if x not in (0, c - 1, c)][1:] + [0, c - 1, c, out[0]])
            alt[n, h] = row
    r3 = oracle.selection_quality(Q, [0] * N, t, K, N, C, alt)
    np.testing.assert_allclose(r3["recall"][full], (Kt - 1) / Kt, atol=0)
    assert (r3["ratio"][full] <= 1.0 + 1e-12).all()
    np.testing.assert_allclose(r3["captured"], (r3["ratio"] * r2["captured"]), rtol=1e-12)
