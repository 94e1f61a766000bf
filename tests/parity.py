"""Parity checks of GPU selections against the oracle (test helper).

Protocol (tolerances from the selection definition: fp32 dot products and
reductions against the oracle's fp64; Select_K of section 3.2 eq 17 with the
lower index winning ties):
  * strict: a (query, KV head) whose oracle run ranked every level with a
    margin of at least `strict` between the last kept and the first dropped
    score must select exactly the oracle's blocks (fp32 scores differ from the
    fp64 ones by a few 1e-6, so no legitimate resolution can differ there);
  * near ties: every other mismatching selection must be the outcome of
    resolving near ties the other way: the oracle's tie-resolution search
    (`reach`) must find a path -- at every ranked level a kept set that drops
    no candidate scoring more than `band` above a kept one -- that ends in
    exactly the GPU's blocks. A selection that needs a larger swap anywhere,
    or that no path reaches (a wrong subtree, a wrong score), fails;
  * every mismatching selection is also checked for structure: ascending,
    distinct, -1 padded, causal, holding the forced blocks, and of size
    min(K_top, eligible leaves);
  * scores of identical selections agree within `score_tol` where finite, and
    the +inf (kept without a score) / -inf (padding) pattern matches exactly.
"""
from __future__ import annotations

import numpy as np


def valid_selection(idx_row, t, C, K_top, causal=True, M1=None):
    got = [int(x) for x in idx_row if x >= 0]
    if list(idx_row[len(got):]) != [-1] * (len(idx_row) - len(got)):
        return "padding not at the end"
    if got != sorted(got) or len(set(got)) != len(got):
        return "not ascending / distinct"
    if causal:
        c = t // C
        if any(x > c for x in got):
            return "future block"
        F = {0, c} | ({c - 1} if c >= 1 else set())
        if not F <= set(got):
            return "forced block missing"
        if len(got) != min(K_top, c + 1):
            return "size %d != %d" % (len(got), min(K_top, c + 1))
    elif M1 is not None and len(got) != min(K_top, M1):
        return "size"
    return None


def route_reach(opyr, Qi, b, t, K_top, causal=True, score_kind="lse", band=1e-3):
    """A `reach` callable for compare(): the oracle's tie-resolution search for the routes
    of queries Qi [n][H_q][d] at positions t of sequence b (n = len(t))."""
    import oracle  # test infrastructure only

    def reach(k, h, target):
        return oracle.route_reach(opyr, Qi[k], [b] * len(k), np.asarray(t)[k], h, target, K_top,
                                  causal=causal, score_kind=score_kind, cap=band)
    return reach


def bsa_reach(opyr, Qi, b, t, K_top, causal=True):
    """A `reach` callable for compare() on the exhaustive selector (one ranked level):
    the cost of a selection is the largest margin by which an unpicked scored leaf's oracle
    score exceeds a picked one's; +inf if it drops a forced block or picks a leaf that is
    not eligible."""
    import oracle  # test infrastructure only

    def reach(k, h, target):
        u = oracle.bsa_scores(opyr, Qi[k], [b] * len(k), np.asarray(t)[k], K_top, causal=causal)
        eps = np.empty(len(k))
        for j in range(len(k)):
            row = u[j, h[j]]
            picked = [int(x) for x in target[j] if x >= 0]
            if any(x >= len(row) or np.isneginf(row[x]) for x in picked):
                eps[j] = np.inf
                continue
            keep_unscored = np.isposinf(row)
            if not set(np.flatnonzero(keep_unscored)) <= set(picked):
                eps[j] = np.inf
                continue
            scored = np.isfinite(row)
            mask = np.zeros(len(row), bool)
            mask[picked] = True
            kept, dropped = row[scored & mask], row[scored & ~mask]
            eps[j] = max(0.0, dropped.max() - kept.min()) if len(kept) and len(dropped) else 0.0
        return eps
    return reach


def compare(gpu_idx, gpu_score, orc, t, C, K_top, causal=True, band=1e-3, score_tol=1e-3, strict=1e-5,
            M1=None, max_near_tie_frac=0.25, score_rtol=0.0, reach=None, tie_tol=5e-5):
    """gpu_idx/gpu_score [n][H][K] numpy, orc = oracle.route(...) dict, t [n] positions.

    band and strict may be arrays broadcastable to [n][H] (per-item bands); scores must
    satisfy |gpu - oracle| <= score_tol + score_rtol * |oracle|. reach(k, h, target) -> eps
    gives, for items (t[k], head h) and GPU selections target [m][K], the smallest
    tie-resolution cost that reproduces each one (required when any selection differs).
    Besides the band, that cost must stay within tie_tol (when given): scores that are
    each within d of the oracle's can only swap candidates less than 2 d apart, and the
    fp32 scores here are within 1e-5 of the fp64 ones."""
    n, H, _ = gpu_idx.shape
    oi, os_, gap = orc["idx"], orc["score"], orc["gap"]
    band = np.broadcast_to(band, (n, H))
    strict = np.broadcast_to(strict, (n, H))
    same = (gpu_idx == oi).all(-1)
    outside = (gap >= strict) & ~same
    bad = np.argwhere(outside)
    assert len(bad) == 0, "index mismatch outside the strict band at (item, head) %s: gpu %s oracle %s gap %s" % (
        bad[0].tolist(), gpu_idx[tuple(bad[0])], oi[tuple(bad[0])], gap[tuple(bad[0])])
    mism = np.argwhere(~same)
    for k, h in mism:
        err = valid_selection(gpu_idx[k, h], int(t[k]), C, K_top, causal, M1)
        assert err is None, "invalid near-tie selection at t=%d h=%d: %s (%s)" % (t[k], h, err, gpu_idx[k, h])
    max_eps = 0.0
    if len(mism):
        assert reach is not None, "%d selections differ from the oracle and no tie-resolution check was given" % len(mism)
        eps = np.asarray(reach(mism[:, 0], mism[:, 1], gpu_idx[mism[:, 0], mism[:, 1]]), dtype=np.float64)
        ok = eps <= band[mism[:, 0], mism[:, 1]]
        if not ok.all():
            j = int(np.flatnonzero(~ok)[0])
            k, h = mism[j]
            raise AssertionError("selection at t=%d h=%d is no tie resolution of the oracle's route within %g: "
                                 "gpu %s oracle %s cost %s (nan: undecided)" % (
                                     t[k], h, band[k, h], gpu_idx[k, h], oi[k, h], eps[j]))
        max_eps = float(eps.max())
        if tie_tol is not None:
            assert max_eps <= tie_tol, "a tie resolution needs a swap of %g, more than fp32 rounding explains" % max_eps
    if gpu_score is not None:
        s_g = gpu_score[same]
        s_o = os_[same]
        fin = np.isfinite(s_o)
        assert (np.isfinite(s_g) == fin).all(), "finite / infinite score pattern differs"
        assert (np.sign(s_g[~fin]) == np.sign(s_o[~fin])).all()
        if fin.any():
            err = np.abs(s_g[fin] - s_o[fin]) - score_rtol * np.abs(s_o[fin])
            assert err.max() <= score_tol, "score error %g > %g" % (err.max(), score_tol)
    near = (gap < band).mean()
    assert near <= max_near_tie_frac, "near-tie fraction %.3f is implausibly high" % near
    return dict(items=int(n * H), mismatched=int((~same).sum()), near_tie=float(near),
                mismatched_outside_strict=int(outside.sum()), invalid_tie_resolutions=0,
                max_tie_resolution_cost=max_eps,
                max_score_err=float(np.abs(gpu_score[same][np.isfinite(os_[same])] - os_[same][np.isfinite(os_[same])]).max())
                if gpu_score is not None and np.isfinite(os_[same]).any() else 0.0)
