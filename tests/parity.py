"""Parity checks of GPU selections against the oracle (test helper).

Protocol (tolerances from the selection definition: fp32 dot products and
reductions against the oracle's fp64):
  * a (query, KV head) whose oracle run ranked every level with a margin of at
    least `band` between the last kept and the first dropped score must
    select exactly the oracle's blocks;
  * inside the band (a near tie) the GPU may legitimately resolve the tie the
    other way, possibly descending into another subtree; there the selection
    must still be valid: ascending, distinct, -1 padded, causal, holding the
    forced blocks, and of size min(K_top, eligible leaves);
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


def compare(gpu_idx, gpu_score, orc, t, C, K_top, causal=True, band=1e-3, score_tol=1e-3, strict=1e-5,
            M1=None, max_near_tie_frac=0.25, score_rtol=0.0):
    """gpu_idx/gpu_score [n][H][K] numpy, orc = oracle.route(...) dict, t [n] positions.

    band may be an array broadcastable to [n][H] (a per-item tie band);
    scores must satisfy |gpu - oracle| <= score_tol + score_rtol * |oracle|."""
    n, H, _ = gpu_idx.shape
    oi, os_, gap = orc["idx"], orc["score"], orc["gap"]
    same = (gpu_idx == oi).all(-1)
    exact = gap >= band
    bad_exact = np.argwhere(exact & ~same)
    assert len(bad_exact) == 0, "index mismatch outside the near-tie band at (item, head) %s: gpu %s oracle %s gap %s" % (
        bad_exact[0].tolist(), gpu_idx[tuple(bad_exact[0])], oi[tuple(bad_exact[0])], gap[tuple(bad_exact[0])])
    for k, h in np.argwhere(~same):
        err = valid_selection(gpu_idx[k, h], int(t[k]), C, K_top, causal, M1)
        assert err is None, "invalid near-tie selection at t=%d h=%d: %s (%s)" % (t[k], h, err, gpu_idx[k, h])
    if gpu_score is not None:
        s_g = gpu_score[same]
        s_o = os_[same]
        fin = np.isfinite(s_o)
        assert (np.isfinite(s_g) == fin).all(), "finite / infinite score pattern differs"
        assert (np.sign(s_g[~fin]) == np.sign(s_o[~fin])).all()
        if fin.any():
            err = np.abs(s_g[fin] - s_o[fin]) - score_rtol * np.abs(s_o[fin])
            assert err.max() <= score_tol, "score error %g > %g" % (err.max(), score_tol)
    near = (~exact).mean()
    assert near <= max_near_tie_frac, "near-tie fraction %.3f is implausibly high" % near
    return dict(items=int(n * H), mismatched=int((~same).sum()), near_tie=float(near),
                mismatched_outside_strict=int(((gap >= strict) & ~same).sum()),
                max_score_err=float(np.abs(gpu_score[same][np.isfinite(os_[same])] - os_[same][np.isfinite(os_[same])]).max())
                if gpu_score is not None and np.isfinite(os_[same]).any() else 0.0)
