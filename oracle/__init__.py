"""CPU oracle for PISA pyramid Top-K block selection -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The GPU library (``hierarchical_top_amd``)
never imports it and shares no code with it.

The arithmetic lives in ``pisa_oracle.c`` (plain C, IEEE double, one definition
per function, each citing the passage of "Block Sparse Attention with
Log-Linear Complexity" it follows). This module only compiles it with gcc and
marshals numpy arrays in and out. Inputs are passed as float32 arrays holding
the exact values given to the GPU (bf16 values convert to float32 exactly).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "pisa_oracle.c"
_LIB = _HERE / "libpisa_oracle.so"
# A test that plants mistakes in a copy of the C source points this at the copy.
_LIB_OVERRIDE = os.environ.get("PISA_ORACLE_LIB")
MAX_LEVELS = 40

_lib = None


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(".so.tmp%d" % os.getpid())
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fPIC",
             "-shared", "-pthread", str(_SRC), "-o", str(tmp), "-lm"],
            check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build(force=False)
            lib = ctypes.CDLL(str(_LIB))
        P = ctypes.c_void_p
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.orc_levels.argtypes = [i64, i32, i32, P]
        lib.orc_levels.restype = i32
        lib.orc_build_pyramid.argtypes = [P, i32, i64, i64, i32, i32, i32, i32, P, P]
        lib.orc_build_pyramid.restype = None
        lib.orc_route.argtypes = [P, P, P, i64, P, P, P, i32, i64, i64, i32, i32, i32, i32,
                                  i32, i32, i32, P, P, P, P, i32]
        lib.orc_route.restype = i32
        lib.orc_route_scored.argtypes = [P, P, P, i64, P, P, P, i32, i64, i64, i32, i32, i32, i32,
                                         i32, i32, i32, i32, P, P, P, P, i32]
        lib.orc_route_scored.restype = i32
        lib.orc_sparse_attn_bwd.argtypes = [P, P, P, i64, P, P, P, P, i32, i64, i64, i32, i32, i32,
                                            i32, P, i32, i32, P, P, P, i32]
        lib.orc_sparse_attn_bwd.restype = i32
        lib.orc_selection_quality.argtypes = [P, P, P, i64, P, i32, i64, i64, i32, i32, i32, i32, P,
                                              i32, P, P, P, P, P, i32]
        lib.orc_selection_quality.restype = i32
        lib.orc_bsa.argtypes = [P, P, P, i64, P, P, i32, i64, i32, i32, i32, i32, i32, i32,
                                i32, P, P, P, i32]
        lib.orc_bsa.restype = i32
        lib.orc_route_reach.argtypes = [P, P, P, P, i64, P, P, P, i32, i64, i64, i32, i32, i32, i32,
                                        i32, i32, i32, i32, P, dbl, i64, P, i32]
        lib.orc_route_reach.restype = i32
        lib.orc_bsa_scores.argtypes = [P, P, P, i64, P, P, i32, i64, i32, i32, i32, i32, i32, i32,
                                       i32, P]
        lib.orc_bsa_scores.restype = i32
        lib.orc_sparse_attn.argtypes = [P, P, P, i64, P, P, i32, i64, i64, i32, i32, i32, i32,
                                        P, i32, i32, P, P, i32]
        lib.orc_sparse_attn.restype = i32
        lib.orc_score.argtypes = [P, i64, i32, i32, i64, P, P, P, i32, i64, i64, i32, i32, i32,
                                  i32]
        lib.orc_score.restype = dbl
        lib.orc_score_kind.argtypes = [P, i64, i32, i32, i64, P, P, P, i32, i64, i64, i32, i32,
                                       i32, i32, i32]
        lib.orc_score_kind.restype = dbl
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def default_threads() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


def levels(N: int, C: int, g: int) -> list[int]:
    """[M_0, M_1, ..., M_L] (eq 7, 10, 13)."""
    M = np.zeros(MAX_LEVELS + 1, dtype=np.int64)
    L = _load().orc_levels(int(N), int(C), int(g), _ptr(M))
    if L < 1:
        raise ValueError("bad pyramid geometry")
    return [int(x) for x in M[:L + 1]]


class Pyramid:
    """fp64 summaries of levels 1..L for keys K [B][N_alloc][H][d] (first N tokens)."""

    def __init__(self, K, N: int, C: int, g: int):
        K = _f32(K)
        self.K = K
        self.B, self.N_alloc, self.H, self.d = K.shape
        self.N, self.C, self.g = int(N), int(C), int(g)
        self.M = levels(N, C, g)
        self.L = len(self.M) - 1
        off = np.zeros(MAX_LEVELS + 2, dtype=np.int64)
        o = 0
        for l in range(1, self.L + 1):
            off[l] = o
            o += self.B * self.H * self.M[l] * self.d
        self.off = off
        self.buf = np.zeros(max(o, 1), dtype=np.float64)
        _load().orc_build_pyramid(_ptr(K), self.B, self.N_alloc, self.N, self.H, self.d,
                                  self.C, self.g, _ptr(self.buf), _ptr(off))

    def level(self, l: int) -> np.ndarray:
        """Level-l summaries as a [B][H][M_l][d] view."""
        n = self.B * self.H * self.M[l] * self.d
        return self.buf[self.off[l]:self.off[l] + n].reshape(self.B, self.H, self.M[l], self.d)


def _items(item_b, item_t):
    return (np.ascontiguousarray(item_b, dtype=np.int64),
            np.ascontiguousarray(item_t, dtype=np.int64))


# block scores (section 4.4): PISA's log-sum-exp, PISA-1 (mean), PISA-2 (mean + var / 2)
SCORE_KINDS = {"lse": 0, "mean": 1, "mean_var": 2}


def route(pyr: Pyramid, Qi, item_b, item_t, K_top: int, causal: bool = True,
          trace: bool = False, threads: int | None = None, score_kind: str = "lse"):
    """PISA route of queries Qi [n][H_q][d] at positions item_t of sequences item_b,
    with block score score_kind ("lse", or the PISA-1 / PISA-2 scores "mean", "mean_var").

    Returns dict(idx [n][H][K_top] int32, score [n][H][K_top] f64, gap [n][H] f64,
    trace [n][H][L+1][2] int32 or None).
    """
    Qi = _f32(Qi)
    n, H_q, d = Qi.shape
    b, t = _items(item_b, item_t)
    H = pyr.H
    idx = np.empty((n, H, K_top), dtype=np.int32)
    score = np.empty((n, H, K_top), dtype=np.float64)
    gap = np.empty((n, H), dtype=np.float64)
    tr = np.zeros((n, H, pyr.L + 1, 2), dtype=np.int32) if trace else None
    rc = _load().orc_route_scored(_ptr(Qi), _ptr(b), _ptr(t), n, _ptr(pyr.K), _ptr(pyr.buf),
                                  _ptr(pyr.off), pyr.B, pyr.N_alloc, pyr.N, H, H_q, d, pyr.C, pyr.g,
                                  int(K_top), int(bool(causal)), SCORE_KINDS[score_kind], _ptr(idx),
                                  _ptr(score), _ptr(gap), _ptr(tr), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle route rejected its arguments")
    return dict(idx=idx, score=score, gap=gap, trace=tr)


def route_reach(pyr: Pyramid, Qi, item_b, item_t, item_h, target, K_top: int, causal: bool = True,
                score_kind: str = "lse", cap: float = 1e-3, budget: int = 200000,
                threads: int | None = None):
    """Smallest tie-resolution cost at which the route of each item can end in a given
    selection: item k is query Qi[k] [H_q][d] at position item_t[k] of sequence item_b[k],
    routed for KV head item_h[k]; target [n][K_top] is the selection to explain (-1 padded).

    At every ranked level a kept set may drop a candidate that scores up to `cost` above a
    kept one (Select_K resolved the other way within that margin); a path costs its largest
    such margin. Returns eps [n]: 0 when target is the oracle's own selection, the smallest
    path cost <= cap that reaches target, +inf when none does, NaN when the search hit its
    budget before finding a path."""
    Qi = _f32(Qi)
    n, H_q, d = Qi.shape
    b, t = _items(item_b, item_t)
    hh = np.ascontiguousarray(item_h, dtype=np.int32)
    tg = np.ascontiguousarray(target, dtype=np.int32).reshape(n, int(K_top))
    eps = np.empty(n, dtype=np.float64)
    rc = _load().orc_route_reach(_ptr(Qi), _ptr(b), _ptr(t), _ptr(hh), n, _ptr(pyr.K), _ptr(pyr.buf),
                                 _ptr(pyr.off), pyr.B, pyr.N_alloc, pyr.N, pyr.H, H_q, d, pyr.C, pyr.g,
                                 int(K_top), int(bool(causal)), SCORE_KINDS[score_kind], _ptr(tg),
                                 float(cap), int(budget), _ptr(eps), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle reachability check rejected its arguments")
    return eps


def bsa_scores(pyr: Pyramid, Qi, item_b, item_t, K_top: int, causal: bool = True):
    """Every leaf's BSA score u [n][H][M_1] for queries Qi [n][H_q][d]: the per-head softmax
    over the scored leaves summed over the group for a scored leaf, +inf for a leaf kept
    without a score, -inf for a leaf after the query."""
    Qi = _f32(Qi)
    n, H_q, d = Qi.shape
    b, t = _items(item_b, item_t)
    u = np.empty((n, pyr.H, pyr.M[1]), dtype=np.float64)
    rc = _load().orc_bsa_scores(_ptr(Qi), _ptr(b), _ptr(t), n, _ptr(pyr.buf), _ptr(pyr.off), pyr.B,
                                pyr.N, pyr.H, H_q, d, pyr.C, pyr.g, int(K_top), int(bool(causal)), _ptr(u))
    if rc != 0:
        raise ValueError("oracle bsa scores rejected its arguments")
    return u


def bsa(pyr: Pyramid, Qi, item_b, item_t, K_top: int, causal: bool = True,
        threads: int | None = None):
    """Exhaustive BSA-style selection (per-head softmax over leaf means, head sum)."""
    Qi = _f32(Qi)
    n, H_q, d = Qi.shape
    b, t = _items(item_b, item_t)
    H = pyr.H
    idx = np.empty((n, H, K_top), dtype=np.int32)
    score = np.empty((n, H, K_top), dtype=np.float64)
    gap = np.empty((n, H), dtype=np.float64)
    rc = _load().orc_bsa(_ptr(Qi), _ptr(b), _ptr(t), n, _ptr(pyr.buf), _ptr(pyr.off), pyr.B,
                         pyr.N, H, H_q, d, pyr.C, pyr.g, int(K_top), int(bool(causal)),
                         _ptr(idx), _ptr(score), _ptr(gap), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle bsa rejected its arguments")
    return dict(idx=idx, score=score, gap=gap)


def sparse_attn(Qi, item_b, item_t, K, V, N: int, C: int, sel, causal: bool = True,
                threads: int | None = None):
    """Block-sparse attention (eq 6) of queries Qi [n][H_q][d] over sel [n][H][k]."""
    Qi, K, V = _f32(Qi), _f32(K), _f32(V)
    n, H_q, d = Qi.shape
    B, N_alloc, H, _ = K.shape
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    b, t = _items(item_b, item_t)
    out = np.empty((n, H_q, d), dtype=np.float64)
    lse = np.empty((n, H_q), dtype=np.float64)
    rc = _load().orc_sparse_attn(_ptr(Qi), _ptr(b), _ptr(t), n, _ptr(K), _ptr(V), B, N_alloc,
                                 int(N), H, H_q, d, int(C), _ptr(sel), sel.shape[2],
                                 int(bool(causal)), _ptr(out), _ptr(lse),
                                 threads or default_threads())
    if rc != 0:
        raise ValueError("oracle attention rejected its arguments")
    return dict(out=out, lse=lse)


def sparse_attn_bwd(Qi, item_b, item_t, K, V, dO, N: int, C: int, sel, causal: bool = True,
                    threads: int | None = None, O=None):
    """Gradients of block-sparse attention (eq 6) for queries Qi [n][H_q][d] over
    sel [n][H][k] with upstream gradient dO [n][H_q][d]: dict(dQ [n][H_q][d],
    dK, dV [B][N_alloc][H][d]) in float64; dK and dV hold the given items' parts.
    O: the saved forward output [n][H_q][d] whose dO . O replaces sum_j p_j dp_j."""
    Qi, K, V, dO = _f32(Qi), _f32(K), _f32(V), _f32(dO)
    Os = _f32(O) if O is not None else None
    n, H_q, d = Qi.shape
    B, N_alloc, H, _ = K.shape
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    b, t = _items(item_b, item_t)
    dQ = np.empty((n, H_q, d), dtype=np.float64)
    dK = np.empty((B, N_alloc, H, d), dtype=np.float64)
    dV = np.empty((B, N_alloc, H, d), dtype=np.float64)
    rc = _load().orc_sparse_attn_bwd(_ptr(Qi), _ptr(b), _ptr(t), n, _ptr(K), _ptr(V), _ptr(dO), _ptr(Os), B,
                                     N_alloc, int(N), H, H_q, d, int(C), _ptr(sel), sel.shape[2],
                                     int(bool(causal)), _ptr(dQ), _ptr(dK), _ptr(dV),
                                     threads or default_threads())
    if rc != 0:
        raise ValueError("oracle attention backward rejected its arguments")
    return dict(dQ=dQ, dK=dK, dV=dV)


def selection_quality(Qi, item_b, item_t, K, N: int, C: int, sel, with_mass: bool = False,
                      threads: int | None = None):
    """Block-selection quality of sel [n][H][K_top] against full attention (eq 35-36,
    55-57) for causal queries Qi [n][H_q][d] at positions item_t of sequences item_b.
    Returns dict(recall, captured, ratio [n][H] f64, ref [n][H][K_top] int32 (the
    full-attention reference set), mass [n][H][M_1] f64 or None)."""
    Qi, K = _f32(Qi), _f32(K)
    n, H_q, d = Qi.shape
    B, N_alloc, H, _ = K.shape
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    Kt = sel.shape[2]
    b, t = _items(item_b, item_t)
    M1 = -(-int(N) // int(C))
    mass = np.empty((n, H, M1)) if with_mass else None
    ref = np.empty((n, H, Kt), dtype=np.int32)
    rec, cap, rat = (np.empty((n, H)) for _ in range(3))
    rc = _load().orc_selection_quality(_ptr(Qi), _ptr(b), _ptr(t), n, _ptr(K), B, N_alloc, int(N), H, H_q,
                                       d, int(C), _ptr(sel), Kt, _ptr(mass), _ptr(ref), _ptr(rec),
                                       _ptr(cap), _ptr(rat), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle selection quality rejected its arguments")
    return dict(recall=rec, captured=cap, ratio=rat, ref=ref, mass=mass)


def score(pyr: Pyramid, q, b: int, h: int, l: int, i: int, kind: str = "lse") -> float:
    """s^(l)_{t,i} of one query head q [d] against node i of level l: the LSE of eq 21,
    or with kind "mean" / "mean_var" the PISA-1 / PISA-2 score of eq 33-34."""
    q = _f32(q)
    return float(_load().orc_score_kind(_ptr(q), int(b), int(h), int(l), int(i), _ptr(pyr.K),
                                        _ptr(pyr.buf), _ptr(pyr.off), pyr.B, pyr.N_alloc, pyr.N,
                                        pyr.H, pyr.d, pyr.C, pyr.g, SCORE_KINDS[kind]))
