"""Algorithmic work of the selection path, counted from the pyramid geometry alone.

Used to turn measured times into roofline figures. Under causal routing with
the forced set (first, previous and current leaf and their ancestors), the
number of candidates and of scored candidates at every level depends only on
the query position t, not on the data ("Block Sparse Attention with
Log-Linear Complexity", section 3.2 eq 16-20 and appendix B):

* a kept node other than the current one (the ancestor of t's leaf) ends
  before the current node starts, so all its g children exist and are
  eligible; the current node is always kept and has
  floor(t / span_{l-1}) - g * anc_l(t) + 1 eligible children;
* a level with more than K_top candidates scores all but the forced ones and
  keeps K_top; otherwise it keeps all and scores none.

Every scored node above the leaves is therefore full (g child summaries) and
every scored leaf holds C keys. Nothing here touches floating-point data.
"""
from __future__ import annotations

import numpy as np


def levels(n: int, C: int, g: int) -> list[int]:
    """[M_0, M_1, ..., M_L] for a sequence of n tokens (section 3.2 eq 7-13)."""
    M = [n, -(-n // C)]
    while M[-1] > 1:
        M.append(-(-M[-1] // g))
    return M


def walk(t, n: int, C: int, g: int, K_top: int):
    """Scored candidates per level for causal queries at positions t (array) of an
    n-token sequence. Returns {level: int64 array aligned with t}."""
    t = np.asarray(t, dtype=np.int64)
    M = levels(n, C, g)
    L = len(M) - 1
    c = t // C
    nA = np.ones_like(t)
    scored = {}
    for l in range(L, 0, -1):
        den = g ** (l - 1)
        ac = c // den
        ap = np.where(c >= 1, (c - 1) // den, 0)
        nF = 1 + (ac != 0) + ((c >= 1) & (ap != 0) & (ap != ac))
        keep_all = nA <= K_top
        scored[l] = np.where(keep_all, 0, nA - nF)
        kept = np.minimum(nA, K_top)
        if l > 1:
            child_span = C * g ** (l - 2)
            nA = (kept - 1) * g + (t // child_span - ac * g + 1)
    return scored


def route_work(B: int, n: int, H_kv: int, G: int, d: int, C: int, g: int, K_top: int, positions=None):
    """Multiply-accumulates and exponentials of routing (fused or two-stage).

    positions: query positions routed (default: all of 0..n-1). Returns a dict
    with 'upper_mac' (levels L..2), 'leaf_mac' (level 1), 'upper_exp',
    'leaf_exp', 'scored_leaves' and 'scored_upper' (summed over queries and KV
    heads and batch).
    """
    t = np.arange(n, dtype=np.int64) if positions is None else np.asarray(positions, dtype=np.int64)
    s = walk(t, n, C, g, K_top)
    up = int(sum(int(v.sum()) for l, v in s.items() if l >= 2))
    leaf = int(s[1].sum())
    per = B * H_kv * G
    return dict(upper_mac=per * up * g * d, leaf_mac=per * leaf * C * d, upper_exp=per * up * g,
                leaf_exp=per * leaf * C, scored_leaves=B * H_kv * leaf, scored_upper=B * H_kv * up)


def decode_work(lengths, H_kv: int, G: int, d: int, C: int, g: int, K_top: int, kv_bytes: int = 2):
    """Work of one decode routing step over sequences of the given lengths (the new
    token sits at n - 1). Bytes are the gathered summaries (fp32) and leaf keys,
    plus the queries and the index output."""
    mac = 0
    gathered = 0
    for n in lengths:
        s = walk([n - 1], int(n), C, g, K_top)
        up = int(sum(int(v[0]) for l, v in s.items() if l >= 2))
        leaf = int(s[1][0])
        mac += H_kv * G * d * (up * g + leaf * C)
        gathered += H_kv * (up * g * d * 4 + leaf * C * d * kv_bytes)
    nb = len(lengths)
    q_bytes = nb * H_kv * G * d * kv_bytes
    out_bytes = nb * H_kv * K_top * 4
    return dict(mac=mac, bytes=gathered + q_bytes + out_bytes)


def build_bytes(B: int, n: int, H_kv: int, d: int, C: int, g: int, k_bytes: int = 2) -> int:
    """Compulsory bytes of a pyramid build: read the keys once, write every level."""
    M = levels(n, C, g)
    return B * n * H_kv * d * k_bytes + sum(B * H_kv * m * d * 4 for m in M[1:])


def bsa_work(B: int, n: int, H_kv: int, G: int, d: int, C: int, K_top: int):
    """One-pass work of the exhaustive selector: every eligible non-forced leaf mean
    is scored once per query head (section 3.1 eq 3-5)."""
    t = np.arange(n, dtype=np.int64)
    c = t // C
    E = c + 1
    nF = 1 + (c != 0) + (c >= 2)
    scored = np.where(E <= K_top, 0, E - nF)
    tot = int(scored.sum())
    return dict(mac=B * H_kv * G * d * tot, exp=B * H_kv * G * tot)


def attn_work(B: int, n: int, H_q: int, d: int, C: int, K_top: int):
    """Work of causal block-sparse attention when every query holds its current
    block plus min(K_top, c + 1) - 1 full past blocks (section 3.1 eq 6)."""
    t = np.arange(n, dtype=np.int64)
    c = t // C
    keys = (np.minimum(K_top, c + 1) - 1) * C + (t - c * C + 1)
    k = int(keys.sum())
    return dict(mac=2 * B * H_q * d * k, exp=B * H_q * k, keys=B * H_q * k)


def attn_bwd_work(B: int, n: int, H_q: int, d: int, C: int, K_top: int):
    """Work of the attention backward for the same selection: per (query head, visible
    key) five d-long products -- the recomputed score, dP = dO . v, and the dV, dK and
    dQ updates -- and one exponential."""
    f = attn_work(B, n, H_q, d, C, K_top)
    return dict(mac=f["mac"] // 2 * 5, exp=f["exp"], keys=f["keys"])
