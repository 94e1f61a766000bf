"""Seeded synthetic workloads for PISA routing (inputs only, no routing arithmetic).

The selection benchmark of "Block Sparse Attention with Log-Linear Complexity"
(appendix B, "Block-selection benchmarks") draws random BF16 queries and keys
from a fixed seed. The workloads below follow that recipe at five shapes:

  tiny    1 x 1024 tokens, 1 query / 1 KV head, d=64, C=16, g=2, K_top=4, fp32
  p16k    1 x 16384, 16 / 4 heads, d=128, C=64, g=4, K_top=8, bf16, planted
  p64k    1 x 65536, 32 / 8 heads, same routing parameters, planted, with V
  p256k   1 x 262144, 16 / 4 heads, same routing parameters, planted
  decode  32 sequences x 262144-token cache, 32 / 8 heads, d=128, C=64, g=4,
          K_top=8, bf16, no planting, 256 appended tokens

and at the appendix's own selection-benchmark shape (``paper_shape``): batch 1,
32 query heads sharing 2 KV heads, d=64, C=64, g=2, K_top=8, bf16, no planting,
at any length N (the appendix sweeps 4K to 256K tokens).

Every tensor is drawn as float32 N(0, 1) from a torch generator seeded per
workload, in the order Q, K, V, planted ids, then rounded to bf16 with
round-to-nearest-even (``.to(torch.bfloat16)``) for the bf16 workloads.
Planted blocks: for every KV head, 32 distinct leaf blocks drawn with
``randperm(M_1)[:32]``; the float32 keys of those blocks are multiplied by 3
before rounding, which gives strong-match targets. This module is shared by
the tests, the benchmark and the oracle callers; it computes nothing of the
selection method itself.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    N: int
    H_q: int
    H_kv: int
    d: int
    C: int
    g: int
    K_top: int
    dtype: str          # "f32" or "bf16"
    planted: int        # planted blocks per KV head (0 = none)
    seed: int
    with_v: bool
    steps: int = 0      # decode: appended tokens

    @property
    def G_Q(self) -> int:
        return self.H_q // self.H_kv

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1024, 1, 1, 64, 16, 2, 4, "f32", 0, 1, True),
    "p16k": Workload("p16k", 1, 16384, 16, 4, 128, 64, 4, 8, "bf16", 32, 2, True),
    "p64k": Workload("p64k", 1, 65536, 32, 8, 128, 64, 4, 8, "bf16", 32, 3, True),
    "p256k": Workload("p256k", 1, 262144, 16, 4, 128, 64, 4, 8, "bf16", 32, 4, False),
    "decode": Workload("decode", 32, 262144, 32, 8, 128, 64, 4, 8, "bf16", 0, 5, True, 256),
}


def paper_shape(N: int, seed: int = 40) -> Workload:
    """The appendix B selection-benchmark shape at N tokens (random Q and K)."""
    return Workload("paper%dk" % (N // 1024) if N % 1024 == 0 else "paper%d" % N,
                    1, N, 32, 2, 64, 64, 2, 8, "bf16", 0, seed, False)


def workload(name: str, **over) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **over) if over else w


def make_prefill(w: Workload, device="cpu"):
    """Q [B,N,H_q,d], K [B,N,H_kv,d], V (or None) and planted ids [B,H_kv,planted].

    Drawn on the CPU from ``torch.Generator().manual_seed(w.seed)`` so that the
    values do not depend on the device; then moved to ``device``.
    """
    gen = torch.Generator().manual_seed(w.seed)
    Q = torch.randn(w.B, w.N, w.H_q, w.d, generator=gen, dtype=torch.float32)
    K = torch.randn(w.B, w.N, w.H_kv, w.d, generator=gen, dtype=torch.float32)
    V = torch.randn(w.B, w.N, w.H_kv, w.d, generator=gen, dtype=torch.float32) if w.with_v else None
    M1 = (w.N + w.C - 1) // w.C
    planted = torch.empty(w.B, w.H_kv, min(w.planted, M1), dtype=torch.int64)
    if w.planted:
        for b in range(w.B):
            for h in range(w.H_kv):
                ids = torch.randperm(M1, generator=gen)[:planted.shape[2]]
                planted[b, h] = ids
                for i in ids.tolist():
                    K[b, i * w.C:(i + 1) * w.C, h, :] *= 3.0
    dt = w.torch_dtype
    Q, K = Q.to(dt), K.to(dt)
    V = V.to(dt) if V is not None else None
    if device != "cpu":
        Q, K = Q.to(device), K.to(device)
        V = V.to(device) if V is not None else None
    return Q, K, V, planted


def make_decode(w: Workload, device, chunk_tokens: int = 1 << 16):
    """Decode workload drawn on ``device`` with a device generator (seed w.seed).

    Returns (K_cache, V_cache, q_steps, k_steps, v_steps):
      K_cache, V_cache [B, N + steps, H_kv, d]: the first N tokens filled, the
        rest zero (filled by the caller as tokens are appended);
      q_steps [steps, B, H_q, d], k_steps / v_steps [steps, B, H_kv, d].
    The caches are drawn sequence by sequence in chunks of ``chunk_tokens``
    tokens, K before V, then the per-step tensors in the order q, k, v.
    """
    dt = w.torch_dtype
    gen = torch.Generator(device=device).manual_seed(w.seed)
    cap = w.N + w.steps
    Kc = torch.zeros(w.B, cap, w.H_kv, w.d, dtype=dt, device=device)
    Vc = torch.zeros(w.B, cap, w.H_kv, w.d, dtype=dt, device=device)
    for b in range(w.B):
        for which in (Kc, Vc):
            for s in range(0, w.N, chunk_tokens):
                e = min(w.N, s + chunk_tokens)
                which[b, s:e] = torch.randn(e - s, w.H_kv, w.d, generator=gen,
                                            dtype=torch.float32, device=device).to(dt)
    q = torch.randn(w.steps, w.B, w.H_q, w.d, generator=gen, dtype=torch.float32,
                    device=device).to(dt)
    k = torch.randn(w.steps, w.B, w.H_kv, w.d, generator=gen, dtype=torch.float32,
                    device=device).to(dt)
    v = torch.randn(w.steps, w.B, w.H_kv, w.d, generator=gen, dtype=torch.float32,
                    device=device).to(dt)
    return Kc, Vc, q, k, v


def make_grad_out(shape, seed: int, dtype=torch.bfloat16):
    """Upstream gradient of the attention output: N(0, 1) float32 from its own seeded
    generator, rounded to ``dtype`` (RNE)."""
    gen = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(dtype)


def random_selection(seed: int, B: int, H_kv: int, N_q: int, K_top: int, C: int, kv_len, causal: bool = True,
                     empty_rows: float = 0.0):
    """Block ids [B][H_kv][N_q][K_top] int32 with the structure of a causal PISA
    selection, drawn at random (no scores): row r of sequence b sits at position
    kv_len[b] - N_q + r; under causal masking its eligible blocks are 0..c with
    c = position // C, and when more than K_top are eligible it keeps 0, c - 1 and
    c plus K_top - 3 distinct others, one drawn uniformly from each of K_top - 3
    equal strata of 1..c - 2; without causal masking every row keeps K_top of the
    ceil(kv_len / C) blocks the same way (no forced blocks). Ascending, -1 padded.
    A fraction ``empty_rows`` of the rows selects nothing."""
    import numpy as np
    rng = np.random.default_rng(seed)
    out = np.full((B, H_kv, N_q, K_top), -1, np.int32)
    r = np.arange(N_q)
    for b in range(B):
        n = int(kv_len[b])
        M = (n + C - 1) // C
        pos = n - N_q + r
        for h in range(H_kv):
            if causal:
                c = pos // C
                lo, span, nf = 1, c - 2, 3       # strata over 1 .. c - 2, plus 0, c - 1, c
            else:
                c = np.full(N_q, M - 1)
                lo, span, nf = 0, np.full(N_q, M), 0
            E = c + 1
            k_free = K_top - nf
            sel = np.full((N_q, K_top), -1, np.int64)
            small = E <= K_top
            if small.any():
                ar = np.arange(K_top)[None, :]
                sel[small] = np.where(ar < E[small, None], ar, -1)
            big = ~small
            if big.any() and k_free > 0:
                sp = span[big].astype(np.int64)[:, None]
                u = rng.random((int(big.sum()), k_free))
                j = np.arange(k_free + 1)[None, :]
                edge = (j * sp) // k_free                      # integer strata [edge_j, edge_j+1)
                width = edge[:, 1:] - edge[:, :-1]             # >= 1: span >= k_free here
                strata = edge[:, :-1] + np.minimum(np.floor(u * width).astype(np.int64), width - 1) + lo
                if causal:
                    cb = c[big][:, None]
                    picks = np.concatenate([np.zeros_like(cb), strata, cb - 1, cb], axis=1)
                else:
                    picks = strata
                sel[big] = np.sort(picks, axis=1)
            if empty_rows > 0:
                sel[rng.random(N_q) < empty_rows] = -1
            out[b, h] = sel
    return out
