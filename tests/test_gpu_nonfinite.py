"""Non-finite inputs (NaN or inf in Q or K): every router, the decode router and the
exhaustive selector still return valid selections -- ascending, distinct, causal block ids,
-1 padded, the forced blocks present -- and attention runs on them. A candidate whose score
is NaN is never picked, so a row can hold fewer than K_top blocks (the level router's exact
log-sum-exp turns a head whose logits are all NaN into -inf, which still ranks, lowest id
first). Nothing here compares with the oracle: the pages define the selection for finite
inputs only."""
import numpy as np
import pytest
import torch

import oracle
from hierarchical_top_amd import pisa, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _poison(w):
    """Seeded inputs of w with NaN query rows (every 97th position, first head of each group),
    a NaN key in leaf block 5 and an inf key in leaf block 9 of every KV head."""
    Q, K = synth.make_prefill(w)[:2]
    Q, K = Q.clone(), K.clone()
    G = w.H_q // w.H_kv
    Q[:, ::97, ::G] = float("nan")
    K[:, 5 * w.C + 3] = float("nan")
    K[:, 9 * w.C + 1] = float("inf")
    return Q, K


def _check_rows(idx, N, C, K_top, causal=True):
    """idx [B][H][N][K_top] (numpy): every row a valid selection."""
    B, H = idx.shape[:2]
    t = np.arange(N)
    c = t // C
    valid = idx >= 0
    assert ((idx >= 0) | (idx == -1)).all(), "negative id other than the -1 padding"
    # -1 padding only at the end of a row
    assert (np.diff(valid.astype(np.int8), axis=-1) <= 0).all(), "padding before a block id"
    # consecutive block ids strictly increase
    assert (np.diff(idx, axis=-1)[valid[..., 1:]] > 0).all(), "block ids not ascending and distinct"
    assert (idx < -(-N // C)).all(), "block id past the last block"
    if causal:
        assert (np.where(valid, idx, 0) <= c[None, None, :, None]).all(), "future block"
        has = lambda x: ((idx == x[None, None, :, None]).any(-1))
        assert has(np.zeros_like(c)).all(), "first block missing"
        assert has(c).all(), "current block missing"
        assert has(np.maximum(c - 1, 0)).all(), "previous block missing"
    n = valid.sum(-1)
    assert (n >= 1).all() and (n <= K_top).all()
    return float((n < np.minimum(K_top, c + 1)[None, None]).mean())


CASES = [
    # dense top levels, then the leaf (g = 4)
    synth.Workload("nf_dense", 1, 4000, 8, 2, 128, 64, 4, 8, "bf16", 0, 71, True),
    # sparse upper levels (more than 16 parents) and a ragged tail
    synth.Workload("nf_sparse", 1, 70001, 4, 2, 128, 64, 4, 8, "bf16", 0, 72, True),
    # g = 2, 64 candidates per item
    synth.Workload("nf_wide", 1, 20000, 8, 2, 128, 32, 2, 32, "bf16", 0, 73, True),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_routers_return_valid_selections_on_nonfinite_inputs(w):
    print("case", w.name, flush=True)
    Q, K = _poison(w)
    Qd, Kd = Q.cuda(), K.cuda()
    pyr = pisa.Pyramid(w.B, w.H_kv, w.d, w.C, w.g, w.N)
    pyr.build(Kd, w.N)
    for name, mode in (("levels", pisa.LEVELS), ("fused", pisa.FUSED), ("two_stage", pisa.TWO_STAGE)):
        print("router", name, flush=True)
        idx, _ = pisa.route_prefill(pyr, Qd, Kd, w.N, w.K_top, mode=mode, with_score=True)
        torch.cuda.synchronize()
        short = _check_rows(idx.cpu().numpy(), w.N, w.C, w.K_top)
        print(w.name, name, "rows with fewer blocks than K_top", short)
    if w.K_top <= 16:
        print("exhaustive selector", flush=True)
        idx, _ = pisa.bsa_select(pyr, Qd, w.N, w.K_top, with_score=True)
        torch.cuda.synchronize()
        _check_rows(idx.cpu().numpy(), w.N, w.C, w.K_top)
    # attention over the level router's selection (per-row and clustered)
    idx, _ = pisa.route_prefill(pyr, Qd, Kd, w.N, w.K_top, mode=pisa.LEVELS, with_score=True)
    V = torch.randn(K.shape, generator=torch.Generator().manual_seed(5)).to(K.dtype).cuda()
    for fn in (pisa.sparse_attn, pisa.sparse_attn_clustered):
        O = fn(Qd, Kd, V, idx, w.C, w.N)
        torch.cuda.synchronize()
        assert O.shape == Qd.shape


def test_decode_returns_valid_selections_on_nonfinite_inputs():
    B, H_q, H, d, C, g, K_top = 4, 8, 2, 128, 64, 4, 8
    lens = [5000, 4097, 1300, 700]
    cap = max(lens)
    gen = torch.Generator().manual_seed(74)
    K = torch.randn(B, cap, H, d, generator=gen).to(torch.bfloat16)
    q = torch.randn(B, H_q, d, generator=gen).to(torch.bfloat16)
    K[0, 5 * C + 3] = float("nan")
    K[1, 9 * C + 1] = float("inf")
    q[2, 0] = float("nan")
    K, q = K.cuda(), q.cuda()
    pyr = pisa.Pyramid(B, H, d, C, g, cap)
    for b in range(B):  # one build per length: sequence b's pyramid covers its own prefix
        one = pisa.Pyramid(1, H, d, C, g, cap)
        one.build(K[b:b + 1].contiguous(), lens[b])
        for l in range(1, len(oracle.levels(lens[b], C, g))):
            pyr.level(l)[b].copy_(one.level(l)[0])
    seqlen = torch.tensor(lens, dtype=torch.int64, device="cuda")
    idx, _ = pisa.route_decode(pyr, q, K, seqlen, K_top, with_score=True)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()  # [B][H][K_top]: the newest position of each sequence
    for b in range(B):
        n = lens[b]
        c = (n - 1) // C
        for h in range(H):
            row = [int(x) for x in idx[b, h]]
            got = [x for x in row if x >= 0]
            assert row[len(got):] == [-1] * (K_top - len(got)), row
            assert got == sorted(set(got)) and all(0 <= x <= c for x in got), row
            assert {0, c, max(c - 1, 0)} <= set(got), row
