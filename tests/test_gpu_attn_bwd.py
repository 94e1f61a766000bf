"""GPU parity of the block-sparse attention backward (pisa_sparse_attn_bwd) against
the CPU oracle's gradients of eq 6, through the C ABI.

The backward takes the forward's output O and log-normaliser; D = sum_e dO * O
stands for sum_j p_j dp_j (equal for the exact output). Two protocols:
  * kernel parity: O (rounded to bf16) and lse (rounded to fp32) come from the
    oracle's forward, and the oracle's backward is handed the same O. What is
    left is the kernel's own arithmetic -- P and dS as two bf16 terms (2^-17),
    fp32 sums and exp2 -- so per tensor max |gpu - oracle| <= 1e-4 of max |oracle|;
  * end to end: O and lse from the GPU forward, against the oracle's exact
    gradients. The bf16 output moves D by dO . (O - o), about 2^-9 of |dO| |O|,
    which shifts every dS_j by p_j times that; rows near the start see few keys,
    so |O| is large there. Per tensor max |gpu - oracle| <= 1e-2 of max |oracle|
    (dV, which does not involve D, 1e-4).
A wrong term (a missing -D, a transposed operand, a scale) moves a result by O(1)
of its size."""
import numpy as np
import pytest
import torch

import oracle
from hierarchical_top_amd import pisa, synth

pytestmark = pytest.mark.gpu

TIGHT = {"dQ": 1e-4, "dK": 1e-4, "dV": 1e-4}
END_TO_END = {"dQ": 1e-2, "dK": 1e-2, "dV": 1e-4}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs(B, N_alloc, N_q, H_q, H_kv, d, seed):
    gen = torch.Generator().manual_seed(seed)
    Q = torch.randn(B, N_q, H_q, d, generator=gen).to(torch.bfloat16)
    K = torch.randn(B, N_alloc, H_kv, d, generator=gen).to(torch.bfloat16)
    V = torch.randn(B, N_alloc, H_kv, d, generator=gen).to(torch.bfloat16)
    dO = synth.make_grad_out((B, N_q, H_q, d), seed + 1000)
    return Q, K, V, dO


def _gpu_grads(Q, K, V, dO, sel, C, N_kv, causal, kv_len=None, O=None, lse=None):
    """GPU gradients; O / lse given (oracle-made) or taken from the GPU forward."""
    Qd, Kd, Vd, dOd = Q.cuda(), K.cuda(), V.cuda(), dO.cuda()
    idx = torch.from_numpy(sel).cuda()
    kl = torch.tensor(kv_len, dtype=torch.int64, device="cuda") if kv_len is not None else None
    if O is None:
        O, lse = pisa.sparse_attn_clustered(Qd, Kd, Vd, idx, C, N_kv, causal=causal, kv_len=kl, with_lse=True)
    else:
        O, lse = O.cuda(), lse.cuda()
    # outputs start as a sentinel: the call must overwrite every element
    out = tuple(torch.full(x.shape, 777.0, dtype=torch.float32, device="cuda") for x in (Qd, Kd, Vd))
    dQ, dK, dV = pisa.sparse_attn_bwd(Qd, Kd, Vd, O, dOd, lse, idx, C, N_kv, causal=causal, kv_len=kl, out=out)
    torch.cuda.synchronize()
    return dQ.double().cpu().numpy(), dK.double().cpu().numpy(), dV.double().cpu().numpy()


def _oracle_forward(Q, K, V, sel, C, kv_len, causal):
    """Oracle forward output rounded to bf16 and log-normaliser rounded to fp32, laid out
    as the GPU forward writes them: O [B][N_q][H_q][d], lse [B][H_q][N_q]."""
    B, N_q, H_q, d = Q.shape
    O = torch.zeros(B, N_q, H_q, d, dtype=torch.bfloat16)
    lse = torch.zeros(B, H_q, N_q, dtype=torch.float32)
    for b in range(B):
        n = int(kv_len[b])
        t = n - N_q + np.arange(N_q)
        f = oracle.sparse_attn(Q[b].float().numpy(), [0] * N_q, t, K[b:b + 1].float().numpy(),
                               V[b:b + 1].float().numpy(), n, C, sel[b].transpose(1, 0, 2), causal=causal)
        O[b] = torch.from_numpy(f["out"]).to(torch.bfloat16)
        lse[b] = torch.from_numpy(f["lse"].T.copy()).float()
    return O, lse


def _oracle_grads(Q, K, V, dO, sel, C, kv_len, causal, O=None):
    B, N_q = Q.shape[:2]
    dQ = np.zeros(Q.shape)
    dK = np.zeros(K.shape)
    dV = np.zeros(V.shape)
    for b in range(B):
        n = int(kv_len[b])
        t = n - N_q + np.arange(N_q)
        g = oracle.sparse_attn_bwd(Q[b].float().numpy(), [0] * N_q, t, K[b:b + 1].float().numpy(),
                                   V[b:b + 1].float().numpy(), dO[b].float().numpy(), n, C,
                                   sel[b].transpose(1, 0, 2), causal=causal,
                                   O=O[b].float().numpy() if O is not None else None)
        dQ[b], dK[b], dV[b] = g["dQ"], g["dK"][0], g["dV"][0]
    return dQ, dK, dV


def _check_all(tol, got, want):
    bad = []
    for name, g, w in zip(("dQ", "dK", "dV"), got, want):
        scale = np.abs(w).max()
        err = np.abs(g - w).max()
        print("%s max |gpu - oracle| %.3g of max |oracle| %.3g (%.2e relative)" % (name, err, scale, err / scale))
        if not err <= tol[name] * scale:
            bad.append("%s: %g > %g" % (name, err, tol[name] * scale))
    assert not bad, bad


def _check(name, got, want, tol):
    scale = np.abs(want).max()
    err = np.abs(got - want).max()
    print("%s max |gpu - oracle| %.3g of max |oracle| %.3g (%.2e relative)" % (name, err, scale, err / scale))
    assert err <= tol[name] * scale, "%s: %g > %g" % (name, err, tol[name] * scale)


CASES = {
    # name: B, N_alloc, N_q, H_q, H_kv, d, C, K_top, causal, kv_len, empty-row fraction
    "ragged_c16": (1, 1000, 1000, 4, 2, 64, 16, 8, True, None, 0.0),
    "d128_c64": (1, 2048, 2048, 16, 4, 128, 64, 8, True, None, 0.02),
    "c32_b2": (2, 2100, 2100, 8, 2, 128, 32, 8, True, None, 0.0),
    "g16_d64": (1, 1024, 1024, 32, 2, 64, 64, 8, True, None, 0.0),
    "g1_noncausal": (1, 777, 777, 2, 2, 64, 32, 6, False, None, 0.0),
    "suffix_rows": (2, 1600, 200, 8, 4, 64, 16, 8, True, [1600, 1111], 0.0),
    "d128_c16_g8": (1, 1500, 1500, 16, 2, 128, 16, 8, True, None, 0.0),
}


@pytest.mark.parametrize("case", list(CASES))
def test_attention_backward_matches_oracle(case):
    B, N_alloc, N_q, H_q, H_kv, d, C, K_top, causal, kv_len, empty = CASES[case]
    print("case", case, flush=True)
    kv = kv_len or [N_alloc] * B
    Q, K, V, dO = _inputs(B, N_alloc, N_q, H_q, H_kv, d, seed=sum(map(ord, case)))
    sel = synth.random_selection(7, B, H_kv, N_q, K_top, C, kv, causal=causal, empty_rows=empty)
    O, lse = _oracle_forward(Q, K, V, sel, C, kv, causal)
    got = _gpu_grads(Q, K, V, dO, sel, C, max(kv), causal, kv_len, O=O, lse=lse)
    _check_all(TIGHT, got, _oracle_grads(Q, K, V, dO, sel, C, kv, causal, O=O))
    print("end to end (GPU forward output)")
    got_e2e = _gpu_grads(Q, K, V, dO, sel, C, max(kv), causal, kv_len)
    _check_all(END_TO_END, got_e2e, _oracle_grads(Q, K, V, dO, sel, C, kv, causal))
    if empty:
        rows = (sel < 0).all(-1)  # [B][H_kv][N_q]
        G = H_q // H_kv
        for h in range(H_kv):
            assert (got[0][0][rows[0, h]][:, h * G:(h + 1) * G] == 0).all()


def test_attention_backward_dense_selection():
    """Every row selects every block (more than 256 rows per block: several chunks per
    block add into the same dK, dV rows): the gradients of dense causal attention."""
    B, N, H_q, H_kv, d, C = 1, 512, 4, 1, 128, 16
    Q, K, V, dO = _inputs(B, N, N, H_q, H_kv, d, seed=77)
    M1 = N // C
    sel = np.tile(np.arange(M1, dtype=np.int32), (B, H_kv, N, 1))
    O, lse = _oracle_forward(Q, K, V, sel, C, [N], True)
    got = _gpu_grads(Q, K, V, dO, sel, C, N, True, O=O, lse=lse)
    _check_all(TIGHT, got, _oracle_grads(Q, K, V, dO, sel, C, [N], True, O=O))


def test_attention_backward_full_size_64k():
    """The 64K attention workload (32 query / 8 KV heads, d=128, C=64, K_top=8) with a
    random causal selection, end to end (GPU forward output): dQ of sampled rows against the oracle (a row's dQ depends on
    that row only), dK and dV of sampled non-forced blocks against the oracle run over
    every row that selected them, and at every size: per (sequence, KV head) the key
    gradients sum to zero and the value gradients to the rows' upstream gradients."""
    w = synth.workload("p64k")
    Q, K, V, _ = synth.make_prefill(w)
    dO = synth.make_grad_out(Q.shape, 303)
    sel = synth.random_selection(8, w.B, w.H_kv, w.N, w.K_top, w.C, [w.N], causal=True)
    dQ, dK, dV = _gpu_grads(Q, K, V, dO, sel, w.C, w.N, True)
    G = w.G_Q
    Kf, Vf = K[0:1].float().numpy(), V[0:1].float().numpy()
    # sampled rows
    t = np.unique(np.concatenate([np.linspace(0, w.N - 1, 300).astype(np.int64), np.arange(2 * w.C)]))
    g = oracle.sparse_attn_bwd(Q[0, t].float().numpy(), [0] * len(t), t, Kf, Vf, dO[0, t].float().numpy(), w.N, w.C,
                               sel[0][:, t].transpose(1, 0, 2))
    _check("dQ", dQ[0, t], g["dQ"], END_TO_END)
    # sampled blocks of two KV heads: the oracle over every row that selected the block
    rng = np.random.default_rng(5)
    for h in (1, 6):
        for blk in rng.choice(np.arange(8, w.N // w.C - 8), size=2, replace=False):
            rows = np.nonzero((sel[0, h] == blk).any(-1))[0]
            gb = oracle.sparse_attn_bwd(Q[0, rows].float().numpy(), [0] * len(rows), rows, Kf, Vf,
                                        dO[0, rows].float().numpy(), w.N, w.C, sel[0][:, rows].transpose(1, 0, 2))
            ks = slice(blk * w.C, (blk + 1) * w.C)
            print("block", blk, "head", h, "rows", len(rows))
            _check("dK", dK[0, ks, h], gb["dK"][0, ks, h], END_TO_END)
            _check("dV", dV[0, ks, h], gb["dV"][0, ks, h], END_TO_END)
    seen = (sel[0] >= 0).any(-1)  # [H_kv][N]
    dOf = dO[0].double().numpy()
    for h in range(w.H_kv):
        sk = dK[0, :, h].sum(0)
        assert np.abs(sk).max() <= 1e-3 * np.abs(dK[0, :, h]).sum(0).max(), "key gradients do not sum to zero"
        want = dOf[seen[h]][:, h * G:(h + 1) * G].sum((0, 1))
        np.testing.assert_allclose(dV[0, :, h].sum(0), want, rtol=0, atol=1e-3 * np.abs(want).max() + 1e-2)


def test_attention_backward_dq_is_deterministic():
    """dQ is summed over a row's blocks in slot order: two runs give identical bits (dK and
    dV take atomics and agree to rounding)."""
    B, N, H_q, H_kv, d, C, K_top = 1, 3000, 8, 2, 128, 64, 8
    Q, K, V, dO = _inputs(B, N, N, H_q, H_kv, d, seed=91)
    sel = synth.random_selection(9, B, H_kv, N, K_top, C, [N], causal=True)
    a = _gpu_grads(Q, K, V, dO, sel, C, N, True)
    b = _gpu_grads(Q, K, V, dO, sel, C, N, True)
    assert np.array_equal(a[0], b[0])
    for x, y in zip(a[1:], b[1:]):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-5 * np.abs(x).max())
