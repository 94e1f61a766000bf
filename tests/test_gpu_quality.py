"""GPU parity of the block-selection quality evaluation (pisa_selection_quality:
full-attention block masses, reference sets, Recall@K, captured mass, mass ratio;
section 4.4 eq 35-36, appendix D.2 eq 55-57) against the CPU oracle, through the
C ABI.

Tolerance: the masses are probabilities computed from fp32 log-sum-exps of bf16
products (fp32 sums, exp and log), so |P_gpu - P_oracle| <= 1e-5. The reference
set must equal the oracle's wherever the oracle's K_top-3-th and next non-forced
masses differ by at least 1e-5; inside that band it must be a valid reference
(forced blocks, distinct, eligible, of the right size) whose captured mass is
within 1e-5 of the oracle's. Recall is then exact and captured mass and ratio
within 1e-5 (3e-5 for the ratio, a quotient of two such sums)."""
import numpy as np
import pytest
import torch

import oracle
from hierarchical_top_amd import pisa, synth

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _gap(mass_row, c, K_top):
    """Oracle margin at the cut of the reference fill (inf when nothing is ranked)."""
    if c + 1 <= K_top:
        return np.inf
    free = np.array([mass_row[B] for B in range(c + 1) if B not in (0, c - 1, c)])
    s = np.sort(free)[::-1]
    k = K_top - 3
    return s[k - 1] - s[k] if k < len(s) else np.inf


def _compare(w, t, got, orc, b):
    M1 = -(-w.N // w.C)
    for h in range(w.H_kv):
        gm = got["mass"][b, h][t].double().cpu().numpy()
        np.testing.assert_allclose(gm, orc["mass"][:, h], rtol=0, atol=TOL)
        gr = got["ref"][b, h][t].cpu().numpy()
        grec = got["recall"][b, h][t].double().cpu().numpy()
        gcap = got["captured"][b, h][t].double().cpu().numpy()
        grat = got["ratio"][b, h][t].double().cpu().numpy()
        near = 0
        for k, pos in enumerate(t):
            c = int(pos) // w.C
            if (gr[k] == orc["ref"][k, h]).all():
                assert np.float32(grec[k]) == np.float32(orc["recall"][k, h])  # hits / K_top in fp32
            else:
                near += 1
                assert _gap(orc["mass"][k, h], c, w.K_top) < TOL, "reference differs outside the band at t=%d" % pos
                row = [int(x) for x in gr[k] if x >= 0]
                assert row == sorted(set(row)) and max(row) <= c and {0, c - 1, c} <= set(row)
                assert len(row) == w.K_top
                assert abs(orc["mass"][k, h][row].sum() - orc["mass"][k, h][orc["ref"][k, h]].sum()) < TOL
            np.testing.assert_allclose(gcap[k], orc["captured"][k, h], rtol=0, atol=TOL)
            np.testing.assert_allclose(grat[k], orc["ratio"][k, h], rtol=0, atol=3 * TOL)
        assert (gm.shape[1] == M1)
        print("b", b, "h", h, "near ties", near, "of", len(t))


CASES = {
    "d128_c64": synth.Workload("q1", 1, 2048, 8, 2, 128, 64, 4, 8, "bf16", 16, 61, False),
    "ragged_g16": synth.Workload("q2", 1, 1000, 32, 2, 64, 16, 2, 8, "bf16", 0, 62, False),
    "b2_c32_k12": synth.Workload("q3", 2, 1500, 4, 4, 64, 32, 4, 12, "bf16", 8, 63, False),
}


@pytest.mark.parametrize("case", list(CASES))
def test_selection_quality_matches_oracle(case):
    w = CASES[case]
    print("case", case, flush=True)
    Q, K, _, _ = synth.make_prefill(w)
    sel = synth.random_selection(11, w.B, w.H_kv, w.N, w.K_top, w.C, [w.N] * w.B, causal=True, empty_rows=0.01)
    got = pisa.selection_quality(Q.cuda(), K.cuda(), torch.from_numpy(sel).cuda(), w.C, with_mass=True, with_ref=True)
    torch.cuda.synchronize()
    t = np.arange(w.N)
    for b in range(w.B):
        orc = oracle.selection_quality(Q[b].float().numpy(), [b] * w.N, t, K.float().numpy(), w.N, w.C,
                                       sel[b].transpose(1, 0, 2), with_mass=True)
        _compare(w, t, got, orc, b)


def test_selection_quality_16k_sampled():
    """The 16K routing workload (16 / 4 heads, d=128, C=64, planted blocks) with the
    oracle's own PISA selection on sampled rows."""
    w = synth.workload("p16k")
    Q, K, _, _ = synth.make_prefill(w)
    t = np.unique(np.concatenate([np.linspace(0, w.N - 1, 160).astype(np.int64), np.arange(3 * w.C)]))
    opyr = oracle.Pyramid(K.float().numpy(), w.N, w.C, w.g)
    osel = oracle.route(opyr, Q[0, t].float().numpy(), [0] * len(t), t, w.K_top)["idx"]  # [n][H][K]
    full = np.full((1, w.H_kv, w.N, w.K_top), -1, np.int32)
    full[0][:, t] = osel.transpose(1, 0, 2)
    got = pisa.selection_quality(Q.cuda(), K.cuda(), torch.from_numpy(full).cuda(), w.C, with_mass=True,
                                 with_ref=True)
    torch.cuda.synchronize()
    orc = oracle.selection_quality(Q[0, t].float().numpy(), [0] * len(t), t, K.float().numpy(), w.N, w.C, osel,
                                   with_mass=True)
    _compare(w, t, got, orc, 0)
