"""GPU parity of the pyramid build and of prefill routing (fused and two-stage)
against the CPU oracle, through the C ABI (hierarchical_top_amd.pisa)."""
import functools

import numpy as np
import pytest
import torch

import oracle
from hierarchical_top_amd import pisa, synth
from tests.parity import compare, route_reach

pytestmark = pytest.mark.gpu

MODES = {"two_stage": pisa.TWO_STAGE, "fused": pisa.FUSED, "levels": pisa.LEVELS}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def custom(name, **kw):
    return synth.workload(name, **kw)


CASES = {
    "tiny": custom("tiny"),
    # ragged tail (partial leaf and partial nodes), grouped heads, bf16
    "ragged": synth.Workload("ragged", 1, 1000, 4, 2, 64, 16, 4, 8, "bf16", 0, 21, False),
    # two sequences, eight-head groups, d=128
    "batch2_g8": synth.Workload("b2g8", 2, 3000, 16, 2, 128, 32, 2, 8, "bf16", 4, 22, False),
    # the page's grouping (16 query heads per KV head), g=2, d=64
    "paper_shape": synth.Workload("paper", 1, 4096, 32, 2, 64, 64, 2, 8, "bf16", 0, 23, False),
    # fp32 with two-head groups
    "f32_g2": synth.Workload("f32g2", 1, 777, 4, 2, 64, 16, 2, 6, "f32", 0, 24, False),
    "p16k": custom("p16k"),
    # large enough that the level router scores an upper level sparsely (more than 16 parents)
    "sparse64k": synth.Workload("s64k", 1, 65536, 8, 2, 128, 64, 4, 8, "bf16", 0, 26, False),
    # the page's benchmark shape at a length whose upper levels are scored sparsely
    "paper64k": synth.paper_shape(65536, seed=27),
    # ragged length: sparse levels 3 and 2 with tail nodes missing grandchildren, two-head groups
    "ragged_big": synth.Workload("rbig", 1, 70001, 4, 2, 128, 64, 4, 8, "bf16", 0, 25, False),
    # g=2 with K_top above 16 (level nodes 625, 313, 157, 79, 40, 20, 10, ...): at K_top=18 the top
    # ranked level is scored densely and the rest sparsely, at K_top=32 every upper level sparsely
    "g2_wide": synth.Workload("g2w", 1, 20000, 8, 2, 128, 32, 2, 8, "bf16", 0, 28, False),
}


@functools.lru_cache(maxsize=1)  # the routers of one case run back to back
def _inputs(w):
    Q, K, V, _ = synth.make_prefill(w)
    return Q, K


def _oracle_route(w, Q, K, K_top, causal, t, score_kind="lse"):
    pyr = oracle.Pyramid(K.float().numpy(), w.N, w.C, w.g)
    res = []
    for b in range(w.B):
        res.append(oracle.route(pyr, Q[b, t].float().numpy(), [b] * len(t), t, K_top, causal=causal,
                                score_kind=score_kind))
    return pyr, res


def _gpu_route(w, Q, K, K_top, causal, mode, score_kind="lse"):
    Qd, Kd = Q.cuda(), K.cuda()
    pyr = pisa.Pyramid(w.B, w.H_kv, w.d, w.C, w.g, w.N)
    pyr.build(Kd, w.N)
    # outputs start as a sentinel so that nothing left in reused memory can pass for a result
    out = torch.full((w.B, w.H_kv, w.N, K_top), -7, dtype=torch.int32, device="cuda")
    sco = torch.full((w.B, w.H_kv, w.N, K_top), 12345.0, dtype=torch.float32, device="cuda")
    idx, score = pisa.route_prefill(pyr, Qd, Kd, w.N, K_top, causal=causal, mode=mode, with_score=True, out=out,
                                    score_out=sco, score_kind=score_kind)
    torch.cuda.synchronize()
    return pyr, idx.cpu().numpy(), score.cpu().numpy()


@pytest.mark.parametrize("case", ["tiny", "ragged", "batch2_g8", "p16k"])
def test_pyramid_build_matches_oracle(case):
    """fp32 sums in token order vs fp64: |err| <= (n - 1) * 2^-24 * sum|x| / n + ulp, bounded
    here by 4e-5 for |x| <= 20 (planted keys are N(0,1) * 3 rounded to bf16)."""
    w = CASES[case]
    Q, K = _inputs(w)
    opyr = oracle.Pyramid(K.float().numpy(), w.N, w.C, w.g)
    pyr = pisa.Pyramid(w.B, w.H_kv, w.d, w.C, w.g, w.N)
    pyr.build(K.cuda(), w.N)
    torch.cuda.synchronize()
    for l in range(1, opyr.L + 1):
        got = pyr.level(l)[:, :, :opyr.M[l]].double().cpu().numpy()
        np.testing.assert_allclose(got, opyr.level(l), rtol=0, atol=4e-5, err_msg="level %d" % l)


def _positions(w, sample):
    if sample is None or sample >= w.N:
        return np.arange(w.N)
    t = np.unique(np.concatenate([np.linspace(0, w.N - 1, sample).astype(np.int64), np.arange(3 * w.C),
                                  np.arange(w.N - w.C, w.N)]))
    return t


@pytest.mark.parametrize("mode", ["two_stage", "fused", "levels"])
@pytest.mark.parametrize("case,K_top,causal,sample", [
    ("tiny", 4, True, None),
    ("tiny", 32, True, None),
    ("tiny", 64, True, None),
    ("tiny", 4, False, None),
    ("ragged", 8, True, None),
    ("ragged", 8, False, None),
    ("batch2_g8", 8, True, None),
    ("paper_shape", 8, True, None),
    ("f32_g2", 6, True, None),
    ("p16k", 8, True, None),
    ("sparse64k", 8, True, 600),
    ("ragged_big", 8, True, 600),
    ("paper64k", 8, True, 600),
    ("g2_wide", 18, True, 600),
    ("g2_wide", 32, True, 600),
])
def test_route_matches_oracle(mode, case, K_top, causal, sample):
    w = CASES[case]
    print("case", case, "mode", mode, "K_top", K_top, "causal", causal, flush=True)
    Q, K = _inputs(w)
    t = _positions(w, sample)
    opyr, orc = _oracle_route(w, Q, K, K_top, causal, t)
    _, idx, score = _gpu_route(w, Q, K, K_top, causal, MODES[mode])
    M1 = -(-w.N // w.C)
    for b in range(w.B):
        gi = idx[b][:, t].transpose(1, 0, 2)
        gs = score[b][:, t].transpose(1, 0, 2)
        # the share of items whose oracle route has a cut within the band grows with K_top: at
        # g=2 and K_top > 16 about five levels of ~60 candidates are ranked and the oracle's own
        # near-tie share on g2_wide is 0.24 (K_top=18) and 0.26 (K_top=32)
        stats = compare(gi, gs, orc[b], t, w.C, K_top, causal=causal, M1=M1,
                        max_near_tie_frac=0.35 if K_top > 16 else 0.25,
                        reach=route_reach(opyr, Q[b, t].float().numpy(), b, t, K_top, causal))
        print(case, mode, b, stats)


@pytest.mark.parametrize("mode", ["levels", "fused"])
@pytest.mark.parametrize("kind", ["mean", "mean_var"])
@pytest.mark.parametrize("case,K_top,causal,sample", [
    ("tiny", 4, True, None),          # fp32: LDS-staged and register-row scoring, dense top levels
    ("tiny", 4, False, None),
    ("ragged", 8, True, None),        # bf16, g=4, two-head groups: streaming kernels, partial leaf and nodes
    ("batch2_g8", 8, True, None),     # two sequences, g=2, eight-head groups, C=32
    ("paper_shape", 8, True, None),   # sixteen-head groups: LDS-staged scoring
    ("f32_g2", 6, True, None),
    ("p16k", 8, True, None),
    ("sparse64k", 8, True, 600),      # sparse upper levels
    ("ragged_big", 8, True, 600),     # tail nodes missing grandchildren at sparse levels
    ("g2_wide", 32, True, 600),       # g=2, 64 candidates per item at every ranked level
])
def test_route_pisa1_pisa2_match_oracle(kind, case, K_top, causal, sample, mode):
    """PISA-1 (mean logit) and PISA-2 (mean + half the variance) block scores of section 4.4,
    on the level-synchronous and the fused per-query routers: same protocol as the LSE score."""
    w = CASES[case]
    print("case", case, "score", kind, "mode", mode, "K_top", K_top, "causal", causal, flush=True)
    Q, K = _inputs(w)
    t = _positions(w, sample)
    opyr, orc = _oracle_route(w, Q, K, K_top, causal, t, score_kind=kind)
    _, idx, score = _gpu_route(w, Q, K, K_top, causal, MODES[mode], score_kind=kind)
    M1 = -(-w.N // w.C)
    # PISA-1's upper-level scores are logits of mean keys, whose spread shrinks with the span of
    # the node, so more items than under LSE have a ranked level inside the 1e-3 band (26 % on
    # the 70,001-token case, 24 % under PISA-2); the cap only guards against a vacuous comparison
    cap = 0.4
    for b in range(w.B):
        gi = idx[b][:, t].transpose(1, 0, 2)
        gs = score[b][:, t].transpose(1, 0, 2)
        stats = compare(gi, gs, orc[b], t, w.C, K_top, causal=causal, M1=M1, max_near_tie_frac=cap,
                        reach=route_reach(opyr, Q[b, t].float().numpy(), b, t, K_top, causal, score_kind=kind))
        print(case, kind, b, stats)


def test_pisa1_leaf_score_is_the_summary_logit():
    """The mean of a leaf's raw-key logits is the logit of the leaf's mean key (linearity):
    PISA-1's leaf scores must equal the head sums of q . kbar^(1) / sqrt(d), computed here in
    fp64 from the GPU-built level-1 summaries."""
    w = CASES["ragged"]
    Q, K = _inputs(w)
    pyr, idx, score = _gpu_route(w, Q, K, 8, True, pisa.LEVELS, score_kind="mean")
    lv1 = pyr.level(1)[0].double().cpu()                      # [H_kv][M1][d]
    G = w.H_q // w.H_kv
    q = Q[0].double().reshape(w.N, w.H_kv, G, w.d)           # [N][H_kv][G][d]
    n_checked = 0
    for h in range(w.H_kv):
        logits = torch.einsum("tgd,md->tgm", q[:, h], lv1[h, :-(-w.N // w.C)]).sum(1) / w.d ** 0.5  # [N][M1]
        sel, sc = idx[0, h], score[0, h]
        fin = np.isfinite(sc)
        tt, kk = np.nonzero(fin)
        want = logits[tt, sel[tt, kk]].numpy()
        np.testing.assert_allclose(sc[tt, kk], want, rtol=0, atol=1e-4)
        n_checked += len(tt)
    assert n_checked > 1000


def test_routers_agree_and_are_deterministic():
    w = CASES["p16k"]
    Q, K = _inputs(w)
    _, i1, s1 = _gpu_route(w, Q, K, 8, True, pisa.TWO_STAGE)
    _, i2, s2 = _gpu_route(w, Q, K, 8, True, pisa.TWO_STAGE)
    _, i3, s3 = _gpu_route(w, Q, K, 8, True, pisa.FUSED)
    _, i4, s4 = _gpu_route(w, Q, K, 8, True, pisa.LEVELS)
    _, i5, s5 = _gpu_route(w, Q, K, 8, True, pisa.LEVELS)
    assert (i1 == i2).all() and np.array_equal(s1, s2, equal_nan=True)  # bit-identical reruns
    assert (i4 == i5).all() and np.array_equal(s4, s5, equal_nan=True)
    for other, name in ((i3, "fused"), (i4, "levels")):
        diff = (i1 != other).any(-1).mean()
        assert diff < 0.01, "%s and two-stage disagree on %.4f of the selections" % (name, diff)


def test_outputs_are_fully_written():
    w = CASES["ragged"]
    Q, K = _inputs(w)
    Qd, Kd = Q.cuda(), K.cuda()
    pyr = pisa.Pyramid(w.B, w.H_kv, w.d, w.C, w.g, w.N)
    pyr.build(Kd, w.N)
    for mode in (pisa.TWO_STAGE, pisa.FUSED, pisa.LEVELS):
        ws = torch.full((pisa.route_workspace_bytes(pyr, w.N, w.H_q, 8, mode) + 1,), 0x5A, dtype=torch.uint8,
                        device="cuda")  # stale workspace contents must not matter
        out = torch.full((w.B, w.H_kv, w.N, 8), -7, dtype=torch.int32, device="cuda")
        sc = torch.full((w.B, w.H_kv, w.N, 8), 12345.0, dtype=torch.float32, device="cuda")
        pisa.route_prefill(pyr, Qd, Kd, w.N, 8, mode=mode, with_score=True, out=out, score_out=sc,
                           workspace=ws if ws.numel() > 1 else None)
        torch.cuda.synchronize()
        assert not (out == -7).any() and not (sc == 12345.0).any()
