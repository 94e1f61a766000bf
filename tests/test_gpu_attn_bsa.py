"""GPU parity of block-sparse attention and of the exhaustive (BSA-style)
selector against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from hierarchical_top_amd import pisa, synth
from tests.parity import bsa_reach, compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


W = {
    "tiny": synth.workload("tiny"),
    "ragged": synth.Workload("ragged", 1, 1000, 4, 2, 64, 16, 4, 8, "bf16", 0, 31, True),
    "c32_b2": synth.Workload("c32b2", 2, 2100, 8, 2, 128, 32, 4, 8, "bf16", 3, 32, True),
    "paper_shape": synth.Workload("paper", 1, 4096, 32, 2, 64, 64, 2, 8, "bf16", 0, 33, True),
    "f32_g4": synth.Workload("f32g4", 1, 600, 8, 2, 128, 32, 2, 5, "f32", 0, 34, True),
    "p64k": synth.workload("p64k"),
}
# attention output tolerance: bf16 outputs 2e-2 absolute; fp32 inputs go through two bf16 terms
ATOL = {"bf16": 2e-2, "f32": 2e-4}


def _positions(w, sample):
    if sample is None or sample >= w.N:
        return np.arange(w.N)
    return np.unique(np.concatenate([np.linspace(0, w.N - 1, sample).astype(np.int64), np.arange(3 * w.C),
                                     np.arange(w.N - w.C, w.N)]))


def _attn(entry, *args, **kw):
    """The per-row entry point or the one clustered by selected block (bf16)."""
    fn = pisa.sparse_attn if entry == "rows" else pisa.sparse_attn_clustered
    return fn(*args, **kw)


@pytest.mark.parametrize("entry", ["rows", "clustered"])
@pytest.mark.parametrize("case,causal,sample,dense", [
    ("tiny", True, None, False),
    ("tiny", True, None, True),
    ("tiny", False, None, False),
    ("ragged", True, None, False),
    ("ragged", True, None, True),  # bf16, every row selects all 63 blocks (clustered: 63 slots per row)
    ("ragged", False, None, False),
    ("c32_b2", True, None, False),
    ("paper_shape", True, 1024, False),
    ("f32_g4", True, None, False),
    ("p64k", True, 1024, False),
])
def test_sparse_attention_matches_oracle(case, causal, sample, dense, entry):
    w = W[case]
    if entry == "clustered" and w.dtype != "bf16":
        pytest.skip("the clustered entry point takes bf16 inputs")
    print("case", case, "causal", causal, "dense", dense, "entry", entry, flush=True)
    Q, K, V, _ = synth.make_prefill(w)
    t = _positions(w, sample)
    M1 = -(-w.N // w.C)
    K_top = M1 if dense else w.K_top
    opyr = oracle.Pyramid(K.float().numpy(), w.N, w.C, w.g)
    Kf, Vf = K.float().numpy(), V.float().numpy()
    Qd, Kd, Vd = Q.cuda(), K.cuda(), V.cuda()
    for b in range(w.B):
        if dense:
            sel = np.tile(np.arange(M1, dtype=np.int32), (len(t), w.H_kv, 1))
        else:
            sel = oracle.route(opyr, Q[b, t].float().numpy(), [b] * len(t), t, K_top, causal=causal)["idx"]
        want = oracle.sparse_attn(Q[b, t].float().numpy(), [0] * len(t), t, Kf[b:b + 1], Vf[b:b + 1], w.N, w.C,
                                  sel, causal=causal)
        # GPU: full [B][H][N][K] index tensor, rows outside the sample select nothing
        full = np.full((w.B, w.H_kv, w.N, K_top), -1, np.int32)
        full[b][:, t] = sel.transpose(1, 0, 2)
        idx = torch.from_numpy(full).cuda()
        O, lse = _attn(entry, Qd, Kd, Vd, idx, w.C, w.N, causal=causal, with_lse=True)
        torch.cuda.synchronize()
        got = O[b, t].float().cpu().numpy()
        err = np.abs(got - want["out"]).max()
        print(case, "b", b, "max |O - oracle|", err)
        assert err <= ATOL[w.dtype], err
        gl = lse[b][:, t].t().cpu().numpy()
        np.testing.assert_allclose(gl, want["lse"], atol=1e-3 if w.dtype == "bf16" else 1e-4)


def test_clustered_attention_every_row_64k():
    """The 64K workload (32 query / 8 KV heads, d=128, C=64, K_top=8) with EVERY row selecting
    blocks -- a structured random causal selection (first, previous and current block plus one
    block from each of five strata of the older ones), drawn without scores -- so that every
    block's cluster spans many chunks, as in the benchmark. Sampled rows against the oracle."""
    w = W["p64k"]
    Q, K, V, _ = synth.make_prefill(w)
    sel_all = synth.random_selection(61, w.B, w.H_kv, w.N, w.K_top, w.C, [w.N], causal=True)
    t = _positions(w, 900)
    print("rows", w.N, "sampled", len(t), flush=True)
    O, lse = pisa.sparse_attn_clustered(Q.cuda(), K.cuda(), V.cuda(), torch.from_numpy(sel_all).cuda(), w.C, w.N,
                                        with_lse=True)
    torch.cuda.synchronize()
    sel = np.ascontiguousarray(sel_all[0][:, t].transpose(1, 0, 2))  # [n][H][K]
    want = oracle.sparse_attn(Q[0, t].float().numpy(), [0] * len(t), t, K.float().numpy(), V.float().numpy(), w.N,
                              w.C, sel)
    err = np.abs(O[0, t].float().cpu().numpy() - want["out"]).max()
    print("max |O - oracle|", err)
    assert err <= ATOL["bf16"], err
    np.testing.assert_allclose(lse[0][:, t].t().cpu().numpy(), want["lse"], atol=1e-3)


@pytest.mark.parametrize("entry", ["rows", "clustered"])
def test_attention_decode_rows_and_empty_rows(entry):
    """N_q = 1 with per-sequence lengths (decode shape); a row whose blocks are all
    masked or absent returns zeros and lse = -inf."""
    w = synth.Workload("dec", 3, 700, 8, 2, 64, 16, 4, 6, "bf16", 0, 35, True)
    Q, K, V, _ = synth.make_prefill(w)
    lens = np.array([700, 513, 1])
    opyr = None
    q = torch.stack([Q[b, lens[b] - 1] for b in range(3)])  # [B][H_q][d]
    sel = np.full((3, w.H_kv, 1, w.K_top), -1, np.int32)
    want = []
    for b in range(3):
        n = int(lens[b])
        opyr = oracle.Pyramid(K[b:b + 1, :n].float().numpy(), n, w.C, w.g)
        r = oracle.route(opyr, q[b:b + 1].float().numpy(), [0], [n - 1], w.K_top)
        sel[b, :, 0] = r["idx"][0]
        want.append(oracle.sparse_attn(q[b:b + 1].float().numpy(), [0], [n - 1], K[b:b + 1].float().numpy(),
                                       V[b:b + 1].float().numpy(), n, w.C, r["idx"]))
    sel_d = torch.from_numpy(sel).cuda()
    kv = torch.from_numpy(lens.astype(np.int64)).cuda()
    O, lse = _attn(entry, q.unsqueeze(1).contiguous().cuda(), K.cuda(), V.cuda(), sel_d, w.C, w.N,
                   kv_len=kv, with_lse=True)
    torch.cuda.synchronize()
    for b in range(3):
        np.testing.assert_allclose(O[b, 0].float().cpu().numpy(), want[b]["out"][0], atol=2e-2)
    # empty selection -> zeros, -inf
    none = torch.full_like(sel_d, -1)
    O2, lse2 = _attn(entry, q.unsqueeze(1).contiguous().cuda(), K.cuda(), V.cuda(), none, w.C, w.N,
                     kv_len=kv, with_lse=True)
    torch.cuda.synchronize()
    assert (O2 == 0).all() and torch.isneginf(lse2).all()


def _bsa_compare(w, t, causal, K_top):
    Q, K, V, _ = synth.make_prefill(w)
    opyr = oracle.Pyramid(K.float().numpy(), w.N, w.C, w.g)
    pyr = pisa.Pyramid(w.B, w.H_kv, w.d, w.C, w.g, w.N)
    Qd, Kd = Q.cuda(), K.cuda()
    pyr.build(Kd, w.N)
    idx, score = pisa.bsa_select(pyr, Qd, w.N, K_top, causal=causal, with_score=True)
    torch.cuda.synchronize()
    idx, score = idx.cpu().numpy(), score.cpu().numpy()
    for b in range(w.B):
        orc = oracle.bsa(opyr, Q[b, t].float().numpy(), [b] * len(t), t, K_top, causal=causal)
        # tie band relative to the size of the summed probabilities of the last kept leaf
        s = orc["score"]
        fin = np.where(np.isfinite(s), s, np.nan)
        ukth = np.nan_to_num(np.nanmin(fin, axis=-1), nan=1.0)
        band = 1e-4 * np.abs(ukth) + 1e-9
        # strict band a tenth of that: fp32 scores of summed probabilities are within ~1e-7 relative
        stats = compare(idx[b][:, t].transpose(1, 0, 2), score[b][:, t].transpose(1, 0, 2), orc, t, w.C, K_top,
                        causal=causal, band=band, strict=band / 10, score_tol=1e-7, score_rtol=1e-4,
                        M1=-(-w.N // w.C), reach=bsa_reach(opyr, Q[b, t].float().numpy(), b, t, K_top, causal))
        print(w.name, b, stats)


@pytest.mark.parametrize("case,causal,K_top,sample", [
    ("tiny", True, 4, None),
    ("tiny", False, 4, None),
    ("ragged", True, 8, None),
    ("c32_b2", True, 8, None),
    ("paper_shape", True, 8, 1024),
    ("f32_g4", True, 5, None),
    ("p64k", True, 8, 2048),
    # K_top above 8: the selector with 16-entry pick lists (fp32 G=1, bf16 G=2 and G=4, fp32 G=4)
    ("tiny", True, 12, None),
    ("ragged", True, 16, None),
    ("c32_b2", True, 13, None),
    ("f32_g4", True, 16, None),
])
def test_bsa_matches_oracle(case, causal, K_top, sample):
    w = W[case]
    print("case", case, flush=True)
    _bsa_compare(w, _positions(w, sample), causal, K_top)
