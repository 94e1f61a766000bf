"""Pyramid build + level-synchronous routing captured in a HIP graph (torch.cuda.CUDAGraph
over the C-ABI calls on the capturing stream) and replayed: every replay, with eager work
and synchronisations between replays, must reproduce the eager selection bit for bit.
The library clears its cluster counters with a kernel (no memset nodes in the graph)."""
import pytest
import torch

from hierarchical_top_amd import pisa, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("case", ["p16k", "ragged"])
def test_graph_replays_match_eager(case):
    w = synth.workload("p16k") if case == "p16k" else \
        synth.Workload("ragged", 1, 5000, 8, 2, 128, 64, 4, 8, "bf16", 8, 71, False)
    Q, K, _, _ = synth.make_prefill(w)
    Q, K = Q.cuda(), K.cuda()
    pyr = pisa.Pyramid(w.B, w.H_kv, w.d, w.C, w.g, w.N)
    ws = torch.empty(pisa.route_workspace_bytes(pyr, w.N, w.H_q, w.K_top, pisa.LEVELS), dtype=torch.uint8,
                     device="cuda")
    idx = torch.full((w.B, w.H_kv, w.N, w.K_top), -7, dtype=torch.int32, device="cuda")
    sco = torch.empty(w.B, w.H_kv, w.N, w.K_top, dtype=torch.float32, device="cuda")

    def step():
        pyr.build(K, w.N)
        pisa.route_prefill(pyr, Q, K, w.N, w.K_top, mode=pisa.LEVELS, workspace=ws, out=idx, with_score=True,
                           score_out=sco)

    step()
    torch.cuda.synchronize()
    want_i, want_s = idx.clone(), sco.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the side stream before capture
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        idx.fill_(-7)
        sco.fill_(12345.0)
        ws.fill_(0x5A)  # stale workspace between replays must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, want_i), "replay %d differs from the eager selection" % r
        assert torch.equal(sco, want_s), "replay %d scores differ" % r
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(idx, want_i)
