"""GPU behaviour of the stage-timing hooks (pisa_time_stage): armed event pairs are consumed
by the next occurrences of their stage on this thread, in order, and bracket that stage's
kernels on the launch stream."""
import pytest
import torch

from hierarchical_top_amd import pisa, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _events(n):
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in ev:
        e.record()  # HIP events exist only once recorded
    torch.cuda.synchronize()
    return ev


def test_stage_events_bracket_their_stages():
    w = synth.Workload("timing", 1, 20000, 8, 2, 128, 64, 4, 8, "bf16", 8, 81, True)
    Q, K, V, _ = synth.make_prefill(w)
    Q, K, V = Q.cuda(), K.cuda(), V.cuda()
    pyr = pisa.Pyramid(w.B, w.H_kv, w.d, w.C, w.g, w.N)
    ws = torch.empty(pisa.route_workspace_bytes(pyr, w.N, w.H_q, w.K_top, pisa.LEVELS), dtype=torch.uint8,
                     device="cuda")
    b0, b1, l0, l1, u0, u1, u2, u3, t0, t1 = _events(10)
    pisa.time_stage("build", b0, b1)
    pisa.time_stage("leaf", l0, l1)
    pisa.time_stage("upper", u0, u1)   # consumed by the first scored upper level
    pisa.time_stage("upper", u2, u3)   # and by the second
    assert pisa.time_stage_pending("upper") == 2
    total0, total1 = _events(2)
    total0.record()
    pyr.build(K, w.N)
    idx = pisa.route_prefill(pyr, Q, K, w.N, w.K_top, mode=pisa.LEVELS, workspace=ws)
    total1.record()
    torch.cuda.synchronize()
    assert pisa.time_stage_pending("build") == 0 and pisa.time_stage_pending("leaf") == 0
    assert pisa.time_stage_pending("upper") == 0
    whole = total0.elapsed_time(total1)
    for a, b in ((b0, b1), (l0, l1), (u0, u1), (u2, u3)):
        ms = a.elapsed_time(b)
        assert 0 < ms <= whole
    # the first upper level ends before the second starts, and both before the leaf starts
    assert u0.elapsed_time(u2) > 0 and u2.elapsed_time(l0) > 0
    # attention backward stage
    O, lse = pisa.sparse_attn_clustered(Q, K, V, idx, w.C, w.N, with_lse=True)
    pisa.time_stage("attn_bwd", t0, t1)
    pisa.sparse_attn_bwd(Q, K, V, O, torch.randn_like(O), lse, idx, w.C, w.N)
    torch.cuda.synchronize()
    assert pisa.time_stage_pending("attn_bwd") == 0 and t0.elapsed_time(t1) > 0
    # an armed pair that no call consumes stays queued until cleared
    pisa.time_stage("bsa", *_events(2))
    pisa.route_prefill(pyr, Q, K, w.N, w.K_top, mode=pisa.LEVELS, workspace=ws)
    assert pisa.time_stage_pending("bsa") == 1
    pisa.time_stage_clear("bsa")
    assert pisa.time_stage_pending("bsa") == 0
