"""The allocation-free prefill router (pisa_route_prefill_noalloc) through the C ABI: its
output must equal the level router's with a caller workspace, bit for bit (same kernels,
integer selections and identical fp32 scores), on two calls in a row, the second with a
smaller input, so that nothing the first call left in the shared scratch array leaks into
the second; shapes whose workspace exceeds the scratch array are rejected on the host."""
import ctypes

import numpy as np
import pytest
import torch

from hierarchical_top_amd import pisa, synth

pytestmark = pytest.mark.gpu

ENOSPACE = -3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(w, K_top):
    Q, K, _, _ = synth.make_prefill(w)
    Qd, Kd = Q.cuda(), K.cuda()
    pyr = pisa.Pyramid(w.B, w.H_kv, w.d, w.C, w.g, w.N)
    pyr.build(Kd, w.N)
    need = pisa.route_workspace_bytes(pyr, w.N, w.H_q, K_top, pisa.LEVELS)
    assert need <= pisa.NOALLOC_SCRATCH_BYTES
    i_ws, s_ws = pisa.route_prefill(pyr, Qd, Kd, w.N, K_top, mode=pisa.LEVELS, with_score=True)
    out = torch.full_like(i_ws, -7)
    sco = torch.full_like(s_ws, 12345.0)
    i_na, s_na = pisa.route_prefill_noalloc(pyr, Qd, Kd, w.N, K_top, out=out, score_out=sco)
    torch.cuda.synchronize()
    return i_ws.cpu().numpy(), s_ws.cpu().numpy(), i_na.cpu().numpy(), s_na.cpu().numpy()


def test_noalloc_matches_workspace_router_twice():
    # first call: the 16K workload (16 query heads over 4 KV heads, d=128, C=64, g=4, planted)
    big = synth.workload("p16k")
    # second call, smaller: 3,000 tokens, 8 query heads over 2 KV heads, ragged tail, d=64, C=16
    small = synth.Workload("noalloc_small", 1, 3000, 8, 2, 64, 16, 4, 8, "bf16", 4, 31, False)
    for w in (big, small):
        print("noalloc case", w.name, "N", w.N, flush=True)
        i_ws, s_ws, i_na, s_na = _both(w, w.K_top)
        assert np.array_equal(i_ws, i_na), "%s: selections differ" % w.name
        assert np.array_equal(s_ws, s_na, equal_nan=True), "%s: scores differ" % w.name
        assert not (i_na == -7).any() and not (s_na == 12345.0).any()


def test_noalloc_rejects_shapes_beyond_the_scratch_array():
    w = synth.workload("p256k")
    pyr = pisa.Pyramid(w.B, w.H_kv, w.d, w.C, w.g, w.N)
    assert pisa.route_workspace_bytes(pyr, w.N, w.H_q, w.K_top, pisa.LEVELS) > pisa.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 24)  # never dereferenced: the size check fails first
    st = pisa.lib().pisa_route_prefill_noalloc(ctypes.byref(pyr.desc), fake, fake, pisa.BF16, w.N, w.H_q, w.K_top,
                                               1, w.H_q // w.H_kv, fake, None, None)
    assert st == ENOSPACE
