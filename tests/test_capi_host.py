"""Host-only checks of the C ABI (no GPU needed): the library loads, exports every
function include/pisa.h declares, and rejects bad arguments on the host with
the documented status codes before anything is queued."""
import ctypes
import re
from pathlib import Path

import pytest

from hierarchical_top_amd import pisa

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "pisa.h"

OK, EINVAL, EUNSUPPORTED, ENOSPACE = 0, -1, -2, -3


@pytest.fixture(scope="module")
def lib():
    if not pisa.LIB_PATH.exists():
        pytest.skip("libpisa.so is not built")
    return pisa.lib()


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pisa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("pisa_build_pyramid", "pisa_route_prefill", "pisa_route_decode", "pisa_sparse_attn",
              "pisa_pyramid_append", "pisa_bsa_select"):
        assert f in names


def test_library_exports_every_declared_function(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(declared_functions()) <= set(pisa.EXPORTS)
    assert lib.pisa_abi_version() == 1


def test_peaks_library_exports_every_declared_function():
    """The unit-throughput loops timed beside the kernels (include/pisa_peaks.h)."""
    from hierarchical_top_amd import build
    if not build.PEAKS_LIB.exists():
        pytest.skip("libpisa_peaks.so is not built")
    text = re.sub(r"/\*.*?\*/", "", (ROOT / "include" / "pisa_peaks.h").read_text(), flags=re.S)
    names = sorted(set(re.findall(r"\b(pisa_peak_[a-z0-9_]+)\s*\(", text)))
    assert {"pisa_peak_copy", "pisa_peak_read", "pisa_peak_gather"} <= set(names)
    peaks = ctypes.CDLL(str(build.PEAKS_LIB))
    assert [n for n in names if not hasattr(peaks, n)] == []


def test_status_strings(lib):
    for s in (OK, EINVAL, EUNSUPPORTED, ENOSPACE, -4):
        assert lib.pisa_status_str(s)
    assert lib.pisa_status_str(7) == b"unknown status"


def plan(lib, *args):
    d = pisa._PyramidDesc()
    st = lib.pisa_pyramid_plan(ctypes.byref(d), *args)
    return st, d


def test_plan_geometry(lib):
    st, d = plan(lib, 1, 4, 128, 64, 4, 262144)
    assert st == OK
    assert d.L_cap == 7
    assert [d.M_cap[l] for l in range(8)] == [262144, 4096, 1024, 256, 64, 16, 4, 1]
    # per-level offsets are 64-float aligned and non-overlapping
    for l in range(1, 7):
        assert d.off[l] % 64 == 0 and d.off[l + 1] >= d.off[l] + 4 * d.M_cap[l] * 128
    assert d.floats >= d.off[7] + 4 * 128
    st, d = plan(lib, 32, 8, 128, 64, 4, 262400)
    assert st == OK and d.L_cap == 8


@pytest.mark.parametrize("args,status", [
    ((0, 4, 128, 64, 4, 1024), EINVAL),
    ((1, 4, 128, 64, 4, 0), EINVAL),
    ((1, 4, 96, 64, 4, 1024), EUNSUPPORTED),
    ((1, 4, 128, 48, 4, 1024), EUNSUPPORTED),
    ((1, 4, 128, 64, 3, 1024), EUNSUPPORTED),
    ((1, 64, 128, 64, 4, 1024), EUNSUPPORTED),
])
def test_plan_rejects(lib, args, status):
    st, _ = plan(lib, *args)
    assert st == status
    assert lib.pisa_last_error()


def fake_pyramid(lib, B=1, H=4, d=128, C=64, g=4, N=4096):
    st, desc = plan(lib, B, H, d, C, g, N)
    assert st == OK
    desc.buf = 1 << 20  # never dereferenced: every call below fails validation first
    return desc


FAKE = ctypes.c_void_p(1 << 24)


def route(lib, desc, N=4096, H_q=16, K_top=8, causal=1, gqa=4, mode=pisa.TWO_STAGE, Q=FAKE, ws=None, ws_bytes=0,
          dt=pisa.BF16):
    return lib.pisa_route_prefill(ctypes.byref(desc), Q, FAKE, dt, N, H_q, K_top, causal, gqa, mode, FAKE, None,
                                  ws, ws_bytes, None)


def test_route_prefill_validation(lib):
    desc = fake_pyramid(lib)
    assert route(lib, desc, N=0) == EINVAL
    assert route(lib, desc, N=4097) == ENOSPACE
    assert route(lib, desc, H_q=15, gqa=3) == EINVAL
    assert route(lib, desc, gqa=2) == EINVAL                       # gqa_group != H_q / H_kv
    assert route(lib, desc, K_top=2) == EINVAL                     # causal needs room for the forced set
    assert route(lib, desc, K_top=0, causal=0) == EINVAL
    assert route(lib, desc, K_top=65) == EINVAL
    assert route(lib, desc, K_top=32) == EUNSUPPORTED              # g * K_top = 128 candidates
    assert route(lib, desc, dt=7) == EINVAL
    assert route(lib, desc, Q=None) == EINVAL
    assert route(lib, desc, Q=ctypes.c_void_p((1 << 24) + 4)) == EINVAL  # misaligned
    assert route(lib, desc, mode=5) == EINVAL
    # two-stage needs a workspace of the advertised size
    n = ctypes.c_size_t(0)
    assert lib.pisa_route_prefill_workspace(ctypes.byref(desc), 4096, 16, 8, pisa.TWO_STAGE, ctypes.byref(n)) == OK
    assert n.value > 0
    assert route(lib, desc, ws=FAKE, ws_bytes=n.value - 1) == ENOSPACE
    m = ctypes.c_size_t(1)
    assert lib.pisa_route_prefill_workspace(ctypes.byref(desc), 4096, 16, 8, pisa.FUSED, ctypes.byref(m)) == OK
    assert m.value == 0


def test_route_prefill_scored_validation(lib):
    desc = fake_pyramid(lib)

    def scored(kind, mode=pisa.LEVELS, K_top=8):
        return lib.pisa_route_prefill_scored(ctypes.byref(desc), FAKE, FAKE, pisa.BF16, 4096, 16, K_top, 1, 4, mode,
                                             kind, FAKE, None, None, 0, None)

    assert scored(3) == EINVAL
    assert scored(-1) == EINVAL
    # PISA-1 / PISA-2 scores run on the level-synchronous and fused routers, not the two-stage one
    assert scored(pisa.SCORE_KINDS["mean"], mode=pisa.TWO_STAGE) == EUNSUPPORTED
    assert scored(pisa.SCORE_KINDS["mean_var"], mode=pisa.TWO_STAGE) == EUNSUPPORTED
    dec = lib.pisa_route_decode_scored
    assert dec(ctypes.byref(desc), FAKE, FAKE, pisa.BF16, FAKE, 16, 8, 4, 3, FAKE, None, None) == EINVAL
    assert dec(ctypes.byref(desc), FAKE, FAKE, pisa.BF16, None, 16, 8, 4, 1, FAKE, None, None) == EINVAL
    # past the score checks, the usual validation applies: no workspace was given
    for kind in (0, 1, 2):
        assert scored(kind) == ENOSPACE
        assert scored(kind, K_top=2) == EINVAL


def test_workspace_query_validates_descriptor(lib):
    """The workspace query walks the pyramid geometry, so it must reject a zeroed or
    hand-edited descriptor (C = 0 or g = 1 would divide by zero or never terminate)."""
    n = ctypes.c_size_t(7)
    zero = pisa._PyramidDesc()
    for mode in (pisa.LEVELS, pisa.TWO_STAGE, pisa.FUSED):
        assert lib.pisa_route_prefill_workspace(ctypes.byref(zero), 4096, 16, 8, mode, ctypes.byref(n)) == EINVAL
    bad = fake_pyramid(lib)
    bad.g = 1
    assert lib.pisa_route_prefill_workspace(ctypes.byref(bad), 4096, 16, 8, pisa.LEVELS, ctypes.byref(n)) == EUNSUPPORTED
    desc = fake_pyramid(lib)
    assert lib.pisa_route_prefill_workspace(ctypes.byref(desc), 4096, 16, 8, 9, ctypes.byref(n)) == EINVAL
    assert lib.pisa_route_prefill_workspace(ctypes.byref(desc), 4097, 16, 8, pisa.LEVELS, ctypes.byref(n)) == ENOSPACE
    assert lib.pisa_route_prefill_workspace(None, 4096, 16, 8, pisa.LEVELS, ctypes.byref(n)) == EINVAL
    assert n.value == 7  # untouched on error


def test_descriptor_must_come_from_plan(lib):
    desc = fake_pyramid(lib)
    desc.off[2] += 64
    assert route(lib, desc) == EINVAL
    desc = fake_pyramid(lib)
    desc.buf = None
    assert route(lib, desc) == EINVAL
    assert lib.pisa_build_pyramid(None, FAKE, pisa.BF16, 16, None) == EINVAL


def test_build_append_decode_validation(lib):
    desc = fake_pyramid(lib)
    assert lib.pisa_build_pyramid(ctypes.byref(desc), FAKE, pisa.BF16, 0, None) == EINVAL
    assert lib.pisa_build_pyramid(ctypes.byref(desc), FAKE, pisa.BF16, 4097, None) == ENOSPACE
    assert lib.pisa_build_pyramid(ctypes.byref(desc), None, pisa.BF16, 16, None) == EINVAL
    assert lib.pisa_pyramid_append(ctypes.byref(desc), FAKE, pisa.BF16, None, None) == EINVAL
    assert lib.pisa_route_decode(ctypes.byref(desc), FAKE, FAKE, pisa.BF16, None, 16, 8, 4, FAKE, None,
                                 None) == EINVAL
    assert lib.pisa_route_decode(ctypes.byref(desc), FAKE, FAKE, pisa.BF16, FAKE, 16, 2, 4, FAKE, None,
                                 None) == EINVAL


def test_attention_and_bsa_validation(lib):
    a = lib.pisa_sparse_attn
    assert a(FAKE, FAKE, FAKE, pisa.BF16, 1, 10, 5, 10, 8, 2, 128, 64, FAKE, 8, 1, None, FAKE, None, None) == EINVAL
    assert a(FAKE, FAKE, FAKE, pisa.BF16, 1, 10, 10, 10, 8, 3, 128, 64, FAKE, 8, 1, None, FAKE, None, None) == EINVAL
    assert a(FAKE, FAKE, FAKE, pisa.BF16, 1, 10, 10, 10, 8, 2, 80, 64, FAKE, 8, 1, None, FAKE, None,
             None) == EUNSUPPORTED
    assert a(FAKE, FAKE, None, pisa.BF16, 1, 10, 10, 10, 8, 2, 128, 64, FAKE, 8, 1, None, FAKE, None, None) == EINVAL
    desc = fake_pyramid(lib)
    b = lib.pisa_bsa_select
    assert b(ctypes.byref(desc), FAKE, pisa.BF16, 4096, 16, 17, 1, 4, FAKE, None, None) == EUNSUPPORTED
    assert b(ctypes.byref(desc), FAKE, pisa.BF16, 4096, 16, 2, 1, 4, FAKE, None, None) == EINVAL
    assert b(ctypes.byref(desc), FAKE, pisa.BF16, 5000, 16, 8, 1, 4, FAKE, None, None) == ENOSPACE


def test_clustered_attention_validation(lib):
    n = pisa.c_size(0)
    w = lib.pisa_sparse_attn_workspace
    assert w(1, 65536, 65536, 32, 8, 128, 64, 8, ctypes.byref(n)) == OK
    big = n.value
    # entries, partial outputs (G x d fp16) and log-sum-exps + exponents per (row, slot), plus the cluster tables
    assert big >= 65536 * 8 * 8 * (4 + 4 * 8 + 4 * 128 * 2)
    assert w(1, 1024, 65536, 32, 8, 128, 64, 8, ctypes.byref(n)) == OK and n.value < big
    assert w(1, 1024, 1024, 32, 8, 128, 64, 65, ctypes.byref(n)) == EUNSUPPORTED
    assert w(1, 1024, 1024, 32, 8, 96, 64, 8, ctypes.byref(n)) == EUNSUPPORTED
    assert w(1, 1024, 1024, 32, 8, 128, 64, 8, None) == EINVAL
    assert w(1, 1024, 1024, 30, 8, 128, 64, 8, ctypes.byref(n)) == EINVAL
    a = lib.pisa_sparse_attn_clustered
    WS = ctypes.c_void_p(0x100000)  # 256-byte aligned, never dereferenced: rejected before any launch
    need = pisa.sparse_attn_workspace_bytes(1, 10, 10, 8, 2, 128, 64, 8)
    args = [FAKE, FAKE, FAKE, pisa.BF16, 1, 10, 10, 10, 8, 2, 128, 64, FAKE, 8, 1, None, FAKE, None]
    assert a(*args, WS, need - 1, None) == ENOSPACE
    assert a(*args, None, need, None) == EINVAL
    assert a(*args, ctypes.c_void_p(0x100010), need, None) == EINVAL  # misaligned workspace
    f32 = list(args)
    f32[3] = pisa.F32
    assert a(*f32, WS, need, None) == EUNSUPPORTED
    k65 = list(args)
    k65[13] = 65
    assert a(*k65, WS, 1 << 40, None) == EUNSUPPORTED


def test_time_stage_validation(lib):
    assert lib.pisa_time_stage(11, None, None) == EINVAL
    assert lib.pisa_time_stage(-1, None, None) == EINVAL
    assert lib.pisa_time_stage(0, FAKE, None) == EINVAL
    assert lib.pisa_time_stage(0, None, None) == OK  # disarm


def test_attention_backward_validation(lib):
    n = pisa.c_size(0)
    w = lib.pisa_sparse_attn_bwd_workspace
    assert w(1, 65536, 65536, 32, 8, 128, 64, 8, ctypes.byref(n)) == OK
    # one fp32 dQ row of d per (row, selected block, query head), plus the clustering tables
    assert n.value >= 65536 * 32 * 8 * 128 * 4
    assert w(1, 1024, 1024, 32, 8, 96, 64, 8, ctypes.byref(n)) == EUNSUPPORTED
    assert w(1, 1024, 1024, 32, 8, 128, 64, 8, None) == EINVAL
    b = lib.pisa_sparse_attn_bwd
    WS = ctypes.c_void_p(0x100000)
    need = pisa.sparse_attn_bwd_workspace_bytes(1, 10, 10, 8, 2, 128, 64, 8)
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, pisa.BF16, 1, 10, 10, 10, 8, 2, 128, 64, FAKE, 8, 1, None,
            FAKE, FAKE, FAKE]
    assert b(*args, WS, need - 1, None) == ENOSPACE
    assert b(*args, None, need, None) == EINVAL
    assert b(*args, ctypes.c_void_p(0x100010), need, None) == EINVAL  # misaligned workspace
    for k in (3, 4, 5, 19):  # O, dO, lse, dQ missing
        a2 = list(args)
        a2[k] = None
        assert b(*a2, WS, need, None) == EINVAL
    f32 = list(args)
    f32[6] = pisa.F32
    assert b(*f32, WS, need, None) == EUNSUPPORTED
    bad = list(args)
    bad[9] = 5  # N_kv < N_q
    assert b(*bad, WS, need, None) == EINVAL


def test_selection_quality_validation(lib):
    n = pisa.c_size(0)
    w = lib.pisa_selection_quality_workspace
    assert w(1, 16384, 16, 64, ctypes.byref(n)) == OK and n.value == 16 * 16384 * 256 * 4
    assert w(1, 16384, 16, 48, ctypes.byref(n)) == EUNSUPPORTED
    assert w(0, 16384, 16, 64, ctypes.byref(n)) == EINVAL
    q = lib.pisa_selection_quality
    WS = ctypes.c_void_p(0x100000)
    args = [FAKE, FAKE, pisa.BF16, 1, 100, 8, 2, 128, 16, FAKE, 8, None, None, FAKE, FAKE, FAKE]
    need = 8 * 100 * 7 * 4
    assert q(*args, WS, need - 1, None) == ENOSPACE
    k2 = list(args)
    k2[10] = 2
    assert q(*k2, WS, need, None) == EINVAL            # no room for the forced blocks
    k17 = list(args)
    k17[10] = 17
    assert q(*k17, WS, need, None) == EUNSUPPORTED
    g3 = list(args)
    g3[6] = 3
    assert q(*g3, WS, need, None) == EINVAL            # H_q not a multiple of H_kv
    nul = list(args)
    nul[13] = None
    assert q(*nul, WS, need, None) == EINVAL
