"""Host-code sanitizer runs (CPU only, no GPU): the oracle (oracle/pisa_oracle.c) and the
C-ABI validation layer (hierarchical_top_amd/csrc/capi.hip, host side) built with
AddressSanitizer and UndefinedBehaviorSanitizer, each driven by a small C program under
tests/sanitize/ that exercises every entry point. A sanitizer report or a failed check makes
the driver exit non-zero. GPU code is built without sanitizers (-fno-gpu-sanitize): only
host code is instrumented."""
import os
import shutil
import subprocess
import tempfile
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(map(str, cmd)), r.stdout, r.stderr)
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_address_and_undefined_sanitizers():
    with tempfile.TemporaryDirectory() as tmp:
        exe = Path(tmp) / "oracle_driver"
        _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
              "-fno-sanitize-recover=all", "-ffp-contract=off", "-pthread", str(ROOT / "oracle" / "pisa_oracle.c"),
              str(ROOT / "tests" / "sanitize" / "oracle_driver.c"), "-o", str(exe), "-lm"])
        r = _run([str(exe)], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"))
        assert "oracle driver: ok" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")
def test_capi_validation_under_address_and_undefined_sanitizers():
    """capi.hip is rebuilt with host sanitizers and linked with the other objects of the
    library (built by hierarchical_top_amd.build when absent). Leak detection is off: the
    HIP runtime's own process-lifetime allocations are not this library's."""
    from hierarchical_top_amd import build as B
    objs = [B.OBJ / (p.stem + ".o") for p in B.sources() if p.name != "capi.hip"]
    if not all(o.exists() for o in objs):
        B.build()
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", str(ROOT / "include"), "-Xarch_host", "-fsanitize=address", "-Xarch_host",
             "-fsanitize=undefined", "-fno-gpu-sanitize"]
    with tempfile.TemporaryDirectory() as tmp:
        capi_o, drv_o, exe = Path(tmp) / "capi.o", Path(tmp) / "driver.o", Path(tmp) / "capi_driver"
        _run([HIPCC, *flags, "-c", str(B.CSRC / "capi.hip"), "-o", str(capi_o)])
        _run([HIPCC, "-x", "c", "-O1", "-g", "-I", str(ROOT / "include"), "-Xarch_host", "-fsanitize=address",
              "-Xarch_host", "-fsanitize=undefined", "-c", str(ROOT / "tests" / "sanitize" / "capi_driver.c"),
              "-o", str(drv_o)])
        _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
              "-fsanitize=undefined", "-fno-gpu-sanitize", str(drv_o), str(capi_o), *map(str, objs), "-o", str(exe)])
        r = _run([str(exe)], env=dict(ENV, ASAN_OPTIONS="detect_leaks=0"))
        assert "capi driver: ok" in r.stdout
