"""Build libpisa.so (gfx950) from hierarchical_top_amd/csrc with hipcc.

    python -m hierarchical_top_amd.build

Objects go to _build/ at the repository root; the shared library is written
next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
ROOT = PKG.parent
OBJ = ROOT / "_build" / "pisa"
LIB = PKG / "libpisa.so"
# unit-throughput loops timed beside the selection kernels (include/pisa_peaks.h)
PEAKS_SRC = PKG / "peaks" / "peaks.hip"
PEAKS_LIB = PKG / "libpisa_peaks.so"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off: hipcc would otherwise form them from float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", str(ROOT / "include"),
]


def sources():
    return sorted(CSRC.glob("*.hip"))


def _compile(src: Path) -> Path:
    out = OBJ / (src.stem + ".o")
    cmd = [HIPCC, *FLAGS, "-c", str(src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on %s" % src.name)
    return out


def build(jobs: int | None = None) -> Path:
    """Compile every csrc/*.hip for gfx950 and link libpisa.so, then libpisa_peaks.so
    (always rebuilds)."""
    OBJ.mkdir(parents=True, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, sources()))
    tmp = LIB.with_suffix(".so.tmp%d" % os.getpid())
    r = subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libpisa.so failed")
    os.replace(tmp, LIB)
    tmp = PEAKS_LIB.with_suffix(".so.tmp%d" % os.getpid())
    r = subprocess.run([HIPCC, *FLAGS, "-shared", str(PEAKS_SRC), "-o", str(tmp)], capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build of libpisa_peaks.so failed")
    os.replace(tmp, PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
