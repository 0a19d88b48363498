"""Build the HIP library (libpagedkv.so) in-tree for gfx950 with hipcc.

`python -m paged_kv_cache_27_amd.build` compiles every source under csrc/ to an
object in _build/ (in parallel) and links the shared library next to this file; the
measurement-only streaming-read probe (probe/) becomes libpkv_probe.so beside it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = ROOT / "_build"
LIB = PKG / "libpagedkv.so"
PROBE_SRC = PKG / "probe" / "probe_read.hip"
PROBE_LIB = PKG / "libpkv_probe.so"
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # Keep packed fp32 arithmetic out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", str(ROOT / "include"), "-I", str(CSRC),
]


def _compile(src: Path) -> Path:
    obj = BUILD / (src.name + ".o")
    cmd = [HIPCC, *FLAGS, "-c", str(src), "-o", str(obj)]
    if src.suffix == ".cpp":
        cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src.name}")
    noisy = [ln for ln in (r.stderr or "").splitlines() if "packed-fp32-ops" not in ln]
    if noisy:
        sys.stderr.write("\n".join(noisy) + "\n")
    return obj


def build(verbose: bool = True) -> Path:
    BUILD.mkdir(exist_ok=True)
    sources = sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.cpp"))
    jobs = min(len(sources) + 1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16)
    with cf.ThreadPoolExecutor(max_workers=max(jobs, 1)) as ex:
        probe = ex.submit(_compile, PROBE_SRC)
        objs = list(ex.map(_compile, sources))
        probe_obj = probe.result()
    for lib, parts in ((LIB, objs), (PROBE_LIB, [probe_obj])):
        tmp = lib.with_suffix(".so.tmp")
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, parts), "-o", str(tmp)]
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB.name}")
    return LIB


if __name__ == "__main__":
    build()
