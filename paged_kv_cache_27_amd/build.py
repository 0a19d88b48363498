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


ASAN_LIB = BUILD / "asan" / "libpagedkv_asan.so"
# Host code only: each sanitizer flag applies to the host compilation (-Xarch_host); the
# device code is the regular build's.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-g"]


def build_sanitized(verbose: bool = True) -> Path:
    """The library with its host-only sources (api.cpp: argument checks, planning, the
    pool's front end; pool.cpp: the block pool) compiled under AddressSanitizer and
    UndefinedBehaviorSanitizer, linked with the kernels' objects of the regular build
    (built first if missing), into _build/asan/libpagedkv_asan.so.  The CPU test suite
    runs against it with the sanitizer runtime preloaded (tests/test_sanitizers_cpu.py)."""
    out_dir = ASAN_LIB.parent
    out_dir.mkdir(parents=True, exist_ok=True)
    kernels = sorted(CSRC.glob("*.hip"))
    if not all((BUILD / (k.name + ".o")).exists() for k in kernels):
        build(verbose=False)
    objs = [BUILD / (k.name + ".o") for k in kernels]
    for src in sorted(CSRC.glob("*.cpp")):
        obj = out_dir / (src.name + ".o")
        cmd = [HIPCC, *FLAGS, *SANITIZE_FLAGS, "-x", "hip", "-c", str(src), "-o", str(obj)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {src.name} (sanitizer build)")
        objs.append(obj)
    tmp = ASAN_LIB.with_suffix(".so.tmp")
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", *map(str, objs), "-o", str(tmp)],
                   check=True)
    os.replace(tmp, ASAN_LIB)
    if verbose:
        print(f"built {ASAN_LIB}")
    return ASAN_LIB


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
