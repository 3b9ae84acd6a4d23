"""Builds librmsnorm_mi355x.so in-tree: the gfx950 kernels with hipcc, the
C-ABI layer with g++, linked by hipcc."""
from __future__ import annotations

import os
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD = PKG / "_build"
LIB = PKG / "librmsnorm_mi355x.so"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # exactly the arithmetic written: no FMA contraction, no fast-math
    "-ffp-contract=off",
    # no packed fp32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
HIP_SOURCES = ["fwd.hip", "fwd_gated.hip", "fwd_add.hip", "fwd_f16.hip", "bwd.hip", "bwd_gated.hip",
               "bwd_add.hip", "bwd_f16.hip", "gemm.hip", "fwd_elem.hip", "bwd_elem.hip", "bwd_elem_f16.hip",
               "fwd_gated_elem.hip", "fwd_add_elem.hip", "bwd_add_elem.hip", "bwd_gated_elem.hip",
               "fwd_gated_f16.hip", "fwd_gated_elem_f16.hip", "fwd_add_f16.hip", "bwd_gated_f16.hip",
               "bwd_gated_elem_f16.hip", "bwd_add_f16.hip",
               "scratch.hip"]
CXX_SOURCES = ["api.cpp"]


def _includes(src: Path, seen=None) -> set:
    """The project headers `src` includes, directly or through other headers
    (quoted includes found in csrc/ or include/)."""
    seen = set() if seen is None else seen
    for line in src.read_text().splitlines():
        line = line.strip()
        if line.startswith("#include \""):
            name = line.split('"')[1]
            for d in (CSRC, INCLUDE):
                h = d / name
                if h.exists() and h not in seen:
                    seen.add(h)
                    _includes(h, seen)
    return seen


def _stale(src: Path, obj: Path) -> bool:
    """An object is stale when it is older than its source or a header the
    source includes."""
    if not obj.exists():
        return True
    return obj.stat().st_mtime < max(f.stat().st_mtime for f in [src, *_includes(src)])


def build(verbose: bool = False, incremental: bool = False) -> Path:
    """Compiles every source (or, with `incremental`, only those whose object
    is older than the source or a header) and links the library."""
    BUILD.mkdir(exist_ok=True)
    inc = [f"-I{INCLUDE}", f"-I{CSRC}"]
    jobs, objs = [], []
    for src in HIP_SOURCES:
        obj = BUILD / (src + ".o")
        objs.append(obj)
        if not incremental or _stale(CSRC / src, obj):
            jobs.append([HIPCC, *HIP_FLAGS, *inc, "-c", str(CSRC / src), "-o", str(obj)])
    for src in CXX_SOURCES:
        obj = BUILD / (src + ".o")
        objs.append(obj)
        if not incremental or _stale(CSRC / src, obj):
            jobs.append(["g++", "-std=c++17", "-O2", "-fPIC", "-Wall", *inc, "-c",
                         str(CSRC / src), "-o", str(obj)])
    procs = [subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
             for cmd in jobs]
    failed = []
    for cmd, p in zip(jobs, procs):
        out, _ = p.communicate()
        # hipcc's host pass does not know the packed-fp32 feature; harmless
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
        if verbose or p.returncode:
            print("\n".join(lines))
        if p.returncode:
            failed.append(cmd[-3])
    if failed:
        raise RuntimeError(f"compilation failed: {failed}")
    tmp = LIB.with_suffix(".so.tmp")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *map(str, objs),
                    "-o", str(tmp)], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    import sys
    print(build(verbose=True, incremental="--incremental" in sys.argv))
