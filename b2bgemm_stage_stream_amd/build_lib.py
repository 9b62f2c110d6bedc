"""Builds libcf.so (the C-ABI library) from csrc/ with hipcc for gfx950.

Object files go to _build/ next to this file; the instantiation units of the
GEMM + epilogue kernel are compiled in parallel.

    python -m b2bgemm_stage_stream_amd.build_lib          # from the repository root
"""
from __future__ import annotations

import concurrent.futures as cf_futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcf.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
# Packed fp32 VALU instructions are disabled for all device code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def _units():
    """(source, object, extra defines) for every translation unit."""
    units = []
    for f in ("api.cpp", "gemm_epilogue_dispatch.hip", "b2b.hip", "b2b_stream.hip"):
        units.append((os.path.join(CSRC, f), os.path.join(BUILD, os.path.splitext(f)[0] + ".o"), []))
    for in_f32 in (0, 1):
        for b_nk in (0, 1):
            for part in range(17):
                obj = os.path.join(BUILD, f"gemm_epilogue_inst_{in_f32}_{b_nk}_{part}.o")
                units.append((os.path.join(CSRC, "gemm_epilogue_inst.hip"), obj,
                              [f"-DCF_IN_F32={in_f32}", f"-DCF_B_NK={b_nk}", f"-DCF_PART={part}"]))
    return units


def _compile(src, obj, defs):
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC] + FLAGS + defs + lang + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _stale(obj: str) -> bool:
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    deps = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)]
    return any(os.path.getmtime(d) > t for d in deps)


def build(jobs: int | None = None, verbose: bool = True, force: bool = True) -> str:
    """Compile the units and link libcf.so. With force=False only units older
    than a source or header are recompiled."""
    os.makedirs(BUILD, exist_ok=True)
    units = _units()
    if not force:
        objs_all = [u[1] for u in units]
        units = [u for u in units if _stale(u[1])]
    jobs = jobs or min(16, os.cpu_count() or 4)
    with cf_futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, *u) for u in units]
        objs = [f.result() for f in futs]
    if not force:
        objs = objs_all
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(objs)} units", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(force="--incremental" not in sys.argv)
