"""Builds libcf.so (the C-ABI library) from csrc/ with hipcc for gfx950.

This module imports nothing from the package, so it runs on a checkout that
has no library yet:

    python b2bgemm_stage_stream_amd/build_lib.py            # build what is out of date
    python b2bgemm_stage_stream_amd/build_lib.py --force    # rebuild every unit

Importing the package calls ``ensure_built()``: when ``libcf.so`` is missing,
or was built from other sources or flags than the ones in the tree, the
library is (re)built under a file lock before it is loaded.

Up-to-date checks use content hashes, not file times: a stamp next to the
library holds the hash of every source and header plus the compiler flags,
and each object file in ``_build/`` has a stamp of its own, so a copy of the
tree with fresh file times neither rebuilds for nothing nor keeps a stale
library.
"""
from __future__ import annotations

import concurrent.futures as cf_futures
import contextlib
import hashlib
import os
import shutil
import subprocess
import sys
import time
from typing import Callable, Optional

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcf.so")
STAMP = LIB + ".stamp"
LOCK = os.path.join(HERE, ".libcf.lock")

ARCH = "gfx950"
# Packed fp32 VALU instructions are disabled for all device code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]
LINK_FLAGS = [f"--offload-arch={ARCH}", "-shared", "-fPIC"]

# Instantiation parts of the GEMM + epilogue kernel (gemm_epilogue_inst.hip):
# 0-9 and 21-23 for both input dtypes, 10-20 for bf16 inputs only.
PARTS_ALL = list(range(10)) + [21, 22, 23]
PARTS_BF16 = range(10, 21)

Log = Callable[[str], None]


def _stderr(msg: str) -> None:
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def hipcc() -> Optional[str]:
    """The compiler: $HIPCC if set, else hipcc on PATH, else ROCm's default
    location; None when that is not an executable file."""
    h = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return h if os.path.isfile(h) and os.access(h, os.X_OK) else None


def units() -> list[tuple[str, str, list[str]]]:
    """(source, object, extra defines) of every translation unit, the ones that
    take longest to compile first (the pool then finishes sooner)."""
    heavy, light = [], []
    for in_f32 in (0, 1):
        for b_nk in (0, 1):
            parts = list(PARTS_ALL) + (list(PARTS_BF16) if in_f32 == 0 else [])
            for part in parts:
                obj = os.path.join(BUILD, f"gemm_epilogue_inst_{in_f32}_{b_nk}_{part}.o")
                u = (os.path.join(CSRC, "gemm_epilogue_inst.hip"), obj,
                     [f"-DCF_IN_F32={in_f32}", f"-DCF_B_NK={b_nk}", f"-DCF_PART={part}"])
                # the element-masked general path (parts 5-9) compiles slowest
                (heavy if 5 <= part <= 9 else light).append(u)
    base = [(os.path.join(CSRC, f), os.path.join(BUILD, os.path.splitext(f)[0] + ".o"), [])
            for f in ("b2b.hip", "b2b_stream.hip", "api.cpp", "gemm_epilogue_dispatch.hip")]
    return heavy + base[:1] + light + base[1:]


def source_hash() -> str:
    """Hash of every source and header the library is built from, and of the
    flags (with the tree's own include directories by name, so that a copy of
    the tree at another path has the same hash)."""
    h = hashlib.sha256()
    flags = [{INCLUDE: "<include>", CSRC: "<csrc>"}.get(f, f) for f in FLAGS]
    h.update(repr((flags, LINK_FLAGS, list(PARTS_ALL), list(PARTS_BF16))).encode())
    for d in (CSRC, INCLUDE):
        for f in sorted(os.listdir(d)):
            p = os.path.join(d, f)
            if os.path.isfile(p):
                h.update(f.encode() + b"\0")
                with open(p, "rb") as fh:
                    h.update(fh.read())
    return h.hexdigest()


def _unit_hash(src: str, defs: list[str]) -> str:
    """Hash of what one object file is built from: the flags, every header
    (any file that is not itself a translation unit), the unit's own source
    and its defines. Translation units include headers only, so a change to
    one .hip file rebuilds that file's objects alone."""
    h = hashlib.sha256()
    flags = [{INCLUDE: "<include>", CSRC: "<csrc>"}.get(f, f) for f in FLAGS]
    h.update(repr((flags, defs, os.path.basename(src))).encode())
    for d in (CSRC, INCLUDE):
        for f in sorted(os.listdir(d)):
            p = os.path.join(d, f)
            if os.path.isfile(p) and not f.endswith((".hip", ".cpp")):
                h.update(f.encode() + b"\0")
                with open(p, "rb") as fh:
                    h.update(fh.read())
    with open(src, "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()


def _read(path: str) -> str:
    try:
        with open(path) as f:
            return f.read().strip()
    except OSError:
        return ""


def up_to_date() -> bool:
    return os.path.exists(LIB) and _read(STAMP) == source_hash()


def _compile(cc: str, src: str, obj: str, defs: list[str], stamp: str) -> float:
    t0 = time.time()
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [cc] + FLAGS + defs + lang + ["-c", src, "-o", obj + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(obj + ".tmp", obj)
    with open(obj + ".stamp", "w") as f:
        f.write(stamp)
    return time.time() - t0


@contextlib.contextmanager
def _locked():
    import fcntl
    with open(LOCK, "w") as fh:
        fcntl.flock(fh, fcntl.LOCK_EX)
        try:
            yield
        finally:
            fcntl.flock(fh, fcntl.LOCK_UN)


def _jobs() -> int:
    n = os.cpu_count() or 4
    # the GPU hosts give one process 16 cores at most, whatever cpu_count says
    return max(1, min(16, int(os.environ.get("MAX_JOBS", n))))


def build(jobs: Optional[int] = None, force: bool = True, log: Log = _stderr) -> str:
    """Compiles the units (all of them, or with force=False only those whose
    stamp differs) and links libcf.so. Progress goes to `log`, one line per
    unit."""
    cc = hipcc()
    if cc is None:
        raise RuntimeError("hipcc not found (set HIPCC or put ROCm's bin directory on PATH)")
    os.makedirs(BUILD, exist_ok=True)
    src_hash = source_hash()
    todo, objs = [], []
    for src, obj, defs in units():
        st = _unit_hash(src, defs)
        objs.append(obj)
        if force or not os.path.exists(obj) or _read(obj + ".stamp") != st:
            todo.append((src, obj, defs, st))
    jobs = jobs or _jobs()
    t0 = time.time()
    if todo:
        log(f"[libcf] compiling {len(todo)} of {len(objs)} units with {jobs} jobs")
    with cf_futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = {ex.submit(_compile, cc, *u): u for u in todo}
        done = 0
        for fut in cf_futures.as_completed(futs):
            dt = fut.result()
            done += 1
            src, obj, defs, _ = futs[fut]
            log(f"[libcf] {done}/{len(todo)} {os.path.basename(obj)} {dt:.0f} s "
                f"(elapsed {time.time() - t0:.0f} s)")
    tmp = LIB + ".tmp"
    cmd = [cc] + LINK_FLAGS + ["-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    with open(STAMP, "w") as f:
        f.write(src_hash)
    log(f"[libcf] built {LIB} from {len(objs)} units in {time.time() - t0:.0f} s")
    return LIB


def ensure_built(log: Log = _stderr) -> str:
    """Returns the library path, building it first (under a file lock, only
    the out-of-date units) when it is missing or stale."""
    if up_to_date():
        return LIB
    with _locked():
        if up_to_date():   # another process built it meanwhile
            return LIB
        log("[libcf] libcf.so is missing or out of date: building it for gfx950")
        return build(force=False, log=log)


if __name__ == "__main__":
    if "--force" in sys.argv:
        with _locked():
            build(force=True)
    else:
        ensure_built()
