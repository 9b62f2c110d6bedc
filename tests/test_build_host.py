"""The library builder on a checkout without a built library (CPU only): it
loads without the package, sees that the library is missing, reports a
missing compiler as an ImportError of the package, and its up-to-date check
follows the sources' content, not their file times."""
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = "b2bgemm_stage_stream_amd"


def clean_copy(tmp_path):
    """The package, include/ and nothing built: what a fresh checkout holds."""
    dst = tmp_path / "repo"
    shutil.copytree(os.path.join(ROOT, PKG), dst / PKG,
                    ignore=shutil.ignore_patterns("_build", "*.so", "*.so.*", "__pycache__", ".libcf.lock"))
    shutil.copytree(os.path.join(ROOT, "include"), dst / "include")
    return dst


def load_builder(repo):
    spec = importlib.util.spec_from_file_location("cf_build_lib_under_test", str(repo / PKG / "build_lib.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_builder_loads_without_library(tmp_path):
    repo = clean_copy(tmp_path)
    bl = load_builder(repo)
    assert not os.path.exists(bl.LIB)
    assert not bl.up_to_date()
    us = bl.units()
    objs = [u[1] for u in us]
    assert len(objs) == len(set(objs))
    # every instantiation part the dispatch table names is built exactly once
    parts = {tuple(d.split("=")[1] for d in u[2]) for u in us if u[2]}
    for f32 in ("0", "1"):
        for nk in ("0", "1"):
            want = set(range(10)) | {21, 22, 23} | (set(range(10, 21)) if f32 == "0" else set())
            assert {int(p) for a, b, p in parts if (a, b) == (f32, nk)} == want


def test_package_import_without_compiler_is_a_clear_import_error(tmp_path):
    repo = clean_copy(tmp_path)
    env = dict(os.environ, HIPCC=str(tmp_path / "no-such-hipcc"), PATH="/usr/bin:/bin")
    r = subprocess.run([sys.executable, "-c", f"import {PKG}"], cwd=str(repo), env=env,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "hipcc not found" in r.stderr, r.stderr[-2000:]
    assert not os.path.exists(repo / PKG / "libcf.so")


def test_stamp_follows_content_not_file_times(tmp_path):
    repo = clean_copy(tmp_path)
    bl = load_builder(repo)
    # a library with a matching stamp is current, whatever the file times say
    open(bl.LIB, "wb").close()
    with open(bl.STAMP, "w") as f:
        f.write(bl.source_hash())
    assert bl.up_to_date()
    later = os.path.getmtime(bl.LIB) + 1000
    for d in (bl.CSRC, bl.INCLUDE):
        for f in os.listdir(d):
            os.utime(os.path.join(d, f), (later, later))
    assert bl.up_to_date()
    # any change of a source makes it stale
    hdr = os.path.join(bl.CSRC, "cf_launch.h")
    with open(hdr, "a") as f:
        f.write("\n// edited\n")
    assert not bl.up_to_date()


@pytest.mark.skipif(not os.path.exists(os.path.join(ROOT, PKG, "libcf.so")), reason="library not built here")
def test_built_library_is_current():
    bl = load_builder(__import__("pathlib").Path(ROOT))
    assert bl.up_to_date(), "libcf.so is older than the sources: rebuild it"


def test_hash_does_not_depend_on_the_tree_path(tmp_path):
    a = load_builder(clean_copy(tmp_path / "one"))
    b = load_builder(clean_copy(tmp_path / "two" / "deeper"))
    assert a.source_hash() == b.source_hash()


def test_unit_stamps_follow_their_own_source_and_the_headers(tmp_path):
    repo = clean_copy(tmp_path)
    bl = load_builder(repo)
    us = bl.units()
    before = {obj: bl._unit_hash(src, defs) for src, obj, defs in us}
    # the same unit at another path has the same stamp
    other = load_builder(clean_copy(tmp_path / "elsewhere"))
    assert [other._unit_hash(s, d) for s, _, d in other.units()] == list(before.values())
    # one translation unit edited: its objects alone go stale
    with open(os.path.join(bl.CSRC, "b2b_stream.hip"), "a") as f:
        f.write("\n// edited\n")
    after = {obj: bl._unit_hash(src, defs) for src, obj, defs in us}
    stale = {os.path.basename(o) for o in before if before[o] != after[o]}
    assert stale == {"b2b_stream.o"}
    # a header edited: every object goes stale
    with open(os.path.join(bl.INCLUDE, "cf.h"), "a") as f:
        f.write("\n// edited\n")
    again = {obj: bl._unit_hash(src, defs) for src, obj, defs in us}
    assert all(again[o] != after[o] for o in after)
