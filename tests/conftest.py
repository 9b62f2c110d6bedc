import importlib.util
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionstart(session):
    """Brings libcf.so up to date before any test module imports the package.

    A fresh checkout has no library: building it takes minutes, so the
    builder's progress lines go to the terminal past pytest's output capture
    (one line per compiled unit)."""
    path = os.path.join(ROOT, "b2bgemm_stage_stream_amd", "build_lib.py")
    spec = importlib.util.spec_from_file_location("cf_build_lib_conftest", path)
    bl = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bl)
    if bl.up_to_date() or bl.hipcc() is None:
        return   # nothing to do, or the package import reports the missing compiler
    capman = session.config.pluginmanager.getplugin("capturemanager")

    def log(msg):
        if capman is None:
            sys.stderr.write(msg + "\n")
            sys.stderr.flush()
            return
        with capman.global_and_fixture_disabled():
            sys.stderr.write(msg + "\n")
            sys.stderr.flush()

    bl.ensure_built(log=log)
