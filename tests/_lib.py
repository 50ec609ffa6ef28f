"""Locates or builds libpa.so for tests (CPU: builds in-tree when missing)."""
import importlib.util
import os

from tests.conftest import ROOT

LIB = os.path.join(ROOT, "paged_kv_cache_57_amd", "libpa.so")
BUILD_PY = os.path.join(ROOT, "paged_kv_cache_57_amd", "build.py")


def load_build_module():
    # loaded by path: the package itself refuses to import before the library exists
    spec = importlib.util.spec_from_file_location("pa_build", BUILD_PY)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def ensure_built():
    if not os.path.exists(LIB):
        load_build_module().build()
    return LIB
