"""The library builds from sources alone, and its host code is clean under
AddressSanitizer and UndefinedBehaviorSanitizer.  No GPU needed: hipcc
cross-compiles for gfx950, and the C ABI's validation paths return before any
device call.

The tree is copied without any built file (no .so, no object), as a fresh
checkout would be, and built there with both documented commands.
"""

import ctypes  # noqa: F401  (the symbol check below runs in a child process)
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = "expert_ffn_layer_softmax_amd"
BUILT = (".so", ".o", ".tmp")


def _ignore(dirpath, names):
    return [n for n in names
            if n.endswith(BUILT) or n.startswith("_build") or n in ("__pycache__", ".pytest_cache")]


@pytest.fixture(scope="module")
def fresh_tree(tmp_path_factory):
    dst = tmp_path_factory.mktemp("checkout")
    for item in ("include", PKG, "oracle", "synth", "tests"):
        shutil.copytree(os.path.join(ROOT, item), os.path.join(dst, item), ignore=_ignore)
    for item in ("__graft_entry__.py", "pytest.ini"):
        shutil.copy(os.path.join(ROOT, item), os.path.join(dst, item))
    assert not any(f.endswith(".so") for _, _, fs in os.walk(dst) for f in fs)
    return str(dst)


def _run(cmd, cwd, env=None, timeout=600):
    r = subprocess.run(cmd, cwd=cwd, env=env, capture_output=True, text=True, timeout=timeout)
    assert r.returncode == 0, f"{cmd} failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def _declared(tree):
    import re
    text = open(os.path.join(tree, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_build_from_a_fresh_checkout(fresh_tree):
    lib = os.path.join(fresh_tree, PKG, "libmoe_mi355x.so")
    # the package's own build command, then the build entry point (which
    # compiles again and opens the result)
    _run([sys.executable, "-m", f"{PKG}.build"], fresh_tree)
    assert os.path.exists(lib)
    os.remove(lib)
    _run([sys.executable, "-c", "import __graft_entry__ as g; g.build()"], fresh_tree)
    assert os.path.exists(lib)
    # build() also makes the bounds-checking debug variant
    assert os.path.exists(os.path.join(fresh_tree, PKG, "libmoe_mi355x_dbg.so"))
    names = _declared(fresh_tree)
    assert "moe_layer_forward" in names
    probe = ("import ctypes, sys; L = ctypes.CDLL(sys.argv[1]); "
             "missing = [n for n in sys.argv[2:] if not hasattr(L, n)]; "
             "print(missing); sys.exit(1 if missing else 0)")
    _run([sys.executable, "-c", probe, lib, *names], fresh_tree)


def test_abi_host_code_under_asan_and_ubsan(fresh_tree):
    """Every C-ABI validation test, against a build whose host code carries
    ASan and UBSan (any report aborts the run: -fno-sanitize-recover)."""
    _run([sys.executable, "-m", f"{PKG}.build", "--sanitize"], fresh_tree)
    san = os.path.join(fresh_tree, PKG, "libmoe_mi355x_san.so")
    assert os.path.exists(san)
    sys.path.insert(0, os.path.join(fresh_tree, PKG))
    try:
        import importlib.util
        spec = importlib.util.spec_from_file_location("_san_build", os.path.join(fresh_tree, PKG, "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        runtime = mod.sanitizer_runtime()
    finally:
        sys.path.pop(0)
    env = dict(os.environ, LD_PRELOAD=runtime, MOE_MI355X_LIB=san,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
              "tests/test_abi_cpu.py"], fresh_tree, env=env)
    assert "passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
