"""The C ABI's host layer under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library with both sanitizers on its host code
(block_mean_pool_amd/build.py build_sanitized: every -fsanitize flag scoped
to the host pass) and runs the CPU boundary tests -- argument validation,
layouts, workspace sizes, the mask check, the Python binding's tensor checks
-- against that build in a child process with the compiler's ASan runtime
preloaded.  Any sanitizer report aborts the child (halt_on_error), so the
test fails on it.  No GPU is touched: every call there fails validation or
is host-only."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "sa_build", os.path.join(ROOT, "block_mean_pool_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def sanitized():
    b = _build_module()
    try:
        rt = b.asan_runtime()
    except FileNotFoundError as e:  # pragma: no cover
        pytest.skip(str(e))
    return b.build_sanitized(), rt


def _env(lib, rt):
    env = dict(os.environ)
    env.update(SA_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


def test_boundary_tests_pass_under_asan_and_ubsan(sanitized):
    lib, rt = sanitized
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                        os.path.join(ROOT, "tests", "test_binding_checks.py")],
                       cwd=ROOT, env=_env(lib, rt), capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]


def test_the_child_runs_the_sanitized_build(sanitized):
    # the binding loads SA_LIBRARY, and that library runs with the ASan
    # runtime mapped in
    lib, rt = sanitized
    code = ("import block_mean_pool_amd as sa\n"
            "maps = open('/proc/self/maps').read()\n"
            "print(sa.LIB_PATH, 'libsparse_attn_san.so' in maps, 'asan' in maps)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_env(lib, rt),
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    path, has_lib, has_rt = r.stdout.split()
    assert path == lib and has_lib == "True" and has_rt == "True"
