"""The C ABI's host code (argument checks, planning, size queries in api.cpp and
plan.hpp) built for the CPU with AddressSanitizer and UndefinedBehaviorSanitizer,
then every host-side test of tests/test_abi.py run against that build in a
child process with the sanitizer runtimes preloaded.  Runs on CPU."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")


def _runtime(name: str) -> str:
    return subprocess.check_output(["g++", f"-print-file-name={name}"], text=True).strip()


def test_abi_host_checks_under_sanitizers():
    from hyena_long_conv_amd.build import build_hostcheck
    lib = build_hostcheck()
    syms = subprocess.check_output(["nm", "-D", "-u", lib], text=True)
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "build is not instrumented"
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    assert os.path.isabs(asan) and os.path.isabs(ubsan), (asan, ubsan)
    env = dict(os.environ, HYENA_LIB=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("HYENA_FORCE_PATH", None)
    env.pop("HYENA_FOURSTEP_N1", None)
    probe = ("import hyena_long_conv_amd as H; L = H.lib(); "
             "assert H.LIB_PATH.endswith('libhyena_hostcheck.so'), H.LIB_PATH; "
             "assert L.hyena_plan(16, None) == 1; print('loaded', H.LIB_PATH)")
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "loaded" in r.stdout, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join("tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out
    assert " passed" in r.stdout and " skipped" not in r.stdout.splitlines()[-1], out
