"""Sanitizer tier on the CPU: the oracle (gdnref.c) built with gcc's
AddressSanitizer and UBSan runs every oracle pin, and the C ABI's host code
(gdn_api.cpp: validation and dispatch) built with host AddressSanitizer and
UBSan runs every CPU ABI test.  Each build is loaded in a child process with
its compiler's ASan runtime preloaded; any sanitizer finding aborts that
process, so the test passes only on a clean run.  Leak detection is off: the
interpreter itself does not free everything at exit."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FINDINGS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer", "UndefinedBehaviorSanitizer")


def run_child(test_file, env_extra, preload):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    # -s: a sanitizer report is written straight to the child's stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", test_file)], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert r.returncode == 0, "%s under sanitizers failed (rc %d)" % (test_file, r.returncode)
    for f in FINDINGS:
        assert f not in out, "sanitizer finding in %s: %s" % (test_file, f)
    assert " passed" in out


def instrumented(lib):
    """The library calls the sanitizers' report functions (it was built with them)."""
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    return "__asan_report" in syms and "__ubsan_handle" in syms


def test_oracle_pins_under_asan_ubsan(tmp_path):
    import oracle
    lib = oracle.build_sanitized(str(tmp_path / "libgdnref_san.so"))
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc's libasan is not installed")
    assert instrumented(lib)
    run_child("test_oracle_pins.py", {"GDNREF_LIBRARY": lib}, asan)


def test_abi_host_code_under_asan_ubsan(tmp_path):
    from gated_delta_rule_02_amd import _build
    lib = _build.build_sanitized(str(tmp_path))
    assert instrumented(lib)
    run_child("test_abi_cpu.py", {"GDN_LIBRARY": lib}, _build.asan_runtime())
