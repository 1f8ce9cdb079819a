"""The C ABI layer's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

abi.hip (argument checks, workspace layouts, dispatch) is rebuilt with both
sanitizers on its host code (device code untouched) and the host ABI tests run
against that build in a child process, with the ASan runtime preloaded into the
(uninstrumented) Python interpreter.  Any report fails the run: UBSan is set to
halt on the first error and ASan aborts on its first one.  Leak checking is off
(the interpreter itself never frees some of its memory)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_host_tests_clean_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from dflash_block_draft_amd import build
    lib = build.build_sanitized(verbose=False)
    env = dict(os.environ)
    env.update({
        "DFLASH_MLA_LIB": lib,
        "LD_PRELOAD": build.san_runtime(),
        "ASAN_OPTIONS": f"detect_leaks=0:log_path={tmp_path}/asan",
        "UBSAN_OPTIONS": f"print_stacktrace=1:halt_on_error=1:log_path={tmp_path}/ubsan",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"), "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    reports = [p.read_text() for p in tmp_path.iterdir() if p.name.startswith(("asan", "ubsan"))]
    assert not reports, "\n".join(reports)[:4000]
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert " passed" in r.stdout
