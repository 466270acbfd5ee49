"""The library's host code (argument validation, workspace planning, the host-only builders)
under AddressSanitizer and UndefinedBehaviorSanitizer: the C-ABI tests run against a build whose
host code carries both sanitizers (device code unchanged), with the sanitizer runtime preloaded
into the test process.  CPU only: the C-ABI tests make no device calls."""
import os
import subprocess
import sys

from conftest import ROOT
from diffusion_transformer_text_s3_amd import build


def test_abi_tests_clean_under_asan_and_ubsan():
    lib = build.build_sanitized()
    # the build really carries both instrumentations
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle_" in syms
    env = dict(os.environ, ZDIT_TEST_LIB=lib, LD_PRELOAD=build.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "tests/test_abi.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
    assert " passed" in r.stdout
