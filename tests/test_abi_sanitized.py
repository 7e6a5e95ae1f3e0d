"""The host-side ABI checks (tests/abi_host_checks.cpp) against a build of the library
whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer: workspace
sizing, argument validation and every refusal path, run without a GPU."""
import os
import subprocess

import pytest

from draft_block_verification_spec_amd import build


@pytest.fixture(scope="module")
def checks(tmp_path_factory):
    return build.build_host_checks(str(tmp_path_factory.mktemp("hostsan")))


def test_library_host_code_is_instrumented(checks):
    lib = os.path.join(os.path.dirname(checks), "libspecverify.so")
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms
    assert "__ubsan_handle_" in syms


def test_host_abi_checks_under_sanitizers(checks):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([checks], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "host ABI checks passed" in r.stdout
