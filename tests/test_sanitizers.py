"""Sanitizer runs of the host-side code (CPU only, no GPU):

* the library's host code (packer, schedule, every entry point's argument checks) built with
  AddressSanitizer (leak detection on) and UndefinedBehaviorSanitizer on the host side;
* the oracle, every routine in both precisions, under the same two sanitizers;
* the CPU model of the publication protocols under ThreadSanitizer.

Each build is compiled fresh into a temporary directory and must run clean: exit status 0 and
no sanitizer report.
"""

import os
import subprocess

import pytest

pytestmark = pytest.mark.slow

REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer", "WARNING: ThreadSanitizer")


def run_clean(exe, *args, env=None):
    res = subprocess.run([exe, *args], capture_output=True, text=True, timeout=600, env=env)
    text = res.stdout + res.stderr
    assert res.returncode == 0, text[-4000:]
    for marker in REPORTS:
        assert marker not in text, text[-4000:]
    return text


def test_library_host_code_under_asan_and_ubsan(tmp_path):
    from bidirectional_lstm_sequence_amd import _sanitize
    exe = _sanitize.build_host_check(str(tmp_path))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1")
    out = run_clean(exe, env=env)
    assert "host checks: 0 failure(s)" in out


def test_oracle_under_asan_and_ubsan(tmp_path):
    import oracle
    exe = oracle.build_check(str(tmp_path / "oracle_check"))
    out = run_clean(exe, env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert "oracle checks: 0 failure(s)" in out


def test_protocol_model_under_tsan(tmp_path):
    from bidirectional_lstm_sequence_amd import _sanitize
    exe = _sanitize.build_protocol_model_tsan(str(tmp_path))
    out = run_clean(exe, "5000")
    assert "FAIL" not in out
