"""CPU tier under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's host side (argument checks of every entry point, workspace-size
and plan arithmetic, the slot-pool planner, settings parsing) is built with
both sanitizers on the host and driven by tests/sanitize/host_check.cpp with
no HIP device visible, so nothing is launched; the oracle's C source is built
with both sanitizers and driven by tests/sanitize/oracle_check.c.  Any report
(or a failed expectation) fails the test."""

import importlib.util
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SAN_DIR = os.path.join(HERE, "sanitize")


def _build():
    path = os.path.join(SAN_DIR, "build.py")
    if not os.path.exists(path) or not os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("gcc") is None:
        pytest.skip("sanitizer sources or toolchain not present")
    spec = importlib.util.spec_from_file_location("w4_sanitize_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.build()


def _run(exe, extra_env):
    env = dict(os.environ)
    env.update({"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    env.update(extra_env)
    p = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=600)
    report = p.stdout + p.stderr
    assert p.returncode == 0, report[-4000:]
    assert "ERROR: AddressSanitizer" not in report and "runtime error:" not in report, report[-4000:]
    assert "ERROR: LeakSanitizer" not in report, report[-4000:]
    return report


def test_host_side_under_sanitizers():
    out = _build()
    # no device visible: valid calls stop at the device check
    rep = _run(os.path.join(out, "host_check"), {"HIP_VISIBLE_DEVICES": "", "ROCR_VISIBLE_DEVICES": ""})
    assert "host checks: 0 failed" in rep


def test_oracle_under_sanitizers():
    out = _build()
    rep = _run(os.path.join(out, "oracle_check"), {"OMP_NUM_THREADS": "4"})
    assert "oracle checks:" in rep
