"""CPU sanitizer leg: the oracle, the input generator and the host-only half of
the C ABI built with AddressSanitizer and UndefinedBehaviorSanitizer, then run.

`sanitize_driver.cpp` exercises oracle rows and frames on edge cases (V below
K, -inf lanes, signed zeros, invalid tokens and IDs, clamped counts, packed
offsets out of range, completion records), the generator on every recipe and
padding kind, and every host-checkable plan and rejection path of the library
with device = -1, so that no call reaches a launch.  The GPU half is stubbed
(a reached stub aborts).  Host compilers only: no GPU code is built here.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIP_INCLUDE = "/opt/rocm/include"

FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all"]


def _compile(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-4000:]}"


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="host compilers not found")
@pytest.mark.skipif(not os.path.isdir(os.path.join(HIP_INCLUDE, "hip")),
                    reason="HIP headers not found")
def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    d = str(tmp_path)
    src = lambda *p: os.path.join(ROOT, *p)
    _compile(["gcc", "-std=c11", *FLAGS, "-c", src("oracle", "oracle_logprobs.c"), "-o", "oracle.o"], d)
    _compile(["gcc", "-std=c11", *FLAGS, "-c", src("synth", "synth.c"), "-o", "synth.o"], d)
    cxx = ["g++", "-std=c++17", *FLAGS, "-D__HIP_PLATFORM_AMD__", "-I" + HIP_INCLUDE,
           "-I" + src("include")]
    _compile([*cxx, "-c", src("full_vocab_logprob_amd", "csrc", "flp_host.cpp"), "-o", "host.o"], d)
    _compile([*cxx, "-c", src("tests", "sanitize_driver.cpp"), "-o", "driver.o"], d)
    _compile(["g++", *FLAGS, "driver.o", "host.o", "oracle.o", "synth.o", "-lpthread", "-lm",
              "-o", "driver"], d)
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([os.path.join(d, "driver")], cwd=d, capture_output=True, text=True,
                       env=env, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-6000:]
    assert "all checks passed" in r.stdout
    assert "runtime error" not in report and "ERROR: AddressSanitizer" not in report
