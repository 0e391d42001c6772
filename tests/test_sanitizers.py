"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Two builds, each in a child process with its sanitizer runtime preloaded and
every finding fatal:

- the fp64 oracle (pa_oracle.c, gcc) under its pin tests;
- the library's host code (planning, argument checks, the contract check,
  the scratch lookup; hipcc with the sanitizers on the host side only) under
  the C ABI and binding tests, which drive every validation path without a
  GPU.

A child that dies of a finding prints the sanitizer's report; the test shows
its tail."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle import build as obuild  # noqa: E402
from paged_gqa_attention_02_amd import build as pbuild  # noqa: E402

ASAN_OPTIONS = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
UBSAN_OPTIONS = "print_stacktrace=1:halt_on_error=1"


def run_child(tests, env_extra):
    env = dict(os.environ, ASAN_OPTIONS=ASAN_OPTIONS, UBSAN_OPTIONS=UBSAN_OPTIONS,
               **env_extra)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
           "-m", "not gpu"] + tests
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    tail = "\n".join(out.splitlines()[-40:])
    assert res.returncode == 0, f"sanitized run failed ({res.returncode}):\n{tail}"
    for bad in ("runtime error:", "AddressSanitizer", "LeakSanitizer"):
        assert bad not in out, f"sanitizer finding:\n{tail}"
    assert " passed" in out, tail
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    lib = obuild.build(out=str(tmp_path / "libpa_oracle_san.so"), sanitize=True)
    run_child(["tests/test_oracle.py"],
              {"PA_ORACLE_LIB": lib, "LD_PRELOAD": obuild.sanitizer_preload()})


def test_host_api_under_asan_ubsan(tmp_path):
    lib = pbuild.build_host_sanitized(str(tmp_path))
    preload = pbuild.sanitizer_preload()
    if not os.path.exists(preload):
        pytest.fail(f"clang ASan runtime not found at {preload}")
    run_child(["tests/test_abi.py", "tests/test_binding_checks.py"],
              {"PAGED_ATTN_LIB": lib, "LD_PRELOAD": preload})
