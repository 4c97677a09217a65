"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C ABI's host side (argument checks, workspace carving, state handling;
every source's host code) is rebuilt with both sanitizers and the host ABI
checks are run against it; the C oracle is rebuilt with both sanitizers and
its pins are run against it.  Each runs in a child process that preloads the
matching sanitizer runtime; a report fails the child (halt on error)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(env_extra, args):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:detect_odr_violation=0:alloc_dealloc_mismatch=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", *args],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def test_c_abi_host_checks_under_sanitizers():
    from log_linear_token_amd import build_sanitized as S
    lib = S.build()
    rt = S.runtime()
    if not os.path.exists(rt):
        pytest.skip(f"no clang ASan runtime at {rt}")
    _run({"LOGLIN_LIB": lib, "LD_PRELOAD": rt}, ["tests/test_abi_host.py"])


def test_oracle_under_sanitizers():
    rt = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    if not os.path.isabs(rt):
        pytest.skip("gcc has no shared libasan")
    _run({"LLO_SANITIZE": "1", "LD_PRELOAD": rt},
         ["tests/test_oracle_pins.py", "tests/test_oracle_gdn.py", "tests/test_oracle_mutations.py",
          "tests/test_oracle_grads.py"])
