"""The host code of the library under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): a build whose host code is
instrumented (device code as usual) runs thousands of random plans through
the host-only planner entry points and the argument checks of every call
(tests/planner_fuzz.py); a sanitizer report aborts the run."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FUZZ = os.path.join(ROOT, "tests", "planner_fuzz.py")


@pytest.mark.parametrize("sanitize,seed", [("address", 11), ("undefined", 12)])
def test_host_code_under_sanitizer(tmp_path, sanitize, seed):
    from latent_attention_decode_amd import build
    lib = build.build(sanitize=sanitize, out=str(tmp_path / f"libmla_decode_{sanitize}.so"))
    env = dict(os.environ, LD_PRELOAD=build.sanitizer_runtime(sanitize),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, FUZZ, lib, str(seed), "3000"], env=env, capture_output=True, text=True,
                       timeout=900)
    report = "AddressSanitizer" in r.stderr or "runtime error" in r.stderr
    assert r.returncode == 0 and not report, r.stderr[-4000:]
    assert "3000 random plans" in r.stdout
