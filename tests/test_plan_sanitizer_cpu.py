"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer.

The planner parses untrusted slice lists, so it is built here from source with
g++ (host code only, no HIP) and ``-fsanitize=address,undefined`` together with
the fuzz driver ``tests/plan_fuzz.cpp``, which feeds it random valid and
invalid problems and the long-context backward plan.  Any memory error or
undefined behaviour aborts the driver.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PLANNER = os.path.join(ROOT, "flexible_mask_flash_amd", "csrc", "ffa_plan.cpp")
DRIVER = os.path.join(ROOT, "tests", "plan_fuzz.cpp")


@pytest.fixture(scope="module")
def fuzz_binary(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("plan_fuzz") / "plan_fuzz")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", PLANNER, DRIVER, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, f"sanitizer build failed:\n{r.stderr}"
    return out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_planner_is_clean_under_sanitizers(fuzz_binary, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([fuzz_binary, "3000", str(seed)], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, f"plan_fuzz failed (seed {seed}):\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "plans accepted" in r.stdout
