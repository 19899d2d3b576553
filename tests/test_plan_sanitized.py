"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer.

pic_plan.cpp is plain C++17 (no HIP), so it is built here with g++ and the
sanitizers, together with a randomised driver (tests/native/plan_stress.cpp)
that runs every planning entry point on random pools and batches, valid and
malformed, and checks each valid plan for internal consistency.  Any
out-of-bounds access, overflow or undefined shift aborts the driver.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "position_independent_kv_pic_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not available")
    out = str(tmp_path_factory.mktemp("asan") / "plan_stress")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "pic_plan.cpp"), os.path.join(ROOT, "tests", "native", "plan_stress.cpp"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    return out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_planner_is_clean_under_sanitizers(driver, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([driver, str(seed), "300"], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, (res.stdout[-2000:], res.stderr[-4000:])
    assert res.stdout.startswith("ok "), res.stdout
    assert int(res.stdout.split()[1]) > 50, "too few valid plans exercised"
