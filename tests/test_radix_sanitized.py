"""The host radix tree + allocator, and the prefix-shared decode planner,
under AddressSanitizer and UndefinedBehaviorSanitizer: standalone C++ drivers
(tests/native) run seeded random operation streams (resp. random tables)
through the C ABI and check conservation and structure after every op (resp.
the plan's cover, sharing, records and minimal reads).  CPU only; built with
g++ (no HIP code involved)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "prefix_shared_kv_host_amd", "csrc")


@pytest.fixture(scope="module")
def fuzz_bin(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("fuzz") / "radix_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "radix.cpp"), os.path.join(CSRC, "common.cpp"),
           os.path.join(ROOT, "tests", "native", "radix_fuzz.cpp"), "-o", out]
    subprocess.run(cmd, check=True)
    return out


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_radix_fuzz_under_sanitizers(fuzz_bin, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([fuzz_bin, str(seed), "15000"], env=env, capture_output=True, text=True,
                       timeout=600)
    assert p.returncode == 0, p.stdout + p.stderr[-4000:]
    assert "fuzz ok" in p.stdout


@pytest.fixture(scope="module")
def plan_fuzz_bin(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("fuzz") / "cascade_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "cascade_plan.cpp"), os.path.join(CSRC, "common.cpp"),
           os.path.join(ROOT, "tests", "native", "cascade_fuzz.cpp"), "-o", out]
    subprocess.run(cmd, check=True)
    return out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_cascade_plan_fuzz_under_sanitizers(plan_fuzz_bin, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([plan_fuzz_bin, str(seed), "1500"], env=env, capture_output=True, text=True,
                       timeout=600)
    assert p.returncode == 0, p.stdout + p.stderr[-4000:]
    assert "fuzz ok" in p.stdout
