"""The host half of the library (planning, descriptors, assembly: plan.cpp)
built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer, driven
through its C ABI by the plain C11 caller and by a randomised C++ driver.  No
HIP code is compiled here: the device half is not on this path."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.fixture(scope="module")
def sanitized_plan(tmp_path_factory):
    if shutil.which("g++") is None or shutil.which("gcc") is None:
        pytest.skip("no host compiler")
    d = tmp_path_factory.mktemp("san")
    obj = d / "plan.o"
    _run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(ROOT, "ragged_token_log_amd", "csrc", "plan.cpp"), "-o", str(obj)])
    return d, obj


def _env():
    env = dict(os.environ)
    # a preloaded library ahead of the ASan runtime is not an error here
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


def test_plain_c_caller_under_sanitizers(sanitized_plan):
    d, obj = sanitized_plan
    cobj = d / "c_abi_check.o"
    exe = d / "c_abi_check_san"
    _run(["gcc", "-std=c11", *SAN, "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(ROOT, "tests", "native", "c_abi_check.c"), "-o", str(cobj)])
    _run(["g++", *SAN, str(cobj), str(obj), "-lm", "-o", str(exe)])
    res = _run([str(exe)], env=_env(), timeout=120)
    assert res.stdout.strip().endswith("ok"), res.stdout + res.stderr


def test_randomised_driver_under_sanitizers(sanitized_plan):
    d, obj = sanitized_plan
    exe = d / "plan_fuzz_san"
    _run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "tests", "native", "plan_fuzz.cpp"), str(obj), "-o", str(exe)])
    res = _run([str(exe), "3000"], env=_env(), timeout=300)
    last = res.stdout.strip().splitlines()[-1]
    assert last.startswith("ok"), res.stdout + res.stderr
    assert int(last.split()[1]) >= 500, last   # a third of the cases reach a plan
