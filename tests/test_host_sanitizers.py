"""The host code of libns.so (argument validation, batch planner, rank
planner) and the fp64 oracle under AddressSanitizer and
UndefinedBehaviorSanitizer, built with g++ on the CPU (no device code: the
kernel launchers are replaced by host-only stand-ins that fail, and no check
here reaches them). The driver is tests/sanitize/host_check.cpp."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "newton_schulz_04_amd", "csrc")
ROCM = "/opt/rocm"


def _build(tmp_path):
    gxx = shutil.which("g++")
    if not gxx or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers are missing")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    objs = []
    for src, lang in [(os.path.join(CSRC, "ns_api.cpp"), "c++"), (os.path.join(CSRC, "ns_plan.cpp"), "c++"),
                      (os.path.join(CSRC, "ns_ranks.cpp"), "c++"),
                      (os.path.join(HERE, "sanitize", "kernel_stubs.cpp"), "c++"),
                      (os.path.join(HERE, "sanitize", "host_check.cpp"), "c++"),
                      (os.path.join(ROOT, "oracle", "ns_oracle.c"), "c")]:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        std = "-std=c++17" if lang == "c++" else "-std=c11"
        compiler = gxx if lang == "c++" else "gcc"
        cmd = [compiler, std, "-O1", "-g", *san, "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
               f"-I{ROOT}/include", f"-I{CSRC}", "-c", src, "-o", obj]
        if lang == "c":
            cmd[1:1] = ["-ffp-contract=off"]
        subprocess.run(cmd, check=True)
        objs.append(obj)
    exe = str(tmp_path / "host_check")
    subprocess.run([gxx, *san, *objs, "-o", exe, f"-L{ROCM}/lib", f"-Wl,-rpath,{ROCM}/lib",
                    "-lamdhip64", "-lm"], check=True)
    return exe


def test_host_code_under_asan_and_ubsan(tmp_path):
    exe = _build(tmp_path)
    env = dict(os.environ)
    # the HIP runtime keeps process-lifetime allocations; leaks are not what
    # this checks
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["HIP_VISIBLE_DEVICES"] = ""
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=600)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "host_check ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
