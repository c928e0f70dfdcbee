"""The C ABI's host layer under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

tests/host/capi_host_test.cpp links capi.cpp and plan.cpp as shipped against stand-in launchers
that perform every workspace / slab write of the replaced kernels on exact-size host buffers:
argument validation, the *_workspace / *_bytes arithmetic and the placement of every region are
checked for every path, including the vocabulary step above 4096 tokens."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "token_adapter_routing_amd", "csrc")
HIP_INC = "/opt/rocm/include"


def _build(tmp_path, extra_sources=()):
    if shutil.which("g++") is None or not os.path.exists(os.path.join(HIP_INC, "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers are missing")
    exe = str(tmp_path / "capi_host_test")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", f"-I{HIP_INC}", f"-I{os.path.join(ROOT, 'include')}",
           f"-I{CSRC}", os.path.join(CSRC, "capi.cpp"), *extra_sources,
           os.path.join(ROOT, "tests", "host", "capi_host_test.cpp"), "-o", exe]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert p.returncode == 0, p.stdout
    return exe


def test_capi_host_layer_sanitized(tmp_path):
    exe = _build(tmp_path, [os.path.join(CSRC, "plan.cpp")])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    p = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env, timeout=600)
    assert p.returncode == 0, p.stdout[-4000:]
    assert " 0 failures" in p.stdout


def test_sanitized_harness_catches_an_undersized_step_workspace(tmp_path):
    """A planted mistake in a copy of the plan (the step's partials sized for at most 4096
    tokens) must make the harness fail: the stand-in split launches overrun the buffer."""
    src = open(os.path.join(CSRC, "plan.cpp")).read()
    good = "p.part_bytes = split_part_floats(N, d_in, r_pad) * sizeof(float);"
    assert good in src
    bad = tmp_path / "plan_undersized.cpp"
    bad.write_text(src.replace(good, "p.part_bytes = split_part_floats(N < 4096 ? N : 4096, d_in, r_pad) * "
                                     "sizeof(float);").replace('#include "molora_plan.h"',
                                                               f'#include "{os.path.join(CSRC, "molora_plan.h")}"'))
    exe = _build(tmp_path, [str(bad)])
    p = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert p.returncode != 0
    assert "heap-buffer-overflow" in p.stdout or "FAIL" in p.stdout
