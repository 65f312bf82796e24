"""The library's host code (plans, exact CG tables, CSR construction, workspace layouts, argument
validation) built with the address and undefined-behaviour sanitizers and exercised through the C
ABI by tests/native/host_abi_check.cpp (CPU only: no GPU call is made)."""

from __future__ import annotations

import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "clebsch_gordan_tensor_receiver_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_code_under_asan_and_ubsan(tmp_path):
    # Host translation units only (the .hip sources hold the device probes and the static scratch).
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.cpp"))) + [os.path.join(ROOT, "tests", "native", "host_abi_check.cpp")]
    exe = str(tmp_path / "host_abi_check")
    stubs = tmp_path / "stubs.cpp"
    # The .hip translation units export these; host-only builds get stand-ins that refuse.
    stubs.write_text(
        '#include "cgtp.h"\n'
        'extern "C" cgtp_status_t cgtp_measure_peak(int, void*, const void*, size_t, int, void*, double*, double*)'
        ' { return CGTP_ERR_UNSUPPORTED; }\n'
        'extern "C" cgtp_status_t cgtp_conv_forward_static(cgtp_plan_t, cgtp_graph_t, cgtp_schedule_t, const void*,'
        ' const void*, const void*, const void*, const void*, void*, void*) { return CGTP_ERR_UNSUPPORTED; }\n')
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           f"-I{os.path.join(ROOT, 'include')}", *srcs, str(stubs), "-o", exe, f"-L{ROCM}/lib", "-lhiprtc",
           "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-ldl", "-lpthread"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600, env=env)
    print(r.stdout[-3000:])
    assert r.returncode == 0, r.stdout[-4000:]
    assert "0 failure(s)" in r.stdout
