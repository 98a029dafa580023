"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU needed): every library source is compiled with both sanitizers on its
host side, linked with `capi_sanitize_driver.cpp`, and the driver exercises
size queries, layer validation and argument errors, including extreme sizes
(negative, zero, INT_MAX) and 20,000 random layer shapes.  Any sanitizer
report or unexpected status fails the test."""

import os
import shutil
import subprocess

import pytest

from mxfp4_moe_decode_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")

# host-side instrumentation only (device code is built as usual)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


@pytest.mark.timeout(900)
def test_capi_host_code_under_sanitizers(tmp_path):
    hipcc = build.hipcc()
    inc = ["-I", os.path.join(build.ROOT, "include"), "-I", build.CSRC]
    srcs = sorted(f for f in os.listdir(build.CSRC) if f.endswith((".hip", ".cpp")))
    procs, objs = [], []
    for f in srcs + ["driver"]:
        src = os.path.join(HERE, "capi_sanitize_driver.cpp") if f == "driver" else os.path.join(build.CSRC, f)
        obj = str(tmp_path / (f + ".o"))
        cmd = [hipcc, "-O1", "-g", "-std=c++17"] + SAN + inc
        if f.endswith(".hip"):
            cmd += ["-x", "hip", f"--offload-arch={build.ARCH}", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops"]
        cmd += ["-c", src, "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
        objs.append(obj)
    for p in procs:
        out, err = p.communicate(timeout=900)
        assert p.returncode == 0, err[-2000:]
    exe = str(tmp_path / "capi_sanitize")
    link = subprocess.run([hipcc] + SAN[:4] + objs + ["-o", exe], capture_output=True, text=True, timeout=300)
    assert link.returncode == 0, link.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    report = run.stdout + run.stderr
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    assert run.returncode == 0 and "ok: 0 failures" in run.stdout, report[-4000:]
