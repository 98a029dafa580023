"""Build-time properties the kernels rely on, checked with the compiler's
resource report (no GPU needed): the persistent fused decode grid must have
every workgroup resident at once, so no instance of its kernel may use
scratch memory (a dispatch waiting for scratch can hold workgroups back);
and the grouped path's kernels keep their values in registers (a spill to
scratch costs a memory round trip per reload)."""

import os
import re
import shutil
import subprocess

import pytest

from mxfp4_moe_decode_amd import build

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def _resource_report(name, tmp_path):
    src = os.path.join(build.CSRC, name)
    cmd = [build.hipcc()] + build._flags() + ["-x", "hip", f"--offload-arch={build.ARCH}", "-Xclang",
                                               "-target-feature", "-Xclang", "-packed-fp32-ops", "-c", src,
                                               "-o", str(tmp_path / "k.o"), "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    names = re.findall(r"Function Name: (\S+)", out.stderr)
    scratch = [int(v) for v in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", out.stderr)]
    assert len(scratch) == len(names)
    return dict(zip(names, scratch))


@pytest.mark.parametrize("name", ["router.hip", "grouped.hip", "quant.hip", "align_sort.hip"])
def test_grouped_path_kernels_use_no_scratch(name, tmp_path):
    report = _resource_report(name, tmp_path)
    assert report and all(v == 0 for v in report.values()), report


def test_fused_decode_kernel_uses_no_scratch(tmp_path):
    report = _resource_report("decode.hip", tmp_path)
    names = [n for n in report if "fused_decode_kernel" in n]
    scratch = [report[n] for n in names]
    assert len(names) >= 3, "expected the MiniMax, folded MiniMax and run-time shape instances"
    assert len(scratch) == len(names)
    assert all(v == 0 for v in scratch), dict(zip(names, scratch))


def test_grouped_gemm_m0_written_only_by_its_lds_loads(tmp_path):
    """The grouped GEMM kernels set M0 in inline asm before each direct
    global-to-LDS load, and the compiler does not preserve M0 across that asm.
    That is sound only while the compiler itself uses M0 nowhere in those
    kernels: outside the asm blocks their code must not mention M0, and every
    asm block that writes it must issue the load right after."""
    src = os.path.join(build.CSRC, "grouped.hip")
    asm = tmp_path / "grouped.s"
    cmd = [build.hipcc()] + build._flags() + ["-x", "hip", f"--offload-arch={build.ARCH}", "-Xclang",
                                               "-target-feature", "-Xclang", "-packed-fp32-ops",
                                               "--cuda-device-only", "-S", src, "-o", str(asm)]
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    text = asm.read_text()
    kernels = re.findall(r"^(\S*grouped_gemm_kernel\S*):[^\n]*\n(.*?)^\.Lfunc_end", text, re.M | re.S)
    assert len(kernels) >= 4, "expected the grouped GEMM instances"
    for name, body in kernels:
        outside, blocks = [], []
        for i, part in enumerate(re.split(r";;#ASMSTART|;;#ASMEND", body)):
            (blocks if i % 2 else outside).append(part)
        code = [ln.split(";")[0] for part in outside for ln in part.splitlines()]
        assert not any(re.search(r"\bm0\b", ln) for ln in code), f"{name}: the compiler uses M0"
        writers = [b for b in blocks if re.search(r"\bm0\b", b)]
        assert writers, f"{name}: no direct-to-LDS loads found"
        for b in writers:
            ins = [ln.strip() for ln in b.splitlines() if ln.strip() and not ln.strip().startswith(";")]
            assert ins[0].startswith("s_mov_b32 m0,") and ins[-1].startswith("global_load_lds_dword"), (name, ins)
