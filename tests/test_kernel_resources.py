"""Every GEMM kernel instantiation keeps all of its accumulators in AGPRs.

The main loop's MFMAs are inline asm whose accumulator operand is tied to AGPRs, and the hardware
does not interlock other instructions' accumulator accesses against an MFMA in flight. If the
compiler holds part of a tile's accumulators in VGPRs (copying them to and from the AGPRs around
the MFMAs), the sums come out wrong: a 256 x 256 AllReduce instantiation compiled that way (183
AGPRs for 256 accumulators per thread) wrote zeros into most of its partial. The build checks the
compiler's resource remarks; this test checks the checker and the kernels as built."""

import os
import subprocess
import tempfile

import pytest

from allgather_gemm_persistent_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNELS = os.path.join(ROOT, "allgather_gemm_persistent_amd", "csrc", "kernels.hip")
REMARKS = os.path.join(ROOT, "_build", "kernels.resources.txt")


def _remark(name, agprs, vgprs=256):
    tag = "[-Rpass-analysis=kernel-resource-usage]"
    return "\n".join([
        f"kernels.hip:749:1: remark: Function Name: {name} {tag}",
        f"kernels.hip:749:1: remark: VGPRs: {vgprs} {tag}",
        f"kernels.hip:749:1: remark: AGPRs: {agprs} {tag}",
        f"kernels.hip:749:1: remark: VGPRs Spill: 0 {tag}",
    ])


def test_checker_flags_accumulators_outside_agprs():
    ar256 = "_ZN3agg11gemm_kernelILi256ELi256ELi0ELi2EEEvNS_8GemmArgsE"
    fp8 = "_ZN3agg11gemm_kernelILi256ELi224ELi1ELi0EEEvNS_8GemmArgsE"
    small = "_ZN3agg11gemm_kernelILi64ELi64ELi0ELi2EEEvNS_8GemmArgsE"
    copy = "_ZN3agg11copy_kernelENS_8GemmArgsE"
    good = "\n".join([_remark(ar256, 256), _remark(fp8, 224), _remark(small, 16), _remark(copy, 0, 38)])
    res = B.kernel_resources(good)
    assert res[ar256]["AGPRs"] == 256 and res[copy]["VGPRs"] == 38
    assert B.accumulator_problems(res) == []
    # the failure seen: 183 AGPRs for 256 x 256 / 256 threads = 256 accumulators
    bad = B.accumulator_problems(B.kernel_resources("\n".join([_remark(ar256, 183), _remark(small, 16)])))
    assert len(bad) == 1 and "256, 256, 0, 2" in bad[0], bad
    # fp8 256 x 224: 224 per thread, one fewer fails
    assert B.accumulator_problems(B.kernel_resources(_remark(fp8, 223)))


def _remarks_text():
    if os.path.exists(REMARKS) and os.path.getmtime(REMARKS) >= os.path.getmtime(KERNELS):
        return open(REMARKS).read()
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    with tempfile.TemporaryDirectory() as d:
        cmd = [hipcc, *B.HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-c",
               KERNELS, "-o", os.path.join(d, "k.o"), "-Rpass-analysis=kernel-resource-usage"]
        r = subprocess.run(cmd, stderr=subprocess.PIPE, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return r.stderr


def test_built_gemm_kernels_hold_accumulators_in_agprs():
    res = B.kernel_resources(_remarks_text())
    gemm = [n for n in res if B._GEMM_KERNEL.fullmatch(n)]
    # bf16: five tile shapes x three epilogues; fp8: five shapes; the FFN chain's 256 x 256
    assert len(gemm) == 21, sorted(gemm)
    assert B.accumulator_problems(res) == []
