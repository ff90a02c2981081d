"""Occupancy the forward kernels are designed for (CPU only: a device-only compile).

The speed of each variant rests on how many of its workgroups share a compute
unit, which its LDS size and register count decide: the 16-row H <= 16 kernels
at 19 KiB run eight per CU (two waves per SIMD), the four-wave D-split kernel two
per CU. A few stray bytes of LDS silently cost a whole workgroup per CU, so the
compiler's resource report is checked here.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "sparse_attention_top_amd", "csrc", "sparse_mla.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LDS_PER_CU = 160 * 1024

# kernel (demangled template form) -> (workgroups per CU its LDS must allow, waves per SIMD)
EXPECTED = {
    "smla_fwd16_kernel<1, 512>": (8, 2),
    "smla_fwd16_fp8_kernel<2, 512>": (8, 2),
    "smla_fwd_kernel<4, 2>": (2, 2),
    "smla_fwd_kernel<2, 2>": (2, 1),
    "smla_fwd_fp8_kernel<8, 4>": (1, 2),
}

MANGLED = {
    "smla_fwd16_kernel<1, 512>": "smla_fwd16_kernelILi1ELi512EE",
    "smla_fwd16_fp8_kernel<2, 512>": "smla_fwd16_fp8_kernelILi2ELi512EE",
    "smla_fwd_kernel<4, 2>": "15smla_fwd_kernelILi4ELi2EE",
    "smla_fwd_kernel<2, 2>": "15smla_fwd_kernelILi2ELi2EE",
    "smla_fwd_fp8_kernel<8, 4>": "smla_fwd_fp8_kernelILi8ELi4EE",
}


@pytest.fixture(scope="module")
def resources(tmp_path_factory):
    if not os.path.exists(HIPCC) or shutil.which("ld.lld", path="/opt/rocm/llvm/bin") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("occ") / "fwd.o"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-c", "-o", str(out), SRC,
           "-Rpass-analysis=kernel-resource-usage"]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr[-2000:]
    res, cur = {}, None
    for line in proc.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            res[cur] = {}
            continue
        m = re.search(r"remark:\s+(LDS Size \[bytes/block\]|Occupancy \[waves/SIMD\]|VGPRs|AGPRs): (\d+)", line)
        if m and cur:
            res[cur][m.group(1)] = int(m.group(2))
    return res


@pytest.mark.parametrize("kernel", sorted(EXPECTED))
def test_forward_kernel_occupancy(resources, kernel):
    wgs, waves = EXPECTED[kernel]
    hits = [v for k, v in resources.items() if MANGLED[kernel] in k]
    assert hits, "kernel %s not found in the resource report" % kernel
    r = hits[0]
    lds = r["LDS Size [bytes/block]"]
    assert LDS_PER_CU // lds >= wgs, "%s: %d bytes of LDS allow %d workgroups per CU, designed for %d" % (
        kernel, lds, LDS_PER_CU // lds, wgs)
    assert r["Occupancy [waves/SIMD]"] >= waves, "%s: %d waves per SIMD, designed for %d" % (
        kernel, r["Occupancy [waves/SIMD]"], waves)
