"""Occupancy and register use the kernels are designed for (CPU only: device-only compiles).

The speed of each variant rests on how many of its workgroups share a compute
unit, which its LDS size and register count decide: the 16-row H <= 16 kernels
at 19 KiB run eight per CU (two waves per SIMD), the four-wave D-split kernel two
per CU, the persistent 128-head kernel one per CU at one wave per SIMD. A few
stray bytes of LDS silently cost a whole workgroup per CU, and a register spill
puts scratch traffic (sharing the memory counter with the gathers) into the
loop, so the compiler's resource report is checked here: no kernel of the
library may use scratch. The 128-head kernel keeps its accumulators by hand in
the AGPR file; the compiler must not place any value of its own there.
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
    "smla_fwd16_kernel<1, 640>": (8, 2),
    "smla_fwd16_i64_kernel<640>": (8, 2),
    "smla_fwd16_fp8_kernel<2, 512>": (8, 2),
    "smla_fwd_kernel<4, 2>": (2, 2),
    "smla_fwd_kernel<2, 2>": (2, 1),
    "smla_fwd_fp8_kernel<8, 4>": (1, 2),
    "smla_fwd128_kernel<false>": (1, 1),
    "smla_fwd128_kernel<true>": (1, 1),
}

MANGLED = {
    "smla_fwd16_kernel<1, 640>": "smla_fwd16_kernelILi1ELi640EE",
    "smla_fwd16_i64_kernel<640>": "smla_fwd16_i64_kernelILi640EE",
    "smla_fwd16_fp8_kernel<2, 512>": "smla_fwd16_fp8_kernelILi2ELi512EE",
    "smla_fwd_kernel<4, 2>": "15smla_fwd_kernelILi4ELi2EE",
    "smla_fwd_kernel<2, 2>": "15smla_fwd_kernelILi2ELi2EE",
    "smla_fwd_fp8_kernel<8, 4>": "smla_fwd_fp8_kernelILi8ELi4EE",
    "smla_fwd128_kernel<false>": "18smla_fwd128_kernelILb0EE",
    "smla_fwd128_kernel<true>": "18smla_fwd128_kernelILb1EE",
}
BWD = os.path.join(ROOT, "sparse_attention_top_amd", "csrc", "sparse_mla_bwd.hip")


FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "--cuda-device-only"]


def _need_hipcc():
    if not os.path.exists(HIPCC) or shutil.which("ld.lld", path="/opt/rocm/llvm/bin") is None:
        pytest.skip("hipcc not available")


def _report(src, out):
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-c", "-o", str(out), src,
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
        m = re.search(r"remark:\s+(LDS Size \[bytes/block\]|Occupancy \[waves/SIMD\]|VGPRs|AGPRs|"
                      r"ScratchSize \[bytes/lane\]|VGPRs Spill): (\d+)", line)
        if m and cur:
            res[cur][m.group(1)] = int(m.group(2))
    return res


@pytest.fixture(scope="module")
def resources(tmp_path_factory):
    _need_hipcc()
    return _report(SRC, tmp_path_factory.mktemp("occ") / "fwd.o")


@pytest.fixture(scope="module")
def resources_bwd(tmp_path_factory):
    _need_hipcc()
    return _report(BWD, tmp_path_factory.mktemp("occ") / "bwd.o")


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


def test_backward_dq16_occupancy(resources_bwd):
    """The backward's dq phase at H <= 16 runs 16-row tiles so that four one-wave workgroups share a CU (two tiles
    and a 640-entry list of LDS each), one wave on every SIMD."""
    hits = [v for k, v in resources_bwd.items() if "smla_bwd_dq16_kernelILi640EE" in k]
    assert hits, "smla_bwd_dq16_kernel<640> not found in the resource report"
    r = hits[0]
    assert LDS_PER_CU // r["LDS Size [bytes/block]"] >= 4, r["LDS Size [bytes/block]"]
    assert r["Occupancy [waves/SIMD]"] >= 1


def _own(res):
    """The library's own kernels (library templates it instantiates are not checked)."""
    return {k: v for k, v in res.items() if "smla_" in k}


@pytest.mark.parametrize("which", ["forward", "backward"])
def test_no_scratch(resources, resources_bwd, which):
    res = _own(resources if which == "forward" else resources_bwd)
    assert res
    bad = {k: (v.get("ScratchSize [bytes/lane]"), v.get("VGPRs Spill")) for k, v in res.items()
           if v.get("ScratchSize [bytes/lane]", 0) or v.get("VGPRs Spill", 0)}
    assert not bad, "kernels using scratch (bytes per lane, VGPRs spilled): %s" % bad


@pytest.fixture(scope="module")
def forward_asm(tmp_path_factory):
    _need_hipcc()
    out = tmp_path_factory.mktemp("asm") / "fwd.s"
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-S", "-o", str(out), SRC]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr[-2000:]
    return out.read_text()


def _bodies(text, pattern):
    for m in re.finditer(r"^(_Z\S*(?:%s)\S*):" % pattern, text, re.M):
        yield m.group(1), text[m.end():text.index("s_endpgm", m.end())]


def test_fwd128_agprs_left_to_the_accumulators(forward_asm):
    """In the 128-head kernel every AGPR operand must come from the hand-written
    accumulator asm: an AGPR the compiler allocates (for a spill or a copy)
    would overwrite an accumulator."""
    found = 0
    for name, body in _bodies(forward_asm, "smla_fwd128_kernel"):
        found += 1
        in_asm, bad = False, []
        for line in body.split("\n"):
            if ";;#ASMSTART" in line:
                in_asm = True
            elif ";;#ASMEND" in line:
                in_asm = False
            elif not in_asm:
                code = line.split(";")[0].strip()
                if code and re.search(r"\ba\[?\d", code):
                    bad.append(code)
        assert not bad, "%s: compiler-generated AGPR operands: %s" % (name, bad[:5])
    assert found == 2


def _vgprs(operand):
    m = re.match(r"v\[(\d+):(\d+)\]$", operand)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", operand)
    return {int(m.group(1))} if m else set()


# A VALU write of a VGPR read by an MFMA needs wait states in between. The
# compiler inserts them only for the MFMAs it generates itself; the MFMAs of
# the kernels are inline asm, and a constant the compiler materialised with a
# v_mov just before one (a zero operand) was once read stale.
MFMA_SRC_WAIT_STATES = 5


@pytest.mark.parametrize("which", ["forward", "backward"])
def test_no_valu_write_right_before_an_mfma_reads_it(forward_asm, tmp_path, which):
    if which == "forward":
        text = forward_asm
    else:
        out = tmp_path / "bwd.s"
        cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-S", "-o", str(out), BWD]
        proc = subprocess.run(cmd, capture_output=True, text=True)
        assert proc.returncode == 0, proc.stderr[-2000:]
        text = out.read_text()
    checked, bad = 0, []
    for name, body in _bodies(text, "smla_"):
        ins = [l.split(";")[0].strip() for l in body.split("\n")]
        ins = [l for l in ins if l and not l.startswith(".") and not l.endswith(":")]
        for i, line in enumerate(ins):
            if not line.startswith("v_mfma"):
                continue
            checked += 1
            ops = [o.strip() for o in line.split(None, 1)[1].split(",")]
            src = set().union(*(_vgprs(o) for o in ops[1:]))
            ws, j = 0, i - 1
            while j >= 0 and ws < MFMA_SRC_WAIT_STATES:
                prev = ins[j]
                if prev.startswith("s_nop"):
                    ws += int(prev.split()[1], 0) + 1
                elif prev.startswith("v_") and not prev.startswith(("v_mfma", "v_readlane", "v_readfirstlane", "v_cmp")):
                    parts = prev.split(None, 1)
                    dst = _vgprs(parts[1].split(",")[0].strip()) if len(parts) > 1 else set()
                    if prev.startswith(("v_permlane", "v_swap")) and len(parts) > 1:
                        dst |= _vgprs(parts[1].split(",")[1].strip())
                    if dst & src:
                        bad.append("%s: %s -> %s" % (name[-40:], prev, line))
                        break
                    ws += 1
                else:
                    ws += 1
                j -= 1
    assert checked > 0
    assert not bad, "VALU writes read by an MFMA within %d wait states: %s" % (MFMA_SRC_WAIT_STATES, bad[:5])
