"""Every gfx950 kernel of the library keeps its working set in registers and
LDS: no scratch (private memory), no vector-register spills, and LDS within the
160 KiB of a CU (scalar-register spills go to vector-register lanes, not to
memory, and are allowed). Scratch in these kernels means register arrays indexed at run time or
spills, which cost an order of magnitude in speed without changing results, so
no numerical test would notice. Compiles each HIP source for the device only
(same flags as the library build) and reads the compiler's resource remarks.

The same assembly is checked for registers touched while a load into them is
still in flight (isa_hazards): the kernels issue loads from inline asm, whose
results the compiler takes as ready at once."""
import concurrent.futures as cf
import os
import re
import subprocess
import tempfile

import pytest

import isa_hazards
from exact_attention_106_amd import build as B

LDS_LIMIT = 160 * 1024


def remarks(src):
    # compiled to an object (so the assembler checks every instruction, inline
    # asm included) with the intermediate assembly kept for the scan
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [B.hipcc()] + B.common_flags() + B.EXTRA.get(src, []) + [
            "--offload-device-only", "-Rpass-analysis=kernel-resource-usage", "-c", "--save-temps",
            os.path.join(B.CSRC, src), "-o", os.path.join(tmp, "k.o")]
        r = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp)
        s_files = [f for f in os.listdir(tmp) if f.endswith("gfx950.s")]
        asm = open(os.path.join(tmp, s_files[0])).read() if r.returncode == 0 and s_files else ""
    assert r.returncode == 0, r.stderr[-2000:]
    assert asm, "no gfx950 assembly for %s" % src
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        # "<file>: remark: <text>" or, with --save-temps, "remark: <file>: <text>"
        m = re.search(r"remark:.*?Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark:.*?:\s+([A-Za-z ]+?)(?: \[bytes/(?:lane|block)\])?: (\d+) \[-Rpass", line)
        if m and cur:
            kernels[cur][m.group(1).strip()] = int(m.group(2))
    return kernels, asm


@pytest.fixture(scope="module")
def all_remarks():
    with cf.ThreadPoolExecutor(max_workers=min(8, len(B.SOURCES))) as ex:
        return dict(zip(B.SOURCES, ex.map(remarks, B.SOURCES)))


@pytest.mark.parametrize("src", [s for s in B.SOURCES if s != "api.hip"])
def test_no_scratch_no_vgpr_spills(all_remarks, src):
    kernels = all_remarks[src][0]
    assert kernels, "no kernels found in %s" % src
    for name, k in kernels.items():
        assert k.get("ScratchSize", 0) == 0, (src, name, k)
        assert k.get("VGPRs Spill", 0) == 0, (src, name, k)
        assert k.get("LDS Size", 0) <= LDS_LIMIT, (src, name, k)


@pytest.mark.parametrize("src", [s for s in B.SOURCES if s != "api.hip"])
def test_no_register_touched_while_its_load_is_in_flight(all_remarks, src):
    found = isa_hazards.hazards(all_remarks[src][1])
    assert not found, "%s: %d accesses, first: %s" % (src, len(found), found[:3])


def test_quantiser_fits_three_workgroups_per_cu(all_remarks):
    """The quantiser's grid is three persistent workgroups of four waves per CU:
    every instantiation (plain, rotated, and the mixed Q/K/V launch) must fit
    three waves per SIMD, 512 / 3 -> at most 168 registers per lane, and three
    workgroups' LDS."""
    kernels = all_remarks["fp8_quant.hip"][0]
    assert len(kernels) == 3, sorted(kernels)
    for name, k in kernels.items():
        vg = (k.get("VGPRs", 0) + 7) // 8 * 8
        regs = vg + k.get("AGPRs", 0) if k.get("AGPRs", 0) else vg
        assert regs <= 168, (name, k)
        assert 3 * k.get("LDS Size", 0) <= 160 * 1024, (name, k)
