"""The direct-to-LDS tile kernels keep all per-lane state in registers: a kernel that
spills moves fragments or LDS addresses to scratch memory in its main loop (the
unrolled two-stage ring hoists one LDS address per fragment and k-step, which is
why it is limited to 16-bit operands and waves of at most 8 fragments).  This test
builds two translation units of the library to gfx950 assembly, the fp16 NN and
e4m3 NN kernels, and checks every direct-to-LDS kernel's private segment size.

One known exception: the 4-wave 256x256 tiles (128x128 accumulators per wave, all
256 accumulation registers) spill in their split-K partial-sum epilogue; those
configurations run only when forced (SG_FORCE_CONFIG), never by default.

CPU only: hipcc cross-compiles for gfx950 without a GPU."""
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "swiglu_gemm_amd"))

UNITS = ["inst_f16_nn.hip", "inst_e4m3_nn.hip"]
# gemm_dma_kernel<DT, TA, TB, EPI_PARTIAL, 256, 256, BK, S, 2, 2>
KNOWN = re.compile(r"gemm_dma_kernelILi\d+ELb[01]ELb[01]ELi2ELi256ELi256ELi(32|64)ELi[24]ELi2ELi2E")


def assemble(build, src, out_dir):
    out = os.path.join(out_dir, src.replace(".hip", ".s"))
    cmd = [build.hipcc()] + build._flags() + ["-S", "--offload-device-only", "-w",
                                               os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


@pytest.fixture(scope="module")
def asm_files(tmp_path_factory):
    import build
    if shutil.which(build.hipcc()) is None and not os.path.exists(build.hipcc()):
        pytest.skip("hipcc not available")
    d = str(tmp_path_factory.mktemp("asm_scratch"))
    with ThreadPoolExecutor(len(UNITS)) as ex:
        return list(ex.map(lambda u: assemble(build, u, d), UNITS))


def kernels(path):
    """(mangled name, private segment bytes) of every kernel in the assembly file."""
    txt = open(path).read()
    for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", txt, re.S):
        size = re.search(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", m.group(2))
        yield m.group(1), int(size.group(1))


def test_direct_to_lds_kernels_do_not_spill(asm_files):
    seen = 0
    for path in asm_files:
        for name, size in kernels(path):
            if "gemm_dma_kernel" not in name:
                continue
            seen += 1
            if KNOWN.search(name):
                continue
            assert size == 0, "%s: %s uses %d bytes of scratch" % (os.path.basename(path), name,
                                                                   size)
    assert seen > 50, "expected the tile kernels, found %d" % seen
