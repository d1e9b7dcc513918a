"""The direct-to-LDS loads are inline asm that write M0 (their LDS address) and then
issue global_load_lds_dwordx4.  LLVM reserves M0 and warns that an asm statement
clobbering it is not guaranteed to be respected: if the compiler itself kept a
value in M0 across such a statement, the asm would overwrite it.  This test builds
two translation units of the library to gfx950 assembly (the decode kernels and the
e4m3 tile kernels, which between them use every DMA form of the library) and checks:

* outside the asm statements no instruction names M0 or uses it implicitly (moves
  relative to M0, messages, GWS, indexed-register mode, interpolation, LDS append /
  consume, or an LDS-DMA load of the compiler's own), so nothing the compiler holds
  lives in M0;
* inside each asm statement the M0 write is followed by one wait state (s_nop 0)
  before the LDS-DMA load that reads it.

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

UNITS = ["inst_decode_bf16.hip", "inst_e4m3_tt.hip"]
IMPLICIT_M0 = re.compile(r"^\s*(s_movrel|v_movrel|s_sendmsg|ds_gws|s_set_gpr_idx|v_interp|"
                         r"ds_append|ds_consume|s_ttracedata|buffer_load\S*\s.*\blds\b|"
                         r"global_load_lds)")
NAMES_M0 = re.compile(r"\bm0\b")


def assemble(build, src, out_dir):
    out = os.path.join(out_dir, src.replace(".hip", ".s"))
    cmd = [build.hipcc()] + build._flags() + ["-S", "--offload-device-only", "-w",
                                               os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


def instructions(path):
    """(inside_asm, text) for every instruction line of the assembly file."""
    inside = False
    for line in open(path):
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            inside = True
            continue
        if s.startswith(";;#ASMEND"):
            inside = False
            continue
        s = s.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        yield inside, s


@pytest.fixture(scope="module")
def asm_files(tmp_path_factory):
    import build
    if shutil.which(build.hipcc()) is None and not os.path.exists(build.hipcc()):
        pytest.skip("hipcc not available")
    d = str(tmp_path_factory.mktemp("asm"))
    with ThreadPoolExecutor(len(UNITS)) as ex:
        return list(ex.map(lambda u: assemble(build, u, d), UNITS))


def test_compiler_never_uses_m0(asm_files):
    for path in asm_files:
        bad = [s for inside, s in instructions(path)
               if not inside and (NAMES_M0.search(s) or IMPLICIT_M0.match(s))]
        assert not bad, "%s: compiler-generated M0 use: %s" % (os.path.basename(path), bad[:5])


def test_each_m0_write_waits_one_state_before_the_dma(asm_files):
    for path in asm_files:
        ins = list(instructions(path))
        writes = 0
        for i, (inside, s) in enumerate(ins):
            if inside and NAMES_M0.search(s):
                writes += 1
                assert re.match(r"s_mov_b32 m0, s\d+$", s), s
                assert ins[i + 1] == (True, "s_nop 0"), ins[i + 1]
                assert ins[i + 2][0] and ins[i + 2][1].startswith("global_load_lds_dwordx4"), \
                    ins[i + 2]
        assert writes > 100, "%s: expected the DMA asm, found %d M0 writes" % (path, writes)
