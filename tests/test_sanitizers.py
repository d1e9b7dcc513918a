"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer runs (CPU only).

* The fp64 oracle (oracle/oracle.c, built with gcc) under tests/sanitize/
  oracle_driver.c: every entry point, transposes, padded leading dimensions, empty
  shapes, several threads.
* The C ABI's argument checking (swiglu_gemm_amd/csrc/api.hip, host code built by
  hipcc with the sanitizers on the host side only) under tests/sanitize/
  abi_driver.c: every invalid argument of every entry point returns its status
  before any HIP call, so no GPU is needed.  The kernels' objects come from the
  library build (swiglu_gemm_amd/_build).

Operands must not overlap the output ("GEMM o Coração Matemático" §6.1); these runs
check that the host code itself reads and writes only what it owns."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
         "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
         os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"), "-lm",
         "-o", exe])
    r = run([exe], env=ENV, timeout=300)
    assert "ok" in r.stdout


def test_abi_validation_under_asan_ubsan(tmp_path):
    objdir = os.path.join(ROOT, "swiglu_gemm_amd", "_build")
    insts = sorted(os.path.join(objdir, f) for f in os.listdir(objdir)
                   if f.startswith("inst_") and f.endswith(".o")) if os.path.isdir(objdir) else []
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)) or len(insts) < 15:
        pytest.skip("hipcc or the library's kernel objects are not available")
    api_o = str(tmp_path / "api_san.o")
    drv_o = str(tmp_path / "abi_driver.o")
    exe = str(tmp_path / "abi_san")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "swiglu_gemm_amd", "csrc")]
    # sanitizers on the host side of the HIP compile only
    run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-omit-frame-pointer"] + inc +
        ["-c", os.path.join(ROOT, "swiglu_gemm_amd", "csrc", "api.hip"), "-o", api_o])
    run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer"] + inc +
        ["-c", os.path.join(SAN, "abi_driver.c"), "-o", drv_o])
    run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
         "-Xarch_host", "-fsanitize=undefined", drv_o, api_o] + insts + ["-o", exe])
    r = run([exe], env=ENV, timeout=300)
    assert "ok" in r.stdout
