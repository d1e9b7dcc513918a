"""Builds libswiglu_gemm.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m swiglu_gemm_amd.build          # or swiglu_gemm_amd.build.build()
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libswiglu_gemm.so")
# diagnostic library (not the GEMM path): a pure MFMA loop for the power-limited
# MFMA ceiling that bench.py --mfma-ceiling reports
DIAG_SRC = os.path.join(HERE, "diag", "mfma_loop.hip")
DIAG_LIB = os.path.join(HERE, "libswiglu_gemm_diag.so")
SOURCES = ["api.hip"] + ["inst_%s_%s.hip" % (d, t) for d in ("f16", "bf16", "e4m3")
                        for t in ("nn", "nt", "tn", "tt")] + \
    ["inst_decode_%s.hip" % d for d in ("f16", "bf16", "e4m3")]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def source_hash() -> str:
    """16 hex digits of the SHA-256 over the library's sources (kernel and ABI files,
    name and contents, in name order).  Built into the library (sg_build_info) so
    that the binding can tell a library built from other sources."""
    h = hashlib.sha256()
    for d, exts in ((CSRC, (".hip", ".hpp")), (INCLUDE, (".h",))):
        for f in sorted(os.listdir(d)):
            if f.endswith(exts):
                with open(os.path.join(d, f), "rb") as fh:
                    h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _flags() -> list:
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            # packed-fp32 VALU ops are kept out of the generated code on purpose
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    """Compile each translation unit in parallel, then link the shared library."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    ident = ["-DSG_SOURCE_HASH=\"%s\"" % source_hash()]

    def one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [hipcc()] + _flags() + (ident if src == "api.hip" else []) + \
            ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed on %s" % src)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 8)) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed linking libswiglu_gemm.so")
    os.replace(tmp, LIB)
    tmp = DIAG_LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([hipcc()] + _flags() + ["-shared", DIAG_SRC, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on diag/mfma_loop.hip")
    os.replace(tmp, DIAG_LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    srcs = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + \
        [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)]
    return any(os.path.getmtime(s) > t for s in srcs)


if __name__ == "__main__":
    print(build(verbose=True))
