"""Plants plausible mistakes in a copy of the oracle (on the CPU) and checks that
the pins of test_oracle.py catch every one: a transposed operand, a wrong index,
a dropped term, a wrong sign, beta == 0 reading C_old, gate/up swapped, the
dequantisation scale dropped, and wrong exponent biases in the decoders."""
import ctypes
import os
import shutil
import subprocess

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = {
    "opA transposed": ("return ta ? A[p * lda + i] : A[i * lda + p];",
                       "return ta ? A[i * lda + p] : A[p * lda + i];"),
    "opB wrong index": ("return tb ? B[j * ldb + p] : B[p * ldb + j];",
                        "return tb ? B[p * ldb + j] : B[p * ldb + j];"),
    "dropped last term": ("for (int64_t p = 0; p < K; ++p) {\n            double a = opA_at",
                          "for (int64_t p = 0; p + 1 < K; ++p) {\n            double a = opA_at"),
    "beta zero reads C": ("double old = (beta == 0.0) ? 0.0 : beta * C[i * ldc + j];\n            C[i * ldc + j] = alpha * acc[j] + old;",
                          "double old = beta * C[i * ldc + j];\n            C[i * ldc + j] = alpha * acc[j] + old;"),
    "silu sign": ("return x / (1.0 + exp(-x));", "return x / (1.0 + exp(x));"),
    "gate/up swapped": ("double g = s * acc[2 * n];\n            double u = s * acc[2 * n + 1];",
                        "double g = s * acc[2 * n + 1];\n            double u = s * acc[2 * n];"),
    "scale dropped": ("double g = s * acc[2 * n];", "double g = acc[2 * n];"),
    "f16 bias": ("v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    "bf16 subnormal": ("v = ldexp((double)f, -133);", "v = ldexp((double)f, -132);"),
    "e4m3 subnormal": ("v = ldexp((double)f, -9);", "v = ldexp((double)f, -10);"),
    "interleave odd/even": ("memcpy(o + ((k * 2 * N) + 2 * n) * esize, a +",
                            "memcpy(o + ((k * 2 * N) + 2 * n + 1) * esize, a +"),
}

# every pin that takes no fixture other than golden_dir
PIN_FUNCS = [getattr(pins, n) for n in dir(pins) if n.startswith("test_")]


def _run_pins(golden_dir):
    failed = []
    for fn in PIN_FUNCS:
        import inspect
        params = inspect.signature(fn).parameters
        kwargs = {}
        if "golden_dir" in params:
            kwargs["golden_dir"] = golden_dir
        calls = [kwargs]
        if "ta" in params:   # parametrised over transposes
            calls = [dict(kwargs, ta=a, tb=b) for a, b in pins.TRANS]
        for kw in calls:
            try:
                fn(**kw)
            except (AssertionError, ValueError):
                failed.append(fn.__name__)
                break
    return failed


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path, golden_dir, monkeypatch):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found: %s" % name
    mutated = src.replace(old, new, 1)
    path = tmp_path / "oracle_mut.c"
    path.write_text(mutated)
    so = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", str(so),
                    str(path), "-lm"], check=True)
    real = oracle._load()
    mut = ctypes.CDLL(str(so))
    # copy the ctypes signatures from the real library
    for fname in ("oracle_gemm_f64", "oracle_gemm_dot_f64", "oracle_swiglu_f64",
                  "oracle_silu_f64", "oracle_decode_f16", "oracle_decode_bf16",
                  "oracle_decode_e4m3", "oracle_decode_f32", "oracle_interleave",
                  "oracle_deinterleave", "oracle_max_threads"):
        f_real = getattr(real, fname)
        f_mut = getattr(mut, fname)
        f_mut.argtypes = f_real.argtypes
        f_mut.restype = f_real.restype
    monkeypatch.setattr(oracle, "_lib", mut)
    failed = _run_pins(golden_dir)
    assert failed, "no pin caught the planted mistake '%s'" % name
