"""Plants plausible mistakes in a copy of the oracle's epilogue functions (Python,
on the CPU) and checks that the pins of test_oracle_epilogue.py catch every one:
GELU's erf argument not scaled by 1/sqrt 2, a dropped factor 1/2, the tanh form
without its cubic term, a SiLU sign, a per-row instead of per-column bias, the
bias added after the activation, quantisation ties rounded away from zero,
overflow to NaN instead of saturation, and a lost sign bit."""
import inspect
import types

import pytest

import oracle
import test_oracle_epilogue as pins

MUTATIONS = {
    "gelu erf argument": ("erfc(-x / math.sqrt(2.0))", "erfc(-x)"),
    "gelu half dropped": ("return 0.5 * x * erfc(", "return x * erfc("),
    "gelu_tanh cubic dropped": ("(x + 0.044715 * x ** 3)", "(x)"),
    "silu sign": ("return x / (1.0 + np.exp(-x))", "return x / (1.0 + np.exp(x))"),
    "bias per row": ("[:N], bias_dtype)[None, :]", "[:M], bias_dtype)[:, None]"),
    "bias after activation": ("        V = V + decode(np.ascontiguousarray(bias_bits).ravel()[:N], bias_dtype)[None, :]\n    return activation(V, act)",
                              "        return activation(V, act) + decode(np.ascontiguousarray(bias_bits).ravel()[:N], bias_dtype)[None, :]\n    return activation(V, act)"),
    "ties away from zero": ("((d_lo == d_hi) & (lo % 2 == 0))", "((d_lo == d_hi) & False)"),
    "overflow to NaN": ("np.where(a >= table[-1], np.uint8(0x7E), code)",
                        "np.where(a > table[-1], np.uint8(0x7F), code)"),
    "sign lost": ("    code = code | np.where(np.signbit(v), np.uint8(0x80), np.uint8(0))\n", ""),
}

PIN_FUNCS = [getattr(pins, n) for n in dir(pins) if n.startswith("test_")]


def _mutated_module(old, new):
    src = inspect.getsource(oracle)
    assert src.count(old) == 1, "mutation anchor not found once: %r" % old
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = oracle.__file__
    exec(compile(src.replace(old, new), oracle.__file__, "exec"), mod.__dict__)
    return mod


def _run_pins(golden_dir):
    failed = []
    for fn in PIN_FUNCS:
        params = inspect.signature(fn).parameters
        calls = [{}]
        for mark in getattr(fn, "pytestmark", []):      # the pin's own parametrisation
            if mark.name == "parametrize":
                argname, values = mark.args[0], mark.args[1]
                calls = [dict(c, **{argname: v}) for c in calls for v in values]
        for kw in calls:
            if "golden_dir" in params:
                kw = dict(kw, golden_dir=golden_dir)
            try:
                fn(**kw)
            except (AssertionError, ValueError, IndexError):
                failed.append(fn.__name__)
                break
    return failed


def test_pins_pass_on_the_real_oracle(golden_dir):
    assert _run_pins(golden_dir) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, golden_dir, monkeypatch):
    mut = _mutated_module(*MUTATIONS[name])
    for attr in ("activation", "gemm_epilogue", "quantize_e4m3"):
        monkeypatch.setattr(oracle, attr, getattr(mut, attr))
    assert _run_pins(golden_dir), "no pin caught: %s" % name
