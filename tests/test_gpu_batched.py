"""GPU parity of the strided-batched GEMM (every problem of the batch against the
fp64 oracle), through the C ABI: all dtypes, transposes, a broadcast operand
(stride 0), gaps between problems that must stay untouched, both the direct-to-LDS
and the register-staged path, e4m3 operands re-laid with 16-byte rows."""
import os

import numpy as np
import pytest

import oracle
from swiglu_gemm_amd import inputs
from helpers import assert_close, bits_equal, from_dev, out_dtype, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import swiglu_gemm_amd as sg
    sg.lib()
    yield
    os.environ.pop("SG_FORCE_CONFIG", None)


def pack(arrs, stride, fill):
    """Flatten each problem's storage into one buffer, problem b at b*stride."""
    flat = [a.reshape(-1) for a in arrs]
    n = (len(arrs) - 1) * stride + max(f.size for f in flat) if stride else flat[0].size
    buf = np.full(n, fill, dtype=flat[0].dtype)
    for b, f in enumerate(flat):
        buf[b * stride: b * stride + f.size] = f
    return buf


def run_batched(dtype, ta, tb, M, N, K, batch, alpha, beta, bcast_b=False, seed=0, force=None,
                ld_mode="padded"):
    import swiglu_gemm_amd as sg
    probs = [inputs.gemm_problem(180 + seed + b, ta, tb, M, N, K, dtype, "normal",
                                 ld_mode=ld_mode, c_dtype=out_dtype(dtype))
             for b in range(batch)]
    if bcast_b:                       # every problem uses problem 0's B
        for p in probs[1:]:
            p["B"] = probs[0]["B"]
    sa = probs[0]["A"].size + 64      # gaps between problems (16-byte multiples)
    sb = 0 if bcast_b else probs[0]["B"].size + 128
    sc = probs[0]["C"].size + 64
    cst = probs[0]["C"].dtype          # storage of C: a fixed NaN bit pattern fills the gaps
    sentinel = (np.array([0x7FC01234], np.uint32) if cst.itemsize == 4 else
                np.array([0x7E55], np.uint16)).view(cst)[0]
    Ab = pack([p["A"] for p in probs], sa, probs[0]["A"].reshape(-1)[0])
    Bb = pack([p["B"] for p in probs], sb, probs[0]["B"].reshape(-1)[0])
    Cb = pack([p["C"] for p in probs], sc, sentinel)
    A, B, C = to_dev(Ab, dtype), to_dev(Bb, dtype), to_dev(Cb, out_dtype(dtype))
    code = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3}[dtype]
    if dtype == "e4m3":               # alpha carries the per-tensor scales (O(1) outputs)
        alpha *= probs[0]["scale_a"] * probs[0]["scale_b"]
    if force:
        os.environ["SG_FORCE_CONFIG"] = force
    print("batched %s %s%s M=%d N=%d K=%d batch=%d" % (dtype, ta, tb, M, N, K, batch), flush=True)
    try:
        sg.gemm_strided_batched(A, B, C, batch, sa, sb, sc, alpha=alpha, beta=beta, transA=ta,
                                transB=tb, dtype=code, M=M, N=N, K=K, lda=probs[0]["lda"],
                                ldb=probs[0]["ldb"], ldc=probs[0]["ldc"])
        torch.cuda.synchronize()
        desc = sg.last_config()
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    got = from_dev(C)
    od = out_dtype(dtype)
    for b, p in enumerate(probs):
        cb = got[b * sc: b * sc + p["C"].size].reshape(p["C"].shape)
        ref = oracle.gemm(ta, tb, M, N, K, alpha, p["A"], p["lda"], p["B"], p["ldb"], beta,
                          p["C"], p["ldc"], dtype, c_dtype=od)
        if p["ldc"] > N:
            assert bits_equal(cb[:, N:], p["C"][:, N:]), "ld padding written (problem %d)" % b
        assert_close(oracle.decode(cb, od)[:, :N], ref[:, :N], dtype, K,
                     "%s problem %d" % (desc, b))
        if b + 1 < batch:                     # the gap after each problem is untouched
            gap = got[b * sc + p["C"].size: (b + 1) * sc]
            assert bits_equal(gap, np.full(gap.size, sentinel, dtype=gap.dtype)), b
    return desc


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "e4m3"])
@pytest.mark.parametrize("tr", ["NN", "TN", "NT", "TT"])
def test_batched_ragged(dtype, tr):
    run_batched(dtype, tr[0], tr[1], 200, 136, 96, 3, 0.7, 0.3, seed=10)


def test_batched_e4m3_relaid_broadcast():
    """e4m3 leading dimensions off the 16-byte grid: each problem's A re-laid, the
    shared B (stride 0) re-laid once; the tile kernels run the batch."""
    desc = run_batched("e4m3", "N", "T", 200, 136, 96, 3, 0.7, 0.3, bcast_b=True, seed=25)
    assert "gemm8 cfg=" in desc, desc


@pytest.mark.parametrize("dtype", ["f16", "bf16", "e4m3"])
def test_batched_direct_path_and_broadcast(dtype):
    """Shapes the direct-to-LDS kernels take; B shared by every problem."""
    desc = run_batched(dtype, "N", "N", 512, 384, 512, 4, 1.0, 0.0, bcast_b=True, seed=20,
                       ld_mode="tight")
    assert "dma" in desc, desc


@pytest.mark.parametrize("force", ["10,3", "13,1", "0,1"])
def test_batched_forced_configs_no_split(force):
    """Forced configurations (a forced split count is ignored inside a batch)."""
    desc = run_batched("bf16", "N", "T", 384, 512, 1024, 2, 0.5, 0.25, seed=30, force=force)
    assert "splits=1" in desc, desc


def test_batched_quick_return_alpha_zero():
    """alpha = 0: C_b = beta * C_b for every problem, A and B unread."""
    run_batched("bf16", "N", "N", 64, 72, 32, 3, 0.0, 0.5, seed=40)
