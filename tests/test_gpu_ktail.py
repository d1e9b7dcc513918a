"""K tails and ragged rows on the direct-to-LDS kernels: K not a multiple of the tile
depth, and rows of a row-contiguous operand that end inside a 16-byte chunk.  The
last, partial K tile is loaded through registers with zeros past K (a 16-byte chunk
that holds the last k is read whole and its bytes past K cleared; chunks wholly past
K are not read).  Leading-dimension padding holds NaN, so a byte past K that leaks
into a product shows as a non-finite output.  GEMM over the four transposes and every
configuration the chooser uses, K below one tile, split-K whose last split ends in the
tail, the extra-epilogue GEMM, the fused SwiGLU (interleaved and split-weight) and
e4m3 operands, against the fp64 oracle."""
import os

import numpy as np
import pytest

import oracle
from swiglu_gemm_amd import inputs
from helpers import assert_close, from_dev, split_count, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DT = {"f16": 1, "bf16": 2, "e4m3": 3}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import swiglu_gemm_amd as sg
    sg.lib()
    yield
    os.environ.pop("SG_FORCE_CONFIG", None)


def repad(storage, cols, ld, dtype):
    """The same values with leading dimension ld (NaN padding)."""
    return inputs.padded(np.ascontiguousarray(storage[:, :cols]), ld, inputs.NAN_BITS[dtype])


def problem(dtype, ta, tb, M, N, K, seed, lda=None, ldb=None):
    """A GEMM problem with padded leading dimensions (64k + 8 elements) or the given
    ones for the operands (e4m3 rows must stay 16-byte multiples)."""
    od = "bf16" if dtype == "e4m3" else dtype
    p = inputs.gemm_problem(seed, ta, tb, M, N, K, dtype, "normal",
                            ld_mode="tight" if dtype == "e4m3" else "padded", c_dtype=od)
    if lda is not None:
        cols = M if ta == "T" else K
        p["A"], p["lda"] = repad(p["A"], cols, lda, dtype), lda
    if ldb is not None:
        cols = K if tb == "T" else N
        p["B"], p["ldb"] = repad(p["B"], cols, ldb, dtype), ldb
    return p, od


def run(p, dtype, od, ta, tb, M, N, K, alpha, beta, forced=None):
    import swiglu_gemm_amd as sg
    A, B, C = to_dev(p["A"], dtype), to_dev(p["B"], dtype), to_dev(p["C"], od)
    if forced:
        os.environ["SG_FORCE_CONFIG"] = forced
    print("ktail gemm %s %s%s %dx%dx%d lda %d ldb %d forced %s" %
          (dtype, ta, tb, M, N, K, p["lda"], p["ldb"], forced), flush=True)
    try:
        sg.gemm(A, B, C, alpha=alpha, beta=beta, transA=ta, transB=tb, M=M, N=N, K=K,
                lda=p["lda"], ldb=p["ldb"], ldc=p["ldc"], dtype=DT[dtype])
        torch.cuda.synchronize()
        desc = sg.last_config()
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    return oracle.decode(from_dev(C), od), desc


def check_full(dtype, ta, tb, M, N, K, seed, forced=None, lda=None, ldb=None, beta=0.3):
    p, od = problem(dtype, ta, tb, M, N, K, seed, lda, ldb)
    alpha = 0.7 * (p["scale_a"] * p["scale_b"] if dtype == "e4m3" else 1.0)
    got, desc = run(p, dtype, od, ta, tb, M, N, K, alpha, beta, forced)
    ref = oracle.gemm(ta, tb, M, N, K, alpha, p["A"], p["lda"], p["B"], p["ldb"], beta, p["C"],
                      p["ldc"], dtype, c_dtype=od)
    assert_close(got[:, :N], ref[:, :N], dtype, K, desc)
    return desc


@pytest.mark.parametrize("tr", ["NN", "NT", "TN", "TT"])
def test_ragged_1000_takes_dma(tr):
    """bf16 1000 x 1000 x 1000 with padded leading dimensions: K = 1000 is 15 tiles of
    64 and a 40-deep tail; every row is a whole number of 16-byte chunks."""
    desc = check_full("bf16", tr[0], tr[1], 1000, 1000, 1000, 600)
    assert "dma" in desc and " reg " not in desc, desc


@pytest.mark.parametrize("tr", ["NN", "NT", "TN", "TT"])
def test_partial_chunks_4097x3001x2049(tr):
    """K = 2049: in a k-contiguous operand the tail's one valid element shares its
    chunk with 7 NaN padding elements of the row; the row-contiguous operands' rows
    (3001 or 4097 elements) end inside a chunk too.  Every output is compared."""
    M, N, K = 4097, 3001, 2049
    ta, tb = tr
    p, od = problem("bf16", ta, tb, M, N, K, 610)
    got, desc = run(p, "bf16", od, ta, tb, M, N, K, 0.7, 0.3)
    assert "dma" in desc, desc
    ref = oracle.gemm(ta, tb, M, N, K, 0.7, p["A"], p["lda"], p["B"], p["ldb"], 0.3, p["C"],
                      p["ldc"], "bf16", c_dtype=od)
    assert_close(got[:, :N], ref[:, :N], "bf16", K, desc)


CFG16 = [10, 24, 46, 48, 13, 32, 6, 44, 30, 5, 3, 11, 12, 27]


@pytest.mark.parametrize("K", [40, 1000, 2049])
@pytest.mark.parametrize("cfg", CFG16)
def test_ktail_every_16bit_config(cfg, K):
    """Each forced 16-bit direct-to-LDS configuration with a K tail (K = 40: no full
    tile at all; 2049: a partial chunk), transposes alternating over the cases; rows
    of A^T (300 elements) and of B (522) end inside a chunk."""
    tr = ["NN", "NT", "TN", "TT"][(CFG16.index(cfg) + K) % 4]
    dtype = "f16" if cfg % 2 else "bf16"
    desc = check_full(dtype, tr[0], tr[1], 300, 522, K, 620 + cfg, forced="%d,1" % cfg)
    assert "cfg=%d " % cfg in desc, desc


@pytest.mark.parametrize("K,lda", [(48, None), (1040, None), (1000, 1008), (4100, 4112)])
@pytest.mark.parametrize("cfg", [14, 15, 16, 17, 33, 45, 47])
def test_ktail_every_e4m3_config(cfg, K, lda):
    """Forced e4m3 configurations with a K tail; K = 1000 and 4100 leave 8 and 4
    valid bytes in the last chunk of each row (rows padded to 1008 / 4112 bytes)."""
    tb = "T" if cfg in (15, 33) else "N"
    ldb = lda if tb == "T" else None
    desc = check_full("e4m3", "N", tb, 200, 384, K, 640 + cfg, forced="%d,1" % cfg, lda=lda,
                      ldb=ldb)
    assert "cfg=%d " % cfg in desc, desc


def test_ktail_split_k():
    """f16 64 x 384 x 8200: split-K whose last non-empty split ends in an 8-deep tail
    (and whose last split is empty)."""
    desc = check_full("f16", "N", "N", 64, 384, 8200, 650)
    assert "dma" in desc and split_count(desc) > 1, desc


def test_ktail_extra_epilogue():
    """Bias + GELU on a K-tail GEMM (bf16 320 x 520 x 1000)."""
    import swiglu_gemm_amd as sg
    M, N, K = 320, 520, 1000
    p, od = problem("bf16", "N", "N", M, N, K, 660)
    bias_bits = inputs.to_storage(np.random.default_rng(661).standard_normal(N) * 2.0, "f32")
    A, B, C = to_dev(p["A"], "bf16"), to_dev(p["B"], "bf16"), to_dev(p["C"], "bf16")
    print("ktail gemm_ex bf16 NN %dx%dx%d" % (M, N, K), flush=True)
    sg.gemm_ex(A, B, C, alpha=0.7, beta=0.3, bias=to_dev(bias_bits, "f32"), activation="gelu",
               dtype=2, M=M, N=N, K=K, lda=p["lda"], ldb=p["ldb"], ldc=p["ldc"])
    torch.cuda.synchronize()
    desc = sg.last_config()
    assert "dma" in desc, desc
    want = oracle.gemm_epilogue("N", "N", M, N, K, 0.7, p["A"], p["lda"], p["B"], p["ldb"], 0.3,
                                p["C"], p["ldc"], "bf16", c_dtype="bf16", bias_bits=bias_bits,
                                bias_dtype="f32", act="gelu")
    assert_close(oracle.decode(from_dev(C), "bf16")[:, :N], want[:, :N], "bf16", K, desc)


@pytest.mark.parametrize("dtype,M,N,K", [("bf16", 300, 1000, 904), ("bf16", 64, 512, 40),
                                         ("e4m3", 200, 1024, 1040)])
def test_ktail_swiglu(dtype, M, N, K):
    """Fused SwiGLU with a K tail, on W_fused and on separate W1, W2."""
    import swiglu_gemm_amd as sg
    pb = inputs.swiglu_problem(670 + K, M, N, K, dtype)
    sa, sw = pb.get("scale_a", 1.0), pb.get("scale_w", 1.0)
    Wf = oracle.interleave(pb["W1"], pb["W2"])
    ref = oracle.swiglu(M, N, K, pb["A"], Wf, dtype, sa, sw)
    A = to_dev(pb["A"], dtype)
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    print("ktail swiglu %s %dx%dx%d" % (dtype, M, N, K), flush=True)
    sg.swiglu_gemm(A, to_dev(Wf, dtype), Y, sa, sw)
    torch.cuda.synchronize()
    desc = sg.last_config()
    assert "dma" in desc, desc
    assert_close(oracle.decode(from_dev(Y), "bf16"), ref, dtype, K, desc)
    Y.fill_(float("nan"))
    print("ktail swiglu_w12 %s %dx%dx%d" % (dtype, M, N, K), flush=True)
    sg.swiglu_gemm_w12(A, to_dev(pb["W1"], dtype), to_dev(pb["W2"], dtype), Y, sa, sw)
    torch.cuda.synchronize()
    desc = sg.last_config()
    assert desc.startswith("swiglu_w12") and "via W_fused" not in desc, desc
    assert_close(oracle.decode(from_dev(Y), "bf16"), ref, dtype, K, desc)


@pytest.mark.parametrize("dtype,M,N,K,lda", [("bf16", 16, 4096, 1000, None), ("f16", 1, 3000, 2049, None),
                                             ("e4m3", 8, 2048, 1040, None), ("e4m3", 32, 1024, 1000, 1008)])
def test_ktail_decode_sizes(dtype, M, N, K, lda):
    """1..32 token rows with a K tail: the decode kernels need whole 128-byte K tiles,
    so these run on the tile kernels with the tail (weights stored N x K)."""
    desc = check_full(dtype, "N", "T", M, N, K, 680 + M, lda=lda, ldb=lda)
    assert "dma" in desc and not desc.startswith("decode"), desc
