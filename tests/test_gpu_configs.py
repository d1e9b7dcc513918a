"""Every kernel configuration (register-staged and DMA ring), every transpose pair,
each epilogue (alpha/beta, SwiGLU pair, split-K partials + reduction), forced
through SG_FORCE_CONFIG and checked against the fp64 oracle.  Shapes are
multiples of every tile so the DMA configurations are eligible."""
import os

import numpy as np
import pytest

import oracle
from swiglu_gemm_amd import inputs
from helpers import assert_close, bits_equal, from_dev, split_count, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CFGS16 = list(range(14)) + [24, 27, 28, 30, 31, 32, 43, 44, 46, 48]   # every 16-bit id
WIDE = [24]                        # 320-column tiles (640-byte LDS rows)
TRANS = ["NN", "NT", "TN", "TT"]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import swiglu_gemm_amd as sg
    sg.lib()
    yield
    os.environ.pop("SG_FORCE_CONFIG", None)


def forced(cfg, splits=0):
    os.environ["SG_FORCE_CONFIG"] = "%d,%d" % (cfg, splits)


def rne16(x, dtype):
    """Round-to-nearest-even 16-bit codes of float64 values that are exact in fp32
    (numpy's half conversion; torch's CPU float -> bfloat16 cast)."""
    if dtype == "f16":
        return np.asarray(x).astype(np.float16).view(np.uint16)
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def rounding_case(cfg, dtype, M, N, K):
    """A holds one nonzero per row, so every output is a single product that the fp32
    accumulator holds exactly: the stored code must be its round-to-nearest-even
    16-bit code, bit for bit -- ties (checked to occur), fp16 subnormals, signs.
    beta = 0 with NaN in C: the old C is not read."""
    import swiglu_gemm_amd as sg
    gen = np.random.default_rng(900 + cfg)
    a = gen.standard_normal(M) * np.where(gen.random(M) < 0.25, 1e-3, 1.0)
    A = np.zeros((M, K))
    A[np.arange(M), np.arange(M) % K] = a
    B = gen.standard_normal((K, N))
    A_bits, B_bits = rne16(A, dtype), rne16(B, dtype)
    C_bits = np.full((M, N), 0x7E00 if dtype == "f16" else 0x7FC0, dtype=np.uint16)
    ref = oracle.gemm("N", "N", M, N, K, 1.0, A_bits, K, B_bits, N, 0.0, C_bits, N, dtype)
    r32 = ref.astype(np.float32)                       # exact: one 16-bit product
    up = rne16(np.nextafter(r32, np.float32(np.inf)), dtype)
    down = rne16(np.nextafter(r32, np.float32(-np.inf)), dtype)
    assert np.count_nonzero((up != down) & (ref != 0)) > 0, "no rounding ties in the case"
    C = to_dev(C_bits, dtype)
    forced(cfg, 1)
    print("rounding cfg %d %s M=%d N=%d" % (cfg, dtype, M, N), flush=True)
    try:
        sg.gemm(to_dev(A_bits, dtype), to_dev(B_bits, dtype), C, alpha=1.0, beta=0.0,
                dtype={"f16": 1, "bf16": 2}[dtype])
        torch.cuda.synchronize()
        desc = sg.last_config()
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    assert "cfg=%d " % cfg in desc, desc
    got = from_dev(C)
    want = rne16(ref, dtype)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "%s: %d codes differ, first at %s: got %#06x want %#06x (%r)" % (
        desc, len(bad), bad[0], got[tuple(bad[0])], want[tuple(bad[0])], ref[tuple(bad[0])])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("cfg", CFGS16)
def test_output_rounding_bit_exact(cfg, dtype):
    """A few tiles: the register epilogue."""
    rounding_case(cfg, dtype, 512, 256, 64)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("cfg", [10, 24, 46, 48, 13, 30, 32, 43, 44, 5, 8])
def test_output_rounding_bit_exact_many_tiles(cfg, dtype):
    """More work-groups than one round of the CUs: the row-staged epilogue of the
    direct-to-LDS kernels (full tiles) next to the register epilogue (edge tiles:
    N = 4608 is not a multiple of every tile width)."""
    rounding_case(cfg, dtype, 8192, 4608, 64)


@pytest.mark.parametrize("cfg", [14, 15, 17, 33, 45, 47])
def test_e4m3_output_rounding_bit_exact_many_tiles(cfg):
    """e4m3 operands, bf16 output: one product per output (A has one nonzero per row)
    times alpha = 1.0625, exact in fp32 (at most 8 + 5 significant bits) and rounded once
    to bf16 -- ties occur, where a bare e4m3 product (<= 8 bits) would always be exact --
    on more work-groups than one round (row-staged epilogue on full tiles, register
    epilogue on edge tiles)."""
    import swiglu_gemm_amd as sg
    M, N, K = 8192, 4608, 128
    gen = np.random.default_rng(950 + cfg)
    a = torch.from_numpy(gen.standard_normal(M).astype(np.float32) * 8).to(torch.float8_e4m3fn)
    A = torch.zeros((M, K), dtype=torch.float8_e4m3fn)
    A[np.arange(M), np.arange(M) % K] = a
    B = torch.from_numpy(gen.standard_normal((K, N)).astype(np.float32) * 8).to(
        torch.float8_e4m3fn)
    A_bits, B_bits = A.view(torch.uint8).numpy(), B.view(torch.uint8).numpy()
    C_bits = np.full((M, N), 0x7FC0, dtype=np.uint16)
    alpha = 1.0625
    ref = oracle.gemm("N", "N", M, N, K, alpha, A_bits, K, B_bits, N, 0.0, C_bits, N, "e4m3",
                      c_dtype="bf16")
    r32 = ref.astype(np.float32)                       # exact: alpha times one product
    up = rne16(np.nextafter(r32, np.float32(np.inf)), "bf16")
    down = rne16(np.nextafter(r32, np.float32(-np.inf)), "bf16")
    assert np.count_nonzero((up != down) & (ref != 0)) > 0, "no rounding ties in the case"
    C = to_dev(C_bits, "bf16")
    forced(cfg, 1)
    print("e4m3 rounding cfg %d" % cfg, flush=True)
    try:
        sg.gemm(to_dev(A_bits, "e4m3"), to_dev(B_bits, "e4m3"), C, alpha=alpha, beta=0.0,
                dtype=3)
        torch.cuda.synchronize()
        desc = sg.last_config()
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    assert "cfg=%d " % cfg in desc, desc
    got = from_dev(C)
    want = rne16(ref, "bf16")
    bad = np.argwhere(got != want)
    assert bad.size == 0, "%s: %d codes differ, first at %s: got %#06x want %#06x (%r)" % (
        desc, len(bad), bad[0], got[tuple(bad[0])], want[tuple(bad[0])], ref[tuple(bad[0])])


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("tr", TRANS)
@pytest.mark.parametrize("cfg", CFGS16)
def test_gemm_every_config(cfg, tr, splits):
    import swiglu_gemm_amd as sg
    M, N, K = 512, 256, 768
    ta, tb = tr
    dtype = "bf16" if cfg % 2 else "f16"
    p = inputs.gemm_problem(60 + cfg, ta, tb, M, N, K, dtype, "normal", ld_mode="tight")
    A, B, C = to_dev(p["A"], dtype), to_dev(p["B"], dtype), to_dev(p["C"], dtype)
    forced(cfg, splits)
    print("cfg %d %s splits %d" % (cfg, tr, splits), flush=True)
    try:
        sg.gemm(A, B, C, alpha=0.7, beta=0.3, transA=ta, transB=tb, M=M, N=N, K=K,
                lda=p["lda"], ldb=p["ldb"], ldc=p["ldc"], dtype={"f16": 1, "bf16": 2}[dtype])
        torch.cuda.synchronize()
        desc = sg.last_config()
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    assert "cfg=%d " % cfg in desc, desc
    assert split_count(desc) == splits, desc
    ref = oracle.gemm(ta, tb, M, N, K, 0.7, p["A"], p["lda"], p["B"], p["ldb"], 0.3, p["C"],
                      p["ldc"], dtype)
    assert_close(oracle.decode(from_dev(C), dtype), ref, dtype, K, desc)


@pytest.mark.parametrize("splits", [1, 2])
@pytest.mark.parametrize("cfg", CFGS16)
def test_swiglu_every_config(cfg, splits):
    import swiglu_gemm_amd as sg
    M, N, K = 256, 512, 512          # W_fused is 512 x 1024
    pb = inputs.swiglu_problem(70 + cfg, M, N, K, "bf16", w_std=0.05)
    Wf = oracle.interleave(pb["W1"], pb["W2"])
    A, W = to_dev(pb["A"], "bf16"), to_dev(Wf, "bf16")
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    forced(cfg, splits)
    print("swiglu cfg %d splits %d" % (cfg, splits), flush=True)
    try:
        sg.swiglu_gemm(A, W, Y)
        torch.cuda.synchronize()
        desc = sg.last_config()
        y1 = from_dev(Y)
        sg.swiglu_gemm(A, W, Y)
        torch.cuda.synchronize()
        y2 = from_dev(Y)
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    assert "cfg=%d " % cfg in desc, desc
    assert split_count(desc) == splits, desc
    assert bits_equal(y1, y2), "not run-to-run identical"
    ref = oracle.swiglu(M, N, K, pb["A"], Wf, "bf16")
    assert_close(oracle.decode(y1, "bf16"), ref, "bf16", K, desc)


@pytest.mark.parametrize("cfg", CFGS16)
def test_identity_bit_exact_every_config(cfg):
    """A @ I == A bit-exactly through every configuration (layout check)."""
    import swiglu_gemm_amd as sg
    M, K = 256, 256
    gen = np.random.default_rng(cfg)
    Ab = inputs.to_storage(gen.standard_normal((M, K)), "bf16")
    Ib = inputs.to_storage(np.eye(K), "bf16")
    A, I = to_dev(Ab, "bf16"), to_dev(Ib, "bf16")
    C = torch.empty((M, K), dtype=torch.bfloat16, device="cuda:0")
    forced(cfg, 1)
    try:
        sg.gemm(A, I, C)
        torch.cuda.synchronize()
        desc = sg.last_config()
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    assert "cfg=%d " % cfg in desc, desc
    assert bits_equal(from_dev(C), Ab), desc


@pytest.mark.parametrize("splits", [1, 2])
@pytest.mark.parametrize("tr", TRANS)
@pytest.mark.parametrize("cfg", WIDE)
def test_wide_tiles_ragged(cfg, tr, splits):
    """320-column tiles on a shape with two full tiles and a ragged third in N,
    a ragged M tile, and an odd number of 64-deep K tiles per split."""
    import swiglu_gemm_amd as sg
    M, N, K = 520, 1000, 640
    ta, tb = tr
    p = inputs.gemm_problem(110 + cfg, ta, tb, M, N, K, "bf16", "normal", ld_mode="padded")
    A, B, C = to_dev(p["A"], "bf16"), to_dev(p["B"], "bf16"), to_dev(p["C"], "bf16")
    forced(cfg, splits)
    print("wide cfg %d %s splits %d" % (cfg, tr, splits), flush=True)
    try:
        sg.gemm(A, B, C, alpha=0.7, beta=0.3, transA=ta, transB=tb, M=M, N=N, K=K,
                lda=p["lda"], ldb=p["ldb"], ldc=p["ldc"], dtype=2)
        torch.cuda.synchronize()
        desc = sg.last_config()
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    assert "cfg=%d " % cfg in desc, desc
    ref = oracle.gemm(ta, tb, M, N, K, 0.7, p["A"], p["lda"], p["B"], p["ldb"], 0.3, p["C"],
                      p["ldc"], "bf16")
    cbits = from_dev(C)
    assert bits_equal(cbits[:, N:], p["C"][:, N:]), "ld padding of C was written"
    assert_close(oracle.decode(cbits, "bf16")[:, :N], ref[:, :N], "bf16", K, desc)


@pytest.mark.parametrize("cfg", WIDE)
def test_wide_tiles_swiglu_and_identity(cfg):
    """SwiGLU pairing across 320-column tiles (fused N = 9728 / 320 is not whole)
    and A @ I bit-exact with a ragged last column tile."""
    import swiglu_gemm_amd as sg
    M, N, K = 256, 4864, 128
    pb = inputs.swiglu_problem(120 + cfg, M, N, K, "bf16")
    Wf = oracle.interleave(pb["W1"], pb["W2"])
    A, W = to_dev(pb["A"], "bf16"), to_dev(Wf, "bf16")
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    forced(cfg, 1)
    try:
        sg.swiglu_gemm(A, W, Y)
        torch.cuda.synchronize()
        desc = sg.last_config()
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    assert "cfg=%d " % cfg in desc, desc
    ref = oracle.swiglu(M, N, K, pb["A"], Wf, "bf16")
    assert_close(oracle.decode(from_dev(Y), "bf16"), ref, "bf16", K, desc)

    Mi, Ki = 256, 704
    gen = np.random.default_rng(cfg)
    Ab = inputs.to_storage(gen.standard_normal((Mi, Ki)), "bf16")
    Ib = inputs.to_storage(np.eye(Ki), "bf16")
    C = torch.empty((Mi, Ki), dtype=torch.bfloat16, device="cuda:0")
    forced(cfg, 1)
    try:
        sg.gemm(to_dev(Ab, "bf16"), to_dev(Ib, "bf16"), C)
        torch.cuda.synchronize()
        desc = sg.last_config()
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    assert "cfg=%d " % cfg in desc, desc
    assert bits_equal(from_dev(C), Ab), desc


@pytest.mark.parametrize("cfg", [34, 35, 36, 37, 38, 39, 40, 41])
def test_pipeline_study_configs_fp16_nn(cfg):
    """The pipeline-depth study configurations (fp16 NN GEMM only) against the
    oracle, on a ragged shape that spans several tiles; other dtypes reject them."""
    import swiglu_gemm_amd as sg
    M, N, K = 520, 1000, 640
    p = inputs.gemm_problem(170 + cfg, "N", "N", M, N, K, "f16", "normal", ld_mode="padded")
    A, B, C = to_dev(p["A"], "f16"), to_dev(p["B"], "f16"), to_dev(p["C"], "f16")
    forced(cfg, 1)
    print("study cfg %d" % cfg, flush=True)
    try:
        sg.gemm(A, B, C, alpha=0.7, beta=0.3, M=M, N=N, K=K, lda=p["lda"], ldb=p["ldb"],
                ldc=p["ldc"], dtype=1)
        torch.cuda.synchronize()
        desc = sg.last_config()
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    assert "cfg=%d " % cfg in desc, desc
    ref = oracle.gemm("N", "N", M, N, K, 0.7, p["A"], p["lda"], p["B"], p["ldb"], 0.3, p["C"],
                      p["ldc"], "f16")
    cbits = from_dev(C)
    assert bits_equal(cbits[:, N:], p["C"][:, N:]), "ld padding of C was written"
    assert_close(oracle.decode(cbits, "f16")[:, :N], ref[:, :N], "f16", K, desc)
