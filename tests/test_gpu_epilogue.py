"""GPU parity of the fused GEMM epilogue (sg_gemm_ex: bias, activation, e4m3
output quantisation) against the fp64 oracle, through the C ABI, on every kernel
path that stores C: the direct-to-LDS tile kernels, the register-staged kernel
(K tail), split-K with its reduction, the decode path, e4m3 operands re-laid
with 16-byte rows, the fp32 kernel and the K == 0 quick return.  e4m3 outputs: bit-exact codes where
the value before quantisation is exact (ties, subnormals, saturation), otherwise
the code must be the rounding of a value within a tight bound of the oracle's.
Also the two plain-GEMM uses of the pages' epilogue argument: attention scores
with alpha = 1/sqrt(d_h) over a strided batch of heads, and the fused Q, K, V
projection as one GEMM on the concatenated weight."""
import math
import os

import numpy as np
import pytest

import oracle
from swiglu_gemm_amd import inputs
from helpers import assert_close, bits_equal, from_dev, out_dtype, split_count, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DT_CODE = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3}
ACTS = ["none", "relu", "gelu", "gelu_tanh", "silu"]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import swiglu_gemm_amd as sg
    sg.lib()
    yield
    os.environ.pop("SG_FORCE_CONFIG", None)


def bias_vec(N, bdt, seed):
    gen = np.random.default_rng(seed)
    vals = gen.standard_normal(N) * 2.0
    return inputs.to_storage(vals, bdt)


def run_ex(p, ta, tb, M, N, K, alpha, beta, dtype, bias_bits, bdt, act, out_scale=None):
    import swiglu_gemm_amd as sg
    A, B = to_dev(p["A"], dtype), to_dev(p["B"], dtype)
    if out_scale is None:
        C = to_dev(p["C"], out_dtype(dtype))
    else:
        C = torch.full((M, p["ldc"]), 0x55, dtype=torch.uint8, device="cuda:0")
    bias = to_dev(bias_bits, bdt) if bias_bits is not None else None
    print("gemm_ex %s %s%s M=%d N=%d K=%d act=%s bias=%s out8=%s" % (
        dtype, ta, tb, M, N, K, act, bdt if bias is not None else None, out_scale), flush=True)
    sg.gemm_ex(A, B, C, alpha=alpha, beta=beta, transA=ta, transB=tb, bias=bias, activation=act,
               out_scale=out_scale, dtype=DT_CODE[dtype], M=M, N=N, K=K, lda=p["lda"],
               ldb=p["ldb"], ldc=p["ldc"])
    torch.cuda.synchronize()
    return from_dev(C), sg.last_config()


def reference(p, ta, tb, M, N, K, alpha, beta, dtype, bias_bits, bdt, act):
    return oracle.gemm_epilogue(ta, tb, M, N, K, alpha, p["A"], p["lda"], p["B"], p["ldb"], beta,
                                p["C"], p["ldc"], dtype, c_dtype=out_dtype(dtype),
                                bias_bits=bias_bits, bias_dtype=bdt, act=act)


def check_codes(codes, y, mag, K, scale, what):
    """codes (M x N uint8) must be the e4m3 rounding of a value within delta of the
    oracle value y (quantisation is monotone): delta = 1e-3*|y| (the activation's
    fp32 evaluation) + 5e-7*sqrt(K)*mag, mag = |alpha|*sum|a*b| + |bias| (fp32
    accumulation: its error scales with the terms summed, not with the result)."""
    delta = 1e-3 * np.abs(y) + 5e-7 * np.sqrt(K) * mag + 1e-6
    lo = oracle.decode(oracle.quantize_e4m3(y - delta, scale), "e4m3")
    hi = oracle.decode(oracle.quantize_e4m3(y + delta, scale), "e4m3")
    got = oracle.decode(codes, "e4m3")
    bad = ~((got >= lo) & (got <= hi))
    if np.any(bad):
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d/%d e4m3 codes off; first at %s: got %r, allowed [%r, %r]"
                             % (what, int(bad.sum()), bad.size, tuple(i), got[tuple(i)],
                                lo[tuple(i)], hi[tuple(i)]))


def case(dtype, ta, tb, M, N, K, seed, ld_mode="padded"):
    p = inputs.gemm_problem(seed, ta, tb, M, N, K, dtype, "normal", ld_mode=ld_mode,
                            c_dtype=out_dtype(dtype))
    scale = p["scale_a"] * p["scale_b"] if dtype == "e4m3" else 1.0
    return p, scale


def check_ex(dtype, ta, tb, M, N, K, seed, act, bdt, beta=0.3, out8=False, ld_mode="padded",
             expect=None):
    p, scale = case(dtype, ta, tb, M, N, K, seed, "tight" if dtype == "e4m3" or out8 else ld_mode)
    alpha = 0.7 * scale
    beta = 0.0 if out8 else beta
    bias_bits = bias_vec(N, bdt, seed + 1) if bdt else None
    out_scale = 0.125 if out8 else None
    got, desc = run_ex(p, ta, tb, M, N, K, alpha, beta, dtype, bias_bits, bdt, act, out_scale)
    if expect:
        assert expect in desc, desc
    y = reference(p, ta, tb, M, N, K, alpha, beta, dtype, bias_bits, bdt, act)
    what = "%s %s%s act=%s %s" % (dtype, ta, tb, act, desc)
    if out8:
        pa = dict(p, A=np.abs(oracle.decode(p["A"], dtype)), B=np.abs(oracle.decode(p["B"], dtype)))
        C0 = np.zeros((M, p["ldc"]))
        oracle.gemm_f64(ta, tb, M, N, K, abs(alpha), pa["A"].ravel(), p["lda"], pa["B"].ravel(),
                        p["ldb"], 0.0, C0.ravel(), p["ldc"])
        mag = C0[:, :N] + (np.abs(oracle.decode(bias_bits, bdt))[None, :] if bdt else 0.0)
        check_codes(got[:, :N], y, mag, K, out_scale, what)
    else:
        od = out_dtype(dtype)
        assert_close(oracle.decode(got, od)[:, :N], y, od, K, what)
        assert bits_equal(got[:, N:], p["C"][:, N:]), "ld padding of C was written"
    return desc


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32", "e4m3"])
def test_epilogue_tile_kernels(dtype, act):
    """Multi-tile ragged shapes on the large-tile kernels (direct-to-LDS for the
    aligned 16-bit / e4m3 rows), bias in fp32 and in bf16; C rows of 522 elements
    (ldc not a multiple of 8) take the quad-store form of the epilogue; fp32 also on
    its 128 x 128 tiles."""
    check_ex(dtype, "N", "N", 300, 520, 256, 400, act, "f32")
    check_ex(dtype, "N", "T", 257, 384, 512, 401, act, "bf16")
    check_ex(dtype, "N", "T", 300, 522, 256, 402, act, "f32", ld_mode="tight")
    if dtype == "f32":
        check_ex(dtype, "T", "N", 3600, 3500, 40, 403, act, "bf16", expect="128x128")


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32", "e4m3"])
def test_epilogue_e4m3_output(dtype, act):
    check_ex(dtype, "N", "N", 300, 512, 256, 410, act, "bf16", out8=True)


EX16 = [2, 6, 10, 13, 24, 30, 32, 44, 46, 48]     # configurations with the extra steps
EX8 = [14, 15, 16, 17, 33, 45, 47]


@pytest.mark.parametrize("tr", ["NN", "NT", "TN", "TT"])
@pytest.mark.parametrize("cfg", EX16)
def test_epilogue_every_config(cfg, tr):
    """Each 16-bit configuration compiled with the extra epilogue steps, forced, in
    every transpose: bias (fp32) + GELU with beta on a ragged multi-tile shape whose
    sizes are multiples of 8 (so every direct-to-LDS ring is eligible), against the
    oracle."""
    os.environ["SG_FORCE_CONFIG"] = "%d,1" % cfg
    try:
        check_ex("bf16", tr[0], tr[1], 296, 520, 256, 470 + cfg, "gelu", "f32", ld_mode="tight",
                 expect="cfg=%d " % cfg)
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)


@pytest.mark.parametrize("tb", ["N", "T"])
@pytest.mark.parametrize("cfg", EX8)
def test_epilogue_every_config_e4m3(cfg, tb):
    """The same for each e4m3 configuration with the extra steps, B stored either way
    (A untransposed: the 32-row tiles take a transposed A through the re-laid path):
    bias (bf16) + GELU with beta, bf16 output, on a ragged shape of multiples of 16."""
    os.environ["SG_FORCE_CONFIG"] = "%d,1" % cfg
    try:
        check_ex("e4m3", "N", tb, 304, 528, 256, 490 + cfg, "gelu", "bf16",
                 expect="cfg=%d " % cfg)
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)


@pytest.mark.parametrize("act", ["gelu", "silu"])
def test_epilogue_other_paths(act):
    """Register-staged kernel (a leading dimension that is not a 16-byte multiple),
    split-K + reduction, decode path, e4m3 operands with odd rows (re-laid with
    16-byte rows for the tile kernels), each with bias and activation, 16-bit and
    e4m3 outputs."""
    check_ex("bf16", "T", "N", 201, 300, 250, 420, act, "f32", expect=" reg ", ld_mode="tight")
    d = check_ex("f16", "N", "N", 64, 384, 8192, 421, act, "f16")
    assert split_count(d) > 1, d
    check_ex("bf16", "N", "T", 4, 1024, 2048, 422, act, "bf16", expect="decode")
    check_ex("bf16", "N", "T", 4, 1024, 2048, 423, act, "bf16", out8=True, expect="decode")
    check_ex("e4m3", "N", "N", 37, 80, 70, 424, act, "f32", expect="gemm8 cfg=")
    check_ex("e4m3", "N", "N", 37, 80, 70, 425, act, "f32", out8=True, expect="gemm8 cfg=")
    d = check_ex("f16", "N", "N", 64, 384, 8192, 426, act, "bf16", out8=True)
    assert split_count(d) > 1, d


def test_epilogue_quick_return_k0():
    """K == 0: C = out(act(beta * C_old + bias)) without reading A or B."""
    import swiglu_gemm_amd as sg
    M, N = 33, 70
    p, _ = case("bf16", "N", "N", M, N, 1, 430)
    bias_bits = bias_vec(N, "f32", 431)
    C = to_dev(p["C"], "bf16")
    bias = to_dev(bias_bits, "f32")
    dummy = torch.zeros(8, dtype=torch.bfloat16, device="cuda:0")
    sg.gemm_ex(dummy, dummy, C, alpha=1.0, beta=0.5, bias=bias, activation="relu", M=M, N=N, K=0,
               lda=1, ldb=N, ldc=p["ldc"], dtype=2)
    torch.cuda.synchronize()
    assert sg.last_config() == "epilogue_only"
    Cold = oracle.decode(p["C"], "bf16")[:, :N]
    want = oracle.activation(0.5 * Cold + oracle.decode(bias_bits, "f32")[None, :], "relu")
    assert_close(oracle.decode(from_dev(C), "bf16")[:, :N], want, "bf16", 1, "K=0")


@pytest.mark.parametrize("K", [1, 64])
def test_e4m3_output_codes_bit_exact(K):
    """v = A[m, 0] * B[0, j] exactly (other terms zero, powers of two): every code
    must equal the oracle's quantisation -- midpoints (ties to even), subnormals,
    saturation, negative values -- on the register-staged (K = 1) and the
    direct-to-LDS (K = 64) kernels."""
    import swiglu_gemm_amd as sg
    table = oracle.decode(np.arange(0x7F, dtype=np.uint8), "e4m3")
    mids = (table[:-1] + table[1:]) / 2
    vals = np.concatenate([table, mids, -table, -mids, [0.0, -0.0, 448.0, 460.0, 464.0, 500.0,
                                                        8192.0, -4096.0, 2.0 ** -10, 3 * 2.0 ** -11]])
    M = -(-len(vals) // 64) * 64
    a = np.zeros((M, K))
    a[: len(vals), 0] = vals / 4.0       # B[0, j] = 2^(j-2) * 2, out_scale 0.5: v/s = vals*2^(j-2)
    N = 8
    b = np.zeros((K, N))
    b[0, :] = 2.0 ** (np.arange(N) - 2) * 2.0
    A_bits = inputs.to_storage(a, "bf16")
    B_bits = inputs.to_storage(b, "bf16")
    assert np.array_equal(oracle.decode(A_bits, "bf16"), a)     # exactly representable
    assert np.array_equal(oracle.decode(B_bits, "bf16"), b)
    C = torch.full((M, N), 0x55, dtype=torch.uint8, device="cuda:0")
    sg.gemm_ex(to_dev(A_bits, "bf16"), to_dev(B_bits, "bf16"), C, out_scale=0.5, dtype=2)
    torch.cuda.synchronize()
    desc = sg.last_config()
    v = 0.0 + a[:, :1] * b[:1, :]     # a sum: an exact zero is +0, as from the accumulator
    want = oracle.quantize_e4m3(v, 0.5)
    got = from_dev(C)
    assert np.array_equal(got, want), (desc, np.argwhere(got != want)[:5])


def test_attention_scores_alpha_inv_sqrt_dh_batched_heads():
    """S_h = Q_h K_h^T / sqrt(d_h) for 8 heads in one strided-batched NT call
    ("GEMM o Coração Matemático" §1: alpha = 1/sqrt(d_h); §13.2: per-head products)."""
    import swiglu_gemm_amd as sg
    H, L, dh = 8, 200, 64
    gen = np.random.default_rng(440)
    q = inputs.to_storage(gen.standard_normal((H, L, dh)), "bf16")
    k = inputs.to_storage(gen.standard_normal((H, L, dh)), "bf16")
    S = torch.empty((H, L, L), dtype=torch.bfloat16, device="cuda:0")
    alpha = 1.0 / math.sqrt(dh)
    sg.gemm_strided_batched(to_dev(q, "bf16"), to_dev(k, "bf16"), S, H, L * dh, L * dh, L * L,
                            alpha=alpha, transB="T", dtype=2, M=L, N=L, K=dh, lda=dh, ldb=dh,
                            ldc=L)
    torch.cuda.synchronize()
    got = oracle.decode(from_dev(S), "bf16")
    for h in range(H):
        C0 = np.zeros((L, L), dtype=np.uint16)
        ref = oracle.gemm("N", "T", L, L, dh, alpha, q[h], dh, k[h], dh, 0.0, C0, L, "bf16")
        assert_close(got[h], ref, "bf16", dh, "head %d" % h)


def test_fused_qkv_projection_is_one_gemm():
    """[Q K V] = X [W_Q W_K W_V] (N = 3d) in one call equals the three projections
    (§13.1); with the same tile configuration forced the bits are identical."""
    import swiglu_gemm_amd as sg
    M, d = 384, 512
    gen = np.random.default_rng(450)
    X = inputs.to_storage(gen.standard_normal((M, d)), "bf16")
    Ws = [inputs.to_storage(gen.standard_normal((d, d)) * 0.05, "bf16") for _ in range(3)]
    Wqkv = np.concatenate(Ws, axis=1)
    Xd = to_dev(X, "bf16")
    os.environ["SG_FORCE_CONFIG"] = "2,1"
    try:
        QKV = torch.empty((M, 3 * d), dtype=torch.bfloat16, device="cuda:0")
        sg.gemm(Xd, to_dev(Wqkv, "bf16"), QKV)
        sep = []
        for W in Ws:
            O = torch.empty((M, d), dtype=torch.bfloat16, device="cuda:0")
            sg.gemm(Xd, to_dev(W, "bf16"), O)
            sep.append(from_dev(O))
        torch.cuda.synchronize()
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    fused = from_dev(QKV)
    for i in range(3):
        assert bits_equal(fused[:, i * d:(i + 1) * d], sep[i]), i
    ref = oracle.gemm("N", "N", M, 3 * d, d, 1.0, X, d, Wqkv, 3 * d, 0.0,
                      np.zeros((M, 3 * d), np.uint16), 3 * d, "bf16")
    assert_close(oracle.decode(fused, "bf16"), ref, "bf16", d, "qkv")


@pytest.mark.parametrize("dtype,M,N,K", [("bf16", 2048, 4864, 896), ("e4m3", 2048, 2048, 2048)])
def test_epilogue_repeatable(dtype, M, N, K):
    """Repeated calls give identical bits (a wave writing LDS before every wave has
    left the ring would show here): beta + bias + GELU, and the e4m3 output."""
    import swiglu_gemm_amd as sg
    p, scale = case(dtype, "N", "N", M, N, K, 460, ld_mode="tight")
    A, B = to_dev(p["A"], dtype), to_dev(p["B"], dtype)
    bias = to_dev(bias_vec(N, "f32", 461), "f32")
    od = out_dtype(dtype)
    print("repeatable gemm_ex %s %dx%dx%d" % (dtype, M, N, K), flush=True)
    outs = []
    for _ in range(5):
        C = to_dev(p["C"], od)
        C8 = torch.zeros((M, N), dtype=torch.uint8, device="cuda:0")
        sg.gemm_ex(A, B, C, alpha=0.7 * scale, beta=0.5, bias=bias, activation="gelu",
                   dtype=DT_CODE[dtype])
        sg.gemm_ex(A, B, C8, alpha=0.7 * scale, bias=bias, activation="silu", out_scale=0.125,
                   dtype=DT_CODE[dtype])
        torch.cuda.synchronize()
        outs.append((from_dev(C), from_dev(C8)))
    desc = sg.last_config()
    assert "dma" in desc, desc
    for o in outs[1:]:
        assert bits_equal(o[0], outs[0][0]) and bits_equal(o[1], outs[0][1]), desc
