"""Host-only checks of the C ABI: the library loads, exports every function that
include/swiglu_gemm.h declares, and rejects invalid arguments with the documented
negative status before making any HIP call (so these run without a GPU)."""
import ctypes
import os

import pytest

import swiglu_gemm_amd as sg
from swiglu_gemm_amd import build as sgbuild


@pytest.fixture(scope="module")
def L():
    if sgbuild.is_stale():
        sgbuild.build()
    return sg.lib()


def test_exports_every_declared_symbol(L):
    names = sg.declared_symbols()
    assert set(names) >= {"sg_gemm", "sg_swiglu_gemm", "sg_interleave_gate_up", "sg_silu_mul",
                          "sg_status_string", "sg_last_config", "sg_release"}
    for n in names:
        assert hasattr(L, n), "libswiglu_gemm.so does not export %s" % n


def test_no_torch_types_in_header():
    text = open(sg.HEADER).read()
    assert "torch" not in text.lower().replace("torch tensors", "")
    assert 'extern "C"' in text


P = ctypes.c_void_p(0x1000)     # never dereferenced: every call below fails validation
NUL = ctypes.c_void_p(0)


def gemm(L, ta=b"N", tb=b"N", M=2, N=2, K=2, alpha=1.0, A=P, lda=2, B=P, ldb=2, beta=0.0, C=P,
         ldc=2, dtype=0):
    return L.sg_gemm(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype, NUL)


def test_gemm_argument_validation(L):
    assert gemm(L, ta=b"X") == -1
    assert gemm(L, tb=b"C") == -2
    assert gemm(L, M=-1) == -3
    assert gemm(L, N=-1) == -4
    assert gemm(L, K=-1) == -5
    assert gemm(L, A=NUL) == -7
    assert gemm(L, lda=1) == -8                       # 'N': lda >= K
    assert gemm(L, ta=b"T", M=3, lda=2) == -8         # 'T': lda >= M
    assert gemm(L, B=NUL) == -9
    assert gemm(L, ldb=1) == -10                      # 'N': ldb >= N
    assert gemm(L, tb=b"t", K=3, lda=3, ldb=2) == -10  # 'T': ldb >= K
    assert gemm(L, C=NUL) == -12
    assert gemm(L, ldc=1) == -13
    assert gemm(L, dtype=7) == -14
    # quick returns never touch the device
    assert gemm(L, M=0, A=NUL, B=NUL, C=NUL) == 0
    assert gemm(L, N=0, A=NUL, B=NUL, C=NUL, ldb=1, ldc=1) == 0


def test_gemm_ex_argument_validation(L):
    def gx(epi, beta=0.0, **kw):
        args = dict(ta=b"N", tb=b"N", M=2, N=2, K=2, alpha=1.0, A=P, lda=2, B=P, ldb=2, C=P,
                    ldc=2, dtype=2)
        args.update(kw)
        ref = ctypes.byref(epi) if epi is not None else None
        return L.sg_gemm_ex(args["ta"], args["tb"], args["M"], args["N"], args["K"],
                            args["alpha"], args["A"], args["lda"], args["B"], args["ldb"], beta,
                            args["C"], args["ldc"], args["dtype"], ref, NUL)
    E = sg.Epilogue
    gelu = E(None, 0, 2, -1, 1.0)
    assert gx(gelu, ta=b"X") == -1
    assert gx(gelu, M=-1) == -3
    assert gx(gelu, A=NUL) == -7
    assert gx(gelu, ldb=1) == -10
    assert gx(gelu, C=NUL) == -12
    assert gx(gelu, dtype=9) == -14
    assert gx(E(None, 0, 5, -1, 1.0)) == -15                 # unknown activation
    assert gx(E(None, 0, -1, -1, 1.0)) == -15
    assert gx(E(P, 3, 0, -1, 1.0)) == -15                    # e4m3 is not a bias type
    assert gx(E(None, 0, 0, 2, 1.0)) == -15                  # out_dtype: -1 or e4m3 only
    assert gx(E(None, 0, 0, 3, 0.0)) == -15                  # out_scale > 0
    assert gx(E(None, 0, 0, 3, float("nan"))) == -15
    assert gx(E(None, 0, 0, 3, 1.0), beta=0.5) == -11       # C_old would be e4m3 codes
    assert gx(E(None, 0, 9, -1, 1.0), ta=b"X") == -1         # lowest invalid argument first
    assert gx(E(None, 0, 0, 3, 1e-45)) == -15                # 1/out_scale overflows
    # no steps: exactly sg_gemm (its own validation)
    assert gx(None, A=NUL) == -7
    assert gx(E(None, 0, 0, -1, 1.0), ldc=1) == -13
    assert gx(gelu, M=0, A=NUL, B=NUL, C=NUL) == 0           # quick return


def test_swiglu_argument_validation(L):
    def sw(A=P, W=P, Y=P, M=2, N=2, K=2, dt=2, sa=1.0, sw_=1.0):
        return L.sg_swiglu_gemm(A, W, Y, M, N, K, dt, sa, sw_, NUL)
    assert sw(A=NUL) == -1
    assert sw(W=NUL) == -2
    assert sw(Y=NUL) == -3
    assert sw(M=-1) == -4
    assert sw(N=-1) == -5
    assert sw(K=-1) == -6
    assert sw(dt=0) == -7
    assert sw(dt=3, sa=0.0) == -8
    assert sw(dt=3, sa=float("inf")) == -8
    assert sw(dt=3, sw_=float("nan")) == -9
    assert sw(dt=2, sa=2.0) == -8                    # scales must be 1 for bf16
    assert sw(M=0) == 0


def test_swiglu_w12_argument_validation(L):
    def sw(A=P, W1=P, W2=P, Y=P, M=2, N=2, K=2, dt=2, sa=1.0, sw_=1.0):
        return L.sg_swiglu_gemm_w12(A, W1, W2, Y, M, N, K, dt, sa, sw_, NUL)
    assert sw(A=NUL) == -1
    assert sw(W1=NUL) == -2
    assert sw(W2=NUL) == -3
    assert sw(Y=NUL) == -4
    assert sw(M=-1) == -5
    assert sw(N=-1) == -6
    assert sw(K=-1) == -7
    assert sw(dt=0) == -8
    assert sw(dt=3, sa=0.0) == -9
    assert sw(dt=3, sw_=float("inf")) == -10
    assert sw(dt=2, sw_=2.0) == -10                  # scales must be 1 for bf16
    assert sw(N=0) == 0


def test_gemm_strided_batched_validation(L):
    def gb(ta=b"N", tb=b"N", M=2, N=2, K=2, A=P, lda=2, sA=4, B=P, ldb=2, sB=4, C=P, ldc=2,
           sC=4, batch=2, dt=2, alpha=1.0, beta=0.0):
        return L.sg_gemm_strided_batched(ta, tb, M, N, K, alpha, A, lda, sA, B, ldb, sB, beta,
                                         C, ldc, sC, batch, dt, NUL)
    assert gb(ta=b"X") == -1
    assert gb(tb=b"X") == -2
    assert gb(M=-1) == -3
    assert gb(N=-1) == -4
    assert gb(K=-1) == -5
    assert gb(A=NUL) == -7
    assert gb(lda=1) == -8
    assert gb(sA=-1) == -9
    assert gb(B=NUL) == -10
    assert gb(ldb=1) == -11
    assert gb(sB=-1) == -12
    assert gb(C=NUL) == -14
    assert gb(ldc=1) == -15
    assert gb(sC=3) == -16                           # outputs of the problems would overlap
    assert gb(batch=-1) == -17
    assert gb(dt=9) == -18
    assert gb(batch=0) == 0
    assert gb(M=0) == 0
    assert sg.status_string(-18) == "invalid argument 18"


def test_other_entry_points_validation(L):
    assert L.sg_interleave_gate_up(NUL, P, P, 1, 1, 2, NUL) == -1
    assert L.sg_interleave_gate_up(P, P, P, -1, 1, 2, NUL) == -4
    assert L.sg_interleave_gate_up(P, P, P, 1, 1, 9, NUL) == -6
    assert L.sg_interleave_gate_up(P, P, P, 0, 5, 2, NUL) == 0
    assert L.sg_silu_mul(P, P, NUL, 1, 1, 2, NUL) == -3
    assert L.sg_silu_mul(P, P, P, 1, 1, 0, NUL) == -6


def test_status_strings(L):
    assert sg.status_string(0) == "success"
    assert sg.status_string(-8) == "invalid argument 8"
    assert isinstance(sg.last_config(), str)


def test_library_built_from_these_sources(L):
    """The loaded library carries the hash of the sources beside it (a stale build is
    refused by the binding)."""
    info = sg.build_info()
    assert info.startswith("swiglu_gemm source ") and info.endswith(" gfx950"), info
    assert sgbuild.source_hash() in info.split(), (info, sgbuild.source_hash())


def test_stale_library_is_refused(monkeypatch):
    monkeypatch.setattr(sgbuild, "source_hash", lambda: "0123456789abcdef")
    with pytest.raises(sg.SwigluGemmError, match="other sources"):
        sg._check_build(sg.lib())


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(sg, "_lib", None)
    monkeypatch.setattr(sg, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(sg.SwigluGemmError):
        sg.lib()


def test_product_path_does_not_import_oracle():
    here = os.path.dirname(sg.__file__)
    for root, _, files in os.walk(here):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(root, f), encoding="utf-8").read()
                assert "import oracle" not in text and "oracle." not in text.replace(
                    "the oracle", ""), f


def test_diagnostic_library_is_separate():
    """The MFMA-ceiling probe lives in its own library: the GEMM library does not
    export it and the diagnostic library exports only the probe."""
    import ctypes
    from swiglu_gemm_amd import build
    if not os.path.exists(build.DIAG_LIB):
        pytest.skip("diagnostic library not built")
    d = ctypes.CDLL(build.DIAG_LIB)
    assert hasattr(d, "sg_diag_mfma_loop")
    assert not hasattr(d, "sg_gemm")
    import swiglu_gemm_amd as sg
    assert not hasattr(sg.lib(), "sg_diag_mfma_loop")
