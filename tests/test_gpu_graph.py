"""Library calls captured into a HIP graph (torch.cuda.CUDAGraph) and replayed: each
replay must give the bits of the eager call.  Between replays the output is cleared
and other eager work of the library runs on the same stream (so a replay that left
the output untouched, or a captured buffer that eager work overwrote, would show).
Covers the paths a serving loop would capture: the 8-wave tile GEMM, split-K and
the decode kernels through the entry point that allocates nothing, the fused
SwiGLU-GEMM (bf16 and e4m3; bf16 at 128 tokens with the L2 warm-up blocks), the fp32
GEMM and e4m3 operands re-laid with 16-byte rows.  Workspace the library owns is grown by the eager call before capture."""
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import swiglu_gemm_amd as sg
    sg.lib()


def rand(shape, dtype, scale, seed):
    g = torch.Generator(device="cuda:0").manual_seed(seed)
    return (torch.randn(shape, device="cuda:0", generator=g) * scale).to(dtype)


def replay_matches_eager(call, out, other):
    """call() writes out; other() is unrelated eager library work."""
    call()
    torch.cuda.synchronize()
    want = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(3):
        out.zero_()
        other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), want.view(torch.uint8)), "replay %d" % r
    del g


def other_work():
    import swiglu_gemm_amd as sg
    A = rand((96, 4096), torch.bfloat16, 1.0, 9)
    B = rand((2048, 4096), torch.bfloat16, 0.02, 10)
    C = torch.empty(96, 2048, dtype=torch.bfloat16, device="cuda:0")
    return lambda: sg.gemm(A, B, C, transB="T")       # split-K on the library workspace


@pytest.mark.parametrize("case", ["tile", "noalloc_splitk", "noalloc_decode", "fp32",
                                  "e4m3_relaid"])
def test_gemm_graph_replay(case):
    import swiglu_gemm_amd as sg
    print("graph gemm %s" % case, flush=True)
    other = other_work()
    if case == "tile":
        A = rand((2048, 4096), torch.float16, 1 / 64, 1)
        B = rand((4096, 3072), torch.float16, 1 / 64, 2)
        C = torch.empty(2048, 3072, dtype=torch.float16, device="cuda:0")
        call = lambda: sg.gemm(A, B, C)
    elif case == "noalloc_splitk":
        A = rand((64, 4096), torch.bfloat16, 1.0, 3)
        B = rand((4096, 4096), torch.bfloat16, 0.02, 4)
        C = torch.empty(64, 4096, dtype=torch.bfloat16, device="cuda:0")
        call = lambda: sg.gemm_noalloc(A, B, C, alpha=0.5, transB="T")
    elif case == "noalloc_decode":
        A = rand((8, 4096), torch.float16, 1.0, 6)
        B = rand((4096, 4096), torch.float16, 0.02, 7)
        C = torch.empty(8, 4096, dtype=torch.float16, device="cuda:0")
        call = lambda: sg.gemm_noalloc(A, B, C)
    elif case == "fp32":
        A = rand((1000, 600), torch.float32, 1.0, 11)
        B = rand((600, 700), torch.float32, 1.0, 12)
        C = torch.empty(1000, 700, dtype=torch.float32, device="cuda:0")
        call = lambda: sg.gemm(A, B, C, alpha=1.5)
    else:
        A = rand((300, 1000), torch.float32, 1.0, 13).to(torch.float8_e4m3fn)
        B = rand((1000, 1001), torch.float32, 1.0, 14).to(torch.float8_e4m3fn)
        C = torch.empty(300, 1001, dtype=torch.bfloat16, device="cuda:0")
        call = lambda: sg.gemm(A, B, C, alpha=1 / 64)
    call()
    torch.cuda.synchronize()
    desc = sg.last_config()
    if case == "noalloc_splitk":
        assert "splits=1" not in desc, desc
    if case == "noalloc_decode":
        assert "decode" in desc, desc
    if case == "e4m3_relaid":
        assert "gemm8 cfg=" in desc, desc
    replay_matches_eager(call, C, other)


@pytest.mark.parametrize("dtype,M", [("bf16", 2048), ("bf16", 128), ("e4m3", 16)])
def test_swiglu_graph_replay(dtype, M):
    import swiglu_gemm_amd as sg
    print("graph swiglu %s M=%d" % (dtype, M), flush=True)
    N, K = (4864, 896) if dtype == "bf16" else (11008, 4096)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float8_e4m3fn
    A = rand((M, K), torch.float32, 1.0, 20).to(tdt)
    W = rand((K, 2 * N), torch.float32, 0.02 if dtype == "bf16" else 20.0, 21).to(tdt)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda:0")
    s = 1.0 if dtype == "bf16" else 0.01
    call = lambda: sg.swiglu_gemm(A, W, Y, s, s)
    if (dtype, M) == ("bf16", 128):
        call()                       # this size launches the L2 warm-up blocks too
        torch.cuda.synchronize()
        assert "l2warm=" in sg.last_config(), sg.last_config()
    replay_matches_eager(call, Y, other_work())
