"""q4_gemm_smalln_noalloc (the allocation-free entry point) against
q4_gemm_smalln_ws, the entry point whose kernels it shares, through the C
ABI: two calls in a row, the second with a smaller input, each equal to the
workspace call bit for bit and within the accuracy bound of the oracle."""
import numpy as np
import pytest

import cases
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_weight_gemv_amd as q4
    q4.lib()
    oracle.build(force=False)
    return torch, q4, torch.device("cuda:0")


def _case(env, M, K, N, seed):
    torch, q4, dev = env
    W = wl.weights(M, K, seed)
    X = wl.activations(N, K, seed, "swiglu")
    codes, scales, _ = oracle.pack(W)
    Y_ref, S = oracle.gemm(codes, scales, M, K, X)
    c = cases.to_dev(codes, torch, dev)
    s = cases.to_dev(scales.view(np.int16), torch, dev).view(torch.float16)
    Xd = cases.to_dev(X.view(np.int16), torch, dev).view(torch.bfloat16)
    return c, s, Xd, Y_ref, S


def test_noalloc_matches_workspace_call_twice(env):
    torch, q4, dev = env
    for (M, K, N, seed) in ((2048, 11008, 16, 61), (301, 8256, 5, 62)):
        assert q4.q4_gemm_smalln_ws_bytes(M, K, N) > 0  # the split runs
        c, s, Xd, Y_ref, S = _case(env, M, K, N, seed)
        Y = q4.q4_gemm_smalln_noalloc(c, s, Xd)
        torch.cuda.synchronize()
        ws = q4.gemm_workspace(M, K, N, dev)
        Y_ws = q4.q4_gemm_smalln_ws(c, s, Xd, ws)
        torch.cuda.synchronize()
        assert torch.equal(Y, Y_ws), f"M={M} K={K} N={N}: noalloc differs from the workspace call"
        err = np.abs(Y.cpu().numpy().astype(np.float64) - Y_ref)
        assert np.all(err <= 1e-3 * S + 1e-5), f"M={M} K={K} N={N}: worst {np.max(err / (1e-3 * S + 1e-5))}"
        del ws, Y_ws
        # the call itself allocates nothing (Y was allocated by the binding)
        Y2 = torch.empty_like(Y)
        mid = torch.cuda.memory_allocated()
        q4.q4_gemm_smalln_noalloc(c, s, Xd, Y2)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == mid
        assert torch.equal(Y2, Y)


def test_noalloc_without_split_is_the_plain_call(env):
    torch, q4, dev = env
    M, K, N = 3000, 2048, 17  # rows of 2048: no scratch needed
    assert q4.q4_gemm_smalln_ws_bytes(M, K, N) == 0
    c, s, Xd, Y_ref, S = _case(env, M, K, N, 63)
    Y = q4.q4_gemm_smalln_noalloc(c, s, Xd)
    torch.cuda.synchronize()
    assert torch.equal(Y, q4.q4_gemm_smalln(c, s, Xd))


def test_noalloc_in_a_hip_graph(env):
    """Captured in a HIP graph (the callers it is for), the call replays to
    the eager result every time, with eager calls of another shape (sharing
    the same scratch) between the replays."""
    torch, q4, dev = env
    M, K, N = 600, 11008, 9
    c, s, Xd, _, _ = _case(env, M, K, N, 64)
    c2, s2, X2, _, _ = _case(env, 301, 8256, 5, 65)
    eager = q4.q4_gemm_smalln_noalloc(c, s, Xd).clone()
    Y = torch.full((N, M), float("nan"), device=dev)
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            q4.q4_gemm_smalln_noalloc(c, s, Xd, Y, stream=st)
    torch.cuda.synchronize()
    for rep in range(3):
        Y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, eager), f"replay {rep} differs from eager"
        q4.q4_gemm_smalln_noalloc(c2, s2, X2)
        torch.cuda.synchronize()


def test_noalloc_refuses_beyond_its_scratch(env):
    torch, q4, dev = env
    M, K, N = 151936, 4096, 32
    assert q4.q4_gemm_smalln_ws_bytes(M, K, N) > q4.Q4_NOALLOC_SCRATCH_BYTES
    codes = torch.zeros(M * K // 2, dtype=torch.uint8, device=dev).view(M, K // 2)
    scales = torch.zeros((M, K // 64), dtype=torch.float16, device=dev)
    X = torch.zeros((N, K), dtype=torch.bfloat16, device=dev)
    with pytest.raises(q4.Q4Error) as ei:
        q4.q4_gemm_smalln_noalloc(codes, scales, X)
    assert ei.value.status == q4.Q4_ERR_WORKSPACE
