"""The forward that allocates nothing (bitlinear_forward_noalloc), through the
C ABI: its results must be those of bitlinear_forward with a workspace, bit
for bit, on consecutive calls that share the library's scratch array -- the
second call smaller than the first, so it runs on what the first one left --
and under graph capture.  Shapes beyond the scratch are rejected before
anything is enqueued."""
import numpy as np
import pytest

from w1_a8_matmul_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def bl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from w1_a8_matmul_amd import bitlinear

    bitlinear.lib()
    return bitlinear


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def _layer(bl, dev, M, K, N, seed, kind="normal_bf16"):
    W = wl.gen_weight(seed, N, K)
    X, is_bf16 = wl.gen_acts(seed + 5, M, K, kind)
    packed, gamma = bl.quantize_weights(torch.from_numpy(W).to(dev))
    Xt = torch.from_numpy(X).to(dev)
    return (Xt.view(torch.bfloat16) if is_bf16 else Xt), packed, gamma


def test_noalloc_matches_forward_on_consecutive_calls(bl):
    dev = torch.device("cuda:0")
    # large first (the GEMM path, its last round cut along K), then smaller
    # ones on the scratch the first left behind, then the fused small-M path
    cases = [(2048, 6912, 2560, "outlier_bf16", None), (300, 2816, 1040, "normal_bf16", "relu2"),
             (64, 2560, 512, "normal_f32", None), (3, 2560, 256, "normal_bf16", None)]
    for M, K, N, kind, epi in cases:
        X, packed, gamma = _layer(bl, dev, M, K, N, 9100 + M, kind)
        want, dw = bl.forward(X, packed, gamma, N, epilogue=epi, debug=True)
        got, dg = bl.forward_noalloc(X, packed, gamma, N, epilogue=epi, debug=True)
        torch.cuda.synchronize()
        assert torch.equal(got, want), (M, K, N)
        assert torch.equal(dg["acc"], dw["acc"]) and torch.equal(dg["xq"], dw["xq"])


def test_noalloc_repeated_and_graph_replay(bl):
    dev = torch.device("cuda:0")
    M, K, N = 512, 4096, 2048
    X, packed, gamma = _layer(bl, dev, M, K, N, 9200, "student_t3_bf16")
    want = bl.forward(X, packed, gamma, N)
    out = torch.empty_like(want)
    for _ in range(3):
        out.zero_()
        bl.forward_noalloc(X, packed, gamma, N, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, want)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        bl.forward_noalloc(X, packed, gamma, N, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        bl.forward_noalloc(X, packed, gamma, N, out=out)
    for rep in range(3):
        out.fill_(float("nan"))  # eager work between replays
        X2, p2, g2 = _layer(bl, dev, 128, 2560, 256, 9300 + rep)  # another call on the scratch
        bl.forward_noalloc(X2, p2, g2, 256)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {rep}"


def test_noalloc_rejects_oversize(bl):
    dev = torch.device("cuda:0")
    M, K, N = 4096, 8192, 256  # needs more than the 32 MiB scratch
    assert bl.workspace_bytes(M, K, N) > bl.NOALLOC_SCRATCH_BYTES
    X = torch.zeros((M, K), dtype=torch.bfloat16, device=dev)
    packed = torch.zeros(N * K // 4, dtype=torch.uint8, device=dev)
    gamma = torch.ones(1, dtype=torch.float32, device=dev)
    out = torch.full((M, N), 7.0, dtype=torch.float32, device=dev)
    with pytest.raises(bl.BitLinearError, match="scratch"):
        bl.forward_noalloc(X, packed, gamma, N, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)  # nothing was enqueued
