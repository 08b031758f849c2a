"""Parity of the decode FFN in one launch (bitlinear_ffn_chain) with the
oracle, through the C ABI.

h (the squared ReLU, plain or gated, of the up projection) and Y (the down
projection of h) must be the oracle's bits, and the same as two
bitlinear_forward calls.  Inputs come from w1_a8_matmul_amd.workloads;
expected values only from the oracle.
"""
import numpy as np
import pytest

from w1_a8_matmul_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from w1_a8_matmul_amd import bitlinear as bl

    bl.lib()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def bl(dev):
    from w1_a8_matmul_amd import bitlinear

    return bitlinear


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def _gpu(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _weights(bl, orc, seed, N, K, dev, glu=False):
    W = wl.gen_weight(seed, N, K)
    packed, gamma = bl.quantize_weights(_gpu(W, dev), glu=glu)
    _, gc = orc.absmean(W)
    qw = orc.ternarize(W, gc)
    assert gamma.cpu().numpy()[0] == gc
    return packed, gamma, qw, gc


def _acts(X, is_bf16, dev):
    t = _gpu(X, dev)
    return t.view(torch.bfloat16) if is_bf16 else t


def _ws_clean(ws):
    # queue and finished count back at zero, no wait gave up (the generation
    # and the per-tile flags carry over to the next call by design)
    q, fin, err = ws.view(torch.int32)[:3].cpu().tolist()
    return q == 0 and fin == 0 and err == 0


def _expected(orc, X, is_bf16, qu, cu, qd, cd, glu):
    y, *_ = orc.forward(X, qu, cu, bf16=is_bf16)
    h = orc.glu_relu2(y) if glu else orc.relu2(y)
    yd, *_ = orc.forward(h, qd, cd)
    return h, yd


# (K, N_up, gated, N_down, activation kind): the decode pair, the 2B and 7B
# gated FFNs, small shapes (one and two blocks per wave, ragged grids)
SHAPES = [(2560, 6912, False, 2560, "normal_bf16"), (2560, 13824, True, 2560, "normal_bf16"),
          (4096, 22016, True, 4096, "student_t3_bf16"), (256, 256, False, 16, "normal_f32"),
          (512, 512, True, 48, "normal_f32")]


@pytest.mark.parametrize("K,N_up,glu,N_down,kind", SHAPES)
@pytest.mark.parametrize("M", [1, 4])
def test_ffn_chain_matches_oracle(dev, bl, orc, M, K, N_up, glu, N_down, kind):
    F = N_up // 2 if glu else N_up
    pu, gu, qu, cu = _weights(bl, orc, 9950 + K + N_up % 977, N_up, K, dev, glu=glu)
    pd, gd, qd, cd = _weights(bl, orc, 9951 + F, N_down, F, dev)
    X, is_bf16 = wl.gen_acts(9952 + M + K, M, K, kind)
    Xt = _acts(X, is_bf16, dev)
    ws = bl.ffn_chain_workspace(N_up, dev)
    H, Y = bl.ffn_chain(Xt, pu, gu, N_up, pd, gd, N_down, glu=glu, workspace=ws)
    h_ref, y_ref = _expected(orc, X, is_bf16, qu, cu, qd, cd, glu)
    torch.cuda.synchronize()
    assert np.array_equal(H.cpu().numpy(), h_ref)
    assert np.array_equal(Y.cpu().numpy(), y_ref)
    assert _ws_clean(ws)
    # the same bits as two plain launches
    h2 = bl.forward(Xt, pu, gu, N_up, epilogue="relu2_glu" if glu else "relu2")
    assert torch.equal(H, h2)
    assert torch.equal(Y, bl.forward(h2, pd, gd, N_down))


def test_ffn_chain_repeated_and_graph(dev, bl, orc):
    # consecutive calls with a smaller M second, then graph replays with eager
    # work between them, all on one workspace
    K, N_up, N_down = 2560, 6912, 2560
    pu, gu, qu, cu = _weights(bl, orc, 9961, N_up, K, dev)
    pd, gd, qd, cd = _weights(bl, orc, 9962, N_down, N_up, dev)
    ws = bl.ffn_chain_workspace(N_up, dev)
    for M in (3, 1):
        X, _ = wl.gen_acts(9963 + M, M, K, "normal_bf16")
        H, Y = bl.ffn_chain(_acts(X, True, dev), pu, gu, N_up, pd, gd, N_down, workspace=ws)
        h_ref, y_ref = _expected(orc, X, True, qu, cu, qd, cd, False)
        torch.cuda.synchronize()
        assert np.array_equal(H.cpu().numpy(), h_ref) and np.array_equal(Y.cpu().numpy(), y_ref)
    X, _ = wl.gen_acts(9969, 2, K, "normal_bf16")
    Xt = _acts(X, True, dev)
    H = torch.empty((2, N_up), dtype=torch.float32, device=dev)
    Y = torch.empty((2, N_down), dtype=torch.float32, device=dev)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        bl.ffn_chain(Xt, pu, gu, N_up, pd, gd, N_down, workspace=ws, H=H, out=Y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bl.ffn_chain(Xt, pu, gu, N_up, pd, gd, N_down, workspace=ws, H=H, out=Y)
    h_ref, y_ref = _expected(orc, X, True, qu, cu, qd, cd, False)
    for r in range(3):
        H.fill_(0)
        Y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(H.cpu().numpy(), h_ref), r
        assert np.array_equal(Y.cpu().numpy(), y_ref), r
        bl.forward(Xt, pu, gu, N_up, epilogue="relu2")  # eager work between replays
    assert _ws_clean(ws)


def test_ffn_chain_errors(dev, bl):
    X = torch.zeros((5, 256), dtype=torch.bfloat16, device=dev)
    p = torch.zeros(256 * 256 // 4, dtype=torch.uint8, device=dev)
    g = torch.ones(1, dtype=torch.float32, device=dev)
    with pytest.raises(bl.BitLinearError, match="1 <= M <= 4"):
        bl.ffn_chain(X, p, g, 256, p, g, 16)
    with pytest.raises(bl.BitLinearError, match="multiple of 256"):
        bl.ffn_chain(X[:1], p, g, 272, p, g, 16)
