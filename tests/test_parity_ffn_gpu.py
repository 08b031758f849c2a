"""Parity of the gated FFN with the down projection's input quantization
fused into the gate+up launch (bitlinear_forward_glu_quant), and of the
small-M forward from pre-quantized rows (bitlinear_forward_q, M <= 4),
through the C ABI.

h must be the oracle's gated squared ReLU of the plain forward, and its
int8 codes, scale and row sum the oracle's R4 quantization of that h, bit
for bit; the down projection from those codes must give the oracle's
forward of h.  Inputs come from w1_a8_matmul_amd.workloads; expected values
only from the oracle.
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


def _check_h(orc, X, is_bf16, qw, gc, H, Hq, hs, hr):
    y, *_ = orc.forward(X, qw, gc, bf16=is_bf16)
    h_ref = orc.glu_relu2(y)
    q_ref, s_ref, r_ref = orc.quant_acts(h_ref)
    torch.cuda.synchronize()
    assert np.array_equal(H.cpu().numpy(), h_ref)
    assert np.array_equal(Hq.cpu().numpy(), q_ref)
    assert np.array_equal(hs.cpu().numpy(), s_ref)
    assert np.array_equal(hr.cpu().numpy(), r_ref)
    return h_ref


# (K, N of the fused gate+up matrix, activation kind): the 2B FFN, the 7B
# FFN (11008 gated outputs), small and ragged shapes
SHAPES = [(2560, 13824, "normal_bf16"), (4096, 22016, "student_t3_bf16"),
          (256, 32, "normal_f32"), (1280, 96, "normal_bf16")]


@pytest.mark.parametrize("K,N,kind", SHAPES)
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_glu_quant_matches_oracle(dev, bl, orc, M, K, N, kind):
    packed, gamma, qw, gc = _weights(bl, orc, 9900 + N % 991, N, K, dev, glu=True)
    X, is_bf16 = wl.gen_acts(9901 + 10 * M + K, M, K, kind)
    ws = bl.forward_glu_quant_workspace(dev)
    out = bl.forward_glu_quant(_acts(X, is_bf16, dev), packed, gamma, N, workspace=ws)
    _check_h(orc, X, is_bf16, qw, gc, *out)
    assert not ws.cpu().numpy().any()  # the counter is back at zero


def test_glu_quant_then_down(dev, bl, orc):
    # the whole gated FFN of the 2B shapes at one and four tokens: gate+up with
    # h quantized in the same launch, then the down projection from the codes
    pgu, ggu, qgu, cgu = _weights(bl, orc, 9911, 13824, 2560, dev, glu=True)
    pd, gd, qd, cd = _weights(bl, orc, 9912, 2560, 6912, dev)
    ws = bl.forward_glu_quant_workspace(dev)
    for M in (4, 1):  # the same workspace, a smaller call second
        X, _ = wl.gen_acts(9913 + M, M, 2560, "normal_bf16")
        H, Hq, hs, hr = bl.forward_glu_quant(_acts(X, True, dev), pgu, ggu, 13824, workspace=ws)
        y = bl.forward_q(Hq, hs, hr, pd, gd, 2560)
        h_ref = _check_h(orc, X, True, qgu, cgu, H, Hq, hs, hr)
        y_ref, *_ = orc.forward(h_ref, qd, cd)
        assert np.array_equal(y.cpu().numpy(), y_ref)
        assert torch.equal(y, bl.forward(H, pd, gd, 2560))  # the same bits as from float h


def test_glu_quant_graph_replay(dev, bl, orc):
    # the counter returns to zero inside the graph; replays with eager work
    # between them all match the eager result
    K, N, M = 2560, 1024, 2
    packed, gamma, qw, gc = _weights(bl, orc, 9921, N, K, dev, glu=True)
    X, _ = wl.gen_acts(9922, M, K, "normal_bf16")
    Xt = _acts(X, True, dev)
    ws = bl.forward_glu_quant_workspace(dev)
    eager = [t.clone() for t in bl.forward_glu_quant(Xt, packed, gamma, N, workspace=ws)]
    H = torch.empty((M, N // 2), dtype=torch.float32, device=dev)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        outs = bl.forward_glu_quant(Xt, packed, gamma, N, workspace=ws, out=H)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = bl.forward_glu_quant(Xt, packed, gamma, N, workspace=ws, out=H)
    for r in range(3):
        for t in outs:
            t.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b), r
        bl.forward(Xt, packed, gamma, N, epilogue="relu2_glu")  # eager work between replays
    assert not ws.cpu().numpy().any()


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_forward_q_small_m_matches_oracle(dev, bl, orc, M):
    # the pre-quantized rows go to the one-launch decode kernel up to four tokens
    for K, N, epi in [(6912, 2560, None), (2560, 6912, "relu2"), (12288, 64, None)]:
        packed, gamma, qw, gc = _weights(bl, orc, 9930 + K, N, K, dev)
        X, _ = wl.gen_acts(9931 + M + K, M, K, "normal_bf16")
        q, sx, rs = orc.quant_acts(X, bf16=True)
        Y = bl.forward_q(_gpu(q, dev), _gpu(sx, dev), _gpu(rs, dev), packed, gamma, N,
                         epilogue=epi, split_remainder=False)
        y_ref, *_ = orc.forward(X, qw, gc, bf16=True)
        if epi == "relu2":
            y_ref = orc.relu2(y_ref)
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy(), y_ref), (K, N)


def test_glu_quant_errors(dev, bl):
    X = torch.zeros((5, 256), dtype=torch.bfloat16, device=dev)
    packed = torch.zeros(32 * 256 // 4, dtype=torch.uint8, device=dev)
    gamma = torch.ones(1, dtype=torch.float32, device=dev)
    with pytest.raises(bl.BitLinearError, match="M <= 4"):
        bl.forward_glu_quant(X, packed, gamma, 32)
    with pytest.raises(bl.BitLinearError, match="N % 32"):
        bl.forward_glu_quant(X[:1], packed, gamma, 48)
