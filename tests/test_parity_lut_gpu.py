"""Parity of the lookup-table decode GEMV (bitlinear_forward_lut) with the
oracle, through the C ABI.

The table method changes how the int32 sums are formed, not their value:
int8 activations, scale, accumulators and outputs must be the oracle's bits,
and the same as bitlinear_forward's.  Inputs come from
w1_a8_matmul_amd.workloads; expected values only from the oracle.
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


def _weights(bl, orc, seed, N, K, dev, sparse=0.0, glu=False):
    W = wl.gen_weight(seed, N, K, sparse)
    packed, gamma = bl.quantize_weights(_gpu(W, dev), glu=glu)
    _, gc = orc.absmean(W)
    qw = orc.ternarize(W, gc)
    assert gamma.cpu().numpy()[0] == gc
    return packed, gamma, qw, gc


# (K, N, activation kind, epilogue, sparse weights): one and many blocks per
# wave, the decode pair's shapes, the largest K the tables fit, a ragged
# number of blocks per wave (K = 1280: five blocks over four waves)
SHAPES = [(256, 16, "normal_f32", None, 0.0), (2560, 6912, "normal_bf16", "relu2", 0.0),
          (6912, 2560, "normal_f32", None, 0.0), (8192, 64, "normal_bf16", None, 0.0),
          (4096, 512, "student_t3_bf16", None, 0.3), (1280, 48, "outlier_bf16", "relu2", 0.0)]


@pytest.mark.parametrize("K,N,kind,epi,sparse", SHAPES)
def test_forward_lut_matches_oracle(dev, bl, orc, K, N, kind, epi, sparse):
    packed, gamma, qw, gc = _weights(bl, orc, 9800 + K + N, N, K, dev, sparse)
    X, is_bf16 = wl.gen_acts(9900 + K, 1, K, kind)
    Xt = _gpu(X, dev)
    Xt = Xt.view(torch.bfloat16) if is_bf16 else Xt
    y, dbg = bl.forward_lut(Xt, packed, gamma, N, epilogue=epi, debug=True)
    y_ref, qx, sx, acc = orc.forward(X, qw, gc, bf16=is_bf16)
    if epi == "relu2":
        y_ref = orc.relu2(y_ref)
    torch.cuda.synchronize()
    assert np.array_equal(dbg["xq"].cpu().numpy(), qx)
    assert dbg["x_scale"].cpu().numpy()[0] == sx[0]
    assert np.array_equal(dbg["acc"].cpu().numpy(), acc)
    assert np.array_equal(y.cpu().numpy(), y_ref)
    y_dot = bl.forward(Xt, packed, gamma, N, epilogue=epi)  # same bits as the dot path
    assert torch.equal(y, y_dot)


def test_forward_lut_glu(dev, bl, orc):
    K, N = 2560, 1024
    packed, gamma, qw, gc = _weights(bl, orc, 9811, N, K, dev, glu=True)
    X, _ = wl.gen_acts(9812, 1, K, "normal_bf16")
    h, dbg = bl.forward_lut(_gpu(X, dev).view(torch.bfloat16), packed, gamma, N,
                            epilogue="relu2_glu", debug=True)
    y_ref, _, _, acc = orc.forward(X, qw, gc, bf16=True)
    torch.cuda.synchronize()
    assert np.array_equal(dbg["acc"].cpu().numpy(), acc)  # unpermuted row order
    assert np.array_equal(h.cpu().numpy(), orc.glu_relu2(y_ref))


def test_forward_lut_pair_chain(dev, bl, orc):
    # the decode pair: up (ReLU^2) feeds its float output to down
    pu, gu, qu, cu = _weights(bl, orc, 9821, 6912, 2560, dev)
    pd, gd, qd, cd = _weights(bl, orc, 9822, 2560, 6912, dev)
    X, _ = wl.gen_acts(9823, 1, 2560, "normal_bf16")
    h = bl.forward_lut(_gpu(X, dev).view(torch.bfloat16), pu, gu, 6912, epilogue="relu2")
    y = bl.forward_lut(h, pd, gd, 2560)
    h_ref = orc.relu2(orc.forward(X, qu, cu, bf16=True)[0])
    y_ref = orc.forward(h_ref, qd, cd)[0]
    torch.cuda.synchronize()
    assert np.array_equal(h.cpu().numpy(), h_ref)
    assert np.array_equal(y.cpu().numpy(), y_ref)


def test_forward_lut_degenerate(dev, bl, orc):
    # an all-zero token (scale from the 1e-5 guard, every code 0) and an
    # all-zero weight matrix (gamma from the guard, every weight code 0)
    K, N = 512, 32
    packed, gamma, qw, gc = _weights(bl, orc, 9831, N, K, dev)
    X = np.zeros((1, K), np.float32)
    y = bl.forward_lut(_gpu(X, dev), packed, gamma, N)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), orc.forward(X, qw, gc)[0])
    W0 = np.zeros((N, K), np.float32)
    p0, g0 = bl.quantize_weights(_gpu(W0, dev))
    X1, _ = wl.gen_acts(9832, 1, K, "normal_f32")
    y0 = bl.forward_lut(_gpu(X1, dev), p0, g0, N)
    torch.cuda.synchronize()
    assert not y0.cpu().numpy().any()


def test_forward_lut_errors(dev, bl):
    packed = torch.zeros(16 * 8448 // 4, dtype=torch.uint8, device=dev)
    gamma = torch.ones(1, dtype=torch.float32, device=dev)
    with pytest.raises(bl.BitLinearError, match="one token"):
        bl.forward_lut(torch.zeros((2, 256), device=dev), packed, gamma, 16)
    with pytest.raises(bl.BitLinearError, match="exceeds 8192"):
        bl.forward_lut(torch.zeros((1, 8448), device=dev), packed, gamma, 16)
    with pytest.raises(bl.BitLinearError, match="multiple of 256"):
        bl.forward_lut(torch.zeros((1, 320), device=dev), packed, gamma, 16)
