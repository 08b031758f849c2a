"""Parity of the gated squared ReLU epilogue (reading R12: a fused gate+up
matrix, h = max(gate, 0)^2 * up; "BitNet b1.58 2B4T Technical Report" card,
Method Adaptation, and fishai digest: ReLU^2 as the FFN activation) with the
CPU oracle, through the C ABI.

The interleaved packing must match the oracle's byte for byte; outputs are
bit-identical (each half is rescaled exactly as the plain forward does and
combined with the same two float multiplies) and held to the 1e-6 bar.
"""
import numpy as np
import pytest

from w1_a8_matmul_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
REL_TOL = 1e-6


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from w1_a8_matmul_amd import bitlinear as bl  # raises if the library is missing

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


def _acts_gpu(X, is_bf16, dev):
    t = _gpu(X, dev)
    return t.view(torch.bfloat16) if is_bf16 else t


def _rel(a, ref):
    a, ref = np.asarray(a, np.float64), np.asarray(ref, np.float64)
    d = np.abs(a - ref)
    assert not ((ref == 0) & (d != 0)).any()
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.where(ref != 0, d / np.abs(ref), 0.0)
    return float(r.max()) if r.size else 0.0


def _glu_weights(bl, orc, seed, N, K, dev):
    W = wl.gen_weight(seed, N, K)
    packed, gamma = bl.quantize_weights(_gpu(W, dev), glu=True)
    _, gc, qw = orc.quantize_weights(W)
    assert gamma.cpu().numpy()[0] == gc
    assert np.array_equal(packed.cpu().numpy(), orc.pack_glu(qw))
    return packed, gamma, qw, gc


@pytest.mark.parametrize("M,K,N,kind", [(1, 2560, 13824, "normal_bf16"),
                                        (4, 256, 544, "normal_f32"),
                                        (3, 6912, 2080, "student_t3_bf16"),
                                        (5, 2560, 13824, "normal_bf16"),
                                        (130, 2816, 1056, "outlier_bf16"),
                                        (2048, 6912, 5120, "outlier_bf16")])
def test_forward_glu_matches_oracle(dev, bl, orc, M, K, N, kind):
    # M <= 4: the fused GEMV; larger M: quantization + GEMM (2048 x 6912 ->
    # 5120 cuts its last, partial round of tiles along K)
    packed, gamma, qw, gc = _glu_weights(bl, orc, 10100 + N, N, K, dev)
    X, is_bf16 = wl.gen_acts(10200 + M, M, K, kind)
    Y, dbg = bl.forward(_acts_gpu(X, is_bf16, dev), packed, gamma, N, epilogue="relu2_glu",
                        debug=True)
    assert Y.shape == (M, N // 2)
    rows = np.arange(M) if M <= 300 else np.array([0, 5, 1023, 1500, M - 1])
    y_full, xq, sx, acc = orc.forward(X[rows], qw, gc, bf16=is_bf16)
    h_ref = orc.glu_relu2(y_full)
    assert np.array_equal(dbg["acc"].cpu().numpy()[rows], acc)  # unpermuted row order
    h = Y.cpu().numpy()[rows]
    assert _rel(h, h_ref) <= REL_TOL
    assert np.array_equal(h, h_ref)


@pytest.mark.parametrize("M,K,N", [(2048, 2560, 13824), (300, 2816, 1056)])
def test_forward_q_glu_matches_forward(dev, bl, orc, M, K, N):
    packed, gamma, qw, gc = _glu_weights(bl, orc, 10300 + N, N, K, dev)
    X, _ = wl.gen_acts(10400 + M, M, K, "normal_bf16")
    Xt = _acts_gpu(X, True, dev)
    Xq, sx, rs = bl.quantize_acts(Xt)
    a = bl.forward_q(Xq, sx, rs, packed, gamma, N, epilogue="relu2_glu")
    b = bl.forward(Xt, packed, gamma, N, epilogue="relu2_glu")
    assert torch.equal(a, b)
    rows = np.array([0, 7, M // 2, M - 1])
    y_full, *_ = orc.forward(X[rows], qw, gc, bf16=True)
    assert np.array_equal(a.cpu().numpy()[rows], orc.glu_relu2(y_full))


@pytest.mark.parametrize("M", [1, 3, 4, 16, 64])
def test_group_glu_matches_oracle(dev, bl, orc, M):
    # gated gate+up layers next to plain ones, in every grouped mode
    shapes = [(2560, 3840, None), (2560, 13824, "relu2_glu"), (6912, 2560, None),
              (256, 544, "relu2_glu"), (2560, 272, "relu2")]
    layers, refs = [], []
    for i, (K, N, epi) in enumerate(shapes):
        W = wl.gen_weight(10500 + i, N, K)
        glu = epi == "relu2_glu"
        packed, gamma = bl.quantize_weights(_gpu(W, dev), glu=glu)
        _, gc, qw = orc.quantize_weights(W)
        X, is_bf16 = wl.gen_acts(10600 + 10 * M + i, M, K, "normal_bf16")
        layers.append((_acts_gpu(X, is_bf16, dev), packed, gamma, N, epi, None))
        y, *_ = orc.forward(X, qw, gc, bf16=is_bf16)
        refs.append(orc.glu_relu2(y) if glu else (orc.relu2(y) if epi == "relu2" else y))
    grp = bl.Group(layers)
    outs = [t.clone() for t in grp.forward()]
    torch.cuda.synchronize()
    for y, y_ref in zip(outs, refs):
        assert y.shape == y_ref.shape
        assert np.array_equal(y.cpu().numpy(), y_ref)
