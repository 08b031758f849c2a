"""Parity of the fused subln + activation quantization (reading R8: RMSNorm
with a per-feature gain before the per-token absmax quantization; fishai
digest, list of BitLinear parts, and "BitNet b1.58 2B4T Technical Report"
card, Method Adaptation) with the CPU oracle, through the C ABI.

The int8 codes and row sums come from x * g and must be bit-identical.  The
RMS factor comes from a double sum of squares whose order differs between the
GPU reduction and the oracle's index order; it only enters the float scale,
which is held to a relative error of 2^-22 (two float roundings), and the
outputs to the contract's 1e-6.
"""
import numpy as np
import pytest

from w1_a8_matmul_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
REL_TOL = 1e-6
SCALE_TOL = 2.0 ** -22
EPS = 1e-5


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
    assert not ((ref == 0) & (d != 0)).any(), "nonzero where the oracle has an exact zero"
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.where(ref != 0, d / np.abs(ref), 0.0)
    return float(r.max()) if r.size else 0.0


def _weights(bl, orc, seed, N, K, dev):
    W = wl.gen_weight(seed, N, K)
    packed, gamma = bl.quantize_weights(_gpu(W, dev))
    _, gc, qw = orc.quantize_weights(W)
    assert gamma.cpu().numpy()[0] == gc
    return packed, gamma, qw, gc


def _expected(orc, X, is_bf16, g, qw, gc, relu2):
    q, s, _ = orc.quant_acts_rmsnorm(X, g, EPS, bf16=is_bf16)
    y = orc.rescale(orc.int_matmul(q, qw), s, gc)
    return (orc.relu2(y) if relu2 else y), q, s


@pytest.mark.parametrize("M,K,kind", [(1, 2560, "normal_bf16"), (5, 256, "normal_f32"),
                                      (300, 6912, "outlier_bf16"), (64, 4096, "student_t3_bf16"),
                                      (3, 11008, "normal_f32"), (2, 16384, "normal_bf16"),
                                      (2, 20480, "normal_f32")])
def test_quantize_acts_rmsnorm_matches_oracle(dev, bl, orc, M, K, kind):
    X, is_bf16 = wl.gen_acts(9100 + M, M, K, kind)
    g = wl.gen_gain(9200 + K, K)
    Xq, sx, rs = bl.quantize_acts(_acts_gpu(X, is_bf16, dev), norm_gain=_gpu(g, dev),
                                  norm_eps=EPS)
    q_ref, s_ref, r_ref = orc.quant_acts_rmsnorm(X, g, EPS, bf16=is_bf16)
    assert np.array_equal(Xq.cpu().numpy(), q_ref)
    assert np.array_equal(rs.cpu().numpy(), r_ref)
    assert _rel(sx.cpu().numpy(), s_ref) <= SCALE_TOL


def test_quantize_acts_rmsnorm_edge_rows(dev, bl, orc):
    # an all-zero row (the guard), a row with one nonzero, a zero gain entry
    M, K = 4, 512
    X = wl.gen_acts_f32(9300, M, K, "normal")
    X[1] = 0
    X[2] = 0
    X[2, 77] = np.float32(-3.0)
    g = wl.gen_gain(9301, K)
    g[5] = 0
    Xq, sx, rs = bl.quantize_acts(_gpu(X, dev), norm_gain=_gpu(g, dev), norm_eps=EPS)
    q_ref, s_ref, r_ref = orc.quant_acts_rmsnorm(X, g, EPS)
    assert np.array_equal(Xq.cpu().numpy(), q_ref) and np.array_equal(rs.cpu().numpy(), r_ref)
    assert _rel(sx.cpu().numpy(), s_ref) <= SCALE_TOL
    assert np.all(Xq.cpu().numpy()[:, 5] == 0)


@pytest.mark.parametrize("M,K,N,kind,epi", [(1, 2560, 6912, "normal_bf16", "relu2"),
                                            (4, 6912, 2560, "normal_f32", None),
                                            (3, 256, 48, "student_t3_bf16", None),
                                            (5, 2560, 272, "normal_bf16", None),
                                            (130, 2816, 1040, "outlier_bf16", "relu2"),
                                            (2048, 2560, 6912, "outlier_bf16", None)])
def test_forward_rmsnorm_matches_oracle(dev, bl, orc, M, K, N, kind, epi):
    # M <= 4: subln inside the fused GEMV launch; larger M: in the
    # quantization launch before the int8 MFMA GEMM
    packed, gamma, qw, gc = _weights(bl, orc, 9400 + N, N, K, dev)
    X, is_bf16 = wl.gen_acts(9500 + M, M, K, kind)
    g = wl.gen_gain(9600 + K, K)
    Y, dbg = bl.forward(_acts_gpu(X, is_bf16, dev), packed, gamma, N, epilogue=epi, debug=True,
                        norm_gain=_gpu(g, dev), norm_eps=EPS)
    rows = np.arange(M) if M <= 300 else np.array([0, 1, 777, 1500, M - 1])
    y_ref, q_ref, s_ref = _expected(orc, X[rows], is_bf16, g, qw, gc, epi == "relu2")
    assert np.array_equal(dbg["xq"].cpu().numpy()[rows], q_ref)
    assert _rel(dbg["x_scale"].cpu().numpy()[rows], s_ref) <= SCALE_TOL
    assert np.array_equal(dbg["acc"].cpu().numpy()[rows], orc.int_matmul(q_ref, qw))
    assert _rel(Y.cpu().numpy()[rows], y_ref) <= REL_TOL


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 16, 64])
def test_group_rmsnorm_matches_oracle(dev, bl, orc, M):
    # layers with and without a gain in one group; M <= 4 applies subln in
    # the grouped kernel's own quantization, larger M in the quantization
    # launch (then the skinny kernel, or the tiled GEMM above 16 tokens)
    shapes = [(2560, 3840, "normal_bf16", None, True), (2560, 272, "normal_f32", "relu2", False),
              (6912, 2560, "normal_bf16", None, True), (4096, 512, "student_t3_bf16", None, True),
              (256, 16, "normal_f32", None, False)]
    layers, refs = [], []
    for i, (K, N, kind, epi, norm) in enumerate(shapes):
        packed, gamma, qw, gc = _weights(bl, orc, 9700 + i, N, K, dev)
        X, is_bf16 = wl.gen_acts(9800 + 10 * M + i, M, K, kind)
        g = wl.gen_gain(9900 + i, K) if norm else None
        layers.append((_acts_gpu(X, is_bf16, dev), packed, gamma, N, epi, None,
                       _gpu(g, dev) if norm else None, EPS))
        if norm:
            y, _, _ = _expected(orc, X, is_bf16, g, qw, gc, epi == "relu2")
        else:
            y, *_ = orc.forward(X, qw, gc, bf16=is_bf16)
            y = orc.relu2(y) if epi == "relu2" else y
        refs.append((y, norm))
    grp = bl.Group(layers)
    outs = [t.clone() for t in grp.forward()]
    torch.cuda.synchronize()
    for (y_ref, norm), y in zip(refs, outs):
        if norm:
            assert _rel(y.cpu().numpy(), y_ref) <= REL_TOL
        else:
            assert np.array_equal(y.cpu().numpy(), y_ref)  # layers without a gain: unchanged
    for y, y2 in zip(outs, grp.forward()):
        assert torch.equal(y, y2)  # repeatable
