"""Parity of the base-3 layout (five ternary codes per byte, reading R13)
with the oracle, through the C ABI.

The packed bytes (from float weights, from int8 codes, and for a fused
gate+up matrix) must equal the oracle's base-3 packing bit for bit, and the
grouped forward on base-3 weights must give the oracle's outputs bit for bit
(the codes are the same as in the 2-bit layout; only their storage differs).
Inputs come from w1_a8_matmul_amd.workloads; expected values only from the
oracle.
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


@pytest.mark.parametrize("N,K,seed,sparse", [(16, 320, 1, 0.0), (48, 656, 2, 0.0),
                                             (256, 2560, 3, 0.0), (2560, 6912, 4, 0.0),
                                             (64, 4096, 5, 0.3), (32, 16, 6, 0.0)])
def test_quantize_weights_b3_bit_exact(dev, bl, orc, N, K, seed, sparse):
    W = wl.gen_weight(seed, N, K, sparse)
    packed, gamma = bl.quantize_weights_b3(_gpu(W, dev))
    _, gc = orc.absmean(W)
    q = orc.ternarize(W, gc)
    assert gamma.cpu().numpy()[0] == gc
    ref = orc.pack_b3(q)
    got = packed.cpu().numpy()
    assert got.size == ref.size == bl.packed_bytes_b3(N, K)
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} bytes differ"
    back = bl.unpack_ternary_b3(packed, N, K).cpu().numpy()
    assert np.array_equal(back, q)


def test_quantize_weights_b3_glu(dev, bl, orc):
    # a fused gate+up matrix: the rows interleave per 16-row tile as in the
    # 2-bit layout (the oracle's 2-bit packing, unpacked, gives that order)
    N, K = 64, 2560
    W = wl.gen_weight(21, N, K)
    packed, gamma = bl.quantize_weights_b3(_gpu(W, dev), glu=True)
    _, gc = orc.absmean(W)
    q = orc.ternarize(W, gc)
    q_rows = orc.unpack(orc.pack_glu(q), N, K)
    assert np.array_equal(packed.cpu().numpy(), orc.pack_b3(q_rows))


@pytest.mark.parametrize("N,K", [(16, 320), (48, 656), (272, 2560)])
def test_pack_unpack_b3(dev, bl, orc, N, K):
    rng = np.random.default_rng(N + K)
    q = rng.integers(-1, 2, (N, K)).astype(np.int8)
    packed = bl.pack_ternary_b3(_gpu(q, dev))
    assert np.array_equal(packed.cpu().numpy(), orc.pack_b3(q))
    assert np.array_equal(bl.unpack_ternary_b3(packed, N, K).cpu().numpy(), q)
    q2 = rng.integers(-128, 128, (N, K)).astype(np.int8)  # clamped into {-1, 0, 1}
    p2 = bl.pack_ternary_b3(_gpu(q2, dev))
    assert np.array_equal(p2.cpu().numpy(), orc.pack_b3(np.clip(q2, -1, 1)))


# shapes: K padded (656 -> 960, 6912 -> 7040, 11008 -> 11200), K = 16, float
# and bf16 inputs, ReLU^2
B3_SHAPES = [(320, 16, "normal_f32", None), (656, 272, "normal_bf16", "relu2"),
             (6912, 2560, "normal_bf16", None), (16, 48, "normal_f32", "relu2"),
             (4096, 512, "student_t3_bf16", None), (11008, 64, "normal_bf16", None),
             (2560, 3840, "normal_bf16", None)]


def _b3_layers(dev, bl, orc, M, shapes, seed0, gains=False):
    layers, refs = [], []
    for i, (K, N, kind, epi) in enumerate(shapes):
        W = wl.gen_weight(seed0 + 2 * i, N, K)
        X, is_bf16 = wl.gen_acts(seed0 + 2 * i + 1, M, K, kind)
        packed, gamma = bl.quantize_weights_b3(_gpu(W, dev))
        _, gc = orc.absmean(W)
        q = orc.ternarize(W, gc)
        Xt = _gpu(X, dev)
        Xt = Xt.view(torch.bfloat16) if is_bf16 else Xt
        g = wl.gen_gain(seed0 + 2 * i + 7, K) if (gains and i % 2 == 0) else None
        if g is None:
            y_ref, *_ = orc.forward(X, q, gc, bf16=is_bf16)
        else:
            qx, sx, _ = orc.quant_acts_rmsnorm(X, g, 1e-5, bf16=is_bf16)
            y_ref = orc.rescale(orc.int_matmul(qx, q), sx, gc)
        if epi == "relu2":
            y_ref = orc.relu2(y_ref)
        layers.append((Xt, packed, gamma, N, epi, None, None if g is None else _gpu(g, dev)))
        refs.append(y_ref)
    return layers, refs


def _fits_lds(M, K):
    # the skinny kernel holds M token rows of the padded K (plus 16 bytes)
    # and M x 2048 bytes of outputs in 160 KiB of LDS
    kp = (K + 319) // 320 * 320
    return M * (kp + 16) + M * 2048 <= 160 * 1024


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 16])
def test_group_b3_matches_oracle(dev, bl, orc, M):
    shapes = [s for s in B3_SHAPES if _fits_lds(M, s[0])]  # M = 16 drops K = 11008
    layers, refs = _b3_layers(dev, bl, orc, M, shapes, 9400 + 10 * M)
    g = bl.Group(layers, fmt="b3")
    first = [y.clone() for y in g.forward()]
    torch.cuda.synchronize()
    for i, (y, y_ref) in enumerate(zip(first, refs)):
        got = y.cpu().numpy()
        assert np.array_equal(got, y_ref), f"layer {i}: {np.count_nonzero(got != y_ref)} differ"
    for y0, y1 in zip(first, g.forward()):  # the queue is back at zero
        assert torch.equal(y0, y1)


@pytest.mark.parametrize("M", [1, 4])
def test_group_b3_subln(dev, bl, orc, M):
    # layers with and without a subln gain; scales within 2^-22 move nothing
    # here (the codes are exact), outputs within the 1e-6 bar
    layers, refs = _b3_layers(dev, bl, orc, M, B3_SHAPES[:4], 9600 + M, gains=True)
    g = bl.Group(layers, fmt="b3")
    outs = g.forward()
    torch.cuda.synchronize()
    for i, (y, y_ref) in enumerate(zip(outs, refs)):
        got = y.cpu().numpy().astype(np.float64)
        ref = y_ref.astype(np.float64)
        rel = np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)
        assert np.all((rel <= 1e-6) | ((got == 0) & (ref == 0))), i


@pytest.mark.parametrize("M", [1, 4, 16])
def test_group_b3_glu(dev, bl, orc, M):
    K, N = 2560, 1024
    W = wl.gen_weight(9700 + M, N, K)
    X, _ = wl.gen_acts(9701 + M, M, K, "normal_bf16")
    packed, gamma = bl.quantize_weights_b3(_gpu(W, dev), glu=True)
    _, gc = orc.absmean(W)
    q = orc.ternarize(W, gc)
    y_ref, *_ = orc.forward(X, q, gc, bf16=True)
    h_ref = orc.glu_relu2(y_ref)
    Xt = _gpu(X, dev).view(torch.bfloat16)
    g = bl.Group([(Xt, packed, gamma, N, "relu2_glu", None)], fmt="b3")
    h = g.forward()[0]
    torch.cuda.synchronize()
    assert np.array_equal(h.cpu().numpy(), h_ref)


def test_group_b3_mixed_formats_rejected(dev, bl):
    import ctypes

    X = torch.zeros((1, 512), dtype=torch.bfloat16, device=dev)
    Y = torch.zeros((1, 16), dtype=torch.float32, device=dev)
    gamma = torch.ones(1, dtype=torch.float32, device=dev)
    p3 = torch.zeros(bl.packed_bytes_b3(16, 512), dtype=torch.uint8, device=dev)
    p2 = torch.zeros(bl.packed_bytes(16, 512), dtype=torch.uint8, device=dev)
    ops = (bl.GroupOp * 2)()
    for i, (fmt, p) in enumerate([("b3", p3), ("2bit", p2)]):
        ops[i] = bl.GroupOp(X.data_ptr(), bl._dtype_code(X), bl.EPI[None], 512, 16, p.data_ptr(),
                            gamma.data_ptr(), Y.data_ptr(), None, 0.0, bl.FMT[fmt])
    handle = ctypes.c_void_p()
    with pytest.raises(bl.BitLinearError, match="same weight format"):
        bl.check(bl.lib().bitlinear_group_create(ops, 2, 1, None, 0, ctypes.byref(handle)),
                 "bitlinear_group_create")


def test_group_b3_errors(dev, bl):
    X = torch.zeros((17, 320), dtype=torch.bfloat16, device=dev)
    packed = torch.zeros(16 * 320 // 5, dtype=torch.uint8, device=dev)
    gamma = torch.ones(1, dtype=torch.float32, device=dev)
    with pytest.raises(bl.BitLinearError, match="base-3"):
        bl.Group([(X, packed, gamma, 16, None, None)], fmt="b3")  # M > 16
    # K = 11008 pads to 11200: 16 token rows of it exceed LDS
    assert not _fits_lds(16, 11008) and _fits_lds(8, 11008)
    X16 = torch.zeros((16, 11008), dtype=torch.bfloat16, device=dev)
    p16 = torch.zeros(bl.packed_bytes_b3(16, 11008), dtype=torch.uint8, device=dev)
    with pytest.raises(bl.BitLinearError, match="LDS"):
        bl.Group([(X16, p16, gamma, 16, None, None)], fmt="b3")
