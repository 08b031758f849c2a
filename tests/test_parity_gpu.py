"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer and byte results (packed weights, int8 activations, int32
accumulators) must be bit-identical.  Float results (gamma, scales, Y) are
designed to be bit-identical too (same IEEE operations in the same order); the
contract bar for Y is a max relative error of 1e-6, asserted here, and exact
equality is asserted separately.

Inputs come from w1_a8_matmul_amd.workloads (seeded, synthetic); expected
values come only from the oracle.
"""
import numpy as np
import pytest

import oracle
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


def _rel_err(y, ref):
    y = y.astype(np.float64)
    ref = ref.astype(np.float64)
    d = np.abs(y - ref)
    den = np.abs(ref)
    bad_zero = (den == 0) & (d != 0)
    assert not bad_zero.any(), "nonzero result where the oracle has an exact zero"
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.where(den > 0, d / den, 0.0)
    return float(r.max()) if r.size else 0.0


def _quantize_both(bl, orc, W, dev):
    packed, gamma = bl.quantize_weights(_gpu(W, dev))
    p_ref, g_ref, q_ref = orc.quantize_weights(W)
    p = packed.cpu().numpy()
    g = gamma.cpu().numpy()[0]
    assert g == g_ref, (g, g_ref)
    assert np.array_equal(p, p_ref), f"{np.count_nonzero(p != p_ref)} packed bytes differ"
    return packed, gamma, q_ref, g_ref


# ---------------------------------------------------------------------------
# weights: gamma, ternary codes, packing
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,K,seed,sparse", [(256, 256, 1001, 0.0), (16, 256, 7, 0.0),
                                             (48, 768, 8, 0.0), (2560, 6912, 1013, 0.0),
                                             (6912, 2560, 9, 0.3)])
def test_quantize_weights_bit_exact(dev, bl, orc, N, K, seed, sparse):
    W = wl.gen_weight(seed, N, K, sparse)
    _quantize_both(bl, orc, W, dev)


def test_quantize_weights_special_matrices(dev, bl, orc):
    # all zero: gamma = 1e-5, every code 1
    _, gamma, q, g = _quantize_both(bl, orc, np.zeros((32, 512), np.float32), dev)
    assert g == np.float32(1e-5) and np.all(q == 0)
    # two-valued: gamma = c exactly, q = sign
    c = np.float32(0.0625)
    W = np.where(np.random.default_rng(3).random((16, 256)) < 0.5, c, -c).astype(np.float32)
    _, _, q, g = _quantize_both(bl, orc, W, dev)
    assert g == c and np.array_equal(q, np.sign(W).astype(np.int8))
    # exact ties at gamma/2 (w/gamma = 0.5 rounds to 0, 1.5 rounds to 2 -> 1)
    row = np.array([4, 1, -1, 2, 3, -3, 0, 1] * 32, np.float32)  # mean |w| = 15/8
    W = np.tile(row, (16, 1))
    _quantize_both(bl, orc, W, dev)
    # a huge dynamic range within one matrix
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((64, 1024)) * np.exp2(rng.integers(-40, 20, (64, 1024)))).astype(np.float32)
    _quantize_both(bl, orc, W, dev)


def test_quantize_weights_7b_gate_up(dev, bl, orc):
    # the largest matrix of the 7B-like workload: 22016 x 4096 (360 MB fp32)
    W = wl.gen_weight(wl.weight_seed("decode_prefill_7b", 0, 2), 22016, 4096, 0.3)
    _quantize_both(bl, orc, W, dev)


@pytest.mark.parametrize("N,K", [(16, 256), (64, 1280), (272, 2560)])
def test_pack_unpack(dev, bl, orc, N, K):
    rng = np.random.default_rng(N + K)
    q = rng.integers(-1, 2, (N, K)).astype(np.int8)
    packed = bl.pack_ternary(_gpu(q, dev))
    assert np.array_equal(packed.cpu().numpy(), orc.pack(q))
    back = bl.unpack_ternary(packed, N, K)
    assert np.array_equal(back.cpu().numpy(), q)
    # values outside {-1,0,1} are clamped
    q2 = rng.integers(-128, 128, (N, K)).astype(np.int8)
    p2 = bl.pack_ternary(_gpu(q2, dev))
    assert np.array_equal(p2.cpu().numpy(), orc.pack(np.clip(q2, -1, 1)))


# ---------------------------------------------------------------------------
# activations
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,kind", [(4, 256, "normal_f32"), (1, 2560, "normal_bf16"),
                                      (16, 6912, "normal_bf16"), (2048, 2560, "outlier_bf16"),
                                      (64, 11008, "student_t3_bf16"), (3, 4096, "normal_f32"),
                                      # one-pass rows up to 16384 columns (ragged past 12288),
                                      # the two-pass loop beyond
                                      (2, 12304, "student_t3_bf16"), (5, 16384, "normal_bf16"),
                                      (3, 16400, "normal_f32"), (2, 20480, "normal_bf16")])
def test_quantize_acts_bit_exact(dev, bl, orc, M, K, kind):
    X, is_bf16 = wl.gen_acts(M * 7 + K, M, K, kind)
    if not is_bf16:
        X[0] *= 1000.0
        if M > 2:
            X[2] = 0.0
    Xq, sx, rs = bl.quantize_acts(_acts_gpu(X, is_bf16, dev))
    q_ref, s_ref, r_ref = orc.quant_acts(X, bf16=is_bf16)
    assert np.array_equal(Xq.cpu().numpy(), q_ref)
    assert np.array_equal(sx.cpu().numpy(), s_ref)
    assert np.array_equal(rs.cpu().numpy(), r_ref)


def test_quantize_acts_ties_and_tiny(dev, bl, orc):
    X = np.zeros((4, 256), np.float32)
    X[0, :10] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 127, 3, -127, 0]
    X[1, 3] = 3e-6          # below the 1e-5 guard
    X[3] = np.linspace(-1, 1, 256, dtype=np.float32)
    Xq, sx, rs = bl.quantize_acts(_gpu(X, dev))
    q_ref, s_ref, r_ref = orc.quant_acts(X)
    assert np.array_equal(Xq.cpu().numpy(), q_ref)
    assert np.array_equal(sx.cpu().numpy(), s_ref)
    assert np.array_equal(rs.cpu().numpy(), r_ref)


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------
def _check_forward(dev, bl, orc, M, K, N, x_kind, seed, epilogue=None, sparse=0.0,
                   rows=None):
    """Runs the GPU forward with debug outputs and compares with the oracle.
    rows: if given, the accumulators and outputs are compared on those token
    rows only (the int8 activations and scales are compared on all rows)."""
    W = wl.gen_weight(seed, N, K, sparse)
    X, is_bf16 = wl.gen_acts(seed + 5, M, K, x_kind)
    packed, gamma, qw, gc = _quantize_both(bl, orc, W, dev)
    Y, dbg = bl.forward(_acts_gpu(X, is_bf16, dev), packed, gamma, N, epilogue=epilogue,
                        debug=True)
    xq_ref, sx_ref, _ = orc.quant_acts(X, bf16=is_bf16)
    assert np.array_equal(dbg["xq"].cpu().numpy(), xq_ref)
    assert np.array_equal(dbg["x_scale"].cpu().numpy(), sx_ref)
    if rows is None:
        rows = np.arange(M)
    acc_ref = orc.int_matmul(xq_ref[rows], qw)
    y_ref = orc.rescale(acc_ref, sx_ref[rows], gc)
    if epilogue == "relu2":
        y_ref = orc.relu2(y_ref)
    acc = dbg["acc"].cpu().numpy()[rows]
    y = Y.cpu().numpy()[rows]
    assert np.array_equal(acc, acc_ref), f"{np.count_nonzero(acc != acc_ref)} accumulators differ"
    assert _rel_err(y, y_ref) <= REL_TOL
    assert np.array_equal(y, y_ref), f"{np.count_nonzero(y != y_ref)} outputs not bit-identical"
    return Y, y_ref


def test_forward_single_bitlinear_m4(dev, bl, orc):
    # single BitLinear, M=4, K=256, N=256, fp32 weights and activations
    w = wl.WORKLOADS["bitlinear_m4_k256_n256"]
    _check_forward(dev, bl, orc, 4, 256, 256, w.x_kind, wl.weight_seed(w.key, 0, 0))


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 15, 16, 17, 33, 64, 100, 129])
@pytest.mark.parametrize("K,N", [(256, 16), (768, 272), (2560, 256)])
def test_forward_ragged_shapes(dev, bl, orc, M, K, N):
    _check_forward(dev, bl, orc, M, K, N, "normal_bf16", 5000 + M * 31 + K + N)


@pytest.mark.parametrize("M", [1, 4, 16, 64])
def test_forward_relu2_epilogue(dev, bl, orc, M):
    _check_forward(dev, bl, orc, M, 2560, 1024, "normal_bf16", 6000 + M, epilogue="relu2")


def test_forward_degenerate_rows(dev, bl, orc):
    for M in (3, 40):
        W = wl.gen_weight(77, 64, 512)
        W[5] = 0.0
        X = wl.gen_acts_f32(78, M, 512, "normal")
        X[1] = 0.0
        packed, gamma, qw, gc = _quantize_both(bl, orc, W, dev)
        Y = bl.forward(_gpu(X, dev), packed, gamma, 64).cpu().numpy()
        y_ref, *_ = orc.forward(X, qw, gc)
        assert np.array_equal(Y, y_ref)
        assert np.all(Y[:, 5] == 0) and np.all(Y[1] == 0)
    # all-zero weights: every output is +0
    packed, gamma, qw, gc = _quantize_both(bl, orc, np.zeros((32, 256), np.float32), dev)
    X = wl.gen_acts_f32(79, 4, 256, "normal")
    Y = bl.forward(_gpu(X, dev), packed, gamma, 32).cpu().numpy()
    assert np.all(Y == 0)


def test_forward_m0_is_noop(dev, bl):
    X = torch.empty((0, 256), dtype=torch.bfloat16, device=dev)
    packed = torch.zeros(16 * 256 // 4, dtype=torch.uint8, device=dev)
    gamma = torch.ones(1, dtype=torch.float32, device=dev)
    Y = bl.forward(X, packed, gamma, 16)
    assert Y.shape == (0, 16)


def test_forward_q_matches_forward(dev, bl, orc):
    for M in (1, 4, 37):
        W = wl.gen_weight(90 + M, 256, 2560)
        X, _ = wl.gen_acts(91 + M, M, 2560, "normal_bf16")
        packed, gamma, qw, gc = _quantize_both(bl, orc, W, dev)
        Xt = _acts_gpu(X, True, dev)
        Y = bl.forward(Xt, packed, gamma, 256)
        Xq, sx, rs = bl.quantize_acts(Xt)
        Yq = bl.forward_q(Xq, sx, rs, packed, gamma, 256)
        assert torch.equal(Y, Yq)


def test_decode_gemv_pair_chain(dev, bl, orc):
    # up 2560->6912 with ReLU^2, then down 6912->2560 on the float result
    key = "decode_gemv_pair_m1"
    up, down = wl.WORKLOADS[key].linears
    Wu = wl.gen_weight(wl.weight_seed(key, 0, 0), up.N, up.K)
    Wd = wl.gen_weight(wl.weight_seed(key, 0, 1), down.N, down.K)
    X, _ = wl.gen_acts(wl.act_seed(key, 0, 0), 1, up.K, "normal_bf16")
    pu, gu, qu, gcu = _quantize_both(bl, orc, Wu, dev)
    pd, gd, qd, gcd = _quantize_both(bl, orc, Wd, dev)
    H = bl.forward(_acts_gpu(X, True, dev), pu, gu, up.N, epilogue="relu2")
    Y, dbg = bl.forward(H, pd, gd, down.N, debug=True)
    y_up, *_ = orc.forward(X, qu, gcu, bf16=True)
    h_ref = orc.relu2(y_up)
    y_ref, xq_ref, sx_ref, acc_ref = orc.forward(h_ref, qd, gcd)
    assert np.array_equal(H.cpu().numpy(), h_ref)
    assert np.array_equal(dbg["xq"].cpu().numpy(), xq_ref)
    assert np.array_equal(dbg["acc"].cpu().numpy(), acc_ref)
    assert _rel_err(Y.cpu().numpy(), y_ref) <= REL_TOL
    assert np.array_equal(Y.cpu().numpy(), y_ref)


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("li", [0, 1, 2, 3])
def test_decode_step_2b_linears(dev, bl, orc, M, li):
    key = "decode_step_2b"
    lin = wl.LAYER_2B[li]
    _check_forward(dev, bl, orc, M, lin.K, lin.N, "normal_bf16", wl.weight_seed(key, 0, li))


@pytest.mark.parametrize("li", [0, 1])
def test_prefill_m2048_sampled(dev, bl, orc, li):
    key = "prefill_m2048"
    lin = wl.WORKLOADS[key].linears[li]
    rows = np.unique(np.concatenate([[0, 1, 2047], np.random.default_rng(li).integers(0, 2048, 45)]))
    _check_forward(dev, bl, orc, 2048, lin.K, lin.N, "outlier_bf16", wl.weight_seed(key, 0, li),
                   rows=rows)


@pytest.mark.parametrize("M", [1, 64, 512])
@pytest.mark.parametrize("li", [0, 1, 2, 3])
def test_7b_linears(dev, bl, orc, M, li):
    key = "decode_prefill_7b"
    lin = wl.LAYER_7B[li]
    rows = None
    if M > 64:
        rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(M + li).integers(0, M, 14)]))
    _check_forward(dev, bl, orc, M, lin.K, lin.N, "student_t3_bf16", wl.weight_seed(key, 0, li),
                   sparse=0.3, rows=rows)


# ---------------------------------------------------------------------------
# grouped decode forward
# ---------------------------------------------------------------------------
GROUP_SHAPES = [(256, 16, "normal_f32", None), (2560, 272, "normal_bf16", "relu2"),
                (6912, 2560, "normal_bf16", None), (768, 48, "normal_f32", "relu2"),
                (4096, 512, "student_t3_bf16", None), (11008, 64, "normal_bf16", None),
                (12288, 32, "normal_bf16", None)]


def _group_layers(dev, bl, orc, M, shapes, seed0):
    layers, refs = [], []
    for i, (K, N, kind, epi) in enumerate(shapes):
        W = wl.gen_weight(seed0 + 2 * i, N, K)
        X, is_bf16 = wl.gen_acts(seed0 + 2 * i + 1, M, K, kind)
        packed, gamma, qw, gc = _quantize_both(bl, orc, W, dev)
        Xt = _acts_gpu(X, is_bf16, dev)
        y_ref, *_ = orc.forward(X, qw, gc, bf16=is_bf16)
        if epi == "relu2":
            y_ref = orc.relu2(y_ref)
        layers.append((Xt, packed, gamma, N, epi, None))
        refs.append(y_ref)
    return layers, refs


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 11])
def test_group_forward_matches_oracle(dev, bl, orc, M):
    layers, refs = _group_layers(dev, bl, orc, M, GROUP_SHAPES, 7000 + 100 * M)
    g = bl.Group(layers)
    outs = [y.clone() for y in g.forward()]
    torch.cuda.synchronize()
    for (Xt, packed, gamma, N, epi, _), y, y_ref in zip(layers, outs, refs):
        assert np.array_equal(y.cpu().numpy(), y_ref)
        single = bl.forward(Xt, packed, gamma, N, epilogue=epi)
        assert torch.equal(single, y)
    again = g.forward()
    for y, y2 in zip(outs, again):
        assert torch.equal(y, y2)


@pytest.mark.parametrize("M", [4, 16])
def test_group_2b_layer(dev, bl, orc, M):
    # one 2B-shape layer (QKV, O, gate+up, down) at the decode step's token counts
    shapes = [(l.K, l.N, "normal_bf16", None) for l in wl.LAYER_2B]
    layers, refs = _group_layers(dev, bl, orc, M, shapes, 7800 + M)
    g = bl.Group(layers)
    outs = g.forward()
    torch.cuda.synchronize()
    for y, y_ref in zip(outs, refs):
        assert np.array_equal(y.cpu().numpy(), y_ref)


@pytest.mark.parametrize("M", [17, 64, 130])
def test_group_gemm_matches_oracle(dev, bl, orc, M):
    # above 16 tokens a group runs as one persistent tiled GEMM over all layers
    shapes = [(256, 16, "normal_f32", None), (2560, 272, "normal_bf16", "relu2"),
              (6912, 2560, "normal_bf16", None), (4096, 512, "student_t3_bf16", None),
              (12544, 48, "normal_bf16", None)]
    layers, refs = _group_layers(dev, bl, orc, M, shapes, 7300 + M)
    g = bl.Group(layers)
    outs = [y.clone() for y in g.forward()]
    torch.cuda.synchronize()
    for (Xt, packed, gamma, N, epi, _), y, y_ref in zip(layers, outs, refs):
        assert np.array_equal(y.cpu().numpy(), y_ref)
    for y, y2 in zip(outs, g.forward()):
        assert torch.equal(y, y2)


def test_group_2b_layer_graph_replay(dev, bl, orc):
    shapes = [(l.K, l.N, "normal_bf16", None) for l in wl.LAYER_2B]
    layers, refs = _group_layers(dev, bl, orc, 1, shapes, 7900)
    g = bl.Group(layers)
    g.forward()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g.forward()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        g.forward()
    for rep in range(3):
        for y in g.outputs:
            y.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for y, y_ref in zip(g.outputs, refs):
            assert np.array_equal(y.cpu().numpy(), y_ref), f"replay {rep}"


def test_prefill_repeatable(dev, bl, orc):
    # The prefill kernel pipelines copies into LDS across waves; repeated runs
    # of a large shape must give identical bits (a missed wait shows up as
    # run-to-run differences) and match the oracle on sampled rows.
    M, K, N = 1024, 6912, 2560
    W = wl.gen_weight(8101, N, K)
    X, _ = wl.gen_acts(8102, M, K, "normal_bf16")
    packed, gamma, qw, gc = _quantize_both(bl, orc, W, dev)
    Xt = _acts_gpu(X, True, dev)
    first = bl.forward(Xt, packed, gamma, N)
    for _ in range(8):
        assert torch.equal(bl.forward(Xt, packed, gamma, N), first)
    rows = np.array([0, 1, 511, 777, 1023])
    xq, sx, _ = orc.quant_acts(X[rows], bf16=True)
    y_ref = orc.rescale(orc.int_matmul(xq, qw), sx, gc)
    assert np.array_equal(first.cpu().numpy()[rows], y_ref)


# ---------------------------------------------------------------------------
# prefill GEMM: the last, partial round of tiles shared along K
# ---------------------------------------------------------------------------
SPLIT_SHAPES = [
    (2048, 2560, 6912),   # 864 tiles of 128x128: a partial last round
    (2048, 6912, 2560),   # 320 tiles
    (512, 4096, 22016),   # 688 tiles
    (300, 2816, 1040),    # fewer tiles than compute units; ragged M and N; 22 steps
    (130, 256, 16),       # two ragged tiles of two steps
    (4096, 256, 4096),    # 1024 tiles: whole rounds only
]


@pytest.mark.parametrize("M,K,N", SPLIT_SHAPES)
def test_forward_q_split_remainder(dev, bl, orc, M, K, N):
    # int32 partial sums are exact in any order, so sharing tiles along K
    # gives the bits of one workgroup per tile; the tile counters return to
    # zero after every call (the same workspace is reused); sampled rows
    # match the oracle.
    W = wl.gen_weight(8200 + N % 97, N, K)
    X, _ = wl.gen_acts(8300 + M, M, K, "normal_bf16")
    packed, gamma, qw, gc = _quantize_both(bl, orc, W, dev)
    Xq, sx, rs = bl.quantize_acts(_acts_gpu(X, True, dev))
    plain = bl.forward_q(Xq, sx, rs, packed, gamma, N, split_remainder=False)
    ws = bl.forward_q_workspace(M, K, N, dev)
    for _ in range(3):
        assert torch.equal(bl.forward_q(Xq, sx, rs, packed, gamma, N, workspace=ws), plain)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(M).integers(0, M, 6)]))
    xq, sxr, _ = orc.quant_acts(X[rows], bf16=True)
    y_ref = orc.rescale(orc.int_matmul(xq, qw), sxr, gc)
    assert np.array_equal(plain.cpu().numpy()[rows], y_ref)


def test_forward_workspace_contents_do_not_matter(dev, bl, orc):
    # forward clears the GEMM's tile counters itself: a workspace full of
    # 0xff bytes gives the oracle's bits, with ReLU^2 and the debug outputs.
    M, K, N = 300, 2816, 1040
    W = wl.gen_weight(8401, N, K)
    X, _ = wl.gen_acts(8402, M, K, "outlier_bf16")
    packed, gamma, qw, gc = _quantize_both(bl, orc, W, dev)
    ws = torch.full((bl.workspace_bytes(M, K, N),), 0xFF, dtype=torch.uint8, device=dev)
    Y, dbg = bl.forward(_acts_gpu(X, True, dev), packed, gamma, N, epilogue="relu2",
                        debug=True, workspace=ws)
    y_ref, xq_ref, sx_ref, acc_ref = orc.forward(X, qw, gc, bf16=True)
    assert np.array_equal(dbg["acc"].cpu().numpy(), acc_ref)
    assert np.array_equal(Y.cpu().numpy(), orc.relu2(y_ref))


def test_forward_q_split_graph_replay(dev, bl, orc):
    # Replays of a captured call reuse the workspace; each must match eager.
    M, K, N = 2048, 2560, 6912
    W = wl.gen_weight(8501, N, K)
    X, _ = wl.gen_acts(8502, M, K, "normal_bf16")
    packed, gamma, qw, gc = _quantize_both(bl, orc, W, dev)
    Xq, sx, rs = bl.quantize_acts(_acts_gpu(X, True, dev))
    eager = bl.forward_q(Xq, sx, rs, packed, gamma, N, split_remainder=False)
    ws = bl.forward_q_workspace(M, K, N, dev)
    out = torch.empty((M, N), dtype=torch.float32, device=dev)
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        bl.forward_q(Xq, sx, rs, packed, gamma, N, out=out, workspace=ws)  # warm-up
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        bl.forward_q(Xq, sx, rs, packed, gamma, N, out=out, workspace=ws)
    for rep in range(4):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
