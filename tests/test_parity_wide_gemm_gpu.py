"""Parity of the prefill GEMM's 128x256 tiles (four waves of 64x128, two
workgroups per CU) with the CPU oracle, through the C ABI.

The library takes these tiles for one layer above 64 tokens when they make
one round that every CU joins and that fills at least three quarters of the
CUs' resident slots (two per CU).  On a 256-CU MI355X (512 slots) the shapes
below do: 2048 x 6400 (400 tiles), 2000 x 6160 (400, ragged rows and a last
column tile of 16 columns), 2048 x 6144 (384, the least that qualifies),
2048 x 6912 (432, the 2B prefill up projection).  Every output
element is compared on the smaller shapes, through the debug kernel (int32
accumulators too) and the plain one (forward_q), with the plain, squared-ReLU
and gated epilogues.  Expected values come only from the oracle.
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


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


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


def _weights(bl, orc, seed, N, K, dev, glu=False):
    W = wl.gen_weight(seed, N, K)
    packed, gamma = bl.quantize_weights(_gpu(W, dev), glu=glu)
    p_ref, gc, qw = orc.quantize_weights(W)
    assert gamma.cpu().numpy()[0] == gc
    assert np.array_equal(packed.cpu().numpy(), orc.pack_glu(qw) if glu else p_ref)
    return packed, gamma, qw, gc


@pytest.mark.parametrize("M,K,N,kind,epi", [(2048, 256, 6400, "normal_bf16", None),
                                            (2000, 512, 6160, "outlier_bf16", "relu2"),
                                            (2048, 768, 6144, "student_t3_bf16", None)])
def test_wide_tiles_every_element(dev, bl, orc, M, K, N, kind, epi):
    packed, gamma, qw, gc = _weights(bl, orc, 20100 + N + K, N, K, dev)
    X, is_bf16 = wl.gen_acts(20200 + M + K, M, K, kind)
    Xt = _acts_gpu(X, is_bf16, dev)
    Y, dbg = bl.forward(Xt, packed, gamma, N, epilogue=epi, debug=True)
    y_ref, xq, sx, acc = orc.forward(X, qw, gc, bf16=is_bf16)
    if epi == "relu2":
        y_ref = orc.relu2(y_ref)
    assert np.array_equal(dbg["xq"].cpu().numpy(), xq)
    a = dbg["acc"].cpu().numpy()
    assert np.array_equal(a, acc), f"{np.count_nonzero(a != acc)} accumulators differ"
    y = Y.cpu().numpy()
    assert _rel(y, y_ref) <= REL_TOL
    assert np.array_equal(y, y_ref), f"{np.count_nonzero(y != y_ref)} outputs differ"
    # the plain (no debug outputs) kernel from the same int8 rows, twice
    Xq, sxg, rs = bl.quantize_acts(Xt)
    for _ in range(2):
        Yq = bl.forward_q(Xq, sxg, rs, packed, gamma, N, epilogue=epi)
        assert np.array_equal(Yq.cpu().numpy(), y_ref)


def test_wide_tiles_gated_epilogue(dev, bl, orc):
    M, K, N = 2048, 512, 6400
    packed, gamma, qw, gc = _weights(bl, orc, 20300, N, K, dev, glu=True)
    X, _ = wl.gen_acts(20301, M, K, "normal_bf16")
    Xt = _acts_gpu(X, True, dev)
    y_full, *_ = orc.forward(X, qw, gc, bf16=True)
    h_ref = orc.glu_relu2(y_full)
    Y, dbg = bl.forward(Xt, packed, gamma, N, epilogue="relu2_glu", debug=True)
    assert Y.shape == (M, N // 2)
    h = Y.cpu().numpy()
    assert _rel(h, h_ref) <= REL_TOL
    assert np.array_equal(h, h_ref)
    Xq, sx, rs = bl.quantize_acts(Xt)
    assert np.array_equal(bl.forward_q(Xq, sx, rs, packed, gamma, N,
                                       epilogue="relu2_glu").cpu().numpy(), h_ref)


def test_wide_tiles_prefill_up_projection_every_tile(dev, bl, orc):
    # 2048 x 2560 -> 6912, the 2B prefill up projection: two rows of every
    # 128-row tile (its first and last), every column.
    M, K, N = 2048, 2560, 6912
    packed, gamma, qw, gc = _weights(bl, orc, 20400, N, K, dev)
    X, _ = wl.gen_acts(20401, M, K, "outlier_bf16")
    Xq, sx, rs = bl.quantize_acts(_acts_gpu(X, True, dev))
    Y = bl.forward_q(Xq, sx, rs, packed, gamma, N)
    rows = np.unique(np.concatenate([np.arange(0, M, 128), np.arange(127, M, 128)]))
    y_ref, *_ = orc.forward(X[rows], qw, gc, bf16=True)
    y = Y.cpu().numpy()[rows]
    assert _rel(y, y_ref) <= REL_TOL
    assert np.array_equal(y, y_ref)


@pytest.mark.parametrize("M,K,N", [(512, 4096, 22016), (1536, 2560, 6912)])
def test_fewer_wide_tiles_take_square_tiles(dev, bl, orc, M, K, N):
    # 344 and 324 128x256 tiles fill under three quarters of the 512 slots,
    # so these run on 128x128 tiles (688 and 648 of them, one round, no
    # pieces): two rows of every 128-row tile, every column.
    packed, gamma, qw, gc = _weights(bl, orc, 20500 + M, N, K, dev)
    X, _ = wl.gen_acts(20501 + M, M, K, "student_t3_bf16")
    Xq, sx, rs = bl.quantize_acts(_acts_gpu(X, True, dev))
    Y = bl.forward_q(Xq, sx, rs, packed, gamma, N)
    rows = np.unique(np.concatenate([np.arange(0, M, 128), np.arange(127, M, 128)]))
    y_ref, *_ = orc.forward(X[rows], qw, gc, bf16=True)
    y = Y.cpu().numpy()[rows]
    assert _rel(y, y_ref) <= REL_TOL
    assert np.array_equal(y, y_ref)
