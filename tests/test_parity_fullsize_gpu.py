"""Full-size parity of the steps the decode and prefill measurements time.

- The whole 2B decode step: 30 layers x (QKV 2560->3840, O 2560->2560,
  gate+up 2560->13824, down 6912->2560) = 120 linears, 2.08 G weights, as
  one grouped forward at M = 1, 4 and 16 (the persistent kernel with its
  static ranges and shared queue, in the launch configuration the bench
  times), and at M = 1 with every linear in the base-3 layout.
- The whole 7B-like step: 32 layers x (QKV 4096->12288, O 4096->4096,
  gate+up 4096->22016, down 11008->4096) = 128 linears, 6.5 G weights with
  30% near-zero entries, Student-t(3) activations, at M = 1 (skinny kernel)
  and M = 64 (quantization launch + one persistent tiled GEMM).
- Prefill GEMMs at M = 2048 and the 7B linears at M = 512 on stratified rows:
  every 128-row tile contributes rows, compared over all N columns, so every
  output tile (including those cut along K) has checked rows.

Every output element of the grouped steps is compared with the oracle, bit
for bit (the 1e-6 relative bar is asserted as well).  Per linear, gamma must
equal the oracle's and the packed weights must unpack to the oracle's ternary
values.  Weights are drawn on the GPU by torch's seeded generator
(workloads.gen_weight_device) and copied to the host for the oracle;
activations come from the numpy generators.  Expected values come only from
the oracle.
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


def _rel_err(y, ref):
    y = y.astype(np.float64)
    ref = ref.astype(np.float64)
    d = np.abs(y - ref)
    den = np.abs(ref)
    assert not ((den == 0) & (d != 0)).any(), "nonzero result where the oracle has an exact zero"
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.where(den > 0, d / den, 0.0)
    return float(r.max()) if r.size else 0.0


class Step:
    """Packed weights of every linear of one step (on the GPU) and their
    ternary values and scales from the oracle (on the host)."""

    def __init__(self, dev, bl, orc, key):
        wk = wl.WORKLOADS[key]
        self.key, self.wk = key, wk
        self.linears = []  # (layer, index, shape, packed, gamma, q_w, gamma_c)
        for layer, li, shape in wl.step_linears(wk):
            W = wl.gen_weight_device(wl.weight_seed(key, layer, li), shape.N, shape.K,
                                     wk.weight_sparse_frac, dev)
            packed, gamma = bl.quantize_weights(W)
            Wh = W.cpu().numpy()
            del W
            _, gc = orc.absmean(Wh)
            q = orc.ternarize(Wh, gc)
            del Wh
            assert gamma.cpu().numpy()[0] == gc, (layer, li)
            back = bl.unpack_ternary(packed, shape.N, shape.K)
            assert torch.equal(back, torch.from_numpy(q).to(dev)), (layer, li)
            del back
            self.linears.append((layer, li, shape, packed, gamma, q, gc))
        torch.cuda.synchronize()

    def check_grouped(self, dev, bl, orc, M, fmt=None):
        layers, refs = [], []
        for layer, li, shape, packed, gamma, q, gc in self.linears:
            X, is_bf16 = wl.gen_acts(wl.act_seed(self.key, layer, li) + 100 * M, M, shape.K,
                                     self.wk.x_kind)
            assert is_bf16
            Xt = torch.from_numpy(X).to(dev).view(torch.bfloat16)
            if fmt == "b3":
                # the same codes in the base-3 layout, packed on the GPU and
                # checked byte for byte against the oracle's packing
                packed = bl.pack_ternary_b3(torch.from_numpy(q).to(dev))
                assert np.array_equal(packed.cpu().numpy(), orc.pack_b3(q)), (layer, li)
            layers.append((Xt, packed, gamma, shape.N, None, None))
            refs.append((X, q, gc))
        g = bl.Group(layers, fmt=fmt)
        first = [y.clone() for y in g.forward()]
        torch.cuda.synchronize()
        worst = 0.0
        for i, ((X, q, gc), y) in enumerate(zip(refs, first)):
            y_ref, *_ = orc.forward(X, q, gc, bf16=True)
            got = y.cpu().numpy()
            worst = max(worst, _rel_err(got, y_ref))
            assert np.array_equal(got, y_ref), \
                f"linear {i}: {np.count_nonzero(got != y_ref)} outputs differ"
        assert worst <= REL_TOL
        # a second launch (the work queue's counters back at zero) gives the
        # same bits
        again = g.forward()
        torch.cuda.synchronize()
        for i, (y0, y1) in enumerate(zip(first, again)):
            assert torch.equal(y0, y1), f"linear {i} differs on the second launch"


@pytest.fixture(scope="module")
def step_2b(dev, bl, orc):
    return Step(dev, bl, orc, "decode_step_2b")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_step_2b_grouped_full(dev, bl, orc, step_2b, M):
    assert len(step_2b.linears) == 120
    step_2b.check_grouped(dev, bl, orc, M)


@pytest.mark.timeout(900)
def test_decode_step_2b_grouped_full_b3(dev, bl, orc, step_2b):
    # the whole 2B step with every linear in the base-3 layout (418.8 MB)
    step_2b.check_grouped(dev, bl, orc, 1, fmt="b3")
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def step_7b(dev, bl, orc):
    return Step(dev, bl, orc, "decode_prefill_7b")


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("M", [1, 64])
def test_decode_step_7b_grouped_full(dev, bl, orc, step_7b, M):
    assert len(step_7b.linears) == 128
    step_7b.check_grouped(dev, bl, orc, M)


def _stratified_rows(M, tile, per_tile, seed):
    rng = np.random.default_rng(seed)
    rows = [0, M - 1]
    for t0 in range(0, M, tile):
        hi = min(M, t0 + tile)
        rows += [t0, hi - 1] + list(rng.integers(t0, hi, per_tile))
    return np.unique(np.array(rows))


def _check_rows(dev, bl, orc, key, li, lin, M, rows, sparse):
    W = wl.gen_weight(wl.weight_seed(key, 0, li), lin.N, lin.K, sparse)
    X, is_bf16 = wl.gen_acts(wl.act_seed(key, 0, li), M, lin.K, wl.WORKLOADS[key].x_kind)
    packed, gamma = bl.quantize_weights(torch.from_numpy(W).to(dev))
    _, gc = orc.absmean(W)
    qw = orc.ternarize(W, gc)
    assert gamma.cpu().numpy()[0] == gc
    Xt = torch.from_numpy(X).to(dev)
    Xt = Xt.view(torch.bfloat16) if is_bf16 else Xt
    Y, dbg = bl.forward(Xt, packed, gamma, lin.N, debug=True)
    xq_ref, sx_ref, _ = orc.quant_acts(X, bf16=is_bf16)
    assert np.array_equal(dbg["xq"].cpu().numpy(), xq_ref)
    assert np.array_equal(dbg["x_scale"].cpu().numpy(), sx_ref)
    acc_ref = orc.int_matmul(xq_ref[rows], qw)
    y_ref = orc.rescale(acc_ref, sx_ref[rows], gc)
    acc = dbg["acc"].cpu().numpy()[rows]
    y = Y.cpu().numpy()[rows]
    assert np.array_equal(acc, acc_ref), f"{np.count_nonzero(acc != acc_ref)} accumulators differ"
    assert _rel_err(y, y_ref) <= REL_TOL
    assert np.array_equal(y, y_ref)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("li", [0, 1])
def test_prefill_m2048_stratified(dev, bl, orc, li):
    key = "prefill_m2048"
    lin = wl.WORKLOADS[key].linears[li]
    rows = _stratified_rows(2048, 128, 3, 40 + li)
    assert len(rows) >= 16 * 3
    _check_rows(dev, bl, orc, key, li, lin, 2048, rows, 0.0)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("li", [0, 1, 2, 3])
def test_7b_m512_stratified(dev, bl, orc, li):
    key = "decode_prefill_7b"
    lin = wl.LAYER_7B[li]
    rows = _stratified_rows(512, 64, 3, 50 + li)
    _check_rows(dev, bl, orc, key, li, lin, 512, rows, 0.3)
