"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each group of tests names the reading (R1..R8 and R12, stated in oracle/bitlinear_oracle.c)
and what pins it: exact rational arithmetic, closed forms, hand-worked cases
from tests/golden/, invariants, a library routine, or brute force.  Sources:
"BitNet b1.58 2B4T Technical Report" card (ai-papers.xuzou.cn), Method
Adaptation; fishai news digest (news.fishai.com.cn/news/3455510), BitLinear
bullets; dignews.cc article, section 2.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from exact import exact_abs_sum, round_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS = np.float32(1e-5)


def _rng(seed):
    return np.random.default_rng(seed)


def _read_kv(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = v.split()
    return out


# --------------------------------------------------------------------------
# R1: gamma = mean |W| (absmean), fp64 sum, one rounding to float
# --------------------------------------------------------------------------
@pytest.mark.parametrize("shape,seed", [((16, 256), 1), ((64, 512), 2), ((48, 768), 3),
                                        ((256, 256), 4)])
def test_gamma_equals_exactly_rounded_mean(orc, shape, seed):
    W = _rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(0.02)
    g, gc = orc.absmean(W)
    exact = exact_abs_sum(W) / (shape[0] * shape[1])
    assert g == round_to_f32(exact)
    assert gc == g  # far above the 1e-5 guard


def test_gamma_wide_dynamic_range(orc):
    # values spanning many binades, so a float32 running sum would be wrong
    rng = _rng(11)
    W = (rng.standard_normal((32, 1024)) * np.exp2(rng.integers(-30, 10, (32, 1024)))).astype(np.float32)
    g, _ = orc.absmean(W)
    assert g == round_to_f32(exact_abs_sum(W) / W.size)


def test_gamma_large_matrix_within_half_ulp(orc):
    # 17.7M elements (the 2B FFN up-projection shape): a naive float32 sum
    # stalls; the fp64 sum keeps the mean within half an ulp of exact.
    W = _rng(5).standard_normal((6912, 2560), dtype=np.float32) * np.float32(0.02)
    g, _ = orc.absmean(W)
    exact = exact_abs_sum(W) / W.size
    assert abs(Fraction(float(g)) - exact) <= Fraction(float(np.spacing(g))) / 2 * Fraction(1001, 1000)


@pytest.mark.parametrize("j", [-20, -3, 1, 7, 30])
def test_gamma_power_of_two_scaling(orc, j):
    W = _rng(6).standard_normal((32, 256), dtype=np.float32)
    g0, _ = orc.absmean(W)
    g1, _ = orc.absmean(W * np.float32(2.0 ** j))
    assert g1 == np.float32(g0 * np.float32(2.0 ** j))
    gn, _ = orc.absmean(-W)
    assert gn == g0


def test_gamma_two_valued_matrix(orc):
    c = np.float32(0.0625)
    W = np.where(_rng(7).random((16, 512)) < 0.5, c, -c).astype(np.float32)
    g, gc = orc.absmean(W)
    assert g == c and gc == c


def test_gamma_all_zero_guard(orc):
    g, gc = orc.absmean(np.zeros((16, 256), np.float32))
    assert g == 0.0 and gc == EPS


def test_gamma_not_row_or_column_mean(orc):
    # rows with very different magnitudes: a per-row or per-column scale, or a
    # divide by K instead of N*K, cannot give this value
    W = np.ones((16, 256), np.float32)
    W[0] *= 17.0
    g, _ = orc.absmean(W)
    assert g == np.float32((17.0 * 256 + 15 * 256) / (16 * 256))


def test_gamma_gaussian_sanity(orc):
    W = _rng(8).standard_normal((512, 1024), dtype=np.float32) * np.float32(0.02)
    g, _ = orc.absmean(W)
    assert abs(g / 0.02 - np.sqrt(2 / np.pi)) < 0.005


# --------------------------------------------------------------------------
# R2: q_w = clamp(rint(W / gamma_c), -1, 1)
# --------------------------------------------------------------------------
def _closed_form_ternary(W, gc):
    # fl(|w|/g) rounds above 0.5 exactly when |w| > g*(0.5 + 2**-25); the
    # product is exact in double (24-bit x 25-bit significands).
    thr = np.float64(gc) * (0.5 + 2.0 ** -25)
    nz = np.abs(W.astype(np.float64)) > thr
    return (np.sign(W) * nz).astype(np.int8)


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_ternary_closed_form_random(orc, seed):
    W = _rng(seed).standard_normal((64, 512), dtype=np.float32) * np.float32(0.02)
    _, gc = orc.absmean(W)
    q = orc.ternarize(W, gc)
    assert np.array_equal(q, _closed_form_ternary(W, gc))
    assert set(np.unique(q)) <= {-1, 0, 1}


def test_ternary_closed_form_adversarial(orc):
    gc = np.float32(0.0173)
    half = np.float32(gc / np.float32(2))
    vals = [half, np.nextafter(half, np.float32(1)), np.nextafter(half, np.float32(0)),
            np.float32(gc * np.float32(1.5)), np.nextafter(np.float32(gc * np.float32(1.5)), np.float32(0)),
            gc, np.float32(0), np.float32(-0.0), np.float32(10.0)]
    vals += [np.float32(-v) for v in vals]
    for _ in range(200):
        vals.append(np.float32(half * np.float32(1 + _rng(len(vals)).integers(-4, 5) * 2.0 ** -23)))
    W = np.array(vals, np.float32).reshape(1, -1)
    q = orc.ternarize(W, gc)
    assert np.array_equal(q, _closed_form_ternary(W, gc))


def test_ternary_tie_golden(orc):
    kv = _read_kv("tie_cases.txt")
    row = np.array([float(v) for v in kv["weights"]], np.float32)
    W = np.tile(row, (16, 4))  # 16 x 16
    g, gc = orc.absmean(W)
    assert g == np.float32(float(kv["weights_gamma"][0]))
    q = orc.ternarize(W, gc)
    assert np.array_equal(q[0, :4], np.array([int(v) for v in kv["weights_q"]], np.int8))


def test_ternary_exact_values(orc):
    c = np.float32(0.25)
    base = _rng(9).integers(-1, 2, (16, 256)).astype(np.float32)
    W = base * c
    _, gc = orc.absmean(W)
    q = orc.ternarize(W, gc)
    # gamma = c * (fraction of nonzeros) <= c, so every nonzero w has |w/gamma| >= 1
    assert np.array_equal(q, base.astype(np.int8))


def test_ternary_sparse_fraction(orc):
    # Gaussian: P(|w| <= gamma/2) with gamma = sigma*sqrt(2/pi) is about 0.310
    W = _rng(10).standard_normal((256, 1024), dtype=np.float32)
    _, gc = orc.absmean(W)
    q = orc.ternarize(W, gc)
    assert abs(np.mean(q == 0) - 0.3101) < 0.005


# --------------------------------------------------------------------------
# R3: packing, four 2-bit codes per byte in 16x256 tiles
# --------------------------------------------------------------------------
def test_pack_positions_golden(orc):
    with open(os.path.join(GOLDEN, "pack_positions.txt")) as f:
        rows = [list(map(int, l.split())) for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) >= 10
    for N, K, n, k, byte, shift in rows:
        q = np.zeros((N, K), np.int8)
        q[n, k] = 1  # code 2 at (n, k), code 1 everywhere else
        p = orc.pack(q)
        expect = np.full(N * K // 4, 0x55, np.uint8)
        expect[byte] = (0x55 & ~(3 << shift)) | (2 << shift)
        assert np.array_equal(p, expect), (N, K, n, k)


@pytest.mark.parametrize("N,K", [(16, 256), (48, 768), (32, 2560)])
def test_pack_roundtrip_and_codes(orc, N, K):
    q = _rng(N + K).integers(-1, 2, (N, K)).astype(np.int8)
    p = orc.pack(q)
    assert p.size == N * K // 4 == orc.packed_bytes(N, K)
    for s in range(0, 8, 2):
        assert not np.any(((p >> s) & 3) == 3)
    assert np.array_equal(orc.unpack(p, N, K), q)


def test_pack_all_81_patterns_everywhere(orc):
    # every 4-tuple of ternary values at every (word, field) position
    pats = np.array(np.meshgrid(*[[-1, 0, 1]] * 4, indexing="ij")).reshape(4, -1).T  # 81 x 4
    N, K = 32, 512
    for off in range(0, 81, 17):
        q = np.roll(np.tile(pats.ravel(), N * K // pats.size + 1)[: N * K], off).reshape(N, K)
        q = q.astype(np.int8)
        assert np.array_equal(orc.unpack(orc.pack(q), N, K), q)


def test_pack_is_a_permutation_of_canonical_codes(orc):
    # the multiset of codes per 16-row tile equals that of the plain row-major
    # code stream of the same rows (the layout only permutes positions)
    q = _rng(31).integers(-1, 2, (32, 512)).astype(np.int8)
    p = orc.pack(q)
    codes = np.stack([(p >> s) & 3 for s in (0, 2, 4, 6)], axis=1).ravel()
    tile_bytes = 16 * 512 // 4
    for t in range(2):
        got = np.bincount(codes[t * tile_bytes * 4:(t + 1) * tile_bytes * 4], minlength=4)
        want = np.bincount((q[t * 16:(t + 1) * 16] + 1).ravel(), minlength=4)
        assert np.array_equal(got, want)


def test_pack_rejects_bad_input(orc):
    with pytest.raises(ValueError):
        orc.pack(np.zeros((15, 256), np.int8))
    with pytest.raises(ValueError):
        orc.pack(np.full((16, 256), 2, np.int8))
    bad = np.full(16 * 256 // 4, 0xFF, np.uint8)
    with pytest.raises(ValueError):
        orc.unpack(bad, 16, 256)


def test_offset_code_identity(orc):
    # sum(code*x) - sum(x) == sum(q*x): the offset codes lose nothing
    rng = _rng(33)
    q = rng.integers(-1, 2, (16, 256)).astype(np.int8)
    x = rng.integers(-127, 128, 256).astype(np.int64)
    code = q.astype(np.int64) + 1
    assert np.array_equal(code @ x - x.sum(), q.astype(np.int64) @ x)


def test_packed_size_matches_reported_footprint():
    kv = _read_kv("model_2b_footprint.txt")
    from w1_a8_matmul_amd.workloads import WORKLOADS

    wl = WORKLOADS["decode_step_2b"]
    assert wl.layers == int(kv["layers"][0])
    assert wl.weights_per_step == int(kv["weights"][0])
    assert wl.weights_per_step // 4 == int(kv["packed_bytes_2bit"][0])
    log2_3_mb = wl.weights_per_step * np.log2(3) / 8 / 1e6
    assert abs(log2_3_mb / float(kv["reported_mb"][0]) - 1) < 0.05


# --------------------------------------------------------------------------
# R4: per-token absmax int8 activations
# --------------------------------------------------------------------------
def _acts(seed, M, K, scale=1.0):
    return (_rng(seed).standard_normal((M, K), dtype=np.float32) * np.float32(scale))


@pytest.mark.parametrize("M,K,scale", [(4, 256, 1.0), (7, 2560, 3e-3), (3, 6912, 40.0)])
def test_acts_range_and_max(orc, M, K, scale):
    X = _acts(M * K, M, K, scale)
    X[0] *= np.float32(100.0)  # one loud token must not change the others
    q, s, r = orc.quant_acts(X)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    assert np.all(np.abs(q.astype(np.int32)).max(axis=1) == 127)  # per token, every row
    assert np.all((np.sign(q) == np.sign(X)) | (q == 0))
    assert np.array_equal(r, q.astype(np.int32).sum(axis=1))


@pytest.mark.parametrize("seed", [41, 42])
def test_acts_reconstruction_bound(orc, seed):
    X = _acts(seed, 8, 2560)
    q, s, _ = orc.quant_acts(X)
    a = np.abs(X).max(axis=1).astype(np.float64)
    assert np.all(s.astype(np.float64) == (a / 127).astype(np.float32).astype(np.float64))
    err = np.abs(X.astype(np.float64) - q.astype(np.float64) * s[:, None])
    bound = s[:, None].astype(np.float64) * (0.5 + 2.0 ** -14)
    assert np.all(err <= bound)


def test_acts_tie_golden(orc):
    kv = _read_kv("tie_cases.txt")
    x = np.array([float(v) for v in kv["acts"]], np.float32)
    X = np.tile(x, (2, 1))
    q, s, _ = orc.quant_acts(X)
    assert np.array_equal(q[0], np.array([int(v) for v in kv["acts_q"]], np.int8))
    assert s[0] == np.float32(float(kv["acts_scale"][0]))


@pytest.mark.parametrize("j", [-12, -1, 3, 20])
def test_acts_power_of_two_and_sign(orc, j):
    X = _acts(43, 5, 512)
    q0, s0, _ = orc.quant_acts(X)
    q1, s1, _ = orc.quant_acts(X * np.float32(2.0 ** j))
    assert np.array_equal(q0, q1) and np.array_equal(s1, s0 * np.float32(2.0 ** j))
    qn, sn, _ = orc.quant_acts(-X)
    assert np.array_equal(qn, -q0) and np.array_equal(sn, s0)


def test_acts_zero_and_tiny_rows(orc):
    X = np.zeros((3, 256), np.float32)
    X[1, 5] = np.float32(3e-6)  # below the 1e-5 guard
    q, s, r = orc.quant_acts(X)
    assert np.all(q[0] == 0) and s[0] == np.float32(EPS / np.float32(127))
    # guarded: qs = 127/1e-5, so 3e-6 maps to rint(38.1) = 38
    assert q[1, 5] == 38 and s[1] == s[0]


def test_acts_bf16_matches_widened_f32(orc):
    from w1_a8_matmul_amd.workloads import to_bf16_bits

    X = _acts(44, 6, 2560, 2.0)
    bits = to_bf16_bits(X)
    widened = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.abs(widened - X) <= np.abs(X) * 2.0 ** -8)  # it is a bf16 rounding
    qa, sa, ra = orc.quant_acts(bits, bf16=True)
    qb, sb, rb = orc.quant_acts(widened)
    assert np.array_equal(qa, qb) and np.array_equal(sa, sb) and np.array_equal(ra, rb)


# --------------------------------------------------------------------------
# R5: exact int32 contraction
# --------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,K", [(1, 48, 256), (4, 32, 768), (5, 16, 2560)])
def test_int_matmul_matches_numpy(orc, M, N, K):
    rng = _rng(M * N + K)
    qx = rng.integers(-127, 128, (M, K)).astype(np.int8)
    qw = rng.integers(-1, 2, (N, K)).astype(np.int8)
    acc = orc.int_matmul(qx, qw)
    assert acc.shape == (M, N)
    assert np.array_equal(acc.astype(np.int64), qx.astype(np.int64) @ qw.astype(np.int64).T)


def test_int_matmul_k_permutation_and_bound(orc):
    rng = _rng(51)
    qx = rng.integers(-127, 128, (3, 512)).astype(np.int8)
    qw = rng.integers(-1, 2, (16, 512)).astype(np.int8)
    perm = rng.permutation(512)
    a0 = orc.int_matmul(qx, qw)
    a1 = orc.int_matmul(qx[:, perm].copy(), qw[:, perm].copy())
    assert np.array_equal(a0, a1)
    nnz = (qw != 0).sum(axis=1)
    assert np.all(np.abs(a0) <= 127 * nnz[None, :])


def test_int_dot_samples(orc):
    rng = _rng(52)
    qx = rng.integers(-127, 128, (9, 768)).astype(np.int8)
    qw = rng.integers(-1, 2, (40, 768)).astype(np.int8)
    mi = rng.integers(0, 9, 100)
    ni = rng.integers(0, 40, 100)
    got = orc.int_dot_samples(qx, qw, mi, ni)
    full = qx.astype(np.int64) @ qw.astype(np.int64).T
    assert np.array_equal(got, full[mi, ni])


# --------------------------------------------------------------------------
# R6: float rescale, R7: ReLU^2
# --------------------------------------------------------------------------
def test_rescale_close_to_exact_product(orc):
    rng = _rng(61)
    acc = rng.integers(-300000, 300000, (4, 64)).astype(np.int32)
    s = (rng.random(4).astype(np.float32) + np.float32(0.1)) * np.float32(0.03)
    g = np.float32(0.0137)
    y = orc.rescale(acc, s, g)
    exact = acc.astype(np.float64) * s[:, None].astype(np.float64) * np.float64(g)
    rel = np.abs(y - exact) / np.maximum(np.abs(exact), 1e-300)
    assert np.all(rel[acc != 0] <= 2.0 ** -23)
    assert np.all(y[acc == 0] == 0)


def test_rescale_scale_order_is_x_then_gamma(orc):
    # a case where the two orders round differently decides the reading R6
    rng = _rng(62)
    acc = rng.integers(-2 ** 20, 2 ** 20, (64, 64)).astype(np.int32)
    s = rng.random(64).astype(np.float32) * np.float32(0.05)
    g = np.float32(0.0173)
    y = orc.rescale(acc, s, g)
    want = ((acc.astype(np.float32) * s[:, None]).astype(np.float32) * g).astype(np.float32)
    other = ((acc.astype(np.float32) * g).astype(np.float32) * s[:, None]).astype(np.float32)
    assert np.array_equal(y, want)
    assert not np.array_equal(want, other)


def test_relu2(orc):
    y = np.array([-2.0, -0.0, 0.0, 1.5, 3e-20, 1e20], np.float32)
    h = orc.relu2(y)
    assert np.array_equal(h, np.array([0, 0, 0, 2.25, np.float32(3e-20) ** 2, np.float32(np.inf)], np.float32))
    assert not np.signbit(h[1])


def test_forward_integer_special_case(orc):
    # W in {+c, -c} with c a power of two -> gamma = c, q_w = sign(W); X
    # integer-valued with |x| max 127 per row -> s_x = 1, q_x = X; so y is
    # exactly c times the plain integer product.
    rng = _rng(63)
    c = np.float32(2.0 ** -6)
    S = np.where(rng.random((32, 512)) < 0.5, 1, -1).astype(np.int64)
    W = (S * c).astype(np.float32)
    Xi = rng.integers(-126, 127, (4, 512)).astype(np.int64)
    Xi[:, 7] = 127
    X = Xi.astype(np.float32)
    packed, gc, qw = orc.quantize_weights(W)
    assert gc == c
    y, xq, sx, acc = orc.forward(X, qw, gc)
    assert np.all(sx == 1.0) and np.array_equal(xq.astype(np.int64), Xi)
    assert np.array_equal(y.astype(np.float64), (Xi @ S.T).astype(np.float64) * float(c))


@pytest.mark.parametrize("i,j", [(-3, 2), (4, -7)])
def test_forward_power_of_two_scaling(orc, i, j):
    rng = _rng(64)
    W = rng.standard_normal((32, 256), dtype=np.float32) * np.float32(0.02)
    X = rng.standard_normal((3, 256), dtype=np.float32)
    _, g0, q0 = orc.quantize_weights(W)
    y0, *_ = orc.forward(X, q0, g0)
    _, g1, q1 = orc.quantize_weights(W * np.float32(2.0 ** i))
    y1, *_ = orc.forward(X * np.float32(2.0 ** j), q1, g1)
    assert np.array_equal(q0, q1)
    assert np.array_equal(y1, y0 * np.float32(2.0 ** (i + j)))


# --------------------------------------------------------------------------
# Brute force on tiny shapes: the quantized product stays within the bound
# the two quantizers allow around the full-precision product.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,K,seed", [(1, 16, 256, 71), (4, 16, 256, 72), (3, 32, 512, 73)])
def test_forward_brute_force_bound(orc, M, N, K, seed):
    rng = _rng(seed)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    X = rng.standard_normal((M, K), dtype=np.float32)
    _, gc, qw = orc.quantize_weights(W)
    y, xq, sx, acc = orc.forward(X, qw, gc)
    Xd, Wd = X.astype(np.float64), W.astype(np.float64)
    y_true = Xd @ Wd.T
    wq_err = np.abs(np.float64(gc) * qw - Wd)  # |gamma q_w - W|
    bound = (np.abs(Xd) @ wq_err.T
             + np.float64(gc) * sx[:, None].astype(np.float64) * (0.5 + 2.0 ** -14)
             * np.abs(qw).sum(axis=1)[None, :]
             + 1e-6 * np.abs(y))
    assert np.all(np.abs(y - y_true) <= bound)
    # and y is the dequantized product up to float rounding
    deq = (np.float64(gc) * qw.astype(np.float64)) @ (sx[:, None] * xq.astype(np.float64)).T
    assert np.allclose(y, deq.T, rtol=1e-6, atol=0)


def test_forward_zero_rows_and_matrix(orc):
    rng = _rng(81)
    W = rng.standard_normal((32, 256), dtype=np.float32) * np.float32(0.02)
    W[5] = 0
    X = rng.standard_normal((4, 256), dtype=np.float32)
    X[2] = 0
    _, gc, qw = orc.quantize_weights(W)
    y, *_ = orc.forward(X, qw, gc)
    assert np.all(y[:, 5] == 0) and np.all(y[2] == 0)
    _, gz, qz = orc.quantize_weights(np.zeros((16, 256), np.float32))
    assert gz == EPS and np.all(qz == 0)
    yz, *_ = orc.forward(X, qz, gz)
    assert np.all(yz == 0)


# --------------------------------------------------------------------------
# R8: subln read as RMSNorm with a per-feature gain, before R4.  Pins: with a
# unit gain the codes are R4's and the scale ratio normalizes the row to RMS
# 1; a constant row gives closed-form codes and factor; power-of-two scaling
# of the input changes nothing; brute force in double of the plain
# definition (normalize, then quantize) agrees away from rounding ties.
# --------------------------------------------------------------------------
def _gain(seed, K):
    return _rng(seed).uniform(0.5, 1.5, K).astype(np.float32)


@pytest.mark.parametrize("M,K,seed", [(4, 256, 91), (3, 2560, 92), (2, 6912, 93)])
def test_rmsnorm_unit_gain_is_plain_quant_and_normalizes(orc, M, K, seed):
    X = _acts(seed, M, K, 3.0)
    q, s, r = orc.quant_acts_rmsnorm(X, np.ones(K, np.float32), 0.0)
    q0, s0, r0 = orc.quant_acts(X)
    assert np.array_equal(q, q0) and np.array_equal(r, r0)
    f = s.astype(np.float64) / s0.astype(np.float64)  # the RMS factor
    rms = np.sqrt(np.mean((X.astype(np.float64) * f[:, None]) ** 2, axis=1))
    assert np.all(np.abs(rms - 1.0) <= 3e-7)


def _rint_even(v: Fraction) -> int:
    fl = v.numerator // v.denominator
    rem = v - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def test_rmsnorm_constant_row_closed_form(orc):
    K, c, eps = 512, np.float32(2.0 ** -7), float(np.float32(1e-4))
    steps = [Fraction(j, 4) for j in range(-4, 5)]  # gains -1, -0.75, ..., 1
    g = np.array([float(steps[k % 9]) for k in range(K)], np.float32)
    X = np.full((2, K), c, np.float32)
    X[1] = -c
    q, s, r = orc.quant_acts_rmsnorm(X, g, eps)
    want = np.array([_rint_even(127 * steps[k % 9]) for k in range(K)], np.int8)
    assert np.array_equal(q[0], want) and np.array_equal(q[1], -want)
    assert np.array_equal(r, q.astype(np.int32).sum(axis=1))
    # mean x^2 = c^2 exactly, so r = 1/sqrt(c^2 + eps); max |u| = c
    rf = np.float32(1.0 / np.sqrt(float(c) ** 2 + eps))
    assert s[0] == s[1] == np.float32(np.float32(c / np.float32(127)) * rf)


@pytest.mark.parametrize("j", [-6, 5])
def test_rmsnorm_power_of_two_scaling_and_signs(orc, j):
    X = _acts(94, 5, 768)
    g = _gain(95, 768)
    q0, s0, r0 = orc.quant_acts_rmsnorm(X, g, 0.0)
    q1, s1, r1 = orc.quant_acts_rmsnorm(X * np.float32(2.0 ** j), g, 0.0)
    assert np.array_equal(q1, q0) and np.array_equal(s1, s0) and np.array_equal(r1, r0)
    qn, sn, _ = orc.quant_acts_rmsnorm(-X, g, 0.0)
    qg, sg, _ = orc.quant_acts_rmsnorm(X, -g, 0.0)
    assert np.array_equal(qn, -q0) and np.array_equal(sn, s0)
    assert np.array_equal(qg, -q0) and np.array_equal(sg, s0)


@pytest.mark.parametrize("M,K,seed", [(6, 2560, 96), (3, 6912, 97)])
def test_rmsnorm_matches_double_definition(orc, M, K, seed):
    X = _acts(seed, M, K, 2.0)
    g = _gain(seed + 100, K)
    eps = 1e-5
    q, s, rs = orc.quant_acts_rmsnorm(X, g, eps)
    Xd, gd = X.astype(np.float64), g.astype(np.float64)
    rr = 1.0 / np.sqrt((Xd ** 2).mean(axis=1) + eps)
    xh = Xd * rr[:, None] * gd[None, :]  # normalize first, as the definition says
    a = np.abs(xh).max(axis=1)
    t = xh * 127.0 / a[:, None]
    near_tie = np.abs(np.abs(t - np.floor(t)) - 0.5) < 1e-4
    assert np.all((q == np.clip(np.rint(t), -127, 127)) | near_tie)
    assert near_tie.mean() < 1e-3
    assert np.all(np.abs(s.astype(np.float64) / (a / 127.0) - 1.0) <= 3e-7)
    assert np.array_equal(rs, q.astype(np.int32).sum(axis=1))


def test_rmsnorm_zero_row_and_zero_gain(orc):
    X = _acts(98, 3, 256)
    X[1] = 0
    g = _gain(99, 256)
    g[10] = 0
    q, s, _ = orc.quant_acts_rmsnorm(X, g, 1e-5)
    assert np.all(q[:, 10] == 0)
    assert np.all(q[1] == 0)
    eps = np.float64(np.float32(1e-5))  # the epsilon is a float argument
    assert s[1] == np.float32(np.float32(EPS / np.float32(127)) * np.float32(1.0 / np.sqrt(eps)))


def test_rmsnorm_bf16_matches_widened_f32(orc):
    from w1_a8_matmul_amd.workloads import to_bf16_bits

    X = _acts(100, 4, 2560, 2.0)
    g = _gain(101, 2560)
    bits = to_bf16_bits(X)
    widened = (bits.astype(np.uint32) << 16).view(np.float32)
    qa, sa, ra = orc.quant_acts_rmsnorm(bits, g, 1e-5, bf16=True)
    qb, sb, rb = orc.quant_acts_rmsnorm(widened, g, 1e-5)
    assert np.array_equal(qa, qb) and np.array_equal(sa, sb) and np.array_equal(ra, rb)


# --------------------------------------------------------------------------
# R12: gated squared ReLU of a fused gate+up output, and the interleaved
# packing of such a matrix.  Pins: the row order of a 32-row matrix worked
# by hand; hand-computed outputs on small integers (exact in float); the
# up = 1 case is R7; a non-positive gate gives a zero.
# --------------------------------------------------------------------------
def test_glu_pack_row_order_by_hand(orc):
    N, K = 32, 256
    q = np.zeros((N, K), np.int8)
    q[np.arange(N), np.arange(N)] = 1  # row r is marked in column r
    got = orc.unpack(orc.pack_glu(q), N, K)
    order = [int(np.argmax(got[r])) for r in range(N)]
    # tile 0: gate rows 0..7 then up rows 16..23; tile 1: gate 8..15, up 24..31
    assert order == list(range(0, 8)) + list(range(16, 24)) + list(range(8, 16)) + \
        list(range(24, 32))
    q2 = _rng(121).integers(-1, 2, (48, 512)).astype(np.int8)
    assert np.array_equal(np.sort(orc.unpack(orc.pack_glu(q2), 48, 512), axis=0),
                          np.sort(q2, axis=0))  # a permutation of whole rows


def test_glu_relu2_by_hand(orc):
    y = np.array([[1, -2, 3, 4, 5, 6, 7, 8],
                  [-1, 0, 2, -3, 9, -4, -5, 10]], np.float32)
    h = orc.glu_relu2(y)
    assert np.array_equal(h, np.array([[5, 0, 63, 128], [0, 0, -20, 0]], np.float32))


def test_glu_relu2_unit_up_is_relu2_and_nonpositive_gate(orc):
    g = _acts(122, 3, 64)
    y = np.concatenate([g, np.ones_like(g)], axis=1)
    assert np.array_equal(orc.glu_relu2(y), orc.relu2(g))
    y2 = np.concatenate([-np.abs(g), _acts(123, 3, 64)], axis=1)
    assert np.all(orc.glu_relu2(y2) == 0)


# --------------------------------------------------------------------------
# Evaluation order of the float steps (R2, R4, R12; also R8's factor).  The
# pages give the quantizers in words; each reading fixes one order of float
# operations.  Hand-worked separating cases (tests/golden/order_cases.txt)
# and exact-arithmetic sweeps tell the stated order apart from the plausible
# others: x*127/a or x/s_x for R4, a reciprocal multiply for R2, r*(r*up)
# for R12, and a float RMS factor for R8.
# --------------------------------------------------------------------------
def _bits(h) -> np.float32:
    return np.array([int(h, 16)], np.uint32).view(np.float32)[0]


def _fl(q: Fraction) -> Fraction:
    """One rounding of a rational to float32, nearest even (signed)."""
    if q < 0:
        return -Fraction(float(round_to_f32(-q)))
    return Fraction(float(round_to_f32(q)))


def _rint_half_even(v: Fraction) -> int:
    return _rint_even(v)


def _clamp127(v: int) -> int:
    return max(-127, min(127, v))


def test_acts_order_golden(orc):
    kv = _read_kv("order_cases.txt")
    a, x = _bits(kv["r4_amax_bits"][0]), _bits(kv["r4_x_bits"][0])
    row = np.zeros((1, 16), np.float32)
    row[0, 0], row[0, 1] = a, x
    q, s, _ = orc.quant_acts(row)
    assert q[0, 0] == 127
    assert q[0, 1] == int(kv["r4_q"][0]) != int(kv["r4_q_other_orders"][0])
    assert s[0] == np.float32(a / np.float32(127))


def test_acts_order_sweep_exact(orc):
    # For random row maxima a, put x at the float32 values nearest to the
    # points where x * fl(127/a) crosses a half-integer; whenever the stated
    # order (x times fl(127/a)) and x*127/a or x/fl(a/127) round to different
    # codes in exact arithmetic, the oracle must give the stated order's code.
    rng = _rng(131)
    rows, want = [], []
    separating = 0
    for a in rng.uniform(0.05, 40.0, 24).astype(np.float32):
        A = Fraction(float(a))
        qs = _fl(Fraction(127) / A)
        sx = _fl(A / 127)
        xs = []
        for j in range(0, 127, 3):
            c = np.float32(float((Fraction(2 * j + 1, 2)) / qs))
            for d in (-2, -1, 0, 1, 2):
                xv = np.float32(c + np.float32(d) * np.spacing(c))
                if not (0 < xv < a):
                    continue
                X_ = Fraction(float(xv))
                mine = _clamp127(_rint_half_even(_fl(X_ * qs)))
                o1 = _clamp127(_rint_half_even(_fl(_fl(X_ * 127) / A)))
                o2 = _clamp127(_rint_half_even(_fl(X_ / sx)))
                if mine != o1 or mine != o2:
                    separating += 1
                xs.append((xv, mine))
        for i in range(0, len(xs), 255):
            part = xs[i:i + 255]
            r = np.zeros(256, np.float32)
            r[0] = a
            e = np.zeros(256, np.int64)
            e[0] = 127
            for k, (xv, mine) in enumerate(part, start=1):
                r[k], e[k] = xv, mine
            rows.append(r)
            want.append(e)
    assert separating >= 20, separating  # the sweep does tell the orders apart
    q, _, _ = orc.quant_acts(np.array(rows))
    assert np.array_equal(q.astype(np.int64), np.array(want))


def test_ternary_division_golden(orc):
    kv = _read_kv("order_cases.txt")
    g, w = _bits(kv["r2_gamma_bits"][0]), _bits(kv["r2_w_bits"][0])
    q = orc.ternarize(np.array([[w, -w]], np.float32), g)
    assert q[0, 0] == int(kv["r2_q"][0]) != int(kv["r2_q_reciprocal"][0])
    assert q[0, 1] == -int(kv["r2_q"][0])


def test_ternary_division_sweep_near_half(orc):
    # Many scales, and weights within 16 float32 steps of gamma/2: the codes
    # must follow the closed form of a true division, and the sweep must hold
    # weights where a reciprocal multiply would round to the other side.
    rng = _rng(132)
    straddle = 0
    for gc in rng.uniform(1e-3, 0.1, 60).astype(np.float32):
        half = np.float32(gc / np.float32(2))
        vals = [np.float32(half + np.float32(d) * np.spacing(half)) for d in range(-16, 17)]
        W = np.array(vals + [-v for v in vals], np.float32).reshape(1, -1)
        q = orc.ternarize(W, gc)
        assert np.array_equal(q, _closed_form_ternary(W, gc))
        G = Fraction(float(gc))
        inv = _fl(1 / G)
        for v in vals:
            V = Fraction(float(v))
            if (_rint_half_even(_fl(V / G)) != 0) != (_rint_half_even(_fl(V * inv)) != 0):
                straddle += 1
    assert straddle >= 10, straddle


def test_glu_association_golden(orc):
    kv = _read_kv("order_cases.txt")
    g, u = _bits(kv["r12_gate_bits"][0]), _bits(kv["r12_up_bits"][0])
    h = orc.glu_relu2(np.array([[g, u]], np.float32))
    assert h.view(np.uint32)[0, 0] == int(kv["r12_h_bits"][0], 16)
    assert int(kv["r12_h_bits"][0], 16) != int(kv["r12_h_other_association_bits"][0], 16)


def test_glu_association_random_exact(orc):
    # Non-integer gates and ups, where the associations round differently:
    # the result is fl(fl(r*r)*up) exactly.
    rng = _rng(133)
    F = 512
    gate = rng.uniform(-0.1, 0.1, (4, F)).astype(np.float32)
    up = rng.uniform(-2.0, 2.0, (4, F)).astype(np.float32)
    h = orc.glu_relu2(np.concatenate([gate, up], axis=1))
    differ = 0
    for m in range(4):
        for f in range(F):
            r = Fraction(float(max(gate[m, f], np.float32(0))))
            U = Fraction(float(up[m, f]))
            want = _fl(_fl(r * r) * U)
            other = _fl(r * _fl(r * U))
            differ += want != other
            assert Fraction(float(h[m, f])) == want
    assert differ >= 10, differ


def test_rmsnorm_factor_correctly_rounded(orc):
    # With a unit gain the scale is fl(s0 * r), s0 the plain scale and r the
    # RMS factor rounded once to float from (nearly) exact arithmetic: the
    # double sum and square root keep it within 1e-15 of exact, far inside
    # half a float32 step, except at near-ties, which are skipped.
    from decimal import Decimal, getcontext

    getcontext().prec = 50
    M, K = 64, 256
    eps = np.float32(1e-5)
    X = _acts(134, M, K, 1.5)
    X *= np.exp2(_rng(135).integers(-3, 4, (M, 1))).astype(np.float32)
    q, s, _ = orc.quant_acts_rmsnorm(X, np.ones(K, np.float32), float(eps))
    _, s0, _ = orc.quant_acts(X)
    checked = 0
    for m in range(M):
        S = sum(Fraction(float(v)) ** 2 for v in X[m])
        inner = S / K + Fraction(float(eps))
        d = Decimal(inner.numerator) / Decimal(inner.denominator)
        r_exact = Fraction(1 / d.sqrt())
        r = _fl(r_exact)
        ulp = Fraction(float(np.spacing(np.float32(float(r)))))
        if abs(abs(r_exact - r) - ulp / 2) < ulp * Fraction(1, 1 << 20):
            continue  # near a rounding tie
        checked += 1
        assert Fraction(float(s[m])) == _fl(Fraction(float(s0[m])) * r), m
    assert checked >= M - 2


# --------------------------------------------------------------------------
# R13: the base-3 layout, five codes per byte in 16 x 320 tiles (K padded to
# a multiple of 320 with code 0).  Pins: hand-worked positions
# (tests/golden/pack_b3_positions.txt); an all-zero matrix packs to bytes of
# 1+3+9+27+81 = 121; a hand-worked padding case; every one of the 243
# five-code patterns in every byte slot; the 2B footprint.
# --------------------------------------------------------------------------
def test_pack_b3_positions_golden(orc):
    with open(os.path.join(GOLDEN, "pack_b3_positions.txt")) as f:
        rows = [list(map(int, l.split())) for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) >= 10
    for N, K, n, k, byte, digit in rows:
        q = np.zeros((N, K), np.int8)
        assert np.all(orc.pack_b3(q) == 121)  # code 1 in all five digits
        q[n, k] = 1  # code 2 at (n, k)
        p = orc.pack_b3(q)
        expect = np.full(N * K // 5, 121, np.uint8)
        expect[byte] = 121 + 3 ** digit
        assert np.array_equal(p, expect), (N, K, n, k)


def test_pack_b3_padding_by_hand(orc):
    # K = 336 pads to 640: tile 0 holds columns 0..319 (all code 1, bytes of
    # 121); tile 1 holds columns 320..335, which are the first 16 columns of
    # quarter 0: word 0, bytes 0..3, digits 0..3 (u = 0..15) of each row's
    # chunk.  Those bytes are 1+3+9+27 = 40 (digit 4 is padding, code 0);
    # every other byte of tile 1 is all padding, 0.
    q = np.zeros((16, 336), np.int8)
    p = orc.pack_b3(q)
    assert p.size == 16 * 640 // 5 == orc.packed_bytes_b3(16, 336)
    assert np.all(p[:1024] == 121)
    t1 = p[1024:].reshape(64, 16)
    assert np.all(t1[:16, :4] == 40) and np.all(t1[:16, 4:] == 0) and np.all(t1[16:] == 0)
    assert np.array_equal(orc.unpack_b3(p, 16, 336), q)
    bad = p.copy()
    bad[1024 + 4] = 1  # a padding code that is not 0
    with pytest.raises(ValueError):
        orc.unpack_b3(bad, 16, 336)


def test_pack_b3_all_243_patterns(orc):
    # every five-code pattern (as a base-3 number, digit i = code of column
    # 20j + 4i + b) lands as that number in every byte slot (j, b)
    pats = np.array(np.meshgrid(*[[0, 1, 2]] * 5, indexing="ij")).reshape(5, -1).T  # 243 x 5
    value = (pats * np.array([1, 3, 9, 27, 81])).sum(axis=1)
    N, K = 16, 320
    for off in range(0, 243, 61):
        q = np.zeros((N, K), np.int8)
        expect = np.zeros(N * K // 5, np.int64)
        s = off
        for n in range(N):
            for quarter in range(4):
                for j in range(4):
                    for b in range(4):
                        pat = s % 243
                        s += 1
                        for i in range(5):
                            q[n, 80 * quarter + 20 * j + 4 * i + b] = pats[pat, i] - 1
                        expect[(quarter * 16 + n) * 16 + 4 * j + b] = value[pat]
        p = orc.pack_b3(q)
        assert np.array_equal(p.astype(np.int64), expect)
        assert np.array_equal(orc.unpack_b3(p, N, K), q)


@pytest.mark.parametrize("N,K", [(16, 320), (48, 656), (32, 2560), (16, 6912)])
def test_pack_b3_roundtrip_and_range(orc, N, K):
    q = _rng(N * K).integers(-1, 2, (N, K)).astype(np.int8)
    p = orc.pack_b3(q)
    Kp = -(-K // 320) * 320
    assert p.size == N * Kp // 5 == orc.packed_bytes_b3(N, K)
    assert p.max() <= 242
    assert np.array_equal(orc.unpack_b3(p, N, K), q)
    # the digits hold exactly the codes (a permutation), plus code 0 padding
    digits = np.stack([(p.astype(np.int64) // 3 ** i) % 3 for i in range(5)], axis=1).ravel()
    want = np.bincount((q + 1).ravel(), minlength=3)
    got = np.bincount(digits, minlength=3)
    assert got[1] == want[1] and got[2] == want[2] and got[0] == want[0] + N * (Kp - K)


def test_pack_b3_footprint():
    kv = _read_kv("model_2b_footprint.txt")
    from w1_a8_matmul_amd.workloads import WORKLOADS

    wl = WORKLOADS["decode_step_2b"]
    total = wl.layers * sum(l.N * (-(-l.K // 320) * 320) // 5 for l in wl.linears)
    assert total == int(kv["packed_bytes_b3"][0])
    assert abs(total / (wl.weights_per_step * np.log2(3) / 8) - 1) < 0.015


def test_pack_b3_rejects_bad_input(orc):
    with pytest.raises(ValueError):
        orc.pack_b3(np.zeros((15, 320), np.int8))
    with pytest.raises(ValueError):
        orc.pack_b3(np.zeros((16, 100), np.int8))
    with pytest.raises(ValueError):
        orc.pack_b3(np.full((16, 320), 2, np.int8))
    with pytest.raises(ValueError):
        orc.unpack_b3(np.full(1024, 243, np.uint8), 16, 320)
