"""Host-side checks of the C ABI: the library loads, exports every declared
function, and rejects bad arguments before it touches the GPU.

None of these calls launches work: each one fails argument checking (which
runs before any HIP call) or is a documented no-op, so they run without a GPU.
Fake device addresses are never dereferenced.
"""
import ctypes

import pytest

bl = pytest.importorskip("w1_a8_matmul_amd.bitlinear")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE, ERR_WS, ERR_HIP, ERR_ARG = range(8)
A = 0x10000   # a fake, 16-byte aligned address (never dereferenced)
U = 0x10004   # a fake misaligned address


@pytest.fixture(scope="module")
def L():
    return bl.lib()


def test_exports_every_declared_function(L):
    names = bl.declared_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(L, n), n


def test_version_and_strings(L):
    assert L.bitlinear_abi_version() == 7
    for s in range(8):
        assert L.bitlinear_status_string(s).decode()
    assert L.bitlinear_status_string(99).decode() == "unknown status"


def test_packed_and_workspace_sizes(L):
    assert L.bitlinear_packed_bytes(6912, 2560) == 6912 * 2560 // 4
    assert L.bitlinear_packed_bytes(16, 256) == 1024
    assert L.bitlinear_packed_bytes(15, 256) == 0
    assert L.bitlinear_packed_bytes(16, 128) == 0
    assert L.bitlinear_packed_bytes(-16, 256) == 0
    assert L.bitlinear_weights_workspace_bytes(6912, 2560) >= 6912 * 8
    assert L.bitlinear_workspace_bytes(1, 2560, 6912) == 0
    assert L.bitlinear_workspace_bytes(0, 2560, 6912) == 0
    big = L.bitlinear_workspace_bytes(2048, 2560, 6912)
    assert big >= 2048 * 2560 + 2 * 2048 * 4
    assert L.bitlinear_workspace_bytes(-1, 2560, 6912) == ctypes.c_size_t(-1).value
    assert L.bitlinear_workspace_bytes(4, 100, 6912) == ctypes.c_size_t(-1).value
    qws = L.bitlinear_forward_q_workspace_bytes(2048, 2560, 6912)
    assert qws >= 4096 + 256 * 128 * 128 * 4  # counters, a partial tile per piece
    assert big >= 2048 * 2560 + 2 * 2048 * 4 + qws  # forward holds forward_q's workspace
    assert L.bitlinear_forward_q_workspace_bytes(0, 2560, 6912) == 0
    assert L.bitlinear_forward_q_workspace_bytes(8, 100, 6912) == ctypes.c_size_t(-1).value


def _err(L):
    return L.bitlinear_last_error().decode()


def test_quantize_weights_validation(L):
    qw = L.bitlinear_quantize_weights
    assert qw(None, 16, 256, A, A, A, 1 << 20, None) == ERR_NULL
    assert "required" in _err(L)
    assert qw(A, 15, 256, A, A, A, 1 << 20, None) == ERR_SHAPE
    assert qw(A, 16, 100, A, A, A, 1 << 20, None) == ERR_SHAPE
    assert qw(A, 0, 256, A, A, A, 1 << 20, None) == ERR_SHAPE
    assert qw(A, 16, 256 * 70000, A, A, A, 1 << 30, None) == ERR_SHAPE
    assert qw(A, 16, (1 << 23) + 256, A, A, A, 1 << 30, None) == ERR_SHAPE  # K <= 2^23
    assert qw(U, 16, 256, A, A, A, 1 << 20, None) == ERR_ALIGN
    assert qw(A, 16, 256, U, A, A, 1 << 20, None) == ERR_ALIGN
    assert qw(A, 16, 256, A, A, None, 0, None) == ERR_WS
    assert qw(A, 16, 256, A, A, A, 8, None) == ERR_WS
    assert "workspace" in _err(L)


def test_pack_unpack_validation(L):
    assert L.bitlinear_pack_ternary(None, 16, 256, A, None) == ERR_NULL
    assert L.bitlinear_pack_ternary(A, 16, 255, A, None) == ERR_SHAPE
    assert L.bitlinear_pack_ternary(A, 16, 256, U, None) == ERR_ALIGN
    assert L.bitlinear_unpack_ternary(A, 16, 256, None, None) == ERR_NULL
    assert L.bitlinear_unpack_ternary(A, 8, 256, A, None) == ERR_SHAPE
    assert L.bitlinear_unpack_ternary(U, 16, 256, A, None) == ERR_ALIGN


def test_quantize_acts_validation(L):
    qa = L.bitlinear_quantize_acts
    assert qa(A, 7, 4, 256, A, A, A, None) == ERR_DTYPE
    assert qa(A, 0, -1, 256, A, A, A, None) == ERR_SHAPE
    assert qa(A, 0, 4, 100, A, A, A, None) == ERR_SHAPE
    assert qa(None, 1, 4, 256, A, A, A, None) == ERR_NULL
    assert qa(A, 1, 4, 256, A, None, A, None) == ERR_NULL
    assert qa(A, 1, 4, 256, U, A, A, None) == ERR_ALIGN
    assert qa(A, 1, 4, 256, A, A, U, None) == ERR_ALIGN
    # M == 0 is a no-op, even with null pointers
    assert qa(None, 1, 0, 256, None, None, None, None) == OK
    assert _err(L) == ""


def test_forward_validation(L):
    f = L.bitlinear_forward
    assert f(A, 3, 1, 256, 16, A, A, A, 0, None, None, 0, None) == ERR_DTYPE
    assert f(A, 0, 1, 256, 16, A, A, A, 5, None, None, 0, None) == ERR_ARG
    assert f(A, 0, -1, 256, 16, A, A, A, 0, None, None, 0, None) == ERR_SHAPE
    assert f(A, 0, 1, 256, 24, A, A, A, 0, None, None, 0, None) == ERR_SHAPE
    assert f(A, 0, 1, 260, 16, A, A, A, 0, None, None, 0, None) == ERR_SHAPE
    assert f(A, 0, 1, 256, 16, None, A, A, 0, None, None, 0, None) == ERR_NULL
    assert f(A, 0, 1, 256, 16, A, None, A, 0, None, None, 0, None) == ERR_NULL
    assert f(A, 0, 1, 256, 16, A, A, None, 0, None, None, 0, None) == ERR_NULL
    assert f(U, 0, 1, 256, 16, A, A, A, 0, None, None, 0, None) == ERR_ALIGN
    dbg = bl.Debug(U, None, None)
    assert f(A, 0, 1, 256, 16, A, A, A, 0, ctypes.byref(dbg), None, 0, None) == ERR_ALIGN
    # the large-M path needs a workspace
    assert f(A, 1, 2048, 2560, 6912, A, A, A, 0, None, None, 0, None) == ERR_WS
    assert f(A, 1, 2048, 2560, 6912, A, A, A, 0, None, A, 1024, None) == ERR_WS
    assert f(A, 1, 2048, 2560, 6912, A, A, A, 0, None, U, 1 << 30, None) == ERR_ALIGN
    assert f(None, 1, 0, 2560, 6912, None, None, None, 0, None, None, 0, None) == OK


def test_rmsnorm_entry_points_validation(L):
    qa = L.bitlinear_quantize_acts_rmsnorm
    assert qa(A, 1, 4, 256, None, 1e-5, A, A, A, None) == ERR_NULL  # the gain is required
    assert "norm_gain" in _err(L)
    assert qa(A, 1, 4, 256, U, 1e-5, A, A, A, None) == ERR_ALIGN
    assert qa(A, 1, 4, 256, A, -1.0, A, A, A, None) == ERR_ARG
    assert qa(A, 1, 4, 256, A, float("nan"), A, A, A, None) == ERR_ARG
    assert qa(A, 1, 4, 256, A, float("inf"), A, A, A, None) == ERR_ARG
    assert qa(A, 7, 4, 256, A, 1e-5, A, A, A, None) == ERR_DTYPE
    assert qa(A, 0, 4, 100, A, 1e-5, A, A, A, None) == ERR_SHAPE
    assert qa(None, 1, 0, 256, None, 1e-5, None, None, None, None) == OK
    f = L.bitlinear_forward_rmsnorm
    assert f(A, 0, 1, 256, 16, None, 1e-5, A, A, A, 0, None, None, 0, None) == ERR_NULL
    assert f(A, 0, 1, 256, 16, U, 1e-5, A, A, A, 0, None, None, 0, None) == ERR_ALIGN
    assert f(A, 0, 1, 256, 16, A, -0.5, A, A, A, 0, None, None, 0, None) == ERR_ARG
    assert f(A, 0, 1, 256, 24, A, 1e-5, A, A, A, 0, None, None, 0, None) == ERR_SHAPE
    assert f(A, 1, 2048, 2560, 6912, A, 1e-5, A, A, A, 0, None, None, 0, None) == ERR_WS
    assert f(None, 1, 0, 2560, 6912, None, 1e-5, None, None, None, 0, None, None, 0,
             None) == OK


def test_forward_q_validation(L):
    f = L.bitlinear_forward_q
    assert f(A, A, A, 4, 256, 16, A, A, A, 9, None, 0, None) == ERR_ARG
    assert f(A, A, None, 4, 256, 16, A, A, A, 0, None, 0, None) == ERR_NULL
    assert f(A, A, A, 4, 256, 17, A, A, A, 0, None, 0, None) == ERR_SHAPE
    assert f(A, A, A, 4, 256, 16, A, U, A, 0, None, 0, None) == ERR_ALIGN
    # a workspace, when given, must be large enough and aligned
    assert f(A, A, A, 4, 256, 16, A, A, A, 0, A, 1024, None) == ERR_WS
    assert f(A, A, A, 4, 256, 16, A, A, A, 0, U, 1 << 30, None) == ERR_ALIGN
    assert f(None, None, None, 0, 256, 16, None, None, None, 0, None, 0, None) == OK


def test_forward_glu_quant_validation(L):
    f = L.bitlinear_forward_glu_quant
    n = L.bitlinear_forward_glu_quant_workspace_bytes()
    assert n >= 4
    #          X  dt M  K    N   packed g  H  Hq hs hr ws  bytes stream
    assert f(A, 7, 1, 256, 32, A, A, A, A, A, A, A, n, None) == ERR_DTYPE
    assert f(A, 0, 1, 256, 48, A, A, A, A, A, A, A, n, None) == ERR_SHAPE   # N % 32
    assert f(A, 0, 5, 256, 32, A, A, A, A, A, A, A, n, None) == ERR_SHAPE   # M > 4
    assert f(A, 0, 0, 256, 32, A, A, A, A, A, A, A, n, None) == ERR_SHAPE   # M < 1
    assert f(A, 0, 1, 12544, 32, A, A, A, A, A, A, A, n, None) == ERR_SHAPE  # K > 12288
    assert f(A, 0, 1, 256, 32, A, A, A, None, A, A, A, n, None) == ERR_NULL
    assert f(A, 0, 1, 256, 32, A, A, A, A, U, A, A, n, None) == ERR_ALIGN
    assert f(A, 0, 1, 256, 32, A, A, A, A, A, A, None, 0, None) == ERR_WS
    assert f(A, 0, 1, 256, 32, A, A, A, A, A, A, A, n - 1, None) == ERR_WS
    assert f(A, 0, 1, 256, 32, A, A, A, A, A, A, U, n, None) == ERR_ALIGN


def test_ffn_chain_validation(L):
    f = L.bitlinear_ffn_chain
    n = L.bitlinear_ffn_chain_workspace_bytes(256)
    assert n >= 16 + 4 * 16
    assert L.bitlinear_ffn_chain_workspace_bytes(24) == 0
    #        X  dt M  K     Nup  pu g  epi Nd  pd gd H  Y  ws bytes stream
    assert f(A, 7, 1, 256, 256, A, A, 1, 16, A, A, A, A, A, n, None) == ERR_DTYPE
    assert f(A, 0, 1, 256, 256, A, A, 0, 16, A, A, A, A, A, n, None) == ERR_ARG   # no ReLU^2
    assert f(A, 0, 5, 256, 256, A, A, 1, 16, A, A, A, A, A, n, None) == ERR_SHAPE
    assert f(A, 0, 1, 256, 272, A, A, 1, 16, A, A, A, A, A, n, None) == ERR_SHAPE  # F % 256
    assert f(A, 0, 1, 256, 528, A, A, 2, 16, A, A, A, A, A, n, None) == ERR_SHAPE  # glu N % 32
    assert f(A, 0, 1, 12544, 256, A, A, 1, 16, A, A, A, A, A, n, None) == ERR_SHAPE
    assert f(A, 0, 1, 256, 256, A, A, 1, 16, A, None, A, A, A, n, None) == ERR_NULL
    assert f(A, 0, 1, 256, 256, A, A, 1, 16, A, A, U, A, A, n, None) == ERR_ALIGN
    assert f(A, 0, 1, 256, 256, A, A, 1, 16, A, A, A, A, None, 0, None) == ERR_WS
    assert f(A, 0, 1, 256, 256, A, A, 1, 16, A, A, A, A, U, n, None) == ERR_ALIGN


def test_forward_lut_validation(L):
    f = L.bitlinear_forward_lut
    #          X  dt K     N   packed g  Y  epi dbg stream
    assert f(A, 7, 256, 16, A, A, A, 0, None, None) == ERR_DTYPE
    assert f(A, 0, 256, 16, A, A, A, 9, None, None) == ERR_ARG
    assert f(A, 0, 320, 16, A, A, A, 0, None, None) == ERR_SHAPE
    assert f(A, 0, 8448, 16, A, A, A, 0, None, None) == ERR_SHAPE
    assert f(None, 0, 256, 16, A, A, A, 0, None, None) == ERR_NULL
    assert f(A, 0, 256, 16, U, A, A, 0, None, None) == ERR_ALIGN


def test_binding_refuses_cpu_tensors():
    import torch

    with pytest.raises(bl.BitLinearError):
        bl.quantize_acts(torch.zeros(4, 256))


def _gop(X=A, dtype=1, epi=0, K=2560, N=256, packed=A, gamma=A, Y=A, gain=None, eps=0.0):
    return bl.GroupOp(X, dtype, epi, K, N, packed, gamma, Y, gain, eps)


def test_group_validation(L):
    arr = (bl.GroupOp * 2)(_gop(), _gop(K=6912, N=2560))
    need = L.bitlinear_group_workspace_bytes(arr, 2, 1)
    assert need >= 2 * 80 + (2 + 20) * 16 + 8  # layer table, work units, queue
    assert L.bitlinear_group_workspace_bytes(arr, 2, 17) > 0      # M > 16: grouped GEMM
    assert L.bitlinear_group_workspace_bytes(arr, 2, 65537) == 0
    assert L.bitlinear_group_workspace_bytes(arr, 2, 16) > 0      # 16 x 6912 fits in LDS
    big = (bl.GroupOp * 1)(_gop(K=12288, N=16))
    assert L.bitlinear_group_workspace_bytes(big, 1, 11) > 0
    assert L.bitlinear_group_workspace_bytes(big, 1, 12) == 0     # 12 x 12304 + ... > 160 KiB
    assert L.bitlinear_group_workspace_bytes(arr, 0, 1) == 0
    h = ctypes.c_void_p()
    assert L.bitlinear_group_create(arr, 2, 1, A, need, None) == ERR_NULL
    assert L.bitlinear_group_create(None, 2, 1, A, need, ctypes.byref(h)) == ERR_NULL
    assert L.bitlinear_group_create(arr, 2, 0, A, need, ctypes.byref(h)) == ERR_SHAPE
    assert L.bitlinear_group_create(arr, 2, 1, A, need - 1, ctypes.byref(h)) == ERR_WS
    assert L.bitlinear_group_create(arr, 2, 1, U, need, ctypes.byref(h)) == ERR_ALIGN
    bad = [(_gop(dtype=5), ERR_DTYPE), (_gop(epi=3), ERR_ARG), (_gop(N=24), ERR_SHAPE),
           (_gop(K=12288 + 256), ERR_SHAPE), (_gop(Y=None), ERR_NULL), (_gop(X=U), ERR_ALIGN),
           (_gop(gain=U, eps=1e-5), ERR_ALIGN), (_gop(gain=A, eps=-1.0), ERR_ARG)]
    for op, code in bad:
        one = (bl.GroupOp * 1)(op)
        assert L.bitlinear_group_create(one, 1, 1, A, 1 << 30, ctypes.byref(h)) == code
        assert h.value is None
    assert L.bitlinear_group_forward(None, None) == ERR_NULL
    L.bitlinear_group_destroy(None)
