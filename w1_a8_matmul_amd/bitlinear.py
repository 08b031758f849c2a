"""ctypes binding of libbitlinear.so (declared in include/bitlinear.h).

Argument marshalling only: every step of the BitLinear forward runs in the
library's HIP kernels.  torch supplies device memory (outputs and workspaces
are allocated as torch tensors) and the stream (torch's current stream).
If the library is not built, every call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

from .build import LIBRARY, ROOT

HEADER = os.path.join(ROOT, "include", "bitlinear.h")

OK = 0
F32, BF16 = 0, 1
EPI = {"none": 0, None: 0, "relu2": 1, "relu2_glu": 2}


def _out_cols(N: int, epilogue) -> int:
    """Columns of Y: the gated epilogue writes N/2."""
    return N // 2 if EPI[epilogue] == 2 else N

_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_sz = ctypes.c_size_t


class BitLinearError(RuntimeError):
    pass


class Debug(ctypes.Structure):
    _fields_ = [("xq_out", _p), ("xscale_out", _p), ("acc_out", _p)]


FMT = {"2bit": 0, None: 0, "b3": 1}


class GroupOp(ctypes.Structure):
    _fields_ = [("X", _p), ("dtype", ctypes.c_int), ("epi", ctypes.c_int), ("K", _i64),
                ("N", _i64), ("packed", _p), ("gamma", _p), ("Y", _p), ("norm_gain", _p),
                ("norm_eps", ctypes.c_float), ("format", ctypes.c_int)]


_lib = None


def declared_functions() -> list:
    """Names of the functions include/bitlinear.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(bitlinear_[a-z0-9_]+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise BitLinearError(
            f"{LIBRARY} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    L = ctypes.CDLL(LIBRARY)
    L.bitlinear_abi_version.restype = ctypes.c_int
    L.bitlinear_packed_bytes.argtypes = [_i64, _i64]
    L.bitlinear_packed_bytes.restype = _sz
    L.bitlinear_weights_workspace_bytes.argtypes = [_i64, _i64]
    L.bitlinear_weights_workspace_bytes.restype = _sz
    L.bitlinear_workspace_bytes.argtypes = [_i64, _i64, _i64]
    L.bitlinear_workspace_bytes.restype = _sz
    L.bitlinear_forward_q_workspace_bytes.argtypes = [_i64, _i64, _i64]
    L.bitlinear_forward_q_workspace_bytes.restype = _sz
    L.bitlinear_quantize_weights.argtypes = [_p, _i64, _i64, _p, _p, _p, _sz, _p]
    L.bitlinear_quantize_weights_glu.argtypes = [_p, _i64, _i64, _p, _p, _p, _sz, _p]
    L.bitlinear_packed_bytes_b3.argtypes = [_i64, _i64]
    L.bitlinear_packed_bytes_b3.restype = _sz
    L.bitlinear_quantize_weights_b3.argtypes = [_p, _i64, _i64, _p, _p, _p, _sz, ctypes.c_int,
                                                _p]
    L.bitlinear_pack_ternary_b3.argtypes = [_p, _i64, _i64, _p, _p]
    L.bitlinear_unpack_ternary_b3.argtypes = [_p, _i64, _i64, _p, _p]
    L.bitlinear_pack_ternary.argtypes = [_p, _i64, _i64, _p, _p]
    L.bitlinear_unpack_ternary.argtypes = [_p, _i64, _i64, _p, _p]
    L.bitlinear_quantize_acts.argtypes = [_p, ctypes.c_int, _i64, _i64, _p, _p, _p, _p]
    L.bitlinear_quantize_acts_rmsnorm.argtypes = [_p, ctypes.c_int, _i64, _i64, _p,
                                                  ctypes.c_float, _p, _p, _p, _p]
    L.bitlinear_forward.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _p, _p, _p,
                                    ctypes.c_int, ctypes.POINTER(Debug), _p, _sz, _p]
    L.bitlinear_forward_rmsnorm.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _p,
                                            ctypes.c_float, _p, _p, _p, ctypes.c_int, _p, _p,
                                            _sz, _p]
    L.bitlinear_forward_q.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p, _p, _p,
                                      ctypes.c_int, _p, _sz, _p]
    L.bitlinear_forward_noalloc.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _p, _p, _p,
                                            ctypes.c_int, ctypes.POINTER(Debug), _p]
    L.bitlinear_forward_glu_quant_workspace_bytes.argtypes = []
    L.bitlinear_forward_glu_quant_workspace_bytes.restype = _sz
    L.bitlinear_forward_glu_quant.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _p, _p, _p, _p,
                                              _p, _p, _p, _sz, _p]
    L.bitlinear_ffn_chain_workspace_bytes.argtypes = [_i64]
    L.bitlinear_ffn_chain_workspace_bytes.restype = _sz
    L.bitlinear_ffn_chain.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _p, _p, ctypes.c_int,
                                      _i64, _p, _p, _p, _p, _p, _sz, _p]
    L.bitlinear_forward_lut.argtypes = [_p, ctypes.c_int, _i64, _i64, _p, _p, _p, ctypes.c_int,
                                        ctypes.POINTER(Debug), _p]
    for name in ("bitlinear_quantize_weights", "bitlinear_pack_ternary",
                 "bitlinear_unpack_ternary", "bitlinear_quantize_acts", "bitlinear_forward",
                 "bitlinear_forward_q", "bitlinear_forward_noalloc", "bitlinear_forward_lut",
                 "bitlinear_forward_glu_quant", "bitlinear_ffn_chain",
                 "bitlinear_quantize_weights_b3", "bitlinear_pack_ternary_b3",
                 "bitlinear_unpack_ternary_b3"):
        getattr(L, name).restype = ctypes.c_int
    L.bitlinear_group_workspace_bytes.argtypes = [ctypes.POINTER(GroupOp), ctypes.c_int, _i64]
    L.bitlinear_group_workspace_bytes.restype = _sz
    L.bitlinear_group_create.argtypes = [ctypes.POINTER(GroupOp), ctypes.c_int, _i64, _p, _sz,
                                         ctypes.POINTER(_p)]
    L.bitlinear_group_create.restype = ctypes.c_int
    L.bitlinear_group_forward.argtypes = [_p, _p]
    L.bitlinear_group_forward.restype = ctypes.c_int
    L.bitlinear_group_destroy.argtypes = [_p]
    L.bitlinear_group_destroy.restype = None
    L.bitlinear_status_string.argtypes = [ctypes.c_int]
    L.bitlinear_status_string.restype = ctypes.c_char_p
    L.bitlinear_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def check(status: int, fn: str) -> None:
    if status != OK:
        L = lib()
        raise BitLinearError(f"{fn}: {L.bitlinear_status_string(status).decode()} "
                             f"({status}): {L.bitlinear_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise BitLinearError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise BitLinearError("tensors must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise BitLinearError(f"activations must be float32 or bfloat16, got {t.dtype}")


# -- sizes ------------------------------------------------------------------
def abi_version() -> int:
    return lib().bitlinear_abi_version()


def packed_bytes(N: int, K: int) -> int:
    return lib().bitlinear_packed_bytes(N, K)


def weights_workspace_bytes(N: int, K: int) -> int:
    return lib().bitlinear_weights_workspace_bytes(N, K)


def workspace_bytes(M: int, K: int, N: int) -> int:
    return lib().bitlinear_workspace_bytes(M, K, N)


def _empty_bytes(n: int, device) -> torch.Tensor:
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


# -- weights ----------------------------------------------------------------
def quantize_weights(W: torch.Tensor, packed: Optional[torch.Tensor] = None,
                     gamma: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, glu: bool = False):
    """Absmean ternary quantization + packing of float32 W [N][K].

    Returns (packed uint8 [N*K/4], gamma_c float32 [1]).  ``glu=True`` packs a
    fused gate+up matrix (gate rows first) for the "relu2_glu" epilogue."""
    N, K = W.shape
    if W.dtype != torch.float32:
        raise BitLinearError("W must be float32")
    nbytes = packed_bytes(N, K)
    if packed is None:
        packed = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=W.device)
    if gamma is None:
        gamma = torch.empty(4, dtype=torch.float32, device=W.device)[:1]
    if workspace is None:
        workspace = _empty_bytes(weights_workspace_bytes(N, K), W.device)
    fn = lib().bitlinear_quantize_weights_glu if glu else lib().bitlinear_quantize_weights
    st = fn(_ptr(W), N, K, _ptr(packed), _ptr(gamma), _ptr(workspace), workspace.numel(),
            _stream())
    check(st, "bitlinear_quantize_weights_glu" if glu else "bitlinear_quantize_weights")
    return packed, gamma


def packed_bytes_b3(N: int, K: int) -> int:
    return lib().bitlinear_packed_bytes_b3(N, K)


def quantize_weights_b3(W: torch.Tensor, glu: bool = False,
                        workspace: Optional[torch.Tensor] = None):
    """quantize_weights into the base-3 layout (five codes per byte; K padded
    to a multiple of 320).  Returns (packed uint8, gamma_c float32 [1])."""
    N, K = W.shape
    if W.dtype != torch.float32:
        raise BitLinearError("W must be float32")
    packed = torch.empty(max(packed_bytes_b3(N, K), 1), dtype=torch.uint8, device=W.device)
    gamma = torch.empty(4, dtype=torch.float32, device=W.device)[:1]
    if workspace is None:
        workspace = _empty_bytes(max(N, 1) * 8 + 256, W.device)
    check(lib().bitlinear_quantize_weights_b3(_ptr(W), N, K, _ptr(packed), _ptr(gamma),
                                              _ptr(workspace), workspace.numel(), int(glu),
                                              _stream()),
          "bitlinear_quantize_weights_b3")
    return packed, gamma


def pack_ternary_b3(Wq: torch.Tensor) -> torch.Tensor:
    N, K = Wq.shape
    packed = torch.empty(max(packed_bytes_b3(N, K), 1), dtype=torch.uint8, device=Wq.device)
    check(lib().bitlinear_pack_ternary_b3(_ptr(Wq), N, K, _ptr(packed), _stream()),
          "bitlinear_pack_ternary_b3")
    return packed


def unpack_ternary_b3(packed: torch.Tensor, N: int, K: int) -> torch.Tensor:
    Wq = torch.empty((N, K), dtype=torch.int8, device=packed.device)
    check(lib().bitlinear_unpack_ternary_b3(_ptr(packed), N, K, _ptr(Wq), _stream()),
          "bitlinear_unpack_ternary_b3")
    return Wq


def pack_ternary(Wq: torch.Tensor) -> torch.Tensor:
    N, K = Wq.shape
    packed = torch.empty(max(packed_bytes(N, K), 1), dtype=torch.uint8, device=Wq.device)
    check(lib().bitlinear_pack_ternary(_ptr(Wq), N, K, _ptr(packed), _stream()),
          "bitlinear_pack_ternary")
    return packed


def unpack_ternary(packed: torch.Tensor, N: int, K: int) -> torch.Tensor:
    Wq = torch.empty((N, K), dtype=torch.int8, device=packed.device)
    check(lib().bitlinear_unpack_ternary(_ptr(packed), N, K, _ptr(Wq), _stream()),
          "bitlinear_unpack_ternary")
    return Wq


# -- activations ------------------------------------------------------------
def quantize_acts(X: torch.Tensor, norm_gain: Optional[torch.Tensor] = None,
                  norm_eps: float = 1e-5):
    """Per-token absmax int8: returns (Xq int8 [M][K], x_scale [M], x_rowsum [M]).

    With ``norm_gain`` (float32 [K] on the GPU), subln (RMSNorm with that
    gain and ``norm_eps``) runs first, fused into the same launch."""
    M, K = X.shape
    Xq = torch.empty((M, K), dtype=torch.int8, device=X.device)
    sx = torch.empty(M, dtype=torch.float32, device=X.device)
    rs = torch.empty(M, dtype=torch.int32, device=X.device)
    if norm_gain is None:
        check(lib().bitlinear_quantize_acts(_ptr(X), _dtype_code(X), M, K, _ptr(Xq), _ptr(sx),
                                            _ptr(rs), _stream()),
              "bitlinear_quantize_acts")
    else:
        check(lib().bitlinear_quantize_acts_rmsnorm(_ptr(X), _dtype_code(X), M, K,
                                                    _ptr(norm_gain), norm_eps, _ptr(Xq),
                                                    _ptr(sx), _ptr(rs), _stream()),
              "bitlinear_quantize_acts_rmsnorm")
    return Xq, sx, rs


# -- forward ----------------------------------------------------------------
def forward(X: torch.Tensor, packed: torch.Tensor, gamma: torch.Tensor, N: int,
            epilogue: Optional[str] = None, debug: bool = False,
            out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
            norm_gain: Optional[torch.Tensor] = None, norm_eps: float = 1e-5):
    """Y [M][N] float32 = BitLinear(X).  With debug=True returns
    (Y, {"xq": int8 [M][K], "x_scale": [M], "acc": int32 [M][N]}).  With
    ``norm_gain`` (float32 [K]) subln runs first, fused into the quantization."""
    M, K = X.shape
    if out is None:
        out = torch.empty((M, _out_cols(N, epilogue)), dtype=torch.float32, device=X.device)
    ws_need = workspace_bytes(M, K, N)
    if ws_need == ctypes.c_size_t(-1).value:
        ws_need = 0  # the call itself reports the bad shape
    if workspace is None and ws_need > 0:
        workspace = _empty_bytes(ws_need, X.device)
    dbg = None
    dbg_struct = None
    if debug:
        dbg = {"xq": torch.empty((M, K), dtype=torch.int8, device=X.device),
               "x_scale": torch.empty(M, dtype=torch.float32, device=X.device),
               "acc": torch.empty((M, N), dtype=torch.int32, device=X.device)}
        dbg_struct = Debug(_ptr(dbg["xq"]), _ptr(dbg["x_scale"]), _ptr(dbg["acc"]))
    dbg_arg = ctypes.byref(dbg_struct) if dbg_struct is not None else None
    ws_n = workspace.numel() if workspace is not None else 0
    if norm_gain is None:
        st = lib().bitlinear_forward(
            _ptr(X), _dtype_code(X), M, K, N, _ptr(packed), _ptr(gamma), _ptr(out),
            EPI[epilogue], dbg_arg, _ptr(workspace), ws_n, _stream())
        check(st, "bitlinear_forward")
    else:
        st = lib().bitlinear_forward_rmsnorm(
            _ptr(X), _dtype_code(X), M, K, N, _ptr(norm_gain), norm_eps, _ptr(packed),
            _ptr(gamma), _ptr(out), EPI[epilogue], dbg_arg, _ptr(workspace), ws_n, _stream())
        check(st, "bitlinear_forward_rmsnorm")
    return (out, dbg) if debug else out


def forward_noalloc(X: torch.Tensor, packed: torch.Tensor, gamma: torch.Tensor, N: int,
                    epilogue: Optional[str] = None, out: Optional[torch.Tensor] = None,
                    debug: bool = False):
    """The forward without a workspace argument: the library's fixed
    per-GPU scratch array (NOALLOC_SCRATCH_BYTES) serves as workspace.  The
    library allocates nothing; ``out`` (and the debug tensors) are the
    caller's.  Calls that overlap on one GPU race (they share the array)."""
    M, K = X.shape
    if out is None:
        out = torch.empty((M, _out_cols(N, epilogue)), dtype=torch.float32, device=X.device)
    dbg = None
    dbg_struct = None
    if debug:
        dbg = {"xq": torch.empty((M, K), dtype=torch.int8, device=X.device),
               "x_scale": torch.empty(M, dtype=torch.float32, device=X.device),
               "acc": torch.empty((M, N), dtype=torch.int32, device=X.device)}
        dbg_struct = Debug(_ptr(dbg["xq"]), _ptr(dbg["x_scale"]), _ptr(dbg["acc"]))
    dbg_arg = ctypes.byref(dbg_struct) if dbg_struct is not None else None
    st = lib().bitlinear_forward_noalloc(_ptr(X), _dtype_code(X), M, K, N, _ptr(packed),
                                         _ptr(gamma), _ptr(out), EPI[epilogue], dbg_arg,
                                         _stream())
    check(st, "bitlinear_forward_noalloc")
    return (out, dbg) if debug else out


NOALLOC_SCRATCH_BYTES = 32 << 20  # BITLINEAR_NOALLOC_SCRATCH_BYTES


def forward_glu_quant_workspace(device) -> torch.Tensor:
    """The counter workspace of forward_glu_quant, zeroed (reusable)."""
    n = lib().bitlinear_forward_glu_quant_workspace_bytes()
    return torch.zeros(n, dtype=torch.uint8, device=device)


def forward_glu_quant(X: torch.Tensor, packed: torch.Tensor, gamma: torch.Tensor, N: int,
                      workspace: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None):
    """Gated FFN front half (fused gate+up weights, M <= 4): returns
    (H float [M][N/2], Hq int8 [M][N/2], h_scale [M], h_rowsum [M]), the last
    three as quantize_acts(H) would give them, from one launch."""
    M, K = X.shape
    F = N // 2
    if workspace is None:
        workspace = forward_glu_quant_workspace(X.device)
    H = out if out is not None else torch.empty((M, F), dtype=torch.float32, device=X.device)
    Hq = torch.empty((M, F), dtype=torch.int8, device=X.device)
    hs = torch.empty(max(M, 4), dtype=torch.float32, device=X.device)[:M]
    hr = torch.empty(max(M, 4), dtype=torch.int32, device=X.device)[:M]
    check(lib().bitlinear_forward_glu_quant(_ptr(X), _dtype_code(X), M, K, N, _ptr(packed),
                                            _ptr(gamma), _ptr(H), _ptr(Hq), _ptr(hs), _ptr(hr),
                                            _ptr(workspace), workspace.numel(), _stream()),
          "bitlinear_forward_glu_quant")
    return H, Hq, hs, hr


def ffn_chain_workspace(N_up: int, device) -> torch.Tensor:
    """The workspace of ffn_chain for an up projection of N_up rows, zeroed
    (reusable; its third int is the error flag)."""
    n = lib().bitlinear_ffn_chain_workspace_bytes(N_up)
    if n == 0:
        raise BitLinearError(f"bad N_up={N_up}")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def ffn_chain(X: torch.Tensor, packed_up: torch.Tensor, gamma_up: torch.Tensor, N_up: int,
              packed_down: torch.Tensor, gamma_down: torch.Tensor, N_down: int,
              glu: bool = False, workspace: Optional[torch.Tensor] = None,
              H: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """The decode FFN (M <= 4) in one launch: returns (H, Y), h = the squared
    ReLU (gated when ``glu``) of the up projection and Y its down projection."""
    M, K = X.shape
    F = N_up // 2 if glu else N_up
    if workspace is None:
        workspace = ffn_chain_workspace(N_up, X.device)
    if H is None:
        H = torch.empty((M, F), dtype=torch.float32, device=X.device)
    if out is None:
        out = torch.empty((M, N_down), dtype=torch.float32, device=X.device)
    check(lib().bitlinear_ffn_chain(_ptr(X), _dtype_code(X), M, K, N_up, _ptr(packed_up),
                                    _ptr(gamma_up), EPI["relu2_glu" if glu else "relu2"],
                                    N_down, _ptr(packed_down), _ptr(gamma_down), _ptr(H),
                                    _ptr(out), _ptr(workspace), workspace.numel(), _stream()),
          "bitlinear_ffn_chain")
    return H, out


def forward_lut(X: torch.Tensor, packed: torch.Tensor, gamma: torch.Tensor, N: int,
                epilogue: Optional[str] = None, out: Optional[torch.Tensor] = None,
                debug: bool = False):
    """The one-token forward by table lookup (X [1][K], K <= 8192): same
    outputs as forward(); no workspace."""
    M, K = X.shape
    if M != 1:
        raise BitLinearError(f"forward_lut takes one token, got M={M}")
    if out is None:
        out = torch.empty((1, _out_cols(N, epilogue)), dtype=torch.float32, device=X.device)
    dbg = None
    dbg_struct = None
    if debug:
        dbg = {"xq": torch.empty((1, K), dtype=torch.int8, device=X.device),
               "x_scale": torch.empty(4, dtype=torch.float32, device=X.device)[:1],
               "acc": torch.empty((1, N), dtype=torch.int32, device=X.device)}
        dbg_struct = Debug(_ptr(dbg["xq"]), _ptr(dbg["x_scale"]), _ptr(dbg["acc"]))
    dbg_arg = ctypes.byref(dbg_struct) if dbg_struct is not None else None
    check(lib().bitlinear_forward_lut(_ptr(X), _dtype_code(X), K, N, _ptr(packed), _ptr(gamma),
                                      _ptr(out), EPI[epilogue], dbg_arg, _stream()),
          "bitlinear_forward_lut")
    return (out, dbg) if debug else out


def forward_q_workspace(M: int, K: int, N: int, device) -> torch.Tensor:
    """A workspace for forward_q, counters zeroed (reusable across calls)."""
    n = lib().bitlinear_forward_q_workspace_bytes(M, K, N)
    if n == ctypes.c_size_t(-1).value:
        raise BitLinearError(f"bad shape M={M} K={K} N={N}")
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=device)


def forward_q(Xq: torch.Tensor, x_scale: torch.Tensor, x_rowsum: torch.Tensor,
              packed: torch.Tensor, gamma: torch.Tensor, N: int,
              epilogue: Optional[str] = None, out: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, split_remainder: bool = True):
    """Y from pre-quantized activations.  ``workspace`` (from
    forward_q_workspace, counters zero) is allocated when None;
    split_remainder=False runs one workgroup per tile without it."""
    M, K = Xq.shape
    if out is None:
        out = torch.empty((M, _out_cols(N, epilogue)), dtype=torch.float32,
                          device=Xq.device)
    if workspace is None and split_remainder:
        workspace = forward_q_workspace(M, K, N, Xq.device)
    ws = workspace if split_remainder else None
    st = lib().bitlinear_forward_q(_ptr(Xq), _ptr(x_scale), _ptr(x_rowsum), M, K, N,
                                   _ptr(packed), _ptr(gamma), _ptr(out), EPI[epilogue],
                                   _ptr(ws), ws.numel() if ws is not None else 0,
                                   _stream())
    check(st, "bitlinear_forward_q")
    return out


# -- grouped decode forward ----------------------------------------------------
class Group:
    """Independent BitLinear layers sharing M (1..65536), run by one or two
    persistent launches (skinny kernel up to 16 tokens, tiled GEMM above).

    layers: list of (X, packed, gamma, N, epilogue, Y) with X [M][K] on the
    GPU and Y [M][N] float32 (allocated when None), optionally followed by a
    subln gain (float32 [K] or None) and its epsilon (default 1e-5).  The
    tensors must stay alive while the group is used; ``forward()`` enqueues
    on torch's stream.  ``fmt="b3"``: every layer's weights are in the
    base-3 layout (quantize_weights_b3)."""

    def __init__(self, layers, fmt=None):
        L = lib()
        arr = (GroupOp * len(layers))()
        self.keep = []
        self.outputs = []
        M = None
        for i, layer in enumerate(layers):
            X, packed, gamma, N, epilogue, Y = layer[:6]
            gain = layer[6] if len(layer) > 6 else None
            eps = float(layer[7]) if len(layer) > 7 else 1e-5
            m, K = X.shape
            M = m if M is None else M
            if m != M:
                raise BitLinearError("all layers of a group need the same M")
            if Y is None:
                Y = torch.empty((M, _out_cols(N, epilogue)), dtype=torch.float32,
                                device=X.device)
            arr[i] = GroupOp(_ptr(X), _dtype_code(X), EPI[epilogue], K, N, _ptr(packed),
                             _ptr(gamma), _ptr(Y), _ptr(gain), eps if gain is not None else 0.0,
                             FMT[fmt])
            self.keep += [X, packed, gamma] + ([gain] if gain is not None else [])
            self.outputs.append(Y)
        self.M = M
        need = L.bitlinear_group_workspace_bytes(arr, len(layers), M)
        if need == 0:
            check(L.bitlinear_group_create(arr, len(layers), M, None, 0, ctypes.byref(_p())),
                  "bitlinear_group_workspace_bytes")
        self.workspace = torch.empty(need, dtype=torch.uint8, device=layers[0][0].device)
        handle = _p()
        check(L.bitlinear_group_create(arr, len(layers), M, _ptr(self.workspace), need,
                                       ctypes.byref(handle)), "bitlinear_group_create")
        self.handle = handle

    def forward(self):
        check(lib().bitlinear_group_forward(self.handle, _stream()), "bitlinear_group_forward")
        return self.outputs

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.bitlinear_group_destroy(h)
            self.handle = None
