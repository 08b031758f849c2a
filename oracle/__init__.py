"""CPU oracle for the W1.58A8 BitLinear forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (``include/`` and
``w1_a8_matmul_amd/``) never imports it and shares no code with it.

This module is a thin ctypes wrapper over ``bitlinear_oracle.c`` (plain C,
compiled with gcc, no fast-math, no FMA contraction).  The C file states the
readings of the pages it follows; each wrapper below names the reading it
exposes.  Arrays are numpy arrays; bf16 activations travel as their uint16
bit patterns.

Every function here is pinned by ``tests/test_oracle_pins.py`` against
closed forms, exact rational arithmetic, invariants, library routines or
brute force on tiny shapes; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "bitlinear_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

# Flags that keep the C arithmetic exactly IEEE: no fast-math, no contraction.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
          "-ffp-contract=off", "-fno-strict-aliasing", "-Wall", "-Wextra"]


def build(source: str = SOURCE, output: str = LIBRARY, extra_flags=()) -> str:
    """Compile the oracle with gcc into ``output`` and return its path."""
    tmp = output + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


class Oracle:
    """One loaded copy of the oracle library (tests may load mutated copies)."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            raise FileNotFoundError(
                f"{path} is not built; run __graft_entry__.build() or oracle.build()")
        lib = ctypes.CDLL(path)
        self.lib = lib
        self.path = path
        lib.oracle_version.restype = ctypes.c_int
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_absmean.argtypes = [_p, _i64, _i64, _p, _p]
        lib.oracle_ternarize.argtypes = [_p, _i64, ctypes.c_float, _p]
        lib.oracle_packed_bytes.argtypes = [_i64, _i64]
        lib.oracle_packed_bytes.restype = _i64
        lib.oracle_pack.argtypes = [_p, _i64, _i64, _p]
        lib.oracle_pack.restype = ctypes.c_int
        lib.oracle_unpack.argtypes = [_p, _i64, _i64, _p]
        lib.oracle_unpack.restype = ctypes.c_int
        lib.oracle_quant_acts_f32.argtypes = [_p, _i64, _i64, _p, _p, _p]
        lib.oracle_quant_acts_bf16.argtypes = [_p, _i64, _i64, _p, _p, _p]
        lib.oracle_quant_acts_rmsnorm_f32.argtypes = [_p, _p, ctypes.c_float, _i64, _i64, _p,
                                                      _p, _p]
        lib.oracle_quant_acts_rmsnorm_bf16.argtypes = [_p, _p, ctypes.c_float, _i64, _i64,
                                                       _p, _p, _p]
        lib.oracle_int_matmul.argtypes = [_p, _p, _i64, _i64, _i64, _p]
        lib.oracle_int_dot_samples.argtypes = [_p, _p, _i64, _p, _p, _i64, _p]
        lib.oracle_rescale.argtypes = [_p, _p, ctypes.c_float, _i64, _i64, _p]
        lib.oracle_relu2.argtypes = [_p, _i64, _p]
        lib.oracle_packed_bytes_b3.argtypes = [_i64, _i64]
        lib.oracle_packed_bytes_b3.restype = _i64
        lib.oracle_pack_b3.argtypes = [_p, _i64, _i64, _p]
        lib.oracle_pack_b3.restype = ctypes.c_int
        lib.oracle_unpack_b3.argtypes = [_p, _i64, _i64, _p]
        lib.oracle_unpack_b3.restype = ctypes.c_int
        lib.oracle_pack_glu.argtypes = [_p, _i64, _i64, _p]
        lib.oracle_pack_glu.restype = ctypes.c_int
        lib.oracle_glu_relu2.argtypes = [_p, _i64, _i64, _p]
        lib.oracle_forward.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _p,
                                       ctypes.c_float, _p, _p, _p, _p]
        lib.oracle_forward.restype = ctypes.c_int

    # -- threads -----------------------------------------------------------
    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def set_threads(self, n: int) -> None:
        self.lib.oracle_set_threads(int(n))

    # -- R1 / R2: absmean weight quantization -------------------------------
    def absmean(self, W: np.ndarray) -> Tuple[np.float32, np.float32]:
        """(gamma, gamma_c): the float mean |W| and its 1e-5 guard (R1)."""
        W = np.ascontiguousarray(W, dtype=np.float32)
        N, K = W.shape
        g = np.zeros(1, np.float32)
        gc = np.zeros(1, np.float32)
        self.lib.oracle_absmean(_ptr(W), N, K, _ptr(g), _ptr(gc))
        return g[0], gc[0]

    def ternarize(self, W: np.ndarray, gamma_c) -> np.ndarray:
        """q_w = clamp(rint(W / gamma_c), -1, 1) (R2)."""
        W = np.ascontiguousarray(W, dtype=np.float32)
        q = np.empty(W.shape, np.int8)
        self.lib.oracle_ternarize(_ptr(W), W.size, ctypes.c_float(float(gamma_c)), _ptr(q))
        return q

    # -- R3: packed layout ---------------------------------------------------
    def packed_bytes(self, N: int, K: int) -> int:
        return int(self.lib.oracle_packed_bytes(N, K))

    def pack(self, q: np.ndarray) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.int8)
        N, K = q.shape
        out = np.empty(N * K // 4, np.uint8)
        if self.lib.oracle_pack(_ptr(q), N, K, _ptr(out)) != 0:
            raise ValueError("oracle_pack: shape outside the layout or non-ternary value")
        return out

    def unpack(self, packed: np.ndarray, N: int, K: int) -> np.ndarray:
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        assert packed.size == N * K // 4
        q = np.empty((N, K), np.int8)
        if self.lib.oracle_unpack(_ptr(packed), N, K, _ptr(q)) != 0:
            raise ValueError("oracle_unpack: bad shape or invalid code 3")
        return q

    # -- R13: base-3 layout, five codes per byte --------------------------------
    def packed_bytes_b3(self, N: int, K: int) -> int:
        return int(self.lib.oracle_packed_bytes_b3(N, K))

    def pack_b3(self, q: np.ndarray) -> np.ndarray:
        """Five ternary codes per byte in 16 x 320 tiles (K padded to 320)."""
        q = np.ascontiguousarray(q, dtype=np.int8)
        N, K = q.shape
        out = np.empty(self.packed_bytes_b3(N, K), np.uint8)
        if self.lib.oracle_pack_b3(_ptr(q), N, K, _ptr(out)) != 0:
            raise ValueError("oracle_pack_b3: shape outside the layout or non-ternary value")
        return out

    def unpack_b3(self, packed: np.ndarray, N: int, K: int) -> np.ndarray:
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        assert packed.size == self.packed_bytes_b3(N, K)
        q = np.empty((N, K), np.int8)
        if self.lib.oracle_unpack_b3(_ptr(packed), N, K, _ptr(q)) != 0:
            raise ValueError("oracle_unpack_b3: bad shape, byte above 242 or nonzero padding")
        return q

    def quantize_weights(self, W: np.ndarray):
        """R1 + R2 + R3: returns (packed, gamma_c, q_w)."""
        _, gc = self.absmean(W)
        q = self.ternarize(W, gc)
        return self.pack(q), gc, q

    # -- R4: per-token absmax activation quantization -----------------------
    def quant_acts(self, X: np.ndarray, bf16: bool = False):
        """Returns (q_x int8 [M][K], s_x float [M], rowsum int32 [M]).

        ``bf16=True`` means X holds bf16 bit patterns as uint16."""
        if bf16:
            X = np.ascontiguousarray(X, dtype=np.uint16)
        else:
            X = np.ascontiguousarray(X, dtype=np.float32)
        M, K = X.shape
        q = np.empty((M, K), np.int8)
        s = np.empty(M, np.float32)
        r = np.empty(M, np.int32)
        fn = self.lib.oracle_quant_acts_bf16 if bf16 else self.lib.oracle_quant_acts_f32
        fn(_ptr(X), M, K, _ptr(q), _ptr(s), _ptr(r))
        return q, s, r

    # -- R12: gated squared ReLU of a fused gate+up matrix ------------------
    def pack_glu(self, q: np.ndarray) -> np.ndarray:
        """Packs q [N][K] (gate rows, then up rows) with the halves interleaved
        per 16-row tile: tile t = gate rows 8t..8t+7, up rows F+8t..F+8t+7."""
        q = np.ascontiguousarray(q, dtype=np.int8)
        N, K = q.shape
        out = np.empty(self.packed_bytes(N, K), np.uint8)
        if self.lib.oracle_pack_glu(_ptr(q), N, K, _ptr(out)) != 0:
            raise ValueError("bad shape or non-ternary value")
        return out

    def glu_relu2(self, y: np.ndarray) -> np.ndarray:
        """h [M][N/2] = max(y_gate, 0)^2 * y_up for y [M][N] = [gate | up]."""
        y = np.ascontiguousarray(y, dtype=np.float32)
        M, N = y.shape
        h = np.empty((M, N // 2), np.float32)
        self.lib.oracle_glu_relu2(_ptr(y), M, N, _ptr(h))
        return h

    # -- R8: subln (RMSNorm with gain) before the absmax quantization --------
    def quant_acts_rmsnorm(self, X: np.ndarray, g: np.ndarray, eps: float = 1e-5,
                           bf16: bool = False):
        """R8 then R4: returns (q_x int8 [M][K], s_x float [M], rowsum int32 [M]).

        The codes are R4's codes of u = X * g; the scale carries the RMS factor
        r = 1/sqrt(mean x^2 + eps).  ``bf16=True`` means X holds bf16 bits."""
        if bf16:
            X = np.ascontiguousarray(X, dtype=np.uint16)
        else:
            X = np.ascontiguousarray(X, dtype=np.float32)
        M, K = X.shape
        g = np.ascontiguousarray(g, dtype=np.float32)
        assert g.shape == (K,)
        q = np.empty((M, K), np.int8)
        s = np.empty(M, np.float32)
        r = np.empty(M, np.int32)
        fn = (self.lib.oracle_quant_acts_rmsnorm_bf16 if bf16
              else self.lib.oracle_quant_acts_rmsnorm_f32)
        fn(_ptr(X), _ptr(g), ctypes.c_float(eps), M, K, _ptr(q), _ptr(s), _ptr(r))
        return q, s, r

    # -- R5: exact integer contraction --------------------------------------
    def int_matmul(self, qx: np.ndarray, qw: np.ndarray) -> np.ndarray:
        qx = np.ascontiguousarray(qx, dtype=np.int8)
        qw = np.ascontiguousarray(qw, dtype=np.int8)
        M, K = qx.shape
        N, K2 = qw.shape
        assert K == K2
        acc = np.empty((M, N), np.int32)
        self.lib.oracle_int_matmul(_ptr(qx), _ptr(qw), M, N, K, _ptr(acc))
        return acc

    def int_dot_samples(self, qx, qw, m_idx, n_idx) -> np.ndarray:
        qx = np.ascontiguousarray(qx, dtype=np.int8)
        qw = np.ascontiguousarray(qw, dtype=np.int8)
        m_idx = np.ascontiguousarray(m_idx, dtype=np.int64)
        n_idx = np.ascontiguousarray(n_idx, dtype=np.int64)
        assert qx.shape[1] == qw.shape[1] and m_idx.shape == n_idx.shape
        out = np.empty(m_idx.shape, np.int32)
        self.lib.oracle_int_dot_samples(_ptr(qx), _ptr(qw), qx.shape[1], _ptr(m_idx),
                                        _ptr(n_idx), m_idx.size, _ptr(out))
        return out

    # -- R6 / R7 -------------------------------------------------------------
    def rescale(self, acc: np.ndarray, s_x: np.ndarray, gamma_c) -> np.ndarray:
        acc = np.ascontiguousarray(acc, dtype=np.int32)
        s_x = np.ascontiguousarray(s_x, dtype=np.float32)
        M, N = acc.shape
        y = np.empty((M, N), np.float32)
        self.lib.oracle_rescale(_ptr(acc), _ptr(s_x), ctypes.c_float(float(gamma_c)), M, N, _ptr(y))
        return y

    def relu2(self, y: np.ndarray) -> np.ndarray:
        y = np.ascontiguousarray(y, dtype=np.float32)
        h = np.empty_like(y)
        self.lib.oracle_relu2(_ptr(y), y.size, _ptr(h))
        return h

    def forward(self, X: np.ndarray, qw: np.ndarray, gamma_c, bf16: bool = False):
        """R4 -> R5 -> R6 for one layer: returns (y, q_x, s_x, acc)."""
        if bf16:
            X = np.ascontiguousarray(X, dtype=np.uint16)
        else:
            X = np.ascontiguousarray(X, dtype=np.float32)
        qw = np.ascontiguousarray(qw, dtype=np.int8)
        M, K = X.shape
        N = qw.shape[0]
        y = np.empty((M, N), np.float32)
        xq = np.empty((M, K), np.int8)
        sx = np.empty(M, np.float32)
        acc = np.empty((M, N), np.int32)
        rc = self.lib.oracle_forward(_ptr(X), 1 if bf16 else 0, M, K, N, _ptr(qw),
                                     ctypes.c_float(float(gamma_c)), _ptr(y), _ptr(xq),
                                     _ptr(sx), _ptr(acc))
        if rc != 0:
            raise ValueError("oracle_forward failed")
        return y, xq, sx, acc


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The oracle built in-tree (built on first use if it is missing)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build()
        _default = Oracle(LIBRARY)
    return _default
