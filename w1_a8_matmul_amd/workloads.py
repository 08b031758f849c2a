"""Seeded synthetic inputs for the W1.58A8 BitLinear workloads.

This module holds no part of the method's arithmetic: it only draws random
tensors and names the workload shapes.  Both the HIP path and the CPU oracle
receive the arrays made here; neither imports the other.

Shapes follow the BitNet b1.58 2B4T model the pages describe (its linears
replace nn.Linear; ReLU^2 FFN; no biases -- "BitNet b1.58 2B4T Technical
Report" card, section "Method Adaptation") and a 7B-like scale-up (the card's
"Limits" section names 7B and 13B models as future work).  The pages measure
on a trained model and real prompts; seeded Gaussian / heavy-tailed tensors of
the same shapes stand in for them.

Generator: numpy PCG64 (``numpy.random.default_rng(seed)``), float32 draws.
Weights: N(0, 0.02^2).  bf16 activations are float32 draws rounded to bf16 by
torch (round to nearest even).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

WEIGHT_STD = np.float32(0.02)


@dataclass(frozen=True)
class Linear:
    name: str
    K: int  # input features
    N: int  # output features


# One transformer layer of the ~2B shape: hidden 2560, 20 query heads and 5
# key/value heads of size 128 (QKV fused: 2560 + 2*640 = 3840), FFN 6912 with
# gate and up fused (13824).
LAYER_2B: Tuple[Linear, ...] = (
    Linear("qkv", 2560, 3840),
    Linear("o", 2560, 2560),
    Linear("gate_up", 2560, 13824),
    Linear("down", 6912, 2560),
)

# One layer of the 7B-like scale-up: hidden 4096, 32 heads of 128 (QKV fused
# 3 x 4096), FFN 11008 (gate and up fused 22016).
LAYER_7B: Tuple[Linear, ...] = (
    Linear("qkv", 4096, 12288),
    Linear("o", 4096, 4096),
    Linear("gate_up", 4096, 22016),
    Linear("down", 11008, 4096),
)


@dataclass(frozen=True)
class Workload:
    key: str
    description: str
    linears: Tuple[Linear, ...]
    layers: int
    tokens: Tuple[int, ...]
    x_kind: str  # "normal_f32", "normal_bf16", "outlier_bf16", "student_t3_bf16"
    weight_sparse_frac: float = 0.0
    chain_relu2: bool = False
    extra: dict = field(default_factory=dict)

    @property
    def weights_per_step(self) -> int:
        return self.layers * sum(l.N * l.K for l in self.linears)


WORKLOADS = {
    "bitlinear_m4_k256_n256": Workload(
        "bitlinear_m4_k256_n256",
        "single BitLinear, M=4, K=256, N=256; fp32 weights and fp32 activations",
        (Linear("single", 256, 256),), 1, (4,), "normal_f32"),
    "decode_gemv_pair_m1": Workload(
        "decode_gemv_pair_m1",
        "decode GEMV pair, M=1: up 2560->6912, ReLU^2, down 6912->2560; bf16 activations",
        (Linear("up", 2560, 6912), Linear("down", 6912, 2560)), 1, (1,), "normal_bf16",
        chain_relu2=True),
    "decode_step_2b": Workload(
        "decode_step_2b",
        "30 layers of 2B-shape linears (QKV, O, gate+up, down), M in {1,4,16}; bf16 activations",
        LAYER_2B, 30, (1, 4, 16), "normal_bf16"),
    "prefill_m2048": Workload(
        "prefill_m2048",
        "prefill GEMMs, M=2048: 2560->6912 and 6912->2560; bf16 activations with 0.1% x50 outliers",
        (Linear("gemm_a", 2560, 6912), Linear("gemm_b", 6912, 2560)), 1, (2048,), "outlier_bf16"),
    "decode_prefill_7b": Workload(
        "decode_prefill_7b",
        "32 layers of 7B-shape linears, M in {1,64,512}; 30% near-zero weights; Student-t(3) bf16 activations",
        LAYER_7B, 32, (1, 64, 512), "student_t3_bf16", weight_sparse_frac=0.3),
}

# Workload index used in seeds (the five workloads in the order above).
WORKLOAD_INDEX = {k: i + 1 for i, k in enumerate(WORKLOADS)}


def weight_seed(workload: str, layer: int, linear: int) -> int:
    return 1000 * WORKLOAD_INDEX[workload] + 10 * layer + linear


def act_seed(workload: str, layer: int, linear: int) -> int:
    return weight_seed(workload, layer, linear) + 5


def gen_weight(seed: int, N: int, K: int, sparse_frac: float = 0.0) -> np.ndarray:
    """float32 [N][K] ~ N(0, 0.02^2); a uniform ``sparse_frac`` of entries is
    multiplied by 1e-3 ("forced near zero", far below half the absmean)."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K), dtype=np.float32)
    W *= WEIGHT_STD
    if sparse_frac > 0.0:
        mask = rng.random((N, K), dtype=np.float32) < np.float32(sparse_frac)
        W[mask] *= np.float32(1e-3)
    return W


def gen_weight_device(seed: int, N: int, K: int, sparse_frac: float, device):
    """The same distribution as ``gen_weight``, drawn by torch's seeded
    generator on ``device`` (a torch tensor, float32 [N][K]): N(0, 0.02^2),
    and a uniform ``sparse_frac`` of entries multiplied by 1e-3.  For the
    full-size workloads (up to 6.5 G weights per step), where drawing on the
    host takes minutes; a check copies the same tensor to the host for the
    oracle."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    W = torch.randn((N, K), generator=gen, device=device, dtype=torch.float32)
    W *= float(WEIGHT_STD)
    if sparse_frac > 0.0:
        mask = torch.rand((N, K), generator=gen, device=device) < sparse_frac
        W = torch.where(mask, W * 1e-3, W)
    return W


def gen_acts_f32(seed: int, M: int, K: int, kind: str) -> np.ndarray:
    """float32 [M][K] activations before any bf16 rounding.

    kind: "normal" N(0,1); "outlier" N(0,1) with round(0.001*M*K) entries,
    chosen uniformly without replacement, multiplied by 50; "student_t3"
    Student-t with 3 degrees of freedom."""
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return rng.standard_normal((M, K), dtype=np.float32)
    if kind == "outlier":
        X = rng.standard_normal((M, K), dtype=np.float32)
        n_out = int(round(0.001 * M * K))
        idx = rng.choice(M * K, size=n_out, replace=False)
        X.reshape(-1)[idx] *= np.float32(50.0)
        return X
    if kind == "student_t3":
        return rng.standard_t(3.0, size=(M, K)).astype(np.float32)
    raise ValueError(f"unknown activation kind {kind!r}")


def gen_gain(seed: int, K: int) -> np.ndarray:
    """float32 [K] subln gains, uniform on [0.5, 1.5) (a trained norm's gains
    sit around 1; the spread makes every feature's gain matter)."""
    rng = np.random.default_rng(seed)
    return rng.uniform(0.5, 1.5, K).astype(np.float32)


def to_bf16_bits(X: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest even, via torch) and return uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(X, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def gen_acts(seed: int, M: int, K: int, x_kind: str) -> Tuple[np.ndarray, bool]:
    """Activations for a workload's ``x_kind``: (array, is_bf16_bits)."""
    base, _, dtype = x_kind.rpartition("_")
    X = gen_acts_f32(seed, M, K, base)
    if dtype == "f32":
        return X, False
    if dtype == "bf16":
        return to_bf16_bits(X), True
    raise ValueError(f"unknown x_kind {x_kind!r}")


def step_linears(workload: Workload) -> List[Tuple[int, int, Linear]]:
    """(layer, linear index, shape) for every linear in one step."""
    return [(layer, i, lin) for layer in range(workload.layers)
            for i, lin in enumerate(workload.linears)]
