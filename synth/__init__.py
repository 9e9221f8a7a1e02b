"""Seeded synthetic inputs for the SMOE routed-expert layer.

This module is shared by the CPU oracle's tests and by the GPU-path tests,
smoke check and bench. It holds random draws and workload shapes only: no
decoding, packing, blob layout, routing or FFN arithmetic lives here. Callers
pass in the sizes they need (for instance the byte count of a packed code
stream, which the consumer computes from its own layout rules).

Value recipes follow the workloads the S-MoE pages describe ("SMOE
Quantisation", section "Why Quantise": Qwen3-235B experts are three
4096 x 1536 matrices, 8 experts active per token, 94 MoE layers; "Model
Agnosticism": DeepSeek-MoE-16B has d_model 2048 and 64 routed experts):

* packed codes: uniform random bytes, i.e. every code uniform in
  [0, 2^bits) and independent (a byte holds 8/bits codes);
* group scales: lognormal with mu = ln 0.02, sigma = 0.5;
* activations: N(0, 1), rounded to bf16 where the workload says bf16;
* router logits: N(0, 1) in fp32;
* the tiny single-expert case draws fp32 weights N(0, 0.02) with each entry
  independently multiplied by 10 with probability 0.01 (to be quantised by
  the caller).
"""

from __future__ import annotations

import dataclasses

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "rng",
    "normal_f32",
    "round_to_bf16",
    "bf16_bits",
    "uniform_bytes",
    "lognormal_f32",
    "outlier_weights_f32",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one synthetic MoE layer workload."""

    name: str
    d_model: int
    ffn_dim: int
    num_experts: int
    top_k: int
    n_tokens: int
    bits: int
    norm_topk_prob: bool
    shared_ffn_dim: int = 0
    n_layers: int = 1
    x_dtype: str = "bf16"  # "bf16" or "f32"
    seed: int = 0


WORKLOADS = {
    # single expert, top-1, tiny SwiGLU; weights quantised by the MSE grid
    "tiny_swiglu": Workload("tiny_swiglu", 256, 128, 1, 1, 1, 4, True,
                            x_dtype="f32", seed=0),
    # Qwen3-235B-shaped layer, batch-1 decode
    "qwen235b_q4_b1": Workload("qwen235b_q4_b1", 4096, 1536, 128, 8, 1, 4, True,
                               seed=2),
    # same layer, 32 tokens, Q4 and Q2
    "qwen235b_q4_b32": Workload("qwen235b_q4_b32", 4096, 1536, 128, 8, 32, 4, True,
                                seed=3),
    "qwen235b_q2_b32": Workload("qwen235b_q2_b32", 4096, 1536, 128, 8, 32, 2, True,
                                seed=3),
    # DeepSeek-MoE-16B-shaped layer, 8 tokens, plus an always-on shared expert
    "deepseek16b_q4_b8": Workload("deepseek16b_q4_b8", 2048, 1408, 64, 6, 8, 4, False,
                                  shared_ffn_dim=2816, seed=4),
    # small decode batches of the same two layers (1-4 tokens)
    "qwen235b_q4_b4": Workload("qwen235b_q4_b4", 4096, 1536, 128, 8, 4, 4, True, seed=8),
    "deepseek16b_q4_b1": Workload("deepseek16b_q4_b1", 2048, 1408, 64, 6, 1, 4, False,
                                  shared_ffn_dim=2816, seed=9),
    "deepseek16b_q4_b4": Workload("deepseek16b_q4_b4", 2048, 1408, 64, 6, 4, 4, False,
                                  shared_ffn_dim=2816, seed=10),
    # the same layer at prefill-sized batches (matrix-core grouped stages)
    "qwen235b_q4_t512": Workload("qwen235b_q4_t512", 4096, 1536, 128, 8, 512, 4, True,
                                 seed=6),
    "qwen235b_q4_t2048": Workload("qwen235b_q4_t2048", 4096, 1536, 128, 8, 2048, 4, True,
                                  seed=7),
    # 94 stacked Qwen3-235B-shaped layers, batch 1, RMSNorm + residual per layer
    "qwen235b_q4_stack94": Workload("qwen235b_q4_stack94", 4096, 1536, 128, 8, 1, 4, True,
                                    n_layers=94, x_dtype="f32", seed=5),
}


def rng(seed: int) -> np.random.Generator:
    """NumPy PCG64 generator for a workload seed."""
    return np.random.default_rng(seed)


def normal_f32(r: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) draws as float32."""
    return (r.standard_normal(shape) * std).astype(np.float32)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32
    arrays whose values are exactly representable in bf16."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(a.shape)


def bf16_bits(a_bf16_exact: np.ndarray) -> np.ndarray:
    """The uint16 bf16 bit patterns of float32 values already rounded to bf16."""
    a = np.ascontiguousarray(a_bf16_exact, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def uniform_bytes(r: np.random.Generator, n: int) -> np.ndarray:
    """n independent uniform bytes."""
    return r.integers(0, 256, size=int(n), dtype=np.uint8)


def lognormal_f32(r: np.random.Generator, n: int, mu: float = float(np.log(0.02)),
                  sigma: float = 0.5) -> np.ndarray:
    """n lognormal(mu, sigma) draws as float32."""
    return r.lognormal(mu, sigma, size=int(n)).astype(np.float32)


def outlier_weights_f32(r: np.random.Generator, shape, std: float = 0.02,
                        p: float = 0.01, factor: float = 10.0) -> np.ndarray:
    """Weights N(0, std^2); each entry independently multiplied by `factor` with
    probability p. The normal draws come first, then the outlier mask."""
    w = r.standard_normal(shape) * std
    mask = r.random(shape) < p
    w = np.where(mask, w * factor, w)
    return w.astype(np.float32)
