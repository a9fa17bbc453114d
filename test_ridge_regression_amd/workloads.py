"""Seeded synthetic inputs for the GKA forward (shared by the tests, the bench and the oracle checks).

This module only draws random numbers and prepares them the way a caller of the layer would
(unit-norm queries and keys, sigmoid gates, rounding to the storage dtype). It holds none of
the layer's own arithmetic: no state recurrence, no solve, no output.

The five workloads mirror the pages' setting. The prefill shape B=8, T=2048, H=8, D=128 is
the "random regression setup" of Fig. 1(a) on the pith.science page (caption of Figure 1) and
of the "Main Findings" list of the ai.info summary. The gate values a in {0.1, 0.05, 0.02} are
among those studied in Fig. 9 (pith.science page, caption of Figure 9). The pages use no dataset
for the forward itself, so every input is drawn here:

  * q, k, v ~ N(0, 1) with shape [B, T, H, D] (drawn in that order, float64);
  * z ~ N(mu, sd) with shape [B, T, H], gate gamma = sigmoid(z) stored as float32;
  * q and k are divided by their L2 norm over D (the block's l2 normalisation, caption of
    Figure 2 on the pith.science page, is the caller's job);
  * bf16 workloads round q, k, v float64 -> float32 -> bfloat16 (round to nearest even).

The arrays returned are float64 copies of exactly the values the device receives.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    D: int
    chunk: int
    gate_mu: float
    gate_sd: float
    a: float
    iters: int
    dtype: str  # "fp32" or "bf16"
    seed: int
    warmup: int = 0  # decode only: warm-up tokens that build the carried state
    steps: int = 0  # decode only: recurrent steps


WORKLOADS: Dict[str, Workload] = {
    # tiny fp32 case, finished by the oracle in milliseconds
    "tiny_fp32": Workload("tiny_fp32", B=1, T=64, H=1, D=16, chunk=16, gate_mu=2.0, gate_sd=0.5,
                          a=0.1, iters=8, dtype="fp32", seed=1),
    # the pages' figure shape, bf16 training forward
    "prefill_b8_t2048_h8_d128": Workload("prefill_b8_t2048_h8_d128", B=8, T=2048, H=8, D=128,
                                         chunk=64, gate_mu=3.0, gate_sd=1.0, a=0.05, iters=10,
                                         dtype="bf16", seed=2),
    # many small heads
    "prefill_b4_t8192_h32_d64": Workload("prefill_b4_t8192_h32_d64", B=4, T=8192, H=32, D=64,
                                         chunk=64, gate_mu=3.0, gate_sd=1.0, a=0.1, iters=8,
                                         dtype="bf16", seed=3),
    # long context, long memory
    "prefill_b1_t131072_h8_d128": Workload("prefill_b1_t131072_h8_d128", B=1, T=131072, H=8,
                                           D=128, chunk=64, gate_mu=4.0, gate_sd=1.0, a=0.02,
                                           iters=12, dtype="bf16", seed=4),
    # batched recurrent decode on a carried fp32 state
    "decode_b256_h8_d128": Workload("decode_b256_h8_d128", B=256, T=1, H=8, D=128, chunk=64,
                                    gate_mu=3.0, gate_sd=1.0, a=0.05, iters=10, dtype="bf16",
                                    seed=5, warmup=512, steps=1000),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even) via float32; returns float32 values."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    bits = x32.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32).reshape(x32.shape)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x).astype(np.float64)
    if dtype == "fp32":
        return x.astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _unit(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def draw(rng: np.random.Generator, shape_btHD, gate_mu: float, gate_sd: float, dtype: str,
         gamma_override: Optional[float] = None):
    """Draw (q, k, v, gamma) in the fixed order; q/k unit-norm over the last axis."""
    q = rng.standard_normal(shape_btHD)
    k = rng.standard_normal(shape_btHD)
    v = rng.standard_normal(shape_btHD)
    z = rng.normal(gate_mu, gate_sd, shape_btHD[:-1])
    q = round_to(_unit(q), dtype)
    k = round_to(_unit(k), dtype)
    v = round_to(v, dtype)
    if gamma_override is None:
        gamma = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    else:
        gamma = np.full(z.shape, gamma_override, dtype=np.float32)
    return q, k, v, gamma.astype(np.float64)


def make_prefill(B: int, T: int, H: int, D: int, gate_mu: float, gate_sd: float, dtype: str,
                 seed: int, gamma_override: Optional[float] = None):
    """Inputs for one prefill call: q, k, v [B,T,H,D] and gamma [B,T,H], as float64 arrays."""
    rng = np.random.default_rng(seed)
    return draw(rng, (B, T, H, D), gate_mu, gate_sd, dtype, gamma_override)


def make_workload(w: Workload, T: Optional[int] = None, B: Optional[int] = None):
    """Prefill inputs for a named workload (optionally a T or B prefix-shaped variant)."""
    return make_prefill(B or w.B, T or w.T, w.H, w.D, w.gate_mu, w.gate_sd, w.dtype, w.seed)


def make_decode_warmup(w: Workload, B: Optional[int] = None):
    """Warm-up tokens [B, warmup, H, D] that build the carried state before decoding."""
    rng = np.random.default_rng([w.seed, 0])
    return draw(rng, (B or w.B, w.warmup, w.H, w.D), w.gate_mu, w.gate_sd, w.dtype)


def make_decode_step(w: Workload, step: int, B: Optional[int] = None):
    """Inputs of recurrent step ``step`` (0-based): q, k, v [B,H,D], gamma [B,H].

    Each step has its own stream (seed, step+1), so any step can be drawn on its own.
    """
    rng = np.random.default_rng([w.seed, step + 1])
    q, k, v, g = draw(rng, (B or w.B, 1, w.H, w.D), w.gate_mu, w.gate_sd, w.dtype)
    return q[:, 0], k[:, 0], v[:, 0], g[:, 0]
