"""Seeded synthetic inputs for the GKA forward (shared by the tests, the bench and the oracle checks).

This module only draws random numbers and prepares them the way a caller of the layer would
(unit-norm queries and keys, sigmoid gates, rounding to the storage dtype). It holds none of
the layer's own arithmetic: no state recurrence, no solve, no output.

The five workloads mirror the pages' setting. The prefill shape B=8, T=2048, H=8, D=128 is
the "random regression setup" of Fig. 1(a) on the pith.science page (caption of Figure 1) and
of the "Main Findings" list of the ai.info summary. The gate values a in {0.1, 0.05, 0.02} are
among those studied in Fig. 9 (pith.science page, caption of Figure 9). The pages use no dataset
for the forward itself, so every input is drawn here:

  * every (batch row b, head h) and every block of 4096 tokens j has its own PCG64 stream,
    keyed [seed, tag, b, h, j] (tag 0 = prefill, 1 = decode warm-up, 2 = decode steps); from
    it q, k, v ~ N(0, 1) of shape [tokens, D] are drawn in that order (float64), then the gate
    pre-activations z ~ N(mu, sd) of shape [tokens]; gate gamma = sigmoid(z) stored as float32;
  * q and k are divided by their L2 norm over D (the block's l2 normalisation, caption of
    Figure 2 on the pith.science page, is the caller's job);
  * bf16 workloads round q, k, v float64 -> float32 -> bfloat16 (round to nearest even);
  * the optional write gates beta_t (the beta-augmented recurrence) come from streams of their
    own: beta = sigmoid(z), z ~ N(0, 2), stored as float32, which spreads them over (0, 1).

The arrays returned are float64 copies of exactly the values the device receives (the decode
step arrays are float32, which holds every bf16 value exactly). Independent streams per head
let a test regenerate the heads it samples without drawing the rest, and let the full draws run
on a thread pool.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

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
    # a serving step on a packed batch: 8 prompts of 256..2048 tokens and 56 decode rows, each
    # continuing a state built from `warmup` tokens (lengths from varlen_lengths)
    "varlen_b64_h8_d128": Workload("varlen_b64_h8_d128", B=64, T=2048, H=8, D=128, chunk=64,
                                   gate_mu=3.0, gate_sd=1.0, a=0.05, iters=10, dtype="bf16",
                                   seed=6, warmup=64, steps=1),
}


def varlen_lengths(w: Workload):
    """Token counts of the packed serving workload, per sequence: (warm-up tokens, tokens of the
    step). Every eighth sequence is a prompt (no warm-up; length uniform in 256..T from a stream
    keyed [seed, 5]); the others decode one token after w.warmup warm-up tokens."""
    rng = np.random.default_rng([w.seed, 5])
    pre, step = [], []
    for b in range(w.B):
        if b % 8 == 0:
            pre.append(0)
            step.append(int(rng.integers(256, w.T + 1)))
        else:
            pre.append(w.warmup)
            step.append(1)
    return pre, step


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


TOKEN_BLOCK = 4096  # tokens per independent stream
TAG_PREFILL, TAG_WARMUP, TAG_STEPS, TAG_BETA = 0, 1, 2, 3


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def draw_block(key: Sequence[int], n: int, D: int, gate_mu: float, gate_sd: float, dtype: str,
               gamma_override: Optional[float] = None):
    """One stream's tokens: q, k, v [n, D] (q, k unit-norm, rounded to dtype) and gamma [n]."""
    rng = np.random.default_rng(list(key))
    q = rng.standard_normal((n, D))
    k = rng.standard_normal((n, D))
    v = rng.standard_normal((n, D))
    z = rng.normal(gate_mu, gate_sd, n)
    q = round_to(_unit(q), dtype)
    k = round_to(_unit(k), dtype)
    v = round_to(v, dtype)
    if gamma_override is None:
        gamma = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    else:
        gamma = np.full(n, gamma_override, dtype=np.float32)
    return q, k, v, gamma.astype(np.float64)


def _draw_grid(tag: int, cells: List[Tuple[int, int, int, int]], R: int, C: int, T: int, D: int,
               gate_mu: float, gate_sd: float, dtype: str, seed: int,
               gamma_override: Optional[float] = None, out_dtype=np.float64,
               time_major: bool = False):
    """Draw the streams of the cells (r, c, b, h) -- output slot (r, c), stream of head (b, h) --
    into q, k, v [R, T, C, D] and gamma [R, T, C] ([T, R, C, ...] if ``time_major``)."""
    lead = (T, R, C) if time_major else (R, T, C)
    q, k, v = (np.empty(lead + (D,), dtype=out_dtype) for _ in range(3))
    g = np.empty(lead, dtype=np.float64)
    jobs = [(cell, t0) for cell in cells for t0 in range(0, T, TOKEN_BLOCK)]

    def run(job):
        (r, c, b, h), t0 = job
        n = min(TOKEN_BLOCK, T - t0)
        blk = draw_block((seed, tag, b, h, t0 // TOKEN_BLOCK), n, D, gate_mu, gate_sd, dtype,
                         gamma_override)
        idx = (slice(t0, t0 + n), r, c) if time_major else (r, slice(t0, t0 + n), c)
        for dst, src in zip((q, k, v, g), blk):
            dst[idx] = src

    if len(jobs) == 1:
        run(jobs[0])
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(run, jobs))
    return q, k, v, g


def make_prefill(B: int, T: int, H: int, D: int, gate_mu: float, gate_sd: float, dtype: str,
                 seed: int, gamma_override: Optional[float] = None,
                 heads: Optional[Sequence[Tuple[int, int]]] = None):
    """Inputs for one prefill call: q, k, v [B,T,H,D] and gamma [B,T,H], as float64 arrays.

    With ``heads`` (a list of (b, h) pairs) only those heads are drawn and the arrays are
    [1, T, P, D] / [1, T, P], holding exactly the values of those heads in the full draw.
    """
    if heads is None:
        cells = [(b, h, b, h) for b in range(B) for h in range(H)]
        return _draw_grid(TAG_PREFILL, cells, B, H, T, D, gate_mu, gate_sd, dtype, seed,
                          gamma_override)
    cells = [(0, i, b, h) for i, (b, h) in enumerate(heads)]
    return _draw_grid(TAG_PREFILL, cells, 1, len(cells), T, D, gate_mu, gate_sd, dtype, seed,
                      gamma_override)


def make_beta(B: int, T: int, H: int, seed: int, beta_mu: float = 0.0, beta_sd: float = 2.0,
              heads: Optional[Sequence[Tuple[int, int]]] = None) -> np.ndarray:
    """Write gates beta_t = sigmoid(z), z ~ N(beta_mu, beta_sd), stored as float32 (returned as
    float64 copies): [B, T, H], or [1, T, P] for the sampled ``heads``. Each head and block of
    TOKEN_BLOCK tokens has its own stream keyed [seed, TAG_BETA, b, h, j], so the gates of a
    head do not depend on which other heads are drawn, and q, k, v, gamma are unchanged."""
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    out = np.empty((len(pairs), T), dtype=np.float64)
    for i, (b, h) in enumerate(pairs):
        for t0 in range(0, T, TOKEN_BLOCK):
            n = min(TOKEN_BLOCK, T - t0)
            z = np.random.default_rng([seed, TAG_BETA, b, h, t0 // TOKEN_BLOCK]).normal(
                beta_mu, beta_sd, n)
            out[i, t0:t0 + n] = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    if heads is None:
        return np.ascontiguousarray(out.reshape(B, H, T).transpose(0, 2, 1))
    return np.ascontiguousarray(out.T[None])


def make_varlen(lengths: Sequence[int], H: int, D: int, gate_mu: float, gate_sd: float,
                dtype: str, seed: int):
    """A packed batch of sequences with the given lengths: q, k, v [total, H, D], gamma
    [total, H] (float64 copies of the device values, as make_prefill) and the offsets cu
    (int32 [B + 1], sequence b = rows cu[b]..cu[b+1]). Sequence b is make_prefill's single row
    with seed = 1000 seed + b, so any one sequence can be redrawn on its own."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    total = int(cu[-1])
    q, k, v = (np.zeros((total, H, D)) for _ in range(3))
    g = np.zeros((total, H))
    for b, L in enumerate(lengths):
        if L == 0:
            continue
        qb, kb, vb, gb = make_prefill(1, L, H, D, gate_mu, gate_sd, dtype, 1000 * seed + b)
        sl = slice(int(cu[b]), int(cu[b + 1]))
        q[sl], k[sl], v[sl], g[sl] = qb[0], kb[0], vb[0], gb[0]
    return q, k, v, g, cu


def make_workload(w: Workload, T: Optional[int] = None, B: Optional[int] = None,
                  heads: Optional[Sequence[Tuple[int, int]]] = None):
    """Prefill inputs for a named workload (optionally fewer tokens or rows, or sampled heads)."""
    return make_prefill(B or w.B, T or w.T, w.H, w.D, w.gate_mu, w.gate_sd, w.dtype, w.seed,
                        heads=heads)


def make_decode_warmup(w: Workload, rows: Optional[Sequence[int]] = None):
    """Warm-up tokens [R, warmup, H, D] (R = len(rows), default all rows) that build the
    carried state before decoding."""
    rows = list(range(w.B)) if rows is None else list(rows)
    cells = [(i, h, b, h) for i, b in enumerate(rows) for h in range(w.H)]
    return _draw_grid(TAG_WARMUP, cells, len(rows), w.H, w.warmup, w.D, w.gate_mu, w.gate_sd,
                      w.dtype, w.seed)


def make_decode_steps(w: Workload, steps: Optional[int] = None,
                      rows: Optional[Sequence[int]] = None):
    """Inputs of ``steps`` recurrent steps: q, k, v [steps, R, H, D] float32 and gamma
    [steps, R, H] float64, for rows ``rows`` (default all rows). Step s of row b is the
    token s of that row's own stream, so any subset of rows is drawn on its own."""
    steps = w.steps if steps is None else steps
    rows = list(range(w.B)) if rows is None else list(rows)
    cells = [(i, h, b, h) for i, b in enumerate(rows) for h in range(w.H)]
    return _draw_grid(TAG_STEPS, cells, len(rows), w.H, steps, w.D, w.gate_mu, w.gate_sd,
                      w.dtype, w.seed, out_dtype=np.float32, time_major=True)
