"""Helpers shared by the GPU parity tests: device copies of oracle inputs and error measures."""
from __future__ import annotations

import sys

import numpy as np
import torch

from test_ridge_regression_amd import gka

TORCH_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32}
# parity bars: relative L2 of o against the oracle's Chebyshev output, and ||H_t||_F per token
TOL_O = {"bf16": 2e-2, "fp32": 1e-5}
TOL_HNORM = 1e-3
# Tripwires beside those bars: about three times the largest error the kernels show on cases of
# at least TRIP_MIN_TOKENS tokens (bf16 o 1.8e-3, float32 o 6.2e-7; ||H_t||_F 2.1e-4 on the
# write-gated C = 32 path, 2e-5 elsewhere). With fewer tokens a handful of bf16 roundings of o
# decide the figure (6.1e-3 for one token of D = 32), so only the bars apply there. A change
# that makes the kernels several times less accurate fails here, far inside the bars.
TRIP_O = {"bf16": 6e-3, "fp32": 2e-6}
TRIP_HNORM = 6e-4
TRIP_MIN_TOKENS = 64


def tripwire(e_o: float, e_hnorm: float, dtype: str, tokens: int, what: str = ""):
    """Assert the tripwire bars on a parity case's relative L2 of o and ||H_t||_F error."""
    if tokens >= TRIP_MIN_TOKENS:
        assert e_o <= TRIP_O[dtype], f"{what}: rel_l2(o) {e_o:.3e} above the tripwire"
    assert e_hnorm <= TRIP_HNORM, f"{what}: ||H_t||_F error {e_hnorm:.3e} above the tripwire"


def log(msg: str):
    """Name the case on stderr before each GPU step (a fault then still says where it was)."""
    sys.stderr.write(f"[gka-test] {msg}\n")
    sys.stderr.flush()


def dev(x: np.ndarray, dtype: str = "fp32") -> torch.Tensor:
    """Exact device copy of a float64 array whose values are representable in ``dtype``."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")
    return t.to(TORCH_DTYPE[dtype]).contiguous()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got))


def max_rel(got: np.ndarray, ref: np.ndarray, floor: float = 1e-30) -> float:
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), floor)))


def worst_head_rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    """Worst relative L2 over (batch, head) slices of [B, T, H, D] arrays."""
    B, _, H, _ = ref.shape
    return max(rel_l2(got[b, :, h], ref[b, :, h]) for b in range(B) for h in range(H))


def state_to_dev(h, u, n2) -> gka.GkaState:
    return gka.GkaState(dev(h), dev(u), dev(n2))


def run_prefill(q, k, v, g, a, iters, chunk, dtype, state=None, segments=0, return_hnorm=True,
                beta=None):
    """Run gka_fwd_chunked (gka_fwd_chunked_beta with ``beta``) on device copies of float64
    inputs; returns numpy results."""
    st = None if state is None else state_to_dev(*state)
    out = gka.fwd_chunked(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(g), a, iters, chunk,
                          state=st, return_hnorm=return_hnorm, segments=segments,
                          beta=None if beta is None else dev(beta))
    torch.cuda.synchronize()
    o, hn = out if return_hnorm else (out, None)
    res = dict(o=host(o), hnorm=None if hn is None else host(hn))
    if st is not None:
        res.update(h=host(st.h), u=host(st.u), n2=host(st.n2))
    return res
