"""GPU parity of the backward pass (gka_bwd) against the float64 oracle's gradients by implicit
differentiation (gka_backward_ref, Chebyshev mode: the same solver as the forward).

Bars: the kernels compute in float32 from the exact input values, so a gradient's relative
error is about kappa T u (kappa <= (1 + a) / a = 21 at a = 0.05, T <= 70 tokens here, u = 2^-24):
1e-4 relative L2 for every float32 output (all gradients of float32 inputs; dgamma and dbeta
always). dq, dk, dv of bf16 inputs are rounded to bf16: 2e-2, the bar of the forward's output.
"""
import numpy as np
import pytest
import torch

from oracle import gka_backward_ref
from test_ridge_regression_amd import gka
from test_ridge_regression_amd import workloads as W

from gka_testutil import dev, host, log, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    gka.load()


def run(q, k, v, g, do, a, iters, dtype, beta=None):
    out = gka.bwd(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(g), dev(do, dtype), a, iters,
                  beta=None if beta is None else dev(beta))
    torch.cuda.synchronize()
    return dict(zip(("dq", "dk", "dv", "dgamma", "dbeta"), (host(x) for x in out)))


def check(got, ref, dtype, what, gated=True):
    bars = {"dq": 2e-2 if dtype == "bf16" else 1e-4, "dk": 2e-2 if dtype == "bf16" else 1e-4,
            "dv": 2e-2 if dtype == "bf16" else 1e-4, "dgamma": 1e-4, "dbeta": 1e-4}
    errs = {n: rel_l2(got[n], ref[n]) for n in bars}
    log(what + ": " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert np.all(np.isfinite(got[n])), (what, n)
        assert e <= bars[n], (what, n, e)


@pytest.mark.parametrize("dtype,D", [("fp32", 16), ("fp32", 32), ("fp32", 64), ("fp32", 128),
                                     ("bf16", 16), ("bf16", 32), ("bf16", 64), ("bf16", 128)])
@pytest.mark.parametrize("gated", [False, True])
def test_backward_parity(dtype, D, gated):
    B, T, H = 2, 37, 2
    q, k, v, g = W.make_prefill(B, T, H, D, 3.0, 1.0, dtype, seed=1100 + D)
    do = W.make_prefill(B, T, H, D, 0.0, 1.0, dtype, seed=1101 + D)[2]  # values ~ N(0, 1)
    beta = W.make_beta(B, T, H, 1102 + D) if gated else None
    log(f"backward {dtype} D={D} beta={gated}")
    ref = gka_backward_ref(q, k, v, g, do, 0.05, 10, beta=beta)
    got = run(q, k, v, g, do, 0.05, 10, dtype, beta=beta)
    check(got, ref, dtype, f"backward {dtype} D={D} beta={gated}")


@pytest.mark.parametrize("iters", [1, 2, 5])
def test_backward_iteration_counts_and_zero_keys(iters):
    B, T, H, D = 1, 70, 2, 64
    q, k, v, g = W.make_prefill(B, T, H, D, 2.0, 1.0, "fp32", seed=1110 + iters)
    k[0, :3, 1] = 0.0  # ||H_t|| = 0 for the first tokens of head 1: dq_t = 0
    do = W.make_prefill(B, T, H, D, 0.0, 1.0, "fp32", seed=1111)[2]
    ref = gka_backward_ref(q, k, v, g, do, 0.1, iters)
    log(f"backward iters={iters} with zero keys")
    got = run(q, k, v, g, do, 0.1, iters, "fp32")
    check(got, ref, "fp32", f"backward iters={iters}")
    assert np.all(got["dq"][0, :3, 1] == 0.0)


@pytest.mark.slow
def test_backward_at_the_figure_shape_sampled():
    """B8 T2048 H8 D128 (bf16): all heads on the GPU, 2 heads against the oracle."""
    w = W.WORKLOADS["prefill_b8_t2048_h8_d128"]
    q, k, v, g = W.make_workload(w)
    do = W.make_prefill(w.B, w.T, w.H, w.D, 0.0, 1.0, "bf16", seed=1120)[2]
    log("backward B8 T2048 H8 D128")
    got = run(q, k, v, g, do, w.a, w.iters, "bf16")
    for b, h in ((0, 0), (5, 3)):
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        ref = gka_backward_ref(q[sl], k[sl], v[sl], g[sl], do[sl], w.a, w.iters)
        check({n: got[n][sl] for n in got}, ref, "bf16", f"figure shape head ({b}, {h})")


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("fp32", 64), ("fp32", 128)])
def test_backward_several_chunks_with_write_gate(dtype, D):
    # 4 chunks of 64 (16 chunks of 16 for float32 D = 128) and a ragged tail: the chunk-start
    # states of the forward scan and the incoming gradients of the reverse scan
    B, T, H = 1, 230, 2
    q, k, v, g = W.make_prefill(B, T, H, D, 2.0, 1.0, dtype, seed=1130 + D)
    g[0, 100:110, 0] = 0.0  # gates of 0 inside a chunk and across the reverse scan
    do = W.make_prefill(B, T, H, D, 0.0, 1.0, dtype, seed=1131)[2]
    beta = W.make_beta(B, T, H, 1132)
    ref = gka_backward_ref(q, k, v, g, do, 0.05, 10, beta=beta)
    log(f"backward several chunks {dtype} D={D}")
    got = run(q, k, v, g, do, 0.05, 10, dtype, beta=beta)
    check(got, ref, dtype, f"backward several chunks {dtype} D={D}")
