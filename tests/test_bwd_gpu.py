"""GPU parity of the backward pass (gka_bwd) against the float64 oracle's gradients by implicit
differentiation (gka_backward_ref, Chebyshev mode: the same solver as the forward).

Bars, from the arithmetic of each path:
- float32 inputs take the vector sweeps, which compute in float32 from the exact input values.
  A gradient's relative error is then about kappa T u (kappa <= (1 + a) / a = 21 at a = 0.05,
  T <= 70 tokens here, u = 2^-24): 1e-4 relative L2 for every output. bf16 inputs with D = 16
  take the same sweeps: 1e-4 for dgamma and dbeta, 2e-2 for dq, dk, dv (their bf16 rounding).
- bf16 inputs with D = 32, 64, 128 take the matrix-core chunk form. It computes on fp16 operands
  (exact power-of-two scales, u = 2^-11) with float32 accumulation, through the forward walk's
  solves, so every gradient carries the forward's operand rounding: 2e-2, the bar of the
  forward's bf16 output, for all five. Tripwires at about 3x the errors measured on these
  inputs (dq 1.7e-3, the bf16 rounding of y; dk 4.6e-3; dv 2.2e-3; dgamma 2.0e-3; dbeta
  1.7e-3) catch a regression long before the bar.
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


# float32 outputs of the vector sweeps (all gradients of float32 inputs; dgamma, dbeta of bf16 D =
# 16) and the bf16 bar of the forward
BAR_F32, BAR_BF16 = 1e-4, 2e-2
TRIP_MFMA = {"dq": 6e-3, "dk": 1.5e-2, "dv": 7e-3, "dgamma": 7e-3, "dbeta": 6e-3}


def check(got, ref, dtype, what, D):
    mfma = dtype == "bf16" and D >= 32
    if mfma:
        bars = {n: BAR_BF16 for n in TRIP_MFMA}
    else:
        low = BAR_BF16 if dtype == "bf16" else BAR_F32
        bars = {"dq": low, "dk": low, "dv": low, "dgamma": BAR_F32, "dbeta": BAR_F32}
    errs = {n: rel_l2(got[n], ref[n]) for n in bars}
    log(what + ": " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert np.all(np.isfinite(got[n])), (what, n)
        assert e <= bars[n], (what, n, e)
        if mfma:
            assert e <= TRIP_MFMA[n], f"{what}: {n} error {e:.3e} above the tripwire"


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
    check(got, ref, dtype, f"backward {dtype} D={D} beta={gated}", D)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("iters", [1, 2, 5])
def test_backward_iteration_counts_and_zero_keys(iters, dtype):
    B, T, H, D = 1, 70, 2, 64
    q, k, v, g = W.make_prefill(B, T, H, D, 2.0, 1.0, dtype, seed=1110 + iters)
    k[0, :3, 1] = 0.0  # ||H_t|| = 0 for the first tokens of head 1: dq_t = 0
    do = W.make_prefill(B, T, H, D, 0.0, 1.0, dtype, seed=1111)[2]
    ref = gka_backward_ref(q, k, v, g, do, 0.1, iters)
    log(f"backward {dtype} iters={iters} with zero keys")
    got = run(q, k, v, g, do, 0.1, iters, dtype)
    check(got, ref, dtype, f"backward {dtype} iters={iters}", D)
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
        check({n: got[n][sl] for n in got}, ref, "bf16", f"figure shape head ({b}, {h})", w.D)


@pytest.mark.parametrize("dtype,D", [("bf16", 32), ("bf16", 64), ("bf16", 128), ("fp32", 64),
                                     ("fp32", 128)])
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
    check(got, ref, dtype, f"backward several chunks {dtype} D={D}", D)


def test_backward_many_segments_long_sequence():
    """B1 T2565 H1 D64 (bf16): 41 chunks in 14 segments of the forward's plan, so the chunk
    states come from the segment scan and the walk over each segment's chunks; zero gates at a
    segment boundary and inside a chunk, write gates."""
    B, T, H, D = 1, 64 * 40 + 5, 1, 64
    q, k, v, g = W.make_prefill(B, T, H, D, 3.0, 1.0, "bf16", seed=1140)
    g[0, [192, 193, 700], 0] = 0.0
    do = W.make_prefill(B, T, H, D, 0.0, 1.0, "bf16", seed=1141)[2]
    beta = W.make_beta(B, T, H, 1142)
    ref = gka_backward_ref(q, k, v, g, do, 0.05, 10, beta=beta)
    log("backward B1 T2565 H1 D64, many segments")
    got = run(q, k, v, g, do, 0.05, 10, "bf16", beta=beta)
    check(got, ref, "bf16", "backward many segments", D)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("sq,sk,sv,sd", [
    (0, 0, -20, 0), (0, 0, 17, 0), (0, -12, 0, 0), (0, 8, 0, 0), (-12, 0, 0, 0), (10, 0, 0, 0),
    (0, 0, 0, -20), (0, 0, 0, 17), (-6, -12, 17, 5),
])
def test_backward_power_of_two_scaled_inputs(D, sq, sk, sv, sd):
    """q, k, v and do scaled by exact powers of two across the bf16 range (the matrix-core
    path's operands carry power-of-two scales): every gradient at the bar and the tripwires."""
    B, T, H = 1, 3 * 64 + 17, 2
    q, k, v, g = W.make_prefill(B, T, H, D, 3.0, 1.0, "bf16", seed=1150 + D)
    do = W.make_prefill(B, T, H, D, 0.0, 1.0, "bf16", seed=1151 + D)[2]
    q, k, v, do = q * 2.0 ** sq, k * 2.0 ** sk, v * 2.0 ** sv, do * 2.0 ** sd
    ref = gka_backward_ref(q, k, v, g, do, 0.05, 10)
    what = f"backward D={D} scales 2^({sq}, {sk}, {sv}, {sd})"
    log(what)
    got = run(q, k, v, g, do, 0.05, 10, "bf16")
    check(got, ref, "bf16", what, D)
