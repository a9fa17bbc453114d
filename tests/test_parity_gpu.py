"""GPU parity: the HIP path (through the C ABI) against the float64 oracle, element by element.

Bars: relative L2 of o <= 2e-2 for bf16 and <= 1e-5 for fp32 (against the oracle's Chebyshev
output with the same iteration count), and ||H_t||_F within 1e-3 relative per token.
"""
import numpy as np
import pytest
import torch

from oracle import gka_forward_ref, gka_step_ref
from test_ridge_regression_amd import gka
from test_ridge_regression_amd import workloads as W

from gka_testutil import (TOL_HNORM, TOL_O, dev, host, log, max_rel, rel_l2, run_prefill,
                          tripwire, worst_head_rel_l2)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    gka.load()


def zero_state(B, H, D):
    return np.zeros((B, H, D, D)), np.zeros((B, H, D, D)), np.zeros((B, H))


def inputs(B, T, H, D, dtype, seed, mu=3.0, sd=1.0):
    return W.make_prefill(B, T, H, D, mu, sd, dtype, seed)


def check_prefill(got, ref, dtype, what=""):
    e = rel_l2(got["o"], ref["o"])
    eh = max_rel(got["hnorm"], ref["hnorm"])
    log(f"{what}: rel_l2(o)={e:.3e} max_rel(hnorm)={eh:.3e}")
    assert np.all(np.isfinite(got["o"]))
    assert e <= TOL_O[dtype], what
    assert eh <= TOL_HNORM, what
    tripwire(e, eh, dtype, got["o"].shape[1], what)


# ------------------------------------------------------------------------------------------
# the tiny fp32 workload: all conventions at 1e-5
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("segments", [1, 2, 4])
def test_tiny_fp32_prefill(segments):
    w = W.WORKLOADS["tiny_fp32"]
    q, k, v, g = W.make_workload(w)
    ref = gka_forward_ref(q, k, v, g, w.a, w.iters)
    log(f"tiny_fp32 prefill segments={segments}")
    got = run_prefill(q, k, v, g, w.a, w.iters, w.chunk, "fp32", state=zero_state(1, 1, w.D),
                      segments=segments)
    check_prefill(got, ref, "fp32", f"tiny_fp32 S={segments}")
    assert rel_l2(got["h"], ref["h"]) < 1e-6
    assert rel_l2(got["u"], ref["u"]) < 1e-6
    assert max_rel(got["n2"], ref["n2"]) < 1e-5


def test_tiny_fp32_as_decode_steps():
    w = W.WORKLOADS["tiny_fp32"]
    q, k, v, g = W.make_workload(w)
    ref = gka_forward_ref(q, k, v, g, w.a, w.iters)
    st = gka.GkaState.zeros(1, 1, w.D)
    outs = []
    log("tiny_fp32 as 64 gka_step calls")
    for t in range(w.T):
        o = gka.step(dev(q[:, t]), dev(k[:, t]), dev(v[:, t]), dev(g[:, t]), w.a, w.iters, st)
        outs.append(host(o))
    torch.cuda.synchronize()
    o = np.stack(outs, axis=1)
    assert rel_l2(o, ref["o"]) <= TOL_O["fp32"]
    assert max_rel(host(st.n2), ref["n2"]) < 1e-5
    assert rel_l2(host(st.h), ref["h"]) < 1e-6
    assert rel_l2(host(st.u), ref["u"]) < 1e-6


# ------------------------------------------------------------------------------------------
# chunk sizes, head sizes, segment counts, ragged lengths
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("D", [16, 32, 64])
@pytest.mark.parametrize("C", [16, 32, 64])
def test_fp32_chunk_and_head_sizes(D, C):
    T = 200  # ragged: not a multiple of any chunk size
    q, k, v, g = inputs(2, T, 3, D, "fp32", seed=10 + D + C, mu=2.0, sd=0.7)
    ref = gka_forward_ref(q, k, v, g, 0.1, 8)
    log(f"fp32 D={D} C={C} T={T}")
    got = run_prefill(q, k, v, g, 0.1, 8, C, "fp32")
    check_prefill(got, ref, "fp32", f"fp32 D={D} C={C}")


@pytest.mark.parametrize("D,C", [(32, 16), (32, 32), (32, 64), (64, 16), (64, 32), (64, 64),
                                 (128, 16), (128, 32), (128, 64)])
def test_bf16_chunk_and_head_sizes(D, C):
    T = 448
    q, k, v, g = inputs(2, T, 3, D, "bf16", seed=30 + D + C)
    ref = gka_forward_ref(q, k, v, g, 0.05, 10)
    log(f"bf16 D={D} C={C} T={T}")
    got = run_prefill(q, k, v, g, 0.05, 10, C, "bf16")
    check_prefill(got, ref, "bf16", f"bf16 D={D} C={C}")


@pytest.mark.parametrize("D", [64, 128])
def test_bf16_chunk_size_invariance(D):
    """C in {16, 32, 64} (float32 operands, the feature-split walk, the token walk) on the same
    inputs, from a carried state and in 3 segments: each against the oracle, and the final
    states against each other."""
    B, T, H = 1, 5 * 64 + 19, 2
    q, k, v, g = inputs(B, 2 * T, H, D, "bf16", seed=71 + D)
    ref = gka_forward_ref(q, k, v, g, 0.05, 10)
    warm = gka_forward_ref(q[:, :T], k[:, :T], v[:, :T], g[:, :T], 0.05, 10, mode="state")
    st = (warm["h"].astype(np.float32).astype(np.float64),
          warm["u"].astype(np.float32).astype(np.float64),
          warm["n2"].astype(np.float32).astype(np.float64))
    ref2 = gka_forward_ref(q[:, T:], k[:, T:], v[:, T:], g[:, T:], 0.05, 10, h0=st[0], u0=st[1],
                           n2_0=st[2])
    finals = []
    for C in (16, 32, 64):
        log(f"bf16 chunk invariance D={D} C={C}")
        got = run_prefill(q[:, T:], k[:, T:], v[:, T:], g[:, T:], 0.05, 10, C, "bf16", state=st,
                          segments=3)
        check_prefill(got, ref2, "bf16", f"bf16 D={D} C={C} (carried state, 3 segments)")
        finals.append(got)
        assert rel_l2(got["h"], ref["h"]) < 1e-4 and rel_l2(got["u"], ref["u"]) < 1e-4
    for other in finals[1:]:
        assert rel_l2(other["h"], finals[0]["h"]) < 1e-4
        assert rel_l2(other["u"], finals[0]["u"]) < 1e-4


@pytest.mark.parametrize("segments", [1, 2, 3, 5, 16])
def test_segment_count_invariance(segments):
    q, k, v, g = inputs(1, 1024, 2, 64, "bf16", seed=41)
    ref = gka_forward_ref(q, k, v, g, 0.05, 10, h0=None)
    log(f"bf16 segments={segments}")
    got = run_prefill(q, k, v, g, 0.05, 10, 64, "bf16", state=zero_state(1, 2, 64),
                      segments=segments)
    check_prefill(got, ref, "bf16", f"segments={segments}")
    assert rel_l2(got["h"], ref["h"]) < 1e-4
    assert rel_l2(got["u"], ref["u"]) < 1e-4
    assert max_rel(got["n2"], ref["n2"]) < 1e-3


@pytest.mark.parametrize("T", [1, 5, 31, 33, 64, 65, 127])
def test_ragged_and_short_sequences(T):
    q, k, v, g = inputs(2, T, 2, 32, "fp32", seed=50 + T, mu=2.0)
    ref = gka_forward_ref(q, k, v, g, 0.1, 6)
    log(f"fp32 ragged T={T}")
    got = run_prefill(q, k, v, g, 0.1, 6, 32, "fp32", state=zero_state(2, 2, 32))
    check_prefill(got, ref, "fp32", f"T={T}")
    assert rel_l2(got["h"], ref["h"]) < 1e-6
    assert max_rel(got["n2"], ref["n2"]) < 1e-5


def test_empty_sequence_leaves_state():
    st = gka.GkaState(torch.full((1, 2, 16, 16), 3.0, device="cuda"),
                      torch.full((1, 2, 16, 16), 4.0, device="cuda"),
                      torch.full((1, 2), 5.0, device="cuda"))
    e = torch.empty(1, 0, 2, 16, device="cuda")
    gka.fwd_chunked(e, e, e, torch.empty(1, 0, 2, device="cuda"), 0.1, 4, 16, state=st)
    torch.cuda.synchronize()
    assert torch.all(st.h == 3.0) and torch.all(st.u == 4.0) and torch.all(st.n2 == 5.0)


# ------------------------------------------------------------------------------------------
# bf16 with chunks of 64 (the token-owning walk): ragged lengths, iteration counts, states
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("T", [1, 5, 63, 65, 130])
def test_bf16_chunk64_ragged(D, T):
    q, k, v, g = inputs(2, T, 2, D, "bf16", seed=300 + T + D)
    ref = gka_forward_ref(q, k, v, g, 0.05, 10)
    log(f"bf16 C=64 ragged D={D} T={T}")
    got = run_prefill(q, k, v, g, 0.05, 10, 64, "bf16", state=zero_state(2, 2, D))
    check_prefill(got, ref, "bf16", f"bf16 C=64 D={D} T={T}")
    assert rel_l2(got["h"], ref["h"]) < 1e-4
    assert rel_l2(got["u"], ref["u"]) < 1e-4
    assert max_rel(got["n2"], ref["n2"]) < 1e-4


@pytest.mark.parametrize("iters", [1, 2, 3, 4, 11])
def test_bf16_chunk64_iteration_counts(iters):
    q, k, v, g = inputs(1, 200, 2, 64, "bf16", seed=320 + iters)
    ref = gka_forward_ref(q, k, v, g, 0.1, iters)
    log(f"bf16 C=64 iters={iters}")
    got = run_prefill(q, k, v, g, 0.1, iters, 64, "bf16")
    check_prefill(got, ref, "bf16", f"bf16 C=64 iters={iters}")


@pytest.mark.parametrize("D", [64, 128])
def test_bf16_chunk64_nonzero_initial_state(D):
    T = 300
    rng = np.random.default_rng(330 + D)
    Z = rng.standard_normal((1, 2, D, 2 * D))
    h0 = (Z @ np.swapaxes(Z, -1, -2) / D).astype(np.float32).astype(np.float64)
    u0 = rng.standard_normal((1, 2, D, D)).astype(np.float32).astype(np.float64)
    n20 = np.sum(h0 * h0, axis=(-1, -2))
    q, k, v, g = inputs(1, T, 2, D, "bf16", seed=331 + D)
    ref = gka_forward_ref(q, k, v, g, 0.05, 10, h0=h0, u0=u0, n2_0=n20)
    for seg in (1, 3):
        log(f"bf16 C=64 nonzero initial state D={D} segments={seg}")
        got = run_prefill(q, k, v, g, 0.05, 10, 64, "bf16", state=(h0, u0, n20), segments=seg)
        check_prefill(got, ref, "bf16", f"bf16 initial state D={D} S={seg}")
        assert rel_l2(got["h"], ref["h"]) < 1e-4
        assert rel_l2(got["u"], ref["u"]) < 1e-4
        assert max_rel(got["n2"], ref["n2"]) < 1e-4


# ------------------------------------------------------------------------------------------
# carried state: split calls, initial states, prefill -> decode hand-off
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,D,C", [("fp32", 32, 16), ("bf16", 128, 64)])
def test_split_calls_carry_the_state(dtype, D, C):
    T1, T2 = 192, 333
    q, k, v, g = inputs(2, T1 + T2, 2, D, dtype, seed=60 + D)
    ref = gka_forward_ref(q, k, v, g, 0.05, 10)
    log(f"split calls {dtype} D={D}")
    st = gka.GkaState.zeros(2, 2, D)
    o1 = gka.fwd_chunked(dev(q[:, :T1], dtype), dev(k[:, :T1], dtype), dev(v[:, :T1], dtype),
                         dev(g[:, :T1]), 0.05, 10, C, state=st)
    o2 = gka.fwd_chunked(dev(q[:, T1:], dtype), dev(k[:, T1:], dtype), dev(v[:, T1:], dtype),
                         dev(g[:, T1:]), 0.05, 10, C, state=st)
    torch.cuda.synchronize()
    o = np.concatenate([host(o1), host(o2)], axis=1)
    assert rel_l2(o, ref["o"]) <= TOL_O[dtype]
    assert max_rel(host(st.n2), ref["n2"]) < 1e-4
    assert rel_l2(host(st.h), ref["h"]) < (1e-6 if dtype == "fp32" else 1e-4)


def test_nonzero_initial_state_fp32():
    D, T = 32, 96
    rng = np.random.default_rng(70)
    Z = rng.standard_normal((1, 2, D, 2 * D))
    h0 = (Z @ np.swapaxes(Z, -1, -2) / D).astype(np.float32).astype(np.float64)
    u0 = rng.standard_normal((1, 2, D, D)).astype(np.float32).astype(np.float64)
    n20 = np.sum(h0 * h0, axis=(-1, -2))
    q, k, v, g = inputs(1, T, 2, D, "fp32", seed=71, mu=2.0)
    ref = gka_forward_ref(q, k, v, g, 0.1, 8, h0=h0, u0=u0, n2_0=n20)
    for seg in (1, 3):
        log(f"fp32 nonzero initial state segments={seg}")
        got = run_prefill(q, k, v, g, 0.1, 8, 16, "fp32", state=(h0, u0, n20), segments=seg)
        check_prefill(got, ref, "fp32", f"initial state S={seg}")
        assert rel_l2(got["h"], ref["h"]) < 1e-6
        assert rel_l2(got["u"], ref["u"]) < 1e-6


@pytest.mark.parametrize("dtype,D,C", [("fp32", 64, 16), ("bf16", 128, 32), ("bf16", 128, 64)])
def test_prefill_then_step_equals_longer_prefill(dtype, D, C):
    T = 160
    q, k, v, g = inputs(2, T + 3, 2, D, dtype, seed=80 + D)
    ref = gka_forward_ref(q, k, v, g, 0.05, 10)
    log(f"prefill -> step {dtype} D={D}")
    st = gka.GkaState.zeros(2, 2, D)
    gka.fwd_chunked(dev(q[:, :T], dtype), dev(k[:, :T], dtype), dev(v[:, :T], dtype),
                    dev(g[:, :T]), 0.05, 10, C, state=st)
    outs = []
    for t in range(T, T + 3):
        outs.append(host(gka.step(dev(q[:, t], dtype), dev(k[:, t], dtype), dev(v[:, t], dtype),
                                  dev(g[:, t]), 0.05, 10, st)))
    torch.cuda.synchronize()
    o = np.stack(outs, axis=1)
    assert rel_l2(o, ref["o"][:, T:]) <= TOL_O[dtype]
    assert max_rel(host(st.n2), ref["n2"]) < 1e-4


# ------------------------------------------------------------------------------------------
# degenerate cases
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,D,C", [("fp32", 16, 16), ("bf16", 64, 32), ("bf16", 128, 64)])
def test_gamma_zero_closed_form(dtype, D, C):
    """gamma = 0 and unit keys: o_t = (1 - (-1)^r / T_r(1+2a)) v_t (k_t . q_t) / (1 + a)."""
    a, r = 0.05, 7
    q, k, v, _ = inputs(2, 100, 2, D, dtype, seed=90)
    g = np.zeros(q.shape[:-1])
    fac = 1 - (-1) ** r / np.polynomial.chebyshev.chebval(1 + 2 * a, [0] * r + [1])
    kk = np.sum(k * k, -1)
    expect = fac * v * (np.sum(k * q, -1) / ((1 + a) * kk))[..., None]
    log(f"gamma = 0 {dtype}")
    got = run_prefill(q, k, v, g, a, r, C, dtype)
    assert rel_l2(got["o"], expect) <= TOL_O[dtype]
    np.testing.assert_allclose(got["hnorm"], kk, rtol=1e-5)
    st = gka.GkaState.zeros(2, 2, D)
    o = host(gka.step(dev(q[:, 0], dtype), dev(k[:, 0], dtype), dev(v[:, 0], dtype),
                      dev(g[:, 0]), a, r, st))
    assert rel_l2(o, expect[:, 0]) <= TOL_O[dtype]


@pytest.mark.parametrize("dtype,D,C", [("fp32", 32, 32), ("bf16", 64, 32), ("bf16", 64, 64)])
def test_zero_keys_give_zero_output(dtype, D, C):
    q, k, v, g = inputs(1, 96, 2, D, dtype, seed=95)
    k[:, :40] = 0.0  # ||H_t|| = 0 for the first 40 tokens
    ref = gka_forward_ref(q, k, v, g, 0.1, 8)
    log(f"zero keys {dtype}")
    got = run_prefill(q, k, v, g, 0.1, 8, C, dtype)
    assert np.all(np.isfinite(got["o"]))
    assert np.all(got["o"][:, :40] == 0.0)
    assert np.all(got["hnorm"][:, :40] == 0.0)
    assert rel_l2(got["o"], ref["o"]) <= TOL_O[dtype]
    st = gka.GkaState.zeros(1, 2, D)
    o = host(gka.step(dev(q[:, 0], dtype), dev(k[:, 0], dtype), dev(v[:, 0], dtype),
                      dev(g[:, 0]), 0.1, 8, st))
    assert np.all(o == 0.0) and np.all(host(st.n2) == 0.0)


def test_single_iteration():
    q, k, v, g = inputs(1, 64, 2, 64, "fp32", seed=97, mu=2.0)
    ref = gka_forward_ref(q, k, v, g, 0.1, 1)
    log("iters = 1")
    got = run_prefill(q, k, v, g, 0.1, 1, 32, "fp32")
    check_prefill(got, ref, "fp32", "iters=1")


def test_bitwise_deterministic():
    q, k, v, g = inputs(2, 512, 4, 128, "bf16", seed=99)
    args = (dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(g))
    log("determinism")
    o1 = gka.fwd_chunked(*args, 0.05, 10, 64, segments=4)
    o2 = gka.fwd_chunked(*args, 0.05, 10, 64, segments=4)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("a", [3.0, 1e2, 1e4, 1e6])
@pytest.mark.parametrize("dtype,D,C", [("bf16", 128, 64), ("bf16", 64, 32), ("fp32", 32, 16)])
def test_large_ridge_scale(dtype, D, C, a):
    # the iterate is about |q| / a: for large a it would fall below the normal range of the fp16
    # operands of the output products, so it is formed times a power of two near a
    q, k, v, g = inputs(2, 150, 2, D, dtype, seed=900 + D)
    ref = gka_forward_ref(q, k, v, g, a, 8)
    log(f"large a={a:g} {dtype} D={D} C={C}")
    got = run_prefill(q, k, v, g, a, 8, C, dtype, segments=2)
    check_prefill(got, ref, dtype, f"a={a:g} {dtype} D={D} C={C}")


@pytest.mark.parametrize("dtype,D,C", [("bf16", 16, 32), ("bf16", 16, 64), ("fp32", 128, 16)])
@pytest.mark.parametrize("T", [37, 200])
def test_head_sizes_16_and_128_with_state(dtype, D, C, T):
    # bf16 with D = 16 (float32 operands) and float32 with D = 128 (chunks of 16)
    rng = np.random.default_rng(950 + D + T)
    Z = rng.standard_normal((2, 2, D, 2 * D))
    h0 = (Z @ np.swapaxes(Z, -1, -2) / D).astype(np.float32).astype(np.float64)
    u0 = rng.standard_normal((2, 2, D, D)).astype(np.float32).astype(np.float64)
    n20 = np.sum(h0 * h0, axis=(-1, -2))
    q, k, v, g = inputs(2, T, 2, D, dtype, seed=951 + D + T)
    ref = gka_forward_ref(q, k, v, g, 0.05, 10, h0=h0, u0=u0, n2_0=n20)
    for seg in (1, 3):
        log(f"{dtype} D={D} C={C} T={T} segments={seg}")
        got = run_prefill(q, k, v, g, 0.05, 10, C, dtype, state=(h0, u0, n20), segments=seg)
        check_prefill(got, ref, dtype, f"{dtype} D={D} C={C} T={T} S={seg}")
        tol = 1e-6 if dtype == "fp32" else 1e-5
        assert rel_l2(got["h"], ref["h"]) < tol and rel_l2(got["u"], ref["u"]) < tol
    # and a decode step continuing the state
    st = gka.GkaState(dev(ref["h"]), dev(ref["u"]), dev(ref["n2"]))
    q1, k1, v1, g1 = (x[:, 0] for x in inputs(2, 1, 2, D, dtype, seed=952 + D))
    o1 = host(gka.step(dev(q1, dtype), dev(k1, dtype), dev(v1, dtype), dev(g1), 0.05, 10, st))
    o1r, *_ = gka_step_ref(q1, k1, v1, g1, 0.05, 10, ref["h"].astype(np.float32),
                           ref["u"].astype(np.float32), ref["n2"].astype(np.float32))
    assert rel_l2(o1, o1r) <= TOL_O[dtype]
