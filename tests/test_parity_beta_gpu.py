"""GPU parity of the write-gated entry points (gka_fwd_chunked_beta, gka_step_beta) against the
float64 oracle with the same gates.

The write gate beta_t scales each token's write into the statistics (ai.info summary, "Main
Findings": H_t = gamma_t H_{t-1} + beta_t k_t k_t^T, U_t = gamma_t U_{t-1} + beta_t v_t k_t^T).
Bars as for the base entry points: relative L2 of o <= 2e-2 (bf16) / 1e-5 (fp32), ||H_t||_F
within 1e-3 relative per token. Gates are drawn by workloads.make_beta (sigmoid of N(0, 2),
spread over (0, 1)); some cases set whole stretches to 0 or 1.

Bars for the carried state of the bf16 paths. The token-owning walk (chunks of 64) applies the
gate through float32 weights (carry weights, the intra-chunk mask, the norm terms), so its state
is as accurate as without a gate: bars 1e-4 (measured below 1e-5). The feature-split walk
(chunks of 32) applies it as sqrt(beta_t) on the key and value rows where they become fp16
matrix operands; bf16 inputs are exact in fp16, the scaled rows are not: each element picks up a
relative rounding error of at most 2^-12, so H and U (sums of products of two such rows) carry a
relative error of up to about 2 * 2^-11 ~ 1e-3 (||H||_F^2 twice that): bars 1e-3 and 2e-3
(measured 3e-4). The output and ||H_t||_F bars are unchanged.
"""
import numpy as np
import pytest
import torch

from oracle import gka_forward_ref, gka_step_ref
from test_ridge_regression_amd import gka
from test_ridge_regression_amd import workloads as W

from gka_testutil import (TOL_HNORM, TOL_O, dev, host, log, max_rel, rel_l2, run_prefill,
                          tripwire)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    gka.load()


def zero_state(B, H, D):
    return np.zeros((B, H, D, D)), np.zeros((B, H, D, D)), np.zeros((B, H))


def gated_inputs(B, T, H, D, dtype, seed, mu=3.0, sd=1.0):
    q, k, v, g = W.make_prefill(B, T, H, D, mu, sd, dtype, seed)
    return q, k, v, g, W.make_beta(B, T, H, seed)


# relative bars of the carried state (H, U) and of ||H||_F^2 by dtype and chunk (see the module
# docstring)
TOL_STATE = {("fp32", 16): 1e-6, ("fp32", 32): 1e-6, ("fp32", 64): 1e-6,
             ("bf16", 64): 1e-4, ("bf16", 32): 1e-3}
TOL_N2 = {("fp32", 16): 1e-5, ("fp32", 32): 1e-5, ("fp32", 64): 1e-5,
          ("bf16", 64): 1e-4, ("bf16", 32): 2e-3}


def check(got, ref, dtype, what, state=False, chunk=64):
    e = rel_l2(got["o"], ref["o"])
    eh = max_rel(got["hnorm"], ref["hnorm"])
    msg = f"{what}: rel_l2(o)={e:.3e} max_rel(hnorm)={eh:.3e}"
    if state:
        eH, eU = rel_l2(got["h"], ref["h"]), rel_l2(got["u"], ref["u"])
        en = max_rel(got["n2"], ref["n2"])
        msg += f" state H {eH:.3e} U {eU:.3e} n2 {en:.3e}"
    log(msg)
    assert np.all(np.isfinite(got["o"]))
    assert e <= TOL_O[dtype], what
    assert eh <= TOL_HNORM, what
    tripwire(e, eh, dtype, got["o"].shape[1], what)
    if state:
        assert eH < TOL_STATE[dtype, chunk] and eU < TOL_STATE[dtype, chunk], what
        assert en < TOL_N2[dtype, chunk], what


# the token-owning walk (bf16, chunks of 64) with its summaries, ragged lengths, segment counts
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("T", [65, 333])
def test_beta_bf16_chunk64(D, T):
    q, k, v, g, bt = gated_inputs(2, T, 2, D, "bf16", seed=500 + T + D)
    ref = gka_forward_ref(q, k, v, g, 0.05, 10, beta=bt)
    for seg in (1, 3):
        log(f"beta bf16 C=64 D={D} T={T} segments={seg}")
        got = run_prefill(q, k, v, g, 0.05, 10, 64, "bf16", state=zero_state(2, 2, D),
                          segments=seg, beta=bt)
        check(got, ref, "bf16", f"beta bf16 C=64 D={D} T={T} S={seg}", state=True)


# calls from the zero state with 2..4 segments: each walk workgroup composes its segment-start
# state from the summaries before it (no scan); D = 32 takes its summaries from the
# feature-split summary kernel
@pytest.mark.parametrize("D", [32, 128])
def test_beta_bf16_composed_segment_starts(D):
    T = 4 * 64 + 23
    q, k, v, g, bt = gated_inputs(2, T, 2, D, "bf16", seed=560 + D)
    ref = gka_forward_ref(q, k, v, g, 0.05, 10, beta=bt)
    for seg in (2, 3, 4):
        log(f"beta bf16 composed starts D={D} segments={seg}")
        got = run_prefill(q, k, v, g, 0.05, 10, 64, "bf16", segments=seg, beta=bt)
        check(got, ref, "bf16", f"beta bf16 composed starts D={D} S={seg}")


# the feature-split walk and summary: float32 inputs, and bf16 with chunks of 32
@pytest.mark.parametrize("dtype,D,C", [("fp32", 16, 16), ("fp32", 32, 32), ("fp32", 64, 64),
                                       ("bf16", 64, 32), ("bf16", 128, 32)])
def test_beta_feature_split(dtype, D, C):
    T = 150
    q, k, v, g, bt = gated_inputs(2, T, 2, D, dtype, seed=520 + D + C, mu=2.0)
    ref = gka_forward_ref(q, k, v, g, 0.1, 8, beta=bt)
    for seg in (1, 3):
        log(f"beta {dtype} D={D} C={C} segments={seg}")
        got = run_prefill(q, k, v, g, 0.1, 8, C, dtype, state=zero_state(2, 2, D), segments=seg,
                          beta=bt)
        check(got, ref, dtype, f"beta {dtype} D={D} C={C} S={seg}", state=True, chunk=C)


@pytest.mark.parametrize("dtype,D,C", [("bf16", 128, 64), ("bf16", 64, 32), ("fp32", 32, 16)])
def test_beta_ones_is_bitwise_the_base_call(dtype, D, C):
    T = 300
    q, k, v, g = W.make_prefill(1, T, 2, D, 3.0, 1.0, dtype, seed=540 + D)
    ones = torch.ones(1, T, 2, device="cuda", dtype=torch.float32)
    args = (dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(g), 0.05, 10, C)
    for seg in (1, 3):
        log(f"beta = 1 vs base {dtype} D={D} C={C} segments={seg}")
        s0, s1 = gka.GkaState.zeros(1, 2, D), gka.GkaState.zeros(1, 2, D)
        o0, h0 = gka.fwd_chunked(*args, state=s0, return_hnorm=True, segments=seg)
        o1, h1 = gka.fwd_chunked(*args, state=s1, return_hnorm=True, segments=seg, beta=ones)
        torch.cuda.synchronize()
        assert torch.equal(o0, o1) and torch.equal(h0, h1)
        assert torch.equal(s0.h, s1.h) and torch.equal(s0.u, s1.u) and torch.equal(s0.n2, s1.n2)


@pytest.mark.parametrize("dtype,D,C", [("bf16", 128, 64), ("bf16", 64, 32), ("fp32", 32, 16)])
def test_beta_zero_stretches(dtype, D, C):
    # head 0: gates 0 on a whole chunk and on every third token elsewhere; head 1: all gates 0,
    # so from the zero state nothing is ever written (||H_t|| = 0 and o = 0 throughout)
    T = 4 * C + 7
    q, k, v, g, bt = gated_inputs(1, T, 2, D, dtype, seed=560 + D + C)
    bt[0, C:2 * C, 0] = 0.0
    bt[0, ::3, 0] = 0.0
    bt[0, 3 * C:3 * C + 5, 0] = 1.0
    bt[0, :, 1] = 0.0
    ref = gka_forward_ref(q, k, v, g, 0.05, 10, beta=bt)
    assert np.all(ref["o"][:, :, 1] == 0.0) and np.all(ref["hnorm"][:, :, 1] == 0.0)
    for seg in (1, 2):
        log(f"beta zero stretches {dtype} D={D} C={C} segments={seg}")
        got = run_prefill(q, k, v, g, 0.05, 10, C, dtype, state=zero_state(1, 2, D),
                          segments=seg, beta=bt)
        assert np.all(got["o"][:, :, 1] == 0.0) and np.all(got["hnorm"][:, :, 1] == 0.0)
        check(dict(o=got["o"][:, :, :1], hnorm=got["hnorm"][:, :, :1]),
              dict(o=ref["o"][:, :, :1], hnorm=ref["hnorm"][:, :, :1]), dtype,
              f"beta zero stretches {dtype} D={D} C={C} S={seg}")


@pytest.mark.parametrize("dtype,D,C", [("bf16", 128, 64), ("fp32", 32, 16)])
def test_beta_nonzero_initial_state(dtype, D, C):
    T = 300
    rng = np.random.default_rng(580 + D)
    Z = rng.standard_normal((1, 2, D, 2 * D))
    h0 = (Z @ np.swapaxes(Z, -1, -2) / D).astype(np.float32).astype(np.float64)
    u0 = rng.standard_normal((1, 2, D, D)).astype(np.float32).astype(np.float64)
    n20 = np.sum(h0 * h0, axis=(-1, -2))
    q, k, v, g, bt = gated_inputs(1, T, 2, D, dtype, seed=581 + D)
    ref = gka_forward_ref(q, k, v, g, 0.05, 10, h0=h0, u0=u0, n2_0=n20, beta=bt)
    for seg in (1, 3):
        log(f"beta initial state {dtype} D={D} segments={seg}")
        got = run_prefill(q, k, v, g, 0.05, 10, C, dtype, state=(h0, u0, n20), segments=seg,
                          beta=bt)
        check(got, ref, dtype, f"beta initial state {dtype} D={D} S={seg}", state=True,
              chunk=C)


@pytest.mark.parametrize("dtype,D,C", [("fp32", 64, 16), ("bf16", 128, 64), ("bf16", 32, 64)])
def test_beta_prefill_then_steps(dtype, D, C):
    T, S = 160, 4
    q, k, v, g, bt = gated_inputs(2, T + S, 2, D, dtype, seed=600 + D)
    ref = gka_forward_ref(q, k, v, g, 0.05, 10, beta=bt)
    log(f"beta prefill -> step {dtype} D={D}")
    st = gka.GkaState.zeros(2, 2, D)
    gka.fwd_chunked(dev(q[:, :T], dtype), dev(k[:, :T], dtype), dev(v[:, :T], dtype),
                    dev(g[:, :T]), 0.05, 10, C, state=st, beta=dev(bt[:, :T]))
    outs = []
    for t in range(T, T + S):
        outs.append(host(gka.step_beta(dev(q[:, t], dtype), dev(k[:, t], dtype),
                                       dev(v[:, t], dtype), dev(g[:, t]), dev(bt[:, t]), 0.05,
                                       10, st)))
    torch.cuda.synchronize()
    o = np.stack(outs, axis=1)
    e = rel_l2(o, ref["o"][:, T:])
    log(f"beta prefill -> step {dtype} D={D}: rel_l2(o)={e:.3e}")
    assert e <= TOL_O[dtype]
    assert max_rel(host(st.n2), ref["n2"]) < TOL_N2[dtype, C]
    assert rel_l2(host(st.h), ref["h"]) < TOL_STATE[dtype, C]
    assert rel_l2(host(st.u), ref["u"]) < TOL_STATE[dtype, C]


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp32", 16)])
def test_beta_step_from_a_state(dtype, D):
    # one gated step from a random PSD state: the decode kernel against gka_step_ref
    B, H = 3, 4
    rng = np.random.default_rng(620 + D)
    Z = rng.standard_normal((B, H, D, 2 * D))
    h = (Z @ np.swapaxes(Z, -1, -2) / D).astype(np.float32).astype(np.float64)
    u = rng.standard_normal((B, H, D, D)).astype(np.float32).astype(np.float64)
    n2 = np.sum(h * h, axis=(-1, -2))
    q, k, v, g, bt = (x[:, 0] for x in gated_inputs(B, 1, H, D, dtype, seed=621 + D))
    bt[0, 0] = 0.0  # no write: H <- gamma H
    bt[0, 1] = 1.0
    o_ref, h_ref, u_ref, n2_ref = gka_step_ref(q, k, v, g, 0.05, 10, h, u, n2, beta=bt)
    st = gka.GkaState(dev(h), dev(u), dev(n2))
    o = host(gka.step_beta(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(g), dev(bt), 0.05,
                           10, st))
    e = rel_l2(o, o_ref)
    log(f"beta step {dtype} D={D}: rel_l2(o)={e:.3e}")
    assert e <= TOL_O[dtype]
    assert max_rel(host(st.n2), n2_ref) < 1e-5
    assert rel_l2(host(st.h), h_ref) < 1e-6
    assert rel_l2(host(st.u), u_ref) < 1e-6


def test_beta_step_ones_is_bitwise_the_base_step():
    B, H, D = 4, 8, 128
    q, k, v, g = (x[:, 0] for x in W.make_prefill(B, 1, H, D, 3.0, 1.0, "bf16", seed=640))
    rng = np.random.default_rng(641)
    h = rng.standard_normal((B, H, D, D)).astype(np.float32)
    h = h + np.swapaxes(h, -1, -2)
    u = rng.standard_normal((B, H, D, D)).astype(np.float32)
    n2 = np.sum(h.astype(np.float64) ** 2, axis=(-1, -2))
    s0, s1 = (gka.GkaState(dev(h), dev(u), dev(n2)) for _ in range(2))
    args = (dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(g), 0.05, 10)
    o0 = gka.step(*args, s0)
    o1 = gka.step(*args, s1, beta=torch.ones(B, H, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o0, o1)
    assert torch.equal(s0.h, s1.h) and torch.equal(s0.u, s1.u) and torch.equal(s0.n2, s1.n2)


@pytest.mark.slow
def test_beta_full_size_prefill_sampled():
    # the B8 T2048 H8 D128 workload with write gates, in the benchmark's launch configuration
    # (the library's own segment plan); 8 of the 64 heads recomputed by the oracle
    w = W.WORKLOADS["prefill_b8_t2048_h8_d128"]
    q, k, v, g = W.make_workload(w)
    bt = W.make_beta(w.B, w.T, w.H, w.seed)
    need = gka.workspace_bytes(w.B, w.T, w.H, w.D, w.chunk, w.iters, w.a, gka.GKA_BF16)
    ws = torch.empty(max(need, 1), device="cuda", dtype=torch.uint8)
    log("beta full-size prefill B8 T2048 H8 D128")
    o, hn = gka.fwd_chunked(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(g), w.a, w.iters,
                            w.chunk, return_hnorm=True, workspace=ws, beta=dev(bt))
    torch.cuda.synchronize()
    pairs = [(0, 0), (1, 3), (2, 7), (3, 1), (4, 4), (5, 6), (6, 2), (7, 5)]
    qs, ks, vs, gs = W.make_workload(w, heads=pairs)
    bs = W.make_beta(w.B, w.T, w.H, w.seed, heads=pairs)
    ref = gka_forward_ref(qs, ks, vs, gs, w.a, w.iters, beta=bs)
    idx_b = torch.tensor([b for b, _ in pairs], device=o.device)
    idx_h = torch.tensor([h for _, h in pairs], device=o.device)
    got_o = host(o[idx_b, :, idx_h].transpose(0, 1).contiguous())[None]
    got_h = host(hn[idx_b, :, idx_h].transpose(0, 1).contiguous())[None]
    worst = max(rel_l2(got_o[0, :, i], ref["o"][0, :, i]) for i in range(len(pairs)))
    eh = max_rel(got_h, ref["hnorm"])
    log(f"beta full size: worst head rel_l2(o)={worst:.3e} hnorm={eh:.3e}")
    assert worst <= TOL_O["bf16"]
    assert eh <= TOL_HNORM
