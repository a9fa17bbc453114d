"""GPU parity of packed variable-length batches (gka_fwd_varlen) against the float64 oracle
run on every sequence alone, with its own initial state: the serving layout, where one call
carries prompts being prefilled and sequences being decoded (length-1 rows that continue a
carried state). Bars as for gka_fwd_chunked: o within 2e-2 (bf16) / 1e-5 (fp32) relative L2 per
sequence, ||H_t||_F within 1e-3, final states as the dense calls'.
"""
import numpy as np
import pytest
import torch

from oracle import gka_forward_ref
from test_ridge_regression_amd import gka
from test_ridge_regression_amd import workloads as W

from gka_testutil import TOL_HNORM, TOL_O, dev, host, log, max_rel, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    gka.load()


def random_states(B, H, D, seed):
    rng = np.random.default_rng(seed)
    Z = rng.standard_normal((B, H, D, 2 * D))
    h0 = (Z @ np.swapaxes(Z, -1, -2) / (4 * D)).astype(np.float32).astype(np.float64)
    u0 = (0.3 * rng.standard_normal((B, H, D, D))).astype(np.float32).astype(np.float64)
    return h0, u0, np.sum(h0 * h0, axis=(-1, -2))


def run_varlen(q, k, v, g, cu, maxlen, a, iters, C, dtype, state=None, beta=None, segments=0):
    st = None if state is None else gka.GkaState(*(dev(x) for x in state))
    cud = torch.from_numpy(cu).to("cuda")
    o, hn = gka.fwd_varlen(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(g), cud, maxlen, a,
                           iters, C, state=st, beta=None if beta is None else dev(beta),
                           return_hnorm=True, segments=segments)
    torch.cuda.synchronize()
    out = dict(o=host(o), hnorm=host(hn))
    if st is not None:
        out.update(h=host(st.h), u=host(st.u), n2=host(st.n2))
    return out


def check_sequences(got, q, k, v, g, cu, a, iters, dtype, state=None, beta=None, what=""):
    B = len(cu) - 1
    worst_o = worst_h = 0.0
    for b in range(B):
        sl = slice(int(cu[b]), int(cu[b + 1]))
        st = {} if state is None else dict(h0=state[0][b:b + 1], u0=state[1][b:b + 1],
                                           n2_0=state[2][b:b + 1])
        if sl.stop == sl.start:
            if state is not None:  # an empty sequence leaves its state as it was
                np.testing.assert_array_equal(got["h"][b], state[0][b].astype(np.float32))
                np.testing.assert_array_equal(got["n2"][b], state[2][b].astype(np.float32))
            continue
        ref = gka_forward_ref(q[None, sl], k[None, sl], v[None, sl], g[None, sl], a, iters,
                              beta=None if beta is None else beta[None, sl], **st)
        e = rel_l2(got["o"][sl], ref["o"][0])
        eh = max_rel(got["hnorm"][sl], ref["hnorm"][0])
        worst_o, worst_h = max(worst_o, e), max(worst_h, eh)
        assert e <= TOL_O[dtype], f"{what} sequence {b}: {e}"
        assert eh <= TOL_HNORM, f"{what} sequence {b}: {eh}"
        if state is not None:
            tol = 1e-6 if dtype == "fp32" else (1e-3 if beta is not None else 1e-4)
            assert rel_l2(got["h"][b], ref["h"][0]) < tol, f"{what} sequence {b}"
            assert rel_l2(got["u"][b], ref["u"][0]) < tol, f"{what} sequence {b}"
    log(f"{what}: worst sequence rel_l2(o)={worst_o:.3e} max_rel(hnorm)={worst_h:.3e}")


LENGTHS = [0, 1, 63, 64, 65, 200, 1, 130]


@pytest.mark.parametrize("dtype,D,C", [("bf16", 128, 64), ("bf16", 32, 64), ("bf16", 64, 32),
                                       ("fp32", 32, 16), ("fp32", 16, 64)])
@pytest.mark.parametrize("gated", [False, True])
def test_packed_mixed_lengths(dtype, D, C, gated):
    H = 2
    q, k, v, g, cu = W.make_varlen(LENGTHS, H, D, 3.0, 1.0, dtype, seed=800 + D + C)
    beta = W.make_beta(1, len(g), H, 801 + D)[0] if gated else None
    state = random_states(len(LENGTHS), H, D, 802 + D)
    for seg in (0, 1, 3):
        log(f"varlen {dtype} D={D} C={C} beta={gated} segments={seg}")
        got = run_varlen(q, k, v, g, cu, max(LENGTHS), 0.05, 10, C, dtype, state=state,
                         beta=beta, segments=seg)
        check_sequences(got, q, k, v, g, cu, 0.05, 10, dtype, state=state, beta=beta,
                        what=f"varlen {dtype} D={D} C={C} beta={gated} S={seg}")


@pytest.mark.parametrize("dtype,D,C", [("bf16", 128, 64), ("fp32", 32, 16)])
def test_equal_lengths_are_bitwise_the_dense_call(dtype, D, C):
    B, T, H = 3, 150, 2
    q, k, v, g = W.make_prefill(B, T, H, D, 3.0, 1.0, dtype, seed=820)
    cu = (np.arange(B + 1) * T).astype(np.int32)
    for seg in (1, 3):
        log(f"varlen == dense {dtype} D={D} segments={seg}")
        s_d, s_v = gka.GkaState.zeros(B, H, D), gka.GkaState.zeros(B, H, D)
        o_d, h_d = gka.fwd_chunked(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(g), 0.05, 10,
                                   C, state=s_d, return_hnorm=True, segments=seg)
        o_v, h_v = gka.fwd_varlen(dev(q.reshape(B * T, H, D), dtype),
                                  dev(k.reshape(B * T, H, D), dtype),
                                  dev(v.reshape(B * T, H, D), dtype), dev(g.reshape(B * T, H)),
                                  torch.from_numpy(cu).to("cuda"), T, 0.05, 10, C, state=s_v,
                                  return_hnorm=True, segments=seg)
        torch.cuda.synchronize()
        assert torch.equal(o_d.reshape(B * T, H, D), o_v)
        assert torch.equal(h_d.reshape(B * T, H), h_v)
        assert torch.equal(s_d.h, s_v.h) and torch.equal(s_d.u, s_v.u)
        assert torch.equal(s_d.n2, s_v.n2)


@pytest.mark.parametrize("dtype,D,C", [("bf16", 128, 64), ("fp32", 32, 16)])
def test_prefill_then_mixed_decode_batch(dtype, D, C):
    # call 1 prefills four prompts; call 2 is a serving step in which three sequences decode one
    # token and one takes a further chunk of its prompt; both against the oracle on the
    # concatenated sequences
    H = 2
    first, second = [100, 37, 64, 5], [1, 1, 20, 1]
    full = [a + b for a, b in zip(first, second)]
    q, k, v, g, cu = W.make_varlen(full, H, D, 3.0, 1.0, dtype, seed=840 + D)
    idx1 = np.concatenate([np.arange(cu[b], cu[b] + first[b]) for b in range(4)])
    idx2 = np.concatenate([np.arange(cu[b] + first[b], cu[b + 1]) for b in range(4)])
    cu1 = np.concatenate([[0], np.cumsum(first)]).astype(np.int32)
    cu2 = np.concatenate([[0], np.cumsum(second)]).astype(np.int32)
    st = gka.GkaState.zeros(4, H, D)
    put = lambda idx: (dev(q[idx], dtype), dev(k[idx], dtype), dev(v[idx], dtype), dev(g[idx]))
    log(f"varlen prefill -> mixed step {dtype} D={D}")
    gka.fwd_varlen(*put(idx1), torch.from_numpy(cu1).to("cuda"), max(first), 0.05, 10, C,
                   state=st)
    o2 = gka.fwd_varlen(*put(idx2), torch.from_numpy(cu2).to("cuda"), max(second), 0.05, 10, C,
                        state=st)
    torch.cuda.synchronize()
    o2 = host(o2)
    for b in range(4):
        sl = slice(int(cu[b]), int(cu[b + 1]))
        ref = gka_forward_ref(q[None, sl], k[None, sl], v[None, sl], g[None, sl], 0.05, 10)
        got = o2[cu2[b]:cu2[b + 1]]
        e = rel_l2(got, ref["o"][0, first[b]:])
        log(f"  sequence {b}: rel_l2(o) of the second call {e:.3e}")
        assert e <= TOL_O[dtype]
        assert max_rel(host(st.n2)[b], ref["n2"][0]) < 1e-4


@pytest.mark.slow
def test_serving_batch_at_scale():
    """A serving step at B64 H8 D128: 8 prompts of 256..2048 tokens and 56 decode rows that
    continue states built by a 64-token packed prefill; 2 prompts and 6 decode rows are
    recomputed by the oracle."""
    w = W.WORKLOADS["varlen_b64_h8_d128"]
    lens_pre, lens = W.varlen_lengths(w)
    H, D = w.H, w.D
    q, k, v, g, cu = W.make_varlen([a + b for a, b in zip(lens_pre, lens)], H, D, w.gate_mu,
                                   w.gate_sd, w.dtype, w.seed)
    idx1 = np.concatenate([np.arange(cu[b], cu[b] + lens_pre[b]) for b in range(w.B)])
    idx2 = np.concatenate([np.arange(cu[b] + lens_pre[b], cu[b + 1]) for b in range(w.B)])
    cu1 = np.concatenate([[0], np.cumsum(lens_pre)]).astype(np.int32)
    cu2 = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    st = gka.GkaState.zeros(w.B, H, D)
    put = lambda idx: (dev(q[idx], "bf16"), dev(k[idx], "bf16"), dev(v[idx], "bf16"), dev(g[idx]))
    log("serving batch B64: warm-up prefill of the decode rows")
    gka.fwd_varlen(*put(idx1), torch.from_numpy(cu1).to("cuda"), max(max(lens_pre), 1), w.a,
                   w.iters, w.chunk, state=st)
    log("serving batch B64: the mixed step")
    o2, hn2 = gka.fwd_varlen(*put(idx2), torch.from_numpy(cu2).to("cuda"), max(lens), w.a,
                             w.iters, w.chunk, state=st, return_hnorm=True)
    torch.cuda.synchronize()
    o2, hn2 = host(o2), host(hn2)
    prompts = [b for b in range(w.B) if lens_pre[b] == 0][:2]
    decodes = [b for b in range(w.B) if lens_pre[b] > 0][:6]
    for b in prompts + decodes:
        sl = slice(int(cu[b]), int(cu[b + 1]))
        ref = gka_forward_ref(q[None, sl], k[None, sl], v[None, sl], g[None, sl], w.a, w.iters)
        e = rel_l2(o2[cu2[b]:cu2[b + 1]], ref["o"][0, lens_pre[b]:])
        eh = max_rel(hn2[cu2[b]:cu2[b + 1]], ref["hnorm"][0, lens_pre[b]:])
        log(f"  sequence {b} ({lens_pre[b]} + {lens[b]} tokens): rel_l2(o)={e:.3e} hnorm={eh:.3e}")
        assert e <= TOL_O["bf16"] and eh <= TOL_HNORM


def test_many_sequences_without_a_dispatch_order():
    # more than 4096 sequences: the launch keeps the plain order; equal lengths must still give
    # the dense call's results bit for bit
    B, T, H, D = 4100, 3, 1, 32
    q, k, v, g = W.make_prefill(B, T, H, D, 3.0, 1.0, "fp32", seed=860)
    cu = (np.arange(B + 1) * T).astype(np.int32)
    log("varlen B=4100 (no dispatch order) == dense")
    o_d = gka.fwd_chunked(dev(q), dev(k), dev(v), dev(g), 0.05, 6, 16, segments=1)
    o_v = gka.fwd_varlen(dev(q.reshape(B * T, H, D)), dev(k.reshape(B * T, H, D)),
                         dev(v.reshape(B * T, H, D)), dev(g.reshape(B * T, H)),
                         torch.from_numpy(cu).to("cuda"), T, 0.05, 6, 16, segments=1)
    torch.cuda.synchronize()
    assert torch.equal(o_d.reshape(B * T, H, D), o_v)
