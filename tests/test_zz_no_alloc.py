"""The allocation-free prefill gka_fwd_chunked_static against gka_fwd_chunked_beta.

Both run the same kernels on the same segment plan, the static entry point with the segment
states in the library's static scratch instead of a caller's workspace, so o, ||H_t||_F and the
final state must be identical bit for bit. Two calls in a row, the second one smaller: the
scratch keeps the first call's contents, which the second call must not read. The second call
is also held to the oracle at the bf16 bar.
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


def _inputs(B, T, H, D, seed, with_beta):
    q, k, v, g = W.make_prefill(B, T, H, D, 3.0, 1.0, "bf16", seed)
    beta = W.make_beta(B, T, H, seed + 1) if with_beta else None
    t = [dev(x, "bf16") for x in (q, k, v)] + [dev(g)]
    return (q, k, v, g, beta), t + [dev(beta) if beta is not None else None]


def _state(B, H, D, seed):
    """A carried state: the final state of a first base call on other tokens."""
    _, (q, k, v, g, _) = _inputs(B, 96, H, D, seed, False)
    st = gka.GkaState.zeros(B, H, D, device=q.device)
    gka.fwd_chunked(q, k, v, g, 0.05, 10, state=st)
    return st


def _clone(st):
    return None if st is None else gka.GkaState(st.h.clone(), st.u.clone(), st.n2.clone())


def _compare(B, T, H, D, segments, seed, with_beta, with_state):
    (qh, kh, vh, gh, bh), (q, k, v, g, beta) = _inputs(B, T, H, D, seed, with_beta)
    st0 = _state(B, H, D, seed + 7) if with_state else None
    need = gka.workspace_bytes(B, T, H, D, 64, 10, 0.05, gka.GKA_BF16, segments)
    log(f"static prefill B{B} T{T} H{H} D{D} segments={segments} beta={with_beta} "
        f"state={with_state}: workspace {need} bytes")
    assert 0 < need <= gka.GKA_STATIC_SCRATCH_BYTES  # the plan uses the scratch
    sa, sb = _clone(st0), _clone(st0)
    oa, hna = gka.fwd_chunked(q, k, v, g, 0.05, 10, state=sa, beta=beta, segments=segments,
                              return_hnorm=True)
    ob = torch.empty_like(q)
    hnb = torch.empty(B, T, H, device=q.device, dtype=torch.float32)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    gka.fwd_chunked_static(q, k, v, g, 0.05, 10, state=sb, beta=beta, segments=segments,
                           out=ob, hnorm=hnb)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(ob, oa)
    assert torch.equal(hnb, hna)
    if st0 is not None:
        assert torch.equal(sb.h, sa.h) and torch.equal(sb.u, sa.u) and torch.equal(sb.n2, sa.n2)
    return host(ob), host(hnb), (qh, kh, vh, gh, bh)


def test_static_prefill_matches_the_workspace_call_twice():
    # first call: 8 heads of D = 128, 16 chunks in 8 segments, write gate and carried state
    _compare(2, 1024, 4, 128, 8, 101, True, True)
    # second call, smaller: 2 heads of D = 64, 6 chunks (ragged tail) in 3 segments, no state
    o, hn, (q, k, v, g, _) = _compare(1, 5 * 64 + 33, 2, 64, 3, 202, False, False)
    ref = gka_forward_ref(q, k, v, g, 0.05, 10)
    e, eh = rel_l2(o, ref["o"]), max_rel(hn, ref["hnorm"])
    log(f"static prefill second call vs oracle: rel_l2(o)={e:.3e} max_rel(hnorm)={eh:.3e}")
    assert e <= TOL_O["bf16"] and eh <= TOL_HNORM


def test_static_prefill_rejects_a_plan_beyond_the_scratch():
    """64 x 8 heads of D = 128 in 32 segments need 2 GiB of segment states: GKA_ERR_SCRATCH,
    raised before anything runs (o keeps its contents)."""
    B, T, H, D = 64, 32 * 64, 8, 128
    q = torch.zeros(B, T, H, D, device="cuda", dtype=torch.bfloat16)
    g = torch.full((B, T, H), 0.9, device="cuda", dtype=torch.float32)
    o = torch.full_like(q, 3.0)
    with pytest.raises(gka.GkaError) as ex:
        gka.fwd_chunked_static(q, q, q, g, 0.05, 10, segments=32, out=o)
    assert ex.value.status == 8
    assert bool((o == 3.0).all())
