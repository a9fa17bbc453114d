"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph on ROCm) and replayed.

The library enqueues only its own kernels on the caller's stream (no memsets, no allocations,
no host synchronisation), so every entry point can be captured. Each graph is replayed several
times, with eager work and synchronisations between the replays, and every replay is compared
bit for bit with the eager result of the same calls.
"""
import numpy as np
import pytest
import torch

from test_ridge_regression_amd import gka
from test_ridge_regression_amd import workloads as W

from gka_testutil import dev, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    gka.load()


def psd_state(B, H, D, seed):
    rng = np.random.default_rng(seed)
    Z = rng.standard_normal((B, H, D, 2 * D))
    h = (Z @ np.swapaxes(Z, -1, -2) / (4 * D)).astype(np.float32)
    u = (0.3 * rng.standard_normal((B, H, D, D))).astype(np.float32)
    return dev(h), dev(u), dev(np.sum(h.astype(np.float64) ** 2, axis=(-1, -2)))


def test_decode_steps_in_a_graph():
    B, H, D, steps = 8, 4, 128, 6
    h0, u0, n0 = psd_state(B, H, D, 1000)
    q, k, v, g = W.make_prefill(B, steps, H, D, 3.0, 1.0, "bf16", seed=1001)
    qs, ks, vs = (dev(np.ascontiguousarray(np.moveaxis(x, 1, 0)), "bf16") for x in (q, k, v))
    gs = dev(np.ascontiguousarray(np.moveaxis(g, 1, 0)))
    # eager reference
    st = gka.GkaState(h0.clone(), u0.clone(), n0.clone())
    ref = [gka.step(qs[i], ks[i], vs[i], gs[i], 0.05, 10, st) for i in range(steps)]
    torch.cuda.synchronize()
    ref_h, ref_n = st.h.clone(), st.n2.clone()
    # captured: static state and outputs
    sg = gka.GkaState(h0.clone(), u0.clone(), n0.clone())
    outs = torch.empty(steps, B, H, D, device="cuda", dtype=torch.bfloat16)
    for i in range(2):  # warm-up outside the capture (first-call attribute set-up)
        gka.step(qs[0], ks[0], vs[0], gs[0], 0.05, 10, gka.GkaState(h0.clone(), u0.clone(),
                                                                   n0.clone()))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            gka.step(qs[i], ks[i], vs[i], gs[i], 0.05, 10, sg, out=outs[i])
    for rep in range(3):
        log(f"decode graph replay {rep}")
        sg.h.copy_(h0)
        sg.u.copy_(u0)
        sg.n2.copy_(n0)
        outs.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i in range(steps):
            assert torch.equal(outs[i], ref[i]), (rep, i)
        assert torch.equal(sg.h, ref_h) and torch.equal(sg.n2, ref_n)
        # eager work between the replays
        gka.step(qs[0], ks[0], vs[0], gs[0], 0.05, 10,
                 gka.GkaState(h0.clone(), u0.clone(), n0.clone()))
        torch.cuda.synchronize()


@pytest.mark.parametrize("packed", [False, True])
def test_prefill_in_a_graph(packed):
    H, D, C = 2, 128, 64
    if packed:
        lengths = [130, 1, 0, 64, 257]
        q, k, v, g, cu = W.make_varlen(lengths, H, D, 3.0, 1.0, "bf16", seed=1010)
        cud = torch.from_numpy(cu).to("cuda")
        B, T = len(lengths), max(lengths)
        need = gka.varlen_workspace_bytes(B, T, H, D, C, 10, 0.05, gka.GKA_BF16)
    else:
        B, T = 2, 300
        q, k, v, g = W.make_prefill(B, T, H, D, 3.0, 1.0, "bf16", seed=1011)
        need = gka.workspace_bytes(B, T, H, D, C, 10, 0.05, gka.GKA_BF16, 3)
    qd, kd, vd, gd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(g)
    ws = torch.empty(max(need, 1), device="cuda", dtype=torch.uint8)
    h0, u0, n0 = psd_state(B, H, D, 1012)

    def call(st, out, hn):
        if packed:
            return gka.fwd_varlen(qd, kd, vd, gd, cud, T, 0.05, 10, C, state=st, out=out,
                                  workspace=ws)
        return gka.fwd_chunked(qd, kd, vd, gd, 0.05, 10, C, state=st, out=out, workspace=ws,
                               segments=3)

    st = gka.GkaState(h0.clone(), u0.clone(), n0.clone())
    ref = call(st, torch.empty_like(qd), None)
    torch.cuda.synchronize()
    ref_h, ref_n = st.h.clone(), st.n2.clone()
    sg = gka.GkaState(h0.clone(), u0.clone(), n0.clone())
    out = torch.empty_like(qd)
    call(gka.GkaState(h0.clone(), u0.clone(), n0.clone()), torch.empty_like(qd), None)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(sg, out, None)
    for rep in range(3):
        log(f"prefill graph replay {rep} packed={packed}")
        sg.h.copy_(h0)
        sg.u.copy_(u0)
        sg.n2.copy_(n0)
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
        assert torch.equal(sg.h, ref_h) and torch.equal(sg.n2, ref_n), rep
        call(gka.GkaState(h0.clone(), u0.clone(), n0.clone()), torch.empty_like(qd), None)
        torch.cuda.synchronize()


def test_backward_in_a_graph():
    B, T, H, D = 1, 150, 2, 64
    q, k, v, g = W.make_prefill(B, T, H, D, 3.0, 1.0, "bf16", seed=1020)
    do = W.make_prefill(B, T, H, D, 0.0, 1.0, "bf16", seed=1021)[2]
    args = (dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(g), dev(do, "bf16"), 0.05, 10)
    p = gka.make_params(B, T, H, D, 64, 10, 0.05, gka.GKA_BF16)
    ws = torch.empty(int(gka.load().gka_bwd_workspace_bytes(gka.ctypes.byref(p))), device="cuda",
                     dtype=torch.uint8)
    ref = gka.bwd(*args, workspace=ws)
    torch.cuda.synchronize()
    ref = [x.clone() for x in ref]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = gka.bwd(*args, workspace=ws)
    for rep in range(3):
        log(f"backward graph replay {rep}")
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), rep
        gka.bwd(*args, workspace=ws)  # eager work between the replays
        torch.cuda.synchronize()
