"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

The HIP path runs every head of every workload; the float64 oracle recomputes a sample of
heads (heads are independent, so a sampled head is exact, not an approximation). The bars are
the same as for the small cases: relative L2 of o <= 2e-2 (bf16), ||H_t||_F within 1e-3
relative at every token.

  * prefill B8 T2048 H8 D128: 8 of 64 heads over the whole sequence;
  * prefill B4 T8192 H32 D64: 16 of 128 heads over the whole sequence;
  * prefill B1 T131072 H8 D128 (2048 chunks in 32 segments of 4096 tokens): 2 of 8 heads. The
    oracle carries the exact state through all tokens (state-only mode, which still yields
    ||H_t||_F at every token) and runs the solve on four windows of 1024 tokens: the first
    (segment 0 alone), two that straddle inner segment boundaries (tokens 4096 and 65536: the
    ends of segments 0 and 15 and the starts of segments 1 and 16, whose start states come from
    the segment scan), and the last (segment 31, after the whole scan);
  * decode B256 H8 D128: 16 of 256 sequences, all 8 heads, over all 1000 steps, from a carried
    state that the oracle builds from 512 warm-up tokens (the same float32 state on both sides).
"""
import numpy as np
import pytest
import torch

from oracle import gka_forward_ref, gka_step_ref
from test_ridge_regression_amd import gka
from test_ridge_regression_amd import workloads as W

from gka_testutil import TOL_HNORM, TOL_O, dev, host, log, max_rel, rel_l2, tripwire

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    gka.load()


def run_full_prefill(w, q, k, v, g):
    """One gka_fwd_chunked over the whole workload with the library's own segment plan."""
    dt = w.dtype
    qd, kd, vd, gd = dev(q, dt), dev(k, dt), dev(v, dt), dev(g)
    need = gka.workspace_bytes(w.B, w.T, w.H, w.D, w.chunk, w.iters, w.a,
                               gka.GKA_BF16 if dt == "bf16" else gka.GKA_FP32)
    ws = torch.empty(max(need, 1), device="cuda", dtype=torch.uint8)
    o, hn = gka.fwd_chunked(qd, kd, vd, gd, w.a, w.iters, w.chunk, return_hnorm=True,
                            workspace=ws)
    torch.cuda.synchronize()
    return o, hn


def check_sampled(w, o, hn, pairs):
    qs, ks, vs, gs = W.make_workload(w, heads=pairs)  # the same values as those heads' inputs
    ref = gka_forward_ref(qs, ks, vs, gs, w.a, w.iters)
    idx_b = torch.tensor([b for b, _ in pairs], device=o.device)
    idx_h = torch.tensor([h for _, h in pairs], device=o.device)
    got_o = host(o[idx_b, :, idx_h].transpose(0, 1).contiguous())[None]  # [1, T, P, D]
    got_h = host(hn[idx_b, :, idx_h].transpose(0, 1).contiguous())[None]  # [1, T, P]
    e = rel_l2(got_o, ref["o"])
    worst = max(rel_l2(got_o[0, :, i], ref["o"][0, :, i]) for i in range(len(pairs)))
    eh = max_rel(got_h, ref["hnorm"])
    log(f"{w.name}: sampled rel_l2(o)={e:.3e} worst head={worst:.3e} hnorm={eh:.3e}")
    assert np.all(np.isfinite(got_o))
    assert e <= TOL_O[w.dtype]
    assert worst <= TOL_O[w.dtype]
    assert eh <= TOL_HNORM
    tripwire(worst, eh, w.dtype, w.T, w.name)


@pytest.mark.timeout(300)
def test_prefill_b8_t2048_h8_d128_full():
    w = W.WORKLOADS["prefill_b8_t2048_h8_d128"]
    log(f"{w.name}: full prefill")
    q, k, v, g = W.make_workload(w)
    o, hn = run_full_prefill(w, q, k, v, g)
    del q, k, v, g
    check_sampled(w, o, hn, [(b, (3 * b + 1) % w.H) for b in range(w.B)])


@pytest.mark.timeout(300)
def test_prefill_b4_t8192_h32_d64_full():
    w = W.WORKLOADS["prefill_b4_t8192_h32_d64"]
    log(f"{w.name}: full prefill")
    q, k, v, g = W.make_workload(w)
    o, hn = run_full_prefill(w, q, k, v, g)
    del q, k, v, g
    check_sampled(w, o, hn, [(b, h) for b in range(w.B) for h in (0, 9, 22, 31)])


@pytest.mark.timeout(400)
def test_prefill_b1_t131072_h8_d128_full():
    w = W.WORKLOADS["prefill_b1_t131072_h8_d128"]
    log(f"{w.name}: full prefill")
    q, k, v, g = W.make_workload(w)
    o, hn = run_full_prefill(w, q, k, v, g)
    del q, k, v, g
    pairs = [(0, 2), (0, 7)]
    qs, ks, vs, gs = W.make_workload(w, heads=pairs)
    got_o = host(o[0][:, [h for _, h in pairs]])[None]  # [1, T, P, D]
    got_h = host(hn[0][:, [h for _, h in pairs]])[None]
    del o, hn
    T, win = w.T, 1024
    seg_tokens = 64 * w.chunk  # the plan: 2048 chunks in 32 segments of 64
    assert gka.workspace_bytes(w.B, w.T, w.H, w.D, w.chunk, w.iters, w.a, gka.GKA_BF16) > 0
    windows = [(0, win), (seg_tokens - win // 2, seg_tokens + win // 2),
               (16 * seg_tokens - win // 2, 16 * seg_tokens + win // 2), (T - win, T)]
    st = None  # (h, u, n2) after the tokens handled so far
    pos, ref_h, errs = 0, [], []
    for a, b in windows:
        if a > pos:  # carry the state to the window in state-only mode
            log(f"{w.name}: oracle state through tokens {pos}..{a}")
            mid = gka_forward_ref(qs[:, pos:a], ks[:, pos:a], vs[:, pos:a], gs[:, pos:a], w.a,
                                  w.iters, mode="state", **_state_kw(st))
            ref_h.append(mid["hnorm"])
            st = (mid["h"], mid["u"], mid["n2"])
        log(f"{w.name}: oracle solve on tokens {a}..{b}")
        r = gka_forward_ref(qs[:, a:b], ks[:, a:b], vs[:, a:b], gs[:, a:b], w.a, w.iters,
                            **_state_kw(st))
        ref_h.append(r["hnorm"])
        st = (r["h"], r["u"], r["n2"])
        errs.append(rel_l2(got_o[:, a:b], r["o"]))
        pos = b
    eh = max_rel(got_h, np.concatenate(ref_h, axis=1))
    log(f"{w.name}: rel_l2(o) per window " + " ".join(f"{a}..{b}: {e:.3e}"
                                                       for (a, b), e in zip(windows, errs))
        + f"; hnorm={eh:.3e}")
    assert np.all(np.isfinite(got_o))
    assert all(e <= TOL_O[w.dtype] for e in errs)
    assert eh <= TOL_HNORM
    tripwire(max(errs), eh, w.dtype, win, w.name)


def _state_kw(st):
    return {} if st is None else dict(h0=st[0], u0=st[1], n2_0=st[2])


@pytest.mark.timeout(400)
def test_decode_b256_h8_d128_full():
    w = W.WORKLOADS["decode_b256_h8_d128"]
    rows = np.linspace(0, w.B - 1, 16).astype(int)
    r = torch.as_tensor(rows, device="cuda")
    log(f"{w.name}: warm-up of {w.warmup} tokens")
    q, k, v, g = W.make_decode_warmup(w)
    # the library's own warm-up over every sequence (prefill of the warm-up tokens)
    st = gka.GkaState.zeros(w.B, w.H, w.D)
    gka.fwd_chunked(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(g), w.a, w.iters,
                    w.chunk, state=st)
    torch.cuda.synchronize()
    # the oracle's warm-up state of the sampled sequences, rounded to the float32 the library
    # carries; both sides start from exactly these values
    del q, k, v, g
    qw, kw, vw, gw = W.make_decode_warmup(w, rows=rows)
    warm = gka_forward_ref(qw, kw, vw, gw, w.a, w.iters, mode="state")
    h0, u0, n20 = (x.astype(np.float32).astype(np.float64) for x in
                   (warm["h"], warm["u"], warm["n2"]))
    # consistency of the library's prefill warm-up with the oracle's (informational bar)
    e_warm = rel_l2(host(st.h[r]), warm["h"])
    log(f"{w.name}: warm-up state rel err {e_warm:.3e}")
    assert e_warm < 1e-4
    st.h[r] = dev(h0)
    st.u[r] = dev(u0)
    st.n2[r] = dev(n20)
    torch.cuda.synchronize()

    log(f"{w.name}: {w.steps} steps")
    Q, K, V, G = W.make_decode_steps(w)
    outs, n2s = [], []
    for s in range(w.steps):
        o = gka.step(dev(Q[s], "bf16"), dev(K[s], "bf16"), dev(V[s], "bf16"), dev(G[s]), w.a,
                     w.iters, st)
        outs.append(o[r].clone())
        n2s.append(st.n2[r].clone())
    torch.cuda.synchronize()
    del Q, K, V, G
    got_o = np.stack([host(x) for x in outs])
    got_n2 = np.stack([host(x) for x in n2s])
    log(f"{w.name}: oracle over {w.steps} steps")
    Qs, Ks, Vs, Gs = W.make_decode_steps(w, rows=rows)
    ref_o = np.empty_like(got_o)
    ref_n2 = np.empty_like(got_n2)
    h, u, n2 = h0, u0, n20
    for s in range(w.steps):
        ref_o[s], h, u, n2 = gka_step_ref(Qs[s], Ks[s], Vs[s], Gs[s], w.a, w.iters, h, u, n2)
        ref_n2[s] = n2
    e = rel_l2(got_o, ref_o)
    eh = max_rel(np.sqrt(got_n2), np.sqrt(ref_n2))
    es = rel_l2(host(st.h[r]), h)
    log(f"{w.name}: rel_l2(o)={e:.3e} hnorm={eh:.3e} final state={es:.3e}")
    assert np.all(np.isfinite(got_o))
    assert e <= TOL_O["bf16"]
    assert eh <= TOL_HNORM
    assert es < 1e-3
