"""The seeded input generator: determinism, shapes, value ranges and bf16 rounding (CPU only)."""
import numpy as np
import pytest
import torch

from test_ridge_regression_amd import workloads as W


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000),
                        [0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40]])
    ours = W.round_bf16(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)


@pytest.mark.parametrize("name", ["tiny_fp32", "prefill_b8_t2048_h8_d128"])
def test_workload_inputs(name):
    w = W.WORKLOADS[name]
    T = min(w.T, 128)
    q, k, v, g = W.make_workload(w, T=T)
    assert q.shape == (w.B, T, w.H, w.D) and g.shape == (w.B, T, w.H)
    for x in (q, k, v):
        assert x.dtype == np.float64
        np.testing.assert_array_equal(W.round_to(x, w.dtype), x)  # exactly representable
    tol = 1e-2 if w.dtype == "bf16" else 1e-6
    np.testing.assert_allclose(np.linalg.norm(k, axis=-1), 1.0, atol=tol)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1.0, atol=tol)
    assert np.all((g > 0) & (g < 1))
    np.testing.assert_array_equal(g.astype(np.float32).astype(np.float64), g)
    q2, k2, v2, g2 = W.make_workload(w, T=T)
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(g, g2)


def test_decode_streams_are_per_row():
    w = W.WORKLOADS["decode_b256_h8_d128"]
    a = W.make_decode_steps(w, steps=5, rows=[3, 9])
    b = W.make_decode_steps(w, steps=5, rows=[9])
    c = W.make_decode_steps(w, steps=7, rows=[9])
    np.testing.assert_array_equal(a[0][:, 1], b[0][:, 0])
    np.testing.assert_array_equal(c[0][:5], b[0])  # q of more steps extends the same stream
    assert not np.array_equal(a[0][:, 0], a[0][:, 1])
    assert a[0].shape == (5, 2, 8, 128) and a[3].shape == (5, 2, 8)
    np.testing.assert_array_equal(W.round_bf16(a[2]), a[2])
    wq = W.make_decode_warmup(w, rows=[9])
    assert wq[0].shape == (1, w.warmup, 8, 128)
    assert not np.array_equal(wq[0][0, :5], b[0][:, 0])  # warm-up and steps differ


def test_sampled_heads_equal_the_full_draw():
    w = W.WORKLOADS["prefill_b8_t2048_h8_d128"]
    T = 300
    q, k, v, g = W.make_workload(w, T=T, B=3)
    pairs = [(2, 5), (0, 0), (1, 7)]
    qs, ks, vs, gs = W.make_workload(w, T=T, heads=pairs)
    for i, (b, h) in enumerate(pairs):
        for full, samp in ((q, qs), (k, ks), (v, vs), (g, gs)):
            np.testing.assert_array_equal(full[b, :, h], samp[0, :, i])


def test_token_blocks_continue_across_streams():
    # sequences longer than one stream block: the block boundary changes nothing visible
    q, k, v, g = W.make_prefill(1, W.TOKEN_BLOCK + 10, 2, 16, 3.0, 1.0, "bf16", 11)
    assert q.shape == (1, W.TOKEN_BLOCK + 10, 2, 16)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1.0, atol=1e-2)
    q2, *_ = W.make_prefill(1, W.TOKEN_BLOCK, 2, 16, 3.0, 1.0, "bf16", 11)
    np.testing.assert_array_equal(q[:, :W.TOKEN_BLOCK], q2)
