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


def test_decode_steps_are_independent_streams():
    w = W.WORKLOADS["decode_b256_h8_d128"]
    a = W.make_decode_step(w, 3, B=4)
    b = W.make_decode_step(w, 3, B=4)
    c = W.make_decode_step(w, 4, B=4)
    np.testing.assert_array_equal(a[0], b[0])
    assert not np.array_equal(a[0], c[0])
    assert a[0].shape == (4, 8, 128) and a[3].shape == (4, 8)
