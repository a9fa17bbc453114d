"""GPU parity across the bf16 input range: keys, values and queries far from unit scale.

bf16 carries float32's exponent range. The chunk walk and the output pass keep every 16-bit
matrix operand in range with exact powers of two (keys per chunk, queries and solves per token,
the value state per wave) or use bf16 operands, so inputs scaled by powers of two must give the
oracle's result at the bf16 bar. The oracle is float64 and scale-covariant: o is linear in v and
in q, and o(2^e k) = 2^-e o(k) (the system scales by 2^2e, U by 2^e).
"""
import numpy as np
import pytest
import torch

from oracle import gka_forward_ref
from test_ridge_regression_amd import gka
from test_ridge_regression_amd import workloads as W

from gka_testutil import TOL_HNORM, TOL_O, log, max_rel, rel_l2, run_prefill

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    gka.load()


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("sq,sk,sv", [
    (0, 0, -20), (0, 0, 17), (0, -12, 0), (0, 8, 0), (-12, 0, 0), (10, 0, 0), (-6, -12, 17),
])
def test_power_of_two_scaled_inputs(D, sq, sk, sv):
    """q, k, v scaled by 2^sq, 2^sk, 2^sv (exact in bf16): 3 chunks, 2 segments, a carried
    initial state built by a first call at the same scales."""
    B, T, H, a, iters = 2, 3 * 64 + 17, 2, 0.05, 10
    q, k, v, g = W.make_prefill(B, 2 * T, H, D, 3.0, 1.0, "bf16", 77 + D)
    q, k, v = q * 2.0 ** sq, k * 2.0 ** sk, v * 2.0 ** sv
    ref = gka_forward_ref(q, k, v, g, a, iters)
    z = (np.zeros((B, H, D, D)), np.zeros((B, H, D, D)), np.zeros((B, H)))
    log(f"range D={D} q 2^{sq} k 2^{sk} v 2^{sv}")
    first = run_prefill(q[:, :T], k[:, :T], v[:, :T], g[:, :T], a, iters, 64, "bf16", state=z,
                        segments=2)
    got = run_prefill(q[:, T:], k[:, T:], v[:, T:], g[:, T:], a, iters, 64, "bf16",
                      state=(first["h"], first["u"], first["n2"]), segments=2)
    o = np.concatenate([first["o"], got["o"]], axis=1)
    hn = np.concatenate([first["hnorm"], got["hnorm"]], axis=1)
    e, eh = rel_l2(o, ref["o"]), max_rel(hn, ref["hnorm"])
    eH, eU = rel_l2(got["h"], ref["h"]), rel_l2(got["u"], ref["u"])
    log(f"range D={D} q 2^{sq} k 2^{sk} v 2^{sv}: rel_l2(o)={e:.3e} max_rel(hnorm)={eh:.3e} "
        f"state H {eH:.3e} U {eU:.3e}")
    assert np.all(np.isfinite(o))
    assert e <= TOL_O["bf16"]
    assert eh <= TOL_HNORM
    assert eH <= 1e-5 and eU <= 1e-5
