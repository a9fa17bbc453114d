"""MI355X-native forward pass of the Gated KalmaNet (GKA) memory layer.

Two entry points, both hand-written HIP for gfx950 behind a C ABI (``include/gka.h``):

* ``fwd_chunked`` -- chunk-wise prefill / training forward over a whole sequence;
* ``step``        -- one recurrent decode step on a carried (H, U, ||H||_F^2) state.

This module stays import-light: the shared library is loaded on first use by
``test_ridge_regression_amd.gka``; ``workloads`` holds the seeded synthetic inputs.
"""

__all__ = ["gka", "workloads"]
