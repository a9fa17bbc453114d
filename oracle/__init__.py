"""CPU oracle for the GKA forward: test infrastructure, not part of the product.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may import it.
It is plain float64 numpy written from the pages' description of the layer and shares no code,
header, table or helper with the HIP library in ``test_ridge_regression_amd``.
"""
from .gka_oracle import (SOLVERS, agd_solve, cg_solve, chebyshev_rates, chebyshev_solve,
                         chebyshev_weights, cholesky_solve, gd_solve, gka_backward_ref,
                         gka_forward_ref, gka_step_ref, ridge_bruteforce, solver_residuals)

__all__ = ["SOLVERS", "agd_solve", "cg_solve", "chebyshev_rates", "chebyshev_solve",
           "chebyshev_weights", "cholesky_solve", "gd_solve", "gka_backward_ref",
           "gka_forward_ref", "gka_step_ref",
           "ridge_bruteforce", "solver_residuals"]
