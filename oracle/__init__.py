"""fp64 CPU oracle for Fibonacci-spaced sparse attention (test infrastructure).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package. It shares no code with the HIP library.
"""
from .fsa_oracle import (BASES, FIB, MODES, POW2, SCHEDULE_COPRIME,  # noqa: F401
                         SCHEDULE_FIXED, TapTable,
                         SCHEDULE_LINEAR, backward, backward_slab, decode, dkdv_rows,
                         dq_rows, forward, forward_rows, forward_slab,
                         offset_table, rope, schedule, OPT_ADAM, OPT_SGD, THETA_CLAMP,
                         THETA_TANH, alpha_of_theta, dalpha_dtheta, theta_init,
                         theta_step, theta_to_alpha)
