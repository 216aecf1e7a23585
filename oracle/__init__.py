"""CPU oracle for msign by Newton-Schulz iteration (fp64 NumPy).

Test infrastructure only: the tests, the smoke check and the benchmark's
CPU-baseline leg use it; the product path never does.
"""
from .msign_oracle import *  # noqa: F401,F403
from .msign_oracle import (KELLER_ABC, DEFAULT_EPS, DEFAULT_STEPS,  # noqa: F401
                           coefficient_schedule, svd_msign, inverse_sqrt_msign,
                           poly_step, phi, theorem1_xq, ns, ns_single, gram_ns,
                           gram_ns_single, spectral_ns, spectral_ns_single,
                           exact_msign, ns_improved_init, ns_improved_init_single,
                           max_rel_fro_error, dense_ns_flops, symmetric_ns_flops,
                           naive_gram_flops, restart_gram_flops, frobenius_normalize)
