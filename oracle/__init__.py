"""CPU oracle for the S4 DPLR filter path (test infrastructure only).

Only the test-suite, the smoke check in __graft_entry__.py and the benchmark's
CPU-baseline leg may import this package.  The HIP library never does, and the
oracle never imports the library.
"""
from .ssm_oracle import *  # noqa: F401,F403
from .ssm_oracle import (OK, SINGULAR_BILINEAR, RESONANT_DIAGONAL, RESONANT_CORRECTION,  # noqa: F401
                         worst_status)
from . import hippo_oracle  # noqa: F401  (HiPPO generators and their DPLR form)
