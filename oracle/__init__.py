"""CPU oracle of the sparse MoE FFN layer (float64 NumPy).

TEST INFRASTRUCTURE ONLY.  Tests, the smoke check and the bench's CPU
baseline may import this package; the HIP product path never does, and the
two share no code.  Parity status of each function is listed in its module
docstring; every function here is pinned by a CPU test against closed forms,
library routines, brute force, invariants or finite differences.
"""
from . import moe_ref, score_f32  # noqa: F401
