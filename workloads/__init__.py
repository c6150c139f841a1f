"""Seeded synthetic workloads for the CSA2 hot path.

This package only draws inputs in their stored formats; it holds none of the
method's arithmetic (no scoring, selection, softmax or rotation).  Both the
oracle-side tests and the GPU side read the tensors it produces.
"""

from .configs import CONFIGS, Csa2Config, get_config  # noqa: F401
from .gen import make_inputs  # noqa: F401
