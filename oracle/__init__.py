"""Reference (oracle) implementation of the MoDA forward pass and its gradients.

Test infrastructure only: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark, never by the product path.
"""
from .moda_oracle import (  # noqa: F401
    moda_forward,
    moda_forward_scalar,
    depth_utilisation,
)
from .moda_backward import moda_backward, moda_backward_keys  # noqa: F401
