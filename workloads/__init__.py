"""Seeded synthetic inputs for the Clebsch-Gordan tensor-product convolution.

This package only draws inputs: atom positions, the periodic neighbour list,
radial-basis values and random tensors. It holds none of the convolution's
arithmetic (no Clebsch-Gordan coefficients, spherical harmonics, path
enumeration or CSR construction), so both the CPU oracle and the HIP path can
use it without sharing any of the method's code.
"""

from .graphs import (  # noqa: F401
    CONFIGS,
    Workload,
    make_workload,
    normal_tensor,
)
