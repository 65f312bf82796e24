"""Clebsch-Gordan tensor-product convolution on AMD MI355X (gfx950).

The computation lives in ``libcgtp.so`` (C ABI in ``include/cgtp.h``): a host runtime that
builds plans and CSR graphs and generates, compiles and launches gfx950 kernels.  This
package holds its build step (``build``) and the ctypes binding (``_lib``).
"""

from . import _lib  # noqa: F401
from ._lib import (CONVENTIONAL, STREAMED, OP_BACKWARD, OP_DOUBLE_BACKWARD, OP_FORWARD, OP_TRIPLE_BACKWARD,  # noqa: F401
                   CgtpError, Convolution, Graph, Plan, check_edges, conv_backward, conv_double_backward, conv_forward,
                   conv_backward_with_state, conv_forward_keep_state, conv_triple_backward, layout_convert, state_size,
                   workspace_size)
