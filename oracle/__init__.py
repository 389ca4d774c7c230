"""Float64 CPU oracle of the equivariant edge convolution (test infrastructure).

This package is the plain, slow, obviously-correct definition that the HIP
library is checked against.  It is TEST INFRASTRUCTURE ONLY: the product path
(the C-ABI library and its Python binding) never imports, calls or links it.
Only the tests, the smoke check and the CPU-baseline leg of the benchmark use
it.  It shares no code with the HIP path; both take their inputs from the
seeded generators in ``eec_inputs``.

Modules
-------
neighbors : periodic neighbour list (brute force and cell list) and CSR.
sph       : real spherical harmonics l <= 3 from the associated-Legendre
            recurrence, and their gradients.
model     : edge geometry, Bessel basis x polynomial envelope, radial MLP,
            message, quadratic readout, analytic backward, forces, virial,
            and the folded / reassociated forms of the last radial layer.

Every function states the passage it follows.  Parity status of each
function (what pins it) is listed in each module's header.
"""
from .neighbors import neighbors_bruteforce, neighbors_celllist, CSR  # noqa: F401
from . import sph  # noqa: F401
from . import model  # noqa: F401
