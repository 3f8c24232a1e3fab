"""fp64 CPU oracle for GSI. TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__ and bench.py's CPU-baseline leg may import this
package. The HIP library never imports, links or calls it, and it never imports the library.
"""
from . import gsi_calibration, gsi_oracle  # noqa: F401
from .gsi_oracle import (FAST, SLOW, as_f64, dense, forward, gate, gate_only, precompute_image,  # noqa: F401
                         project, ratio, residual, residual_norms, spectral_norm, squared_norms,
                         static_projection)
