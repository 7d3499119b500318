"""Float64 CPU oracle of the sparse MoE layer -- test infrastructure only.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The HIP library and its Python binding never do.
"""
from . import moe_oracle  # noqa: F401
