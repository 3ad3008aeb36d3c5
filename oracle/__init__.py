"""fp64 CPU oracle of the Gated DeltaNet layer (test infrastructure only).

Used by tests/, the smoke check and the benchmark's CPU-baseline leg; the
HIP library and its binding never import it.
"""
from . import gdn_oracle  # noqa: F401
