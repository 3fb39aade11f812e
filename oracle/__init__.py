"""CPU oracle for the KDA gated delta-rule recurrence.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  ``reference`` is the
numpy fp64 form (plus the dense affine form used by the pins); ``native`` is
the same recurrence in plain C (fp64, OpenMP over sequence x head).
"""
from . import reference, native  # noqa: F401
from .reference import rel_err  # noqa: F401
