"""fp64 CPU oracle for MLA latent-cache attention.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its Python binding.
"""

from . import mla_oracle  # noqa: F401
