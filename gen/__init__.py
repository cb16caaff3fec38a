"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This package holds no arithmetic of the method (no repack, no GEMM, no
routing); it only draws random inputs of the documented shapes and
distributions.  See ``gen.synth``.
"""

from .synth import *  # noqa: F401,F403
