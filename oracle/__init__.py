"""CPU oracle of the looped normalized-GPT forward pass.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call anything in this package. The HIP library
never uses it, and it never uses the HIP library: the two share nothing but
the seeded inputs drawn by the `synth` package.

Parity pins (what checks this oracle against something other than itself)
live in tests/test_oracle_*.py; the header of each module lists what pins it.
"""
from .ngpt import LoopedNGPT, OracleConfigError  # noqa: F401
from . import kvspec  # noqa: F401
