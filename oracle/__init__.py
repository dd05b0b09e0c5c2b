"""CPU oracle for attention-mass KV selection and compacted decode attention.

TEST INFRASTRUCTURE ONLY.  Plain, slow, float64 numpy written from the
definitions on the source pages; it shares no code with the HIP library and
imports nothing from it.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import it; the product path never does.
"""
from .kvsel_oracle import *  # noqa: F401,F403
from .kvsel_oracle import __all__  # noqa: F401
