"""CPU oracle for the INT4 single-token decode block.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls, links
or executes anything under ``oracle/``: only the test suite, the smoke check
in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It
shares no code with the HIP library (no kernels, headers, helpers, tables or
constant generators).  Its only common dependency is the seeded input
generator ``int4_quantized_decode_amd.synth``, which holds none of the
method's arithmetic.
"""
from .reference import *  # noqa: F401,F403
