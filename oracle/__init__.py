"""CPU oracle of the n-gram memory hot path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package; the product library never does.
"""
from .pagegram import *  # noqa: F401,F403
from .pagegram import (HASH_VERSION, forward_engram, forward_scalar, gather,  # noqa: F401
                       gather_stored, index, layout_bases, nf4_codebook,
                       nf4_dequantize, nf4_quantize, project, role_constants,
                       splitmix64)
