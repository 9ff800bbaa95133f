"""CPU float64 oracle for vector-quantized decode -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never calls it and it imports nothing
from the GPU library: the two share no code.  See ``oracle/vq.py`` for the
definitions and the passages each one follows.
"""
from .vq import *  # noqa: F401,F403
from .vq import __all__  # noqa: F401
