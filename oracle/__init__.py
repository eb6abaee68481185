"""Plain CPU oracle for the MXFP4 training hot path.

TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers; the library and its Python binding never
import this package. It shares no code, tables or constants with the HIP path.
"""
from .mxfp4 import *  # noqa: F401,F403
