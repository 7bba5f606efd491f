"""CPU oracle for paged-attention decode (fp64).  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package.  The GPU library never does, and this package never imports the GPU library.
"""
from .pa_ref import *  # noqa: F401,F403
