"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the bench's CPU-baseline leg may import this
package.  It shares no code with the HIP path and never touches a GPU.
"""
from . import ref, online, fp8  # noqa: F401
