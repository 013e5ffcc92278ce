"""fp64 CPU oracle for exact attention. Test infrastructure: only the tests, the smoke
check and the bench's CPU-baseline leg use it; the library never does."""
from . import attention  # noqa: F401
