"""CPU oracle (fp64 NumPy) for page-sparse decode attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the product path.
"""
from .page_sparse import *  # noqa: F401,F403
from .page_sparse import __all__  # noqa: F401
