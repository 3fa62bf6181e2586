"""CPU oracle (fp64 NumPy) for page-sparse decode attention and its dense verification.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the product path.
"""
from .page_sparse import *  # noqa: F401,F403
from .page_sparse import __all__ as _page_sparse_all
from .speculative import *  # noqa: F401,F403
from .speculative import __all__ as _speculative_all
from . import control  # noqa: F401  (the sparsity-schedule controller: oracle.control)
from . import top_p  # noqa: F401  (score-mass page selection: oracle.top_p)

__all__ = list(_page_sparse_all) + list(_speculative_all)
