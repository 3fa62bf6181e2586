"""Query-aware page-sparse decode attention for AMD Instinct MI355X (gfx950).

The kernels live in ``libspdec.so`` (HIP, C ABI in ``include/spdec.h``);
``spdec`` is the thin ctypes binding, ``synth`` the seeded input generator and
``build`` compiles the library in-tree.
"""
from . import spdec  # noqa: F401
from .spdec import (  # noqa: F401
    PagedCache, acceptance, append_kv, build_meta, dense_decode, select_pages, sparse_decode,
)
