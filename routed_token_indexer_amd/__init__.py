"""MISA routed token indexer for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libmisa.so`` (C ABI in include/misa.h);
this package holds its build script, a thin ctypes binding and the seeded
synthetic workloads. Importing the package does not load the library; the
first indexer call does, and raises if it has not been built.
"""
__version__ = "0.1.0"

_EXPORTS = ("pool_keys", "route", "score_topk", "hier_rerank", "dsa_index_dense", "indexer", "hier_indexer",
            "debug_scores",
            "workspace_bytes", "timing_begin", "timing_end", "MisaError")


def __getattr__(name):
    if name in _EXPORTS:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
