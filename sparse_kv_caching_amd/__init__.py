"""LoLA chunkwise attention step for one layer on MI355X (gfx950).

The compute lives in the HIP library ``liblola.so`` (C ABI, ``include/lola.h``);
:mod:`sparse_kv_caching_amd.lola` is the thin ctypes binding over it.  The
binding is imported lazily so that :mod:`sparse_kv_caching_amd.workloads` (the
seeded input generators) can be used without the library.
"""

import importlib

__all__ = ["lola", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
