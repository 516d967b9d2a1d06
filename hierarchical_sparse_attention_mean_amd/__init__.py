"""MI355X-native Log-linear Sparse Attention (LLSA) hot path.

The compute lives in ``libllsa.so`` (hand-written HIP for gfx950 behind a C ABI declared in
``include/llsa.h``); :mod:`.llsa` is the thin ctypes binding with the same entry-point names, and
:mod:`.inputs` holds the seeded synthetic input generators and :mod:`.profiling` turns rocprofv3
counter runs into the HBM-traffic summaries kept under ``profiles/``.  Submodules are imported lazily so that
the input generators can be used on hosts without the built library.
"""
import importlib

__all__ = ["llsa", "inputs", "profiling"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
