"""ReplaySSM decode-time state engine for AMD MI355X (gfx950).

The compute path is the C-ABI library ``librssm.so`` (hand-written HIP kernels,
declared in ``include/rssm.h``); :mod:`.rssm` is its thin ctypes binding with
the same entry-point names.  Nothing is loaded at import time: the library is
opened on first use, and every entry point raises if it is missing.
"""
__all__ = ["rssm", "synthetic"]
