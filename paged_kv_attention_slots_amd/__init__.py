"""Paged-KV attention step (store_kv, decode, ragged prefill) for MI355X.

The kernels live in ``libmsgl.so`` (built from ``csrc/`` by ``build.py``)
behind the C ABI in ``include/msgl.h``; ``_lib`` is the ctypes binding with
the same entry-point names, ``runner`` drives a whole step, and ``workloads``
builds seeded synthetic inputs.  Importing ``_lib`` (or ``runner``) raises
when the library has not been built: there is no CPU fallback.
"""

__all__ = ["workloads", "runner", "build"]
