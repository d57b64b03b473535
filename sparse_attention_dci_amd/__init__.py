"""IceCache decode hot path for AMD Instinct MI355X (gfx950).

The library is a C-ABI shared object (``csrc/`` -> ``libice.so``) whose calls
are declared in ``include/ice.h``; ``binding`` is a thin ctypes layer over it
that marshals torch tensors (device memory and streams only).  ``workloads``
draws seeded synthetic inputs.  Nothing here falls back to a CPU path: when
the compiled library is missing, the binding raises.
"""
__all__ = ["binding", "workloads"]
