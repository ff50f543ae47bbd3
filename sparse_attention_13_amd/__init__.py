"""Sparse flash attention for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library ``libsfa.so`` (C-ABI declared in
``include/sfa.h``); ``binding`` is the thin ctypes layer over it and ``api``
the PyTorch-facing calls that allocate outputs and pass pointers and the
current stream.
"""
