"""int4 compressed-domain decode attention for AMD Instinct MI355X (gfx950).

The product is libtq.so (C ABI in include/tq.h); ``tq`` is its ctypes binding and
``workloads`` draws the seeded synthetic inputs.
"""
from . import tq  # noqa: F401
