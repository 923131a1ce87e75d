"""MI355X (gfx950) implementation of the Memory Sparse Attention hot path.

The work is done by libmsa.so (HIP kernels behind the C ABI of
include/msa.h); ``_lib`` is its ctypes binding and ``synth`` draws seeded
synthetic inputs.  Importing the package does not load the library; the
first call through ``_lib`` does, and raises if it has not been built.
"""

from . import synth  # noqa: F401
from ._lib import (  # noqa: F401
    Assembly,
    MSAError,
    RouteCall,
    assemble,
    assemble_workspace_bytes,
    attend_workspace_bytes,
    bank_rows,
    decode_workspace_bytes,
    doc_map,
    doc_map_bytes,
    load,
    pool_encode,
    route,
    route_workspace_bytes,
    sparse_attend,
    sparse_decode,
    sparse_decode_noalloc,
)

__all__ = ["Assembly", "MSAError", "RouteCall", "assemble", "assemble_workspace_bytes", "attend_workspace_bytes", "bank_rows",
           "decode_workspace_bytes", "doc_map", "doc_map_bytes", "load", "pool_encode", "route",
           "route_workspace_bytes", "sparse_attend", "sparse_decode", "sparse_decode_noalloc", "synth"]
