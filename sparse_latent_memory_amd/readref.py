"""ctypes binding of libmsa_readref.so: the reference streaming read in the
tiled router bank's access pattern (include/msa_readref.h).  Measurement
only; bench.py times it on the bank buffer beside the bank scan."""

import ctypes
import os

import torch

from . import _lib

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmsa_readref.so")
EXPORTS = ("msa_ref_read_tiles",)
TILE_BYTES = 32768

_ref = None


def load():
    """Load libmsa_readref.so (after torch, sharing its HIP runtime)."""
    global _ref
    if _ref is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmsa_readref.so is not built ({LIB_PATH}); run "
                               "`python -m sparse_latent_memory_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        lib.msa_ref_read_tiles.argtypes = [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P, P, P]
        lib.msa_ref_read_tiles.restype = ctypes.c_int
        _ref = lib
    return _ref


def read_tiles(buf, grid, nontemporal=True, sink=None, stream=None, events=None):
    """Read the whole 32 KiB tiles of the device tensor `buf` (its bytes
    rounded down to a tile multiple).  Returns (sink, bytes read); sink holds
    grid*256 16-byte XOR folds (int32 [grid*256*4]) whose XOR is the XOR of
    the bytes read."""
    n_bytes = buf.numel() * buf.element_size() // TILE_BYTES * TILE_BYTES
    if n_bytes == 0:
        raise ValueError("buf holds less than one 32 KiB tile")
    if sink is None:
        sink = torch.empty(grid * 256 * 4, dtype=torch.int32, device=buf.device)
    if sink.numel() * sink.element_size() < grid * 256 * 16:
        raise ValueError(f"sink needs {grid * 256 * 16} bytes")
    ev = events if events is not None else (None, None)
    rc = load().msa_ref_read_tiles(_lib._dptr(buf, "buf"), n_bytes, grid, 1 if nontemporal else 0,
                                   _lib._dptr(sink, "sink"), _lib._stream(stream), ev[0], ev[1])
    if rc != 0:
        raise RuntimeError(f"msa_ref_read_tiles returned {rc}")
    return sink, n_bytes
