"""The system's own LZ4 library (liblz4, the reference implementation of the
LZ4 block format), loaded with ctypes when it is installed: an encoder and a
decoder written by someone else, to check the oracle's and the GPU's blocks
against.  Only the tests use it; `available()` is False where it is missing.
"""
import ctypes
import ctypes.util

import numpy as np

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib or None
    name = ctypes.util.find_library("lz4") or "liblz4.so.1"
    try:
        lib = ctypes.CDLL(name)
        for f in ("LZ4_compress_default", "LZ4_decompress_safe", "LZ4_compressBound"):
            getattr(lib, f)
    except (OSError, AttributeError):
        _lib = False
        return None
    lib.LZ4_compress_default.argtypes = [ctypes.c_char_p, ctypes.c_char_p, ctypes.c_int, ctypes.c_int]
    lib.LZ4_compress_fast.argtypes = [ctypes.c_char_p, ctypes.c_char_p, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.LZ4_decompress_safe.argtypes = [ctypes.c_char_p, ctypes.c_char_p, ctypes.c_int, ctypes.c_int]
    lib.LZ4_compressBound.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def available() -> bool:
    return _load() is not None


def version() -> int:
    return int(_load().LZ4_versionNumber())


def compress_block(data: bytes, acceleration: int = 1) -> bytes:
    """One LZ4 block of `data` as the library's fast compressor writes it."""
    lib = _load()
    cap = lib.LZ4_compressBound(len(data))
    out = ctypes.create_string_buffer(max(cap, 1))
    n = lib.LZ4_compress_fast(bytes(data), out, len(data), cap, acceleration)
    assert n > 0 or len(data) == 0, n
    return out.raw[:n]


def decompress_block(comp: bytes, out_size: int):
    """The library's decode of one block into at most out_size bytes: the bytes,
    or None when it rejects the block."""
    lib = _load()
    out = ctypes.create_string_buffer(max(out_size, 1))
    n = lib.LZ4_decompress_safe(bytes(comp), out, len(comp), out_size)
    return None if n < 0 else out.raw[:n]


def compress_blocks(data, block_bytes=65536, acceleration=1):
    """Blocks of `data` (any array, viewed as bytes), each compressed by the
    library, laid end to end: (payload, offsets, sizes) in the layout of
    oracle.lz4_encode_blocks."""
    b = np.ascontiguousarray(data).view(np.uint8).reshape(-1).tobytes()
    comps = [compress_block(b[i:i + block_bytes], acceleration) for i in range(0, len(b), block_bytes)]
    sizes = np.array([len(c) for c in comps], np.uint32)
    offsets = np.concatenate([[0], np.cumsum(sizes, dtype=np.uint64)[:-1]]).astype(np.uint64)
    payload = np.frombuffer(b"".join(comps), np.uint8).copy()
    return payload, offsets, sizes
