"""Thin ctypes binding of libkvpub_floor.so (include/kvpub_floor.h): the
plain-stream floor kernel the benchmark times beside the cache-store, and an
empty kernel (the fixed cost of a launch).
Argument marshalling only; loading fails loudly if the library is not built."""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvpub_floor.so")

KVPUB_FLOOR_WRITE_BACK = 0
KVPUB_FLOOR_NON_TEMPORAL = 1
KVPUB_FLOOR_WRITE_THROUGH = 2
POLICIES = {"write_back": KVPUB_FLOOR_WRITE_BACK, "non_temporal": KVPUB_FLOOR_NON_TEMPORAL,
            "write_through": KVPUB_FLOOR_WRITE_THROUGH}

EXPORTS = ("kvpub_floor_stream", "kvpub_floor_empty")

_lib = None


def load(path=LIB_PATH):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with replicated_fp8_sparse_amd.build."
                          "build_floor_library()")
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    lib.kvpub_floor_stream.restype = ctypes.c_int
    lib.kvpub_floor_stream.argtypes = [vp, ctypes.c_uint64, ctypes.POINTER(vp), ctypes.c_uint32,
                                       ctypes.c_uint64, ctypes.c_uint32, vp]
    lib.kvpub_floor_empty.restype = ctypes.c_int
    lib.kvpub_floor_empty.argtypes = [ctypes.c_uint32, ctypes.c_uint32, vp]
    _lib = lib
    return lib


def kvpub_floor_stream(inp, in_bytes, outs, out_bytes, policy, stream=0):
    arr = (ctypes.c_void_p * max(1, len(outs)))(*outs)
    return load().kvpub_floor_stream(inp, in_bytes, arr, len(outs), out_bytes, policy, stream)


def kvpub_floor_empty(blocks, threads, stream=0):
    return load().kvpub_floor_empty(blocks, threads, stream)
