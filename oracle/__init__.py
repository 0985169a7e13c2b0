"""CPU oracle of the replicated FP8 KV cache-store -- TEST INFRASTRUCTURE ONLY.

The plain C definition lives in ``kvpub_oracle.c`` (see its header for the
passages of the pages it follows and the readings it takes).  This module
only loads the compiled library and marshals numpy arrays into it.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  The GPU library and its Python binding never
do: the two paths share no code.
"""
import ctypes
import os

import numpy as np

from .build import build_oracle, lib_path

MAIN_ROW_BYTES = 656
IDX_CODES_BYTES = 128
SLOTS_PER_PAGE = 64

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)


def _ptr(a, typ):
    return a.ctypes.data_as(typ)


class Oracle:
    """Handle on one build of the oracle library (``plant`` != 0: a planted mistake)."""

    def __init__(self, plant=0, rebuild=False):
        path = lib_path(plant)
        if rebuild or not os.path.exists(path):
            build_oracle(plant)
        self.plant = plant
        self.lib = lib = ctypes.CDLL(path)
        lib.kvo_e4m3_encode.restype = ctypes.c_uint8
        lib.kvo_e4m3_encode.argtypes = [ctypes.c_float]
        lib.kvo_e4m3_encode_array.restype = None
        lib.kvo_e4m3_encode_array.argtypes = [_f32p, ctypes.c_size_t, _u8p]
        lib.kvo_quant_tiles.restype = None
        lib.kvo_quant_tiles.argtypes = [_u16p, ctypes.c_size_t, _u8p, _f32p]
        lib.kvo_encode_rows.restype = None
        lib.kvo_encode_rows.argtypes = [ctypes.c_int64, _u16p, ctypes.c_int64, _u16p,
                                        ctypes.c_int64, _u16p, ctypes.c_int64,
                                        _u8p, _u8p, _u8p]
        lib.kvo_store.restype = ctypes.c_int64
        lib.kvo_store.argtypes = [ctypes.c_uint32, ctypes.POINTER(_u8p), ctypes.POINTER(_u8p),
                                  ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                  ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32,
                                  ctypes.c_int64, _u16p, ctypes.c_int64, _u16p,
                                  ctypes.c_int64, _u16p, ctypes.c_int64, _i64p]
        lib.kvo_dequant_tile.restype = None
        lib.kvo_dequant_tile.argtypes = [_u8p, ctypes.c_float, ctypes.c_size_t, _u16p]
        lib.kvo_gather.restype = ctypes.c_int64
        lib.kvo_gather.argtypes = [_u8p, _u8p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                   ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                   _i64p, _u16p, ctypes.c_int64, _u16p, ctypes.c_int64, _u16p,
                                   ctypes.c_int64]
        lib.kvo_epoch_after.restype = ctypes.c_uint64
        lib.kvo_epoch_after.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.kvo_plant_id.restype = ctypes.c_int
        lib.kvo_plant_id.argtypes = []
        assert lib.kvo_plant_id() == plant

    # -- e4m3 ---------------------------------------------------------
    def e4m3_encode(self, v):
        """Encode a float32 array (any shape) to e4m3fn codes (uint8, same shape)."""
        v = np.ascontiguousarray(v, dtype=np.float32)
        out = np.empty(v.shape, dtype=np.uint8)
        self.lib.kvo_e4m3_encode_array(_ptr(v, _f32p), v.size, _ptr(out, _u8p))
        return out

    # -- tiles --------------------------------------------------------
    def quant_tiles(self, x_bits):
        """x_bits: uint16 bf16 patterns, shape [..., 128].  Returns (codes u8, scales f32)."""
        x = np.ascontiguousarray(x_bits, dtype=np.uint16)
        assert x.shape[-1] == 128
        n = x.size // 128
        codes = np.empty(x.shape, dtype=np.uint8)
        scales = np.empty(x.shape[:-1], dtype=np.float32)
        self.lib.kvo_quant_tiles(_ptr(x, _u16p), n, _ptr(codes, _u8p), _ptr(scales, _f32p))
        return codes, scales

    # -- rows ---------------------------------------------------------
    def encode_rows(self, latent, rope, indexer):
        """Per-token rows: (main [T,656] u8, idx codes [T,128] u8, idx scale bytes [T,4] u8)."""
        latent = np.ascontiguousarray(latent, dtype=np.uint16)
        rope = np.ascontiguousarray(rope, dtype=np.uint16)
        indexer = np.ascontiguousarray(indexer, dtype=np.uint16)
        T = latent.shape[0]
        assert latent.shape == (T, 512) and rope.shape == (T, 64) and indexer.shape == (T, 128)
        main = np.empty((T, MAIN_ROW_BYTES), dtype=np.uint8)
        codes = np.empty((T, IDX_CODES_BYTES), dtype=np.uint8)
        scales = np.empty((T, 4), dtype=np.uint8)
        self.lib.kvo_encode_rows(T, _ptr(latent, _u16p), 512, _ptr(rope, _u16p), 64,
                                 _ptr(indexer, _u16p), 128, _ptr(main, _u8p),
                                 _ptr(codes, _u8p), _ptr(scales, _u8p))
        return main, codes, scales

    # -- the store ----------------------------------------------------
    def store(self, main_replicas, idx_replicas, *, num_pages, main_page_stride,
              main_layer_stride, idx_page_stride, idx_layer_stride, layer,
              latent, rope, indexer, slot_mapping):
        """Insert every valid token into each host replica (uint8 numpy buffers, modified
        in place).  Returns the number of invalid slots."""
        R = len(main_replicas)
        assert len(idx_replicas) == R
        for b in list(main_replicas) + list(idx_replicas):
            assert b.dtype == np.uint8 and b.flags.c_contiguous
        latent = np.ascontiguousarray(latent, dtype=np.uint16)
        rope = np.ascontiguousarray(rope, dtype=np.uint16)
        indexer = np.ascontiguousarray(indexer, dtype=np.uint16)
        slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
        T = slots.shape[0]
        need_main = layer * main_layer_stride + num_pages * main_page_stride
        need_idx = layer * idx_layer_stride + num_pages * idx_page_stride
        for b in main_replicas:
            assert b.size >= need_main
        for b in idx_replicas:
            assert b.size >= need_idx
        mb = (_u8p * R)(*[_ptr(b, _u8p) for b in main_replicas])
        ib = (_u8p * R)(*[_ptr(b, _u8p) for b in idx_replicas])
        return int(self.lib.kvo_store(R, mb, ib, num_pages, main_page_stride,
                                      main_layer_stride, idx_page_stride, idx_layer_stride,
                                      layer, T, _ptr(latent, _u16p), latent.shape[1] if T else 512,
                                      _ptr(rope, _u16p), rope.shape[1] if T else 64,
                                      _ptr(indexer, _u16p), indexer.shape[1] if T else 128,
                                      _ptr(slots, _i64p)))

    # -- the reader ---------------------------------------------------
    def dequant_tile(self, codes, scale):
        """codes: uint8 array (any length) sharing one fp32 scale -> bf16 bit patterns."""
        c = np.ascontiguousarray(codes, dtype=np.uint8)
        out = np.empty(c.shape, dtype=np.uint16)
        self.lib.kvo_dequant_tile(_ptr(c, _u8p), float(np.float32(scale)), c.size, _ptr(out, _u16p))
        return out

    def gather(self, main_replica, idx_replica, *, num_pages, main_page_stride, main_layer_stride,
               idx_page_stride, idx_layer_stride, layer, slot_mapping):
        """Dequantizing gather from one host replica: (latent [T,512], rope [T,64], indexer [T,128])
        as bf16 bit patterns (uint16), and the number of out-of-range slots."""
        for b in (main_replica, idx_replica):
            assert b.dtype == np.uint8 and b.flags.c_contiguous
        slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
        T = slots.shape[0]
        assert main_replica.size >= layer * main_layer_stride + num_pages * main_page_stride
        assert idx_replica.size >= layer * idx_layer_stride + num_pages * idx_page_stride
        lat = np.empty((T, 512), dtype=np.uint16)
        rope = np.empty((T, 64), dtype=np.uint16)
        idx = np.empty((T, 128), dtype=np.uint16)
        bad = self.lib.kvo_gather(_ptr(main_replica, _u8p), _ptr(idx_replica, _u8p), num_pages,
                                  main_page_stride, main_layer_stride, idx_page_stride,
                                  idx_layer_stride, layer, T, _ptr(slots, _i64p),
                                  _ptr(lat, _u16p), 512, _ptr(rope, _u16p), 64, _ptr(idx, _u16p), 128)
        return lat, rope, idx, int(bad)

    def epoch_after(self, e0, n_fences):
        return int(self.lib.kvo_epoch_after(e0, n_fences))


_default = None


def get():
    """The real (unplanted) oracle, built on first use."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
