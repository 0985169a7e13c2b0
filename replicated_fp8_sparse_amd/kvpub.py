"""Thin ctypes binding of libkvpub.so (include/kvpub.h).

Argument marshalling only: every step of the cache-store and the fence runs in
the library's HIP kernels.  Functions keep the C names and return the status
code; ``check()`` turns a non-zero status into ``KvpubError``.  Device
pointers and streams are plain integers (``tensor.data_ptr()``,
``torch.cuda.current_stream().cuda_stream``).

The library must have been built (``replicated_fp8_sparse_amd.build`` or
``__graft_entry__.build()``); loading fails loudly otherwise -- there is no
fallback path.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvpub.so")

KVPUB_OK = 0
KVPUB_ERR_INVALID_ARG = 1
KVPUB_ERR_OUT_OF_MEMORY = 2
KVPUB_ERR_UNSUPPORTED = 3
KVPUB_ERR_HIP = 4
KVPUB_ERR_CAPTURING = 5
KVPUB_ERR_FENCE_TIMEOUT = 6
KVPUB_ERR_IN_USE = 7

KVPUB_FLAG_FENCE_TIMEOUT = 0x1
KVPUB_FLAG_POISONED = 0x2

KVPUB_CONFIG_FENCE_RELEASE_ONLY = 0x1

SLOTS_PER_PAGE = 64
LATENT_DIM = 512
ROPE_DIM = 64
INDEXER_DIM = 128
MAIN_ROW_BYTES = 656
MAIN_PAGE_BYTES = 64 * 656
IDX_PAGE_BYTES = 64 * 128 + 64 * 4
IDX_SCALES_OFFSET = 64 * 128
MAX_REPLICAS = 8

# Every function include/kvpub.h declares.
EXPORTS = ("kvpub_config_init", "kvpub_create", "kvpub_create_static", "kvpub_store", "kvpub_gather", "kvpub_fence",
           "kvpub_fence_host_epoch",
           "kvpub_graph_create", "kvpub_graph_replay", "kvpub_graph_destroy",
           "kvpub_epoch_read", "kvpub_error_read", "kvpub_participant_signal",
           "kvpub_destroy", "kvpub_strerror", "kvpub_abi_version", "kvpub_vmm_create",
           "kvpub_vmm_grow", "kvpub_vmm_pages", "kvpub_vmm_destroy")


class kvpub_config(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32),
                ("num_replicas", ctypes.c_uint32),
                ("num_layers", ctypes.c_uint32),
                ("block_size", ctypes.c_uint32),
                ("num_pages", ctypes.c_uint64),
                ("main_page_stride", ctypes.c_uint64),
                ("main_layer_stride", ctypes.c_uint64),
                ("idx_page_stride", ctypes.c_uint64),
                ("idx_layer_stride", ctypes.c_uint64),
                ("num_lanes", ctypes.c_uint32),
                ("num_participants", ctypes.c_uint32),
                ("fence_timeout_ns", ctypes.c_uint64),
                ("device", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class kvpub_layer_io(ctypes.Structure):
    _fields_ = [("latent", ctypes.c_void_p),
                ("rope", ctypes.c_void_p),
                ("indexer", ctypes.c_void_p),
                ("latent_row_stride", ctypes.c_int64),
                ("rope_row_stride", ctypes.c_int64),
                ("indexer_row_stride", ctypes.c_int64),
                ("slot_mapping", ctypes.c_void_p),
                ("num_tokens", ctypes.c_int64),
                ("layer", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]


class KvpubError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: kvpub status {status} ({strerror(status)})")


_lib = None


def load(path=LIB_PATH):
    """Load libkvpub.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with replicated_fp8_sparse_amd.build."
                          "build_library() (no CPU fallback exists)")
    lib = ctypes.CDLL(path)
    vp, u32, u64, i64, i32 = (ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64,
                              ctypes.c_int64, ctypes.c_int)
    cfgp = ctypes.POINTER(kvpub_config)
    sig = {
        "kvpub_config_init": (None, [cfgp, u32, u32, u64]),
        "kvpub_create": (i32, [cfgp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp)]),
        "kvpub_create_static": (i32, [cfgp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, ctypes.POINTER(vp)]),
        "kvpub_store": (i32, [vp, u32, i64, vp, i64, vp, i64, vp, i64, vp, vp]),
        "kvpub_gather": (i32, [vp, u32, u32, i64, vp, vp, i64, vp, i64, vp, i64, vp]),
        "kvpub_fence": (i32, [vp, u32, vp]),
        "kvpub_fence_host_epoch": (i32, [vp, u32, vp]),
        "kvpub_graph_create": (i32, [vp, ctypes.POINTER(kvpub_layer_io), u32, u32, ctypes.POINTER(vp)]),
        "kvpub_graph_replay": (i32, [vp, vp]),
        "kvpub_graph_destroy": (i32, [vp]),
        "kvpub_epoch_read": (i32, [vp, u32, ctypes.POINTER(u64)]),
        "kvpub_error_read": (i32, [vp, ctypes.POINTER(u64), ctypes.POINTER(u32), i32]),
        "kvpub_participant_signal": (i32, [vp, u32, u32, ctypes.POINTER(ctypes.POINTER(u64))]),
        "kvpub_destroy": (i32, [vp]),
        "kvpub_strerror": (ctypes.c_char_p, [i32]),
        "kvpub_abi_version": (u32, []),
        "kvpub_vmm_create": (i32, [cfgp, u64, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp)]),
        "kvpub_vmm_grow": (i32, [vp, u64, vp]),
        "kvpub_vmm_pages": (i32, [vp, ctypes.POINTER(u64)]),
        "kvpub_vmm_destroy": (i32, [vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def strerror(status):
    try:
        return load().kvpub_strerror(int(status)).decode()
    except ImportError:
        return "library not loaded"


def check(status, what="kvpub"):
    if status != KVPUB_OK:
        raise KvpubError(status, what)
    return status


# -- same names as the C ABI ------------------------------------------------

def kvpub_config_init(num_replicas, num_layers, num_pages):
    cfg = kvpub_config()
    load().kvpub_config_init(ctypes.byref(cfg), num_replicas, num_layers, num_pages)
    return cfg


def kvpub_create(cfg, main_bases, idx_bases):
    """Returns (status, ctx handle or None).  Bases are device addresses (ints)."""
    R = len(main_bases)
    mb = (ctypes.c_void_p * R)(*main_bases)
    ib = (ctypes.c_void_p * R)(*idx_bases)
    out = ctypes.c_void_p()
    st = load().kvpub_create(ctypes.byref(cfg), mb, ib, ctypes.byref(out))
    return st, (out.value if st == KVPUB_OK else None)


def kvpub_create_static(cfg, main_bases, idx_bases, stream=0):
    """Returns (status, ctx handle or None); the context's words live in the
    library's static per-GPU array (no allocation)."""
    R = len(main_bases)
    mb = (ctypes.c_void_p * R)(*main_bases)
    ib = (ctypes.c_void_p * R)(*idx_bases)
    out = ctypes.c_void_p()
    st = load().kvpub_create_static(ctypes.byref(cfg), mb, ib, stream, ctypes.byref(out))
    return st, (out.value if st == KVPUB_OK else None)


def kvpub_store(ctx, layer, num_tokens, latent, latent_row_stride, rope, rope_row_stride,
                indexer, indexer_row_stride, slot_mapping, stream=0):
    return load().kvpub_store(ctx, layer, num_tokens, latent, latent_row_stride, rope,
                              rope_row_stride, indexer, indexer_row_stride, slot_mapping,
                              stream)


def kvpub_gather(ctx, replica, layer, num_tokens, slot_mapping, latent_out, latent_row_stride,
                 rope_out, rope_row_stride, indexer_out, indexer_row_stride, stream=0):
    return load().kvpub_gather(ctx, replica, layer, num_tokens, slot_mapping, latent_out,
                               latent_row_stride, rope_out, rope_row_stride, indexer_out,
                               indexer_row_stride, stream)


def kvpub_fence(ctx, lane=0, stream=0):
    return load().kvpub_fence(ctx, lane, stream)


def kvpub_fence_host_epoch(ctx, lane=0, stream=0):
    return load().kvpub_fence_host_epoch(ctx, lane, stream)


def kvpub_graph_create(ctx, ios, lane=0):
    """ios: sequence of kvpub_layer_io.  Returns (status, graph handle or None)."""
    n = len(ios)
    arr = (kvpub_layer_io * n)(*ios)
    out = ctypes.c_void_p()
    st = load().kvpub_graph_create(ctx, arr, n, lane, ctypes.byref(out))
    return st, (out.value if st == KVPUB_OK else None)


def kvpub_graph_replay(graph, stream=0):
    return load().kvpub_graph_replay(graph, stream)


def kvpub_graph_destroy(graph):
    return load().kvpub_graph_destroy(graph)


def kvpub_epoch_read(ctx, lane=0):
    v = ctypes.c_uint64()
    st = load().kvpub_epoch_read(ctx, lane, ctypes.byref(v))
    return st, v.value


def kvpub_error_read(ctx, clear=False):
    """Returns (status, invalid_slots, flags)."""
    inv = ctypes.c_uint64()
    fl = ctypes.c_uint32()
    st = load().kvpub_error_read(ctx, ctypes.byref(inv), ctypes.byref(fl), 1 if clear else 0)
    return st, inv.value, fl.value


def kvpub_participant_signal(ctx, lane, p):
    """Returns (status, ctypes pointer to the host-coherent uint64 signal word)."""
    out = ctypes.POINTER(ctypes.c_uint64)()
    st = load().kvpub_participant_signal(ctx, lane, p, ctypes.byref(out))
    return st, (out if st == KVPUB_OK else None)


def kvpub_destroy(ctx):
    return load().kvpub_destroy(ctx)


def kvpub_abi_version():
    return load().kvpub_abi_version()


def kvpub_vmm_create(cfg, max_pages):
    """Returns (status, vmm handle or None, main base addresses, idx base addresses);
    cfg's layer strides are updated in place."""
    R = cfg.num_replicas
    mb = (ctypes.c_void_p * max(R, 1))()
    ib = (ctypes.c_void_p * max(R, 1))()
    out = ctypes.c_void_p()
    st = load().kvpub_vmm_create(ctypes.byref(cfg), max_pages, mb, ib, ctypes.byref(out))
    if st != KVPUB_OK:
        return st, None, [], []
    return st, out.value, [mb[r] for r in range(R)], [ib[r] for r in range(R)]


def kvpub_vmm_grow(vmm, num_pages, ctx=None):
    return load().kvpub_vmm_grow(vmm, num_pages, ctx)


def kvpub_vmm_pages(vmm):
    v = ctypes.c_uint64()
    st = load().kvpub_vmm_pages(vmm, ctypes.byref(v))
    return st, v.value


def kvpub_vmm_destroy(vmm):
    return load().kvpub_vmm_destroy(vmm)


def kvpub_strerror(status):
    return strerror(status)


def layer_io(latent, rope, indexer, slot_mapping, num_tokens, layer,
             latent_row_stride=LATENT_DIM, rope_row_stride=ROPE_DIM,
             indexer_row_stride=INDEXER_DIM):
    """Build a kvpub_layer_io from device addresses."""
    return kvpub_layer_io(latent, rope, indexer, latent_row_stride, rope_row_stride,
                          indexer_row_stride, slot_mapping, num_tokens, layer, 0)
