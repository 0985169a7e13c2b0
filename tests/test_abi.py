"""The C-ABI library loads and exports every function include/kvpub.h declares;
host-side argument checks; the product path has no CPU fallback.  No GPU
compute is run here."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

from replicated_fp8_sparse_amd import kvpub

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvpub.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"KVPUB_API\s+[\w\s\*]+?\b(kvpub_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(kvpub.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = kvpub.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", kvpub.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kvpub_\w+)", out))
    assert exported == set(declared_functions())


def test_struct_layouts_match_the_header():
    cfg = kvpub.kvpub_config_init(2, 3, 100)
    assert cfg.struct_size == ctypes.sizeof(kvpub.kvpub_config) == 80
    assert (cfg.num_replicas, cfg.num_layers, cfg.block_size, cfg.num_pages) == (2, 3, 64, 100)
    assert cfg.main_page_stride == 41984 and cfg.idx_page_stride == 8448
    assert cfg.main_layer_stride == 100 * 41984 and cfg.idx_layer_stride == 100 * 8448
    assert ctypes.sizeof(kvpub.kvpub_layer_io) == 72
    assert kvpub.kvpub_abi_version() == 1


def test_strerror_covers_every_status():
    for st in range(7):
        assert kvpub.kvpub_strerror(st) not in ("unknown status", "")
    assert kvpub.kvpub_strerror(99) == "unknown status"


def test_host_side_argument_checks():
    cfg = kvpub.kvpub_config_init(2, 1, 4)
    cfg.num_replicas = 0
    st, ctx = kvpub.kvpub_create(cfg, [16, 32], [16, 32])
    assert st == kvpub.KVPUB_ERR_INVALID_ARG and ctx is None
    cfg = kvpub.kvpub_config_init(2, 1, 4)
    st, ctx = kvpub.kvpub_create(cfg, [16, 0], [16, 32])          # null base
    assert st == kvpub.KVPUB_ERR_INVALID_ARG
    st, ctx = kvpub.kvpub_create(cfg, [16, 40], [16, 32])         # misaligned base
    assert st == kvpub.KVPUB_ERR_INVALID_ARG
    assert kvpub.kvpub_store(None, 0, 4, 16, 512, 16, 64, 16, 128, 16, 0) == kvpub.KVPUB_ERR_INVALID_ARG
    assert kvpub.kvpub_gather(None, 0, 0, 4, 16, 16, 512, 16, 64, 16, 128, 0) == kvpub.KVPUB_ERR_INVALID_ARG
    assert kvpub.kvpub_fence(None, 0, 0) == kvpub.KVPUB_ERR_INVALID_ARG
    assert kvpub.kvpub_fence_host_epoch(None, 0, 0) == kvpub.KVPUB_ERR_INVALID_ARG
    assert kvpub.kvpub_graph_replay(None, 0) == kvpub.KVPUB_ERR_INVALID_ARG
    assert kvpub.kvpub_graph_destroy(None) == kvpub.KVPUB_OK
    assert kvpub.kvpub_destroy(None) == kvpub.KVPUB_OK
    st, _ = kvpub.kvpub_epoch_read(None, 0)
    assert st == kvpub.KVPUB_ERR_INVALID_ARG
    # VMM storage: argument checks come before any HIP call
    cfg = kvpub.kvpub_config_init(2, 1, 4)
    assert kvpub.kvpub_vmm_create(cfg, 3)[0] == kvpub.KVPUB_ERR_INVALID_ARG       # max below the initial pages
    cfg.num_replicas = 0
    assert kvpub.kvpub_vmm_create(cfg, 8)[0] == kvpub.KVPUB_ERR_INVALID_ARG
    cfg = kvpub.kvpub_config_init(2, 1, 4)
    cfg.idx_page_stride = 8 * 1024                                                # below one Indexer-K page
    assert kvpub.kvpub_vmm_create(cfg, 8)[0] == kvpub.KVPUB_ERR_INVALID_ARG
    assert kvpub.kvpub_vmm_grow(None, 8) == kvpub.KVPUB_ERR_INVALID_ARG
    assert kvpub.kvpub_vmm_pages(None)[0] == kvpub.KVPUB_ERR_INVALID_ARG
    assert kvpub.kvpub_vmm_destroy(None) == kvpub.KVPUB_OK


def test_missing_library_fails_loudly(tmp_path):
    saved = kvpub._lib
    kvpub._lib = None
    try:
        with pytest.raises(ImportError):
            kvpub.load(str(tmp_path / "libkvpub.so"))
    finally:
        kvpub._lib = saved


def test_product_code_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "replicated_fp8_sparse_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "kvpub_oracle" not in text and "kvo_" not in text, f


def _cfg(**kw):
    cfg = kvpub.kvpub_config_init(2, 2, 8)
    for k, v in kw.items():
        setattr(cfg, k, v)
    return cfg


@pytest.mark.parametrize("field,value", [
    ("struct_size", 8),                                  # wrong ABI size
    ("num_replicas", 0), ("num_replicas", 9),            # R in 1..8
    ("num_layers", 0),
    ("block_size", 32),                                  # pages hold 64 slots
    ("num_pages", 0), ("num_pages", (1 << 40) + 1),
    ("main_page_stride", 41984 - 16), ("main_page_stride", 41984 + 8),   # >= 64*656, multiple of 16
    ("idx_page_stride", 8448 - 16), ("idx_page_stride", 8448 + 4),       # >= 64*132, multiple of 16
    ("main_layer_stride", 8 * 41984 - 16),               # L > 1: room for every page
    ("idx_layer_stride", 8 * 8448 + 8),                  # L > 1: multiple of 16
    ("num_lanes", 0), ("num_lanes", 65),
    ("num_participants", 0), ("num_participants", 9),
    ("device", -1),
    ("flags", 2), ("flags", 0x80000001),                 # bits other than the release-only option
])
def test_create_rejects_each_bad_config_field(field, value):
    """Every configuration rule is checked on the host before any HIP call."""
    cfg = _cfg(**{field: value})
    st, ctx = kvpub.kvpub_create(cfg, [16, 32], [16, 32])
    assert st == kvpub.KVPUB_ERR_INVALID_ARG and ctx is None


def test_config_init_defaults():
    cfg = kvpub.kvpub_config_init(3, 5, 100)
    assert (cfg.struct_size, cfg.num_replicas, cfg.num_layers, cfg.block_size, cfg.num_pages) == \
        (ctypes.sizeof(kvpub.kvpub_config), 3, 5, 64, 100)
    assert (cfg.main_page_stride, cfg.idx_page_stride) == (64 * 656, 64 * 132)
    assert (cfg.main_layer_stride, cfg.idx_layer_stride) == (100 * 64 * 656, 100 * 64 * 132)
    assert (cfg.num_lanes, cfg.num_participants, cfg.fence_timeout_ns, cfg.device, cfg.flags) == (1, 1, 0, 0, 0)


def test_one_layer_ignores_the_layer_strides():
    """With L == 1 the layer strides address nothing and are not checked; a config with arbitrary ones
    gets past validation (and only then needs a device)."""
    cfg = kvpub.kvpub_config_init(1, 1, 8)
    cfg.main_layer_stride, cfg.idx_layer_stride = 3, 5
    st, ctx = kvpub.kvpub_create(cfg, [16], [16])       # no device here: HIP error, else a context
    assert st != kvpub.KVPUB_ERR_INVALID_ARG
    if ctx is not None:
        kvpub.kvpub_destroy(ctx)


def test_the_abi_from_plain_c(tmp_path):
    """A C99 program built against include/kvpub.h alone links libkvpub.so and
    gets the documented host-side answers (no GPU involved)."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    lib_dir = os.path.dirname(kvpub.LIB_PATH)
    exe = str(tmp_path / "abi_from_c")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-o", exe,
           os.path.join(root, "tests", "c", "abi_from_c.c"), "-I", os.path.join(root, "include"),
           "-L", lib_dir, "-lkvpub", f"-Wl,-rpath,{lib_dir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


FLOOR_HEADER = os.path.join(ROOT, "include", "kvpub_floor.h")


def test_floor_library_exports_its_header():
    """The benchmark's floor-kernel library exports what include/kvpub_floor.h declares
    and rejects bad arguments on the host (nothing launched)."""
    from replicated_fp8_sparse_amd import build, floor
    if not os.path.exists(floor.LIB_PATH):
        build.build_floor_library()
    declared = sorted(set(re.findall(r"KVPUB_FLOOR_API\s+[\w\s\*]+?\b(kvpub_\w+)\s*\(", open(FLOOR_HEADER).read())))
    assert declared == sorted(floor.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", floor.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    assert set(re.findall(r"\bT (kvpub_\w+)", out)) == set(declared)
    f = floor.kvpub_floor_stream
    assert f(0, 16, [16], 16, 0) == 1                      # null input
    assert f(16, 16, [], 16, 0) == 1                       # no output
    assert f(16, 16, [16] * 9, 16, 0) == 1                 # more than 8 outputs
    assert f(16, 24, [16], 16, 0) == 1                     # not a multiple of 16
    assert f(8, 16, [16], 16, 0) == 1                      # misaligned
    assert f(16, 16, [16], 16, 3) == 1                     # unknown policy
    assert f(16, 16, [16], 1 << 32, floor.KVPUB_FLOOR_WRITE_THROUGH) == 1   # 32-bit buffer offsets
    e = floor.kvpub_floor_empty
    assert e(0, 64) == 1                                   # no block
    assert e(1, 32) == 1 and e(1, 100) == 1                # not a multiple of 64 threads
    assert e(1, 2048) == 1                                 # more than 1024 threads
    assert e(1 << 31, 64) == 1                             # grid too large


def test_log_lines_only_when_asked():
    """KVPUB_LOG=1 prints one line per context creation (its configuration and
    status) on stderr; without it the library prints nothing."""
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from replicated_fp8_sparse_amd import kvpub\n"
            "cfg = kvpub.kvpub_config_init(2, 1, 4); cfg.num_replicas = 0\n"
            "st, ctx = kvpub.kvpub_create(cfg, [16, 32], [16, 32])\n"
            "assert st == kvpub.KVPUB_ERR_INVALID_ARG and ctx is None\n"
            "assert kvpub.kvpub_destroy(None) == kvpub.KVPUB_OK\n") % ROOT
    env = {k: v for k, v in os.environ.items() if k != "KVPUB_LOG"}
    quiet = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=120)
    assert quiet.returncode == 0, quiet.stderr
    assert "kvpub:" not in quiet.stderr
    loud = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          env=dict(env, KVPUB_LOG="1"), timeout=120)
    assert loud.returncode == 0, loud.stderr
    lines = [l for l in loud.stderr.splitlines() if l.startswith("kvpub:")]
    assert lines == ["kvpub: create R=0 L=1 pages=4 lanes=1 participants=1 device=0 flags=0 -> invalid argument "
                     "(ctx (nil))"], loud.stderr


def test_valid_calls_without_a_device_fail_cleanly():
    """A valid configuration on a machine with no usable GPU: creation returns a HIP
    (or unsupported-device) status and no handle, and nothing is left to release."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: creation would succeed")
    no_device = (kvpub.KVPUB_ERR_HIP, kvpub.KVPUB_ERR_UNSUPPORTED)
    cfg = kvpub.kvpub_config_init(2, 3, 8)
    st, ctx = kvpub.kvpub_create(cfg, [1 << 20, 2 << 20], [3 << 20, 4 << 20])
    assert st in no_device and ctx is None
    st, ctx = kvpub.kvpub_create_static(cfg, [1 << 20, 2 << 20], [3 << 20, 4 << 20])
    assert st in no_device and ctx is None
    st, vmm, _, _ = kvpub.kvpub_vmm_create(kvpub.kvpub_config_init(2, 3, 8), 16)
    assert st in no_device and vmm is None
