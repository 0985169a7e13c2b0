"""The benchmark's plain-stream floor kernel writes what it documents: each output
piece is the input piece of the same index (past the input's end, its index)."""
import numpy as np
import pytest

from replicated_fp8_sparse_amd import floor

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("policy", sorted(floor.POLICIES))
@pytest.mark.parametrize("in_bytes,out_bytes,n_outs", [(1 << 20, 592 << 10, 2), (4096, 8192, 3), (16, 16, 1)])
def test_floor_stream_bytes(policy, in_bytes, out_bytes, n_outs):
    import torch
    print(f"[gpu-test] floor {policy} in={in_bytes} out={out_bytes} x{n_outs}", flush=True)
    rng = np.random.default_rng(in_bytes + out_bytes)
    src = torch.from_numpy(rng.integers(0, 256, in_bytes, dtype=np.uint8)).to("cuda")
    outs = [torch.zeros(out_bytes, dtype=torch.uint8, device="cuda") for _ in range(n_outs)]
    s = torch.cuda.current_stream().cuda_stream
    assert floor.kvpub_floor_stream(src.data_ptr(), in_bytes, [o.data_ptr() for o in outs], out_bytes,
                                    floor.POLICIES[policy], s) == 0
    torch.cuda.synchronize()
    want = np.empty(out_bytes, np.uint8)
    n = min(in_bytes, out_bytes)
    want[:n] = src.cpu().numpy()[:n]
    if out_bytes > in_bytes:
        idx = np.arange(in_bytes // 16, out_bytes // 16, dtype=np.uint32)
        want[in_bytes:] = np.repeat(idx, 4).view(np.uint8)
    for o in outs:
        assert np.array_equal(o.cpu().numpy(), want)


@pytest.mark.parametrize("blocks,threads", [(1, 64), (256, 256), (1024, 1024)])
def test_floor_empty_launches(blocks, threads):
    """The empty kernel launches with the documented shapes and leaves the stream usable."""
    import torch
    print(f"[gpu-test] floor empty {blocks}x{threads}", flush=True)
    s = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        assert floor.kvpub_floor_empty(blocks, threads, s) == 0
    torch.cuda.synchronize()
    x = torch.arange(8, device="cuda")
    assert int(x.sum()) == 28
