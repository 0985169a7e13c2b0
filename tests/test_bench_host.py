"""CPU checks of the benchmark's host logic (bench.py): the algorithmic byte
count behind the roofline, the committed rocprofv3 record it quotes and the rule
that drops it once the store kernel's source changes, and the one-GPU guard."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_per_launch():
    # per valid token: the bf16 rows read once (latent 512 + RoPE 64 + indexer 128 elements),
    # and per replica the 656-byte Main-KV row plus 128 Indexer-K codes and a 4-byte scale
    assert bench.READ_BYTES_PER_TOKEN == 1408
    assert bench.WRITE_BYTES_PER_TOKEN_PER_REPLICA == 788
    assert bench.alg_bytes(4096, 2) == 12_222_464
    assert bench.alg_bytes(32768, 4) == 149_422_080
    assert bench.alg_bytes(0, 8) == 0


def test_committed_profile_record_is_consistent():
    """The record's traffic is its counters times their calibration factors, for the
    graph layer's algorithmic bytes; while the kernel source still has the recorded
    hash, the benchmark quotes exactly these figures."""
    rec = json.load(open(bench.TRAFFIC_RECORD))
    cal = rec["calibration"]
    want = round(rec["fetch_kib_per_launch"] * cal["fetch_factor"] * 1024
                 + rec["write_kib_per_launch"] * cal["write_factor"] * 1024)
    assert abs(rec["traffic_bytes_per_launch"] - want) <= 0.001 * want
    assert rec["alg_bytes_per_launch"] == bench.alg_bytes(4096, 2)
    assert rec["kernel"] == "store_kernel<2, true, false, true, 4>"
    kt = rec["kernel_trace"]
    assert os.path.exists(os.path.join(ROOT, kt["summary"]))
    assert kt["dispatches"] > 0 and kt["timed_replays_mean_ns"] > 0
    for cmd in rec["commands"] + [kt["command"]]:
        assert "bench.py" in cmd and "_work" not in cmd
    quoted, why = bench.profile_record()
    if quoted is None:
        pytest.skip(f"not quoted by the benchmark: {why}")
    traffic, how = bench.measured_traffic()
    assert traffic == rec["traffic_bytes_per_launch"] and "FETCH_SIZE" in how
    assert bench.traced_durations()["dispatches"] == kt["dispatches"]


def test_profile_record_is_dropped_when_the_kernel_source_changes(tmp_path, monkeypatch):
    src = tmp_path / "store_kernel.hip"
    src.write_bytes(open(bench.KERNEL_SOURCE, "rb").read() + b"\n// edited\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(src))
    rec, why = bench.profile_record()
    assert rec is None and "changed" in why
    assert bench.measured_traffic() == (None, why)
    assert bench.traced_durations() is None
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(tmp_path / "missing.json"))
    assert bench.profile_record() == (None, "no profile record")


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8", "--steps", "3"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env=e, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_an_auxiliary_leg_that_fails_is_recorded_not_fatal(capsys):
    assert bench.aux_leg("ok leg", lambda: {"x": 1}) == {"x": 1}

    def broken():
        raise RuntimeError("no VMM on this device")

    assert bench.aux_leg("vmm leg", broken) == {"error": "RuntimeError: no VMM on this device"}
    assert "vmm leg failed" in capsys.readouterr().err
