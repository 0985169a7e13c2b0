#!/usr/bin/env python3
"""Benchmark of the replicated FP8 cache-store + device-epoch fence on one MI355X.

A step is one replay of the captured graph of the model shape: 61 sparse
layers, each a kvpub_store of T=4096 tokens into R=2 replica caches of 8192
64-slot pages followed by one kvpub_fence (system-scope release, then acquire
wait on the epoch), so every part of the hot path runs: slot decode, row
loads, tile amax, scale, e4m3 quantization, row packing, the R-way fan-out
stores, the fence, graph replay.  Inputs are seeded N(0,1) bf16 rows already
resident in HBM; the cache layout is the one the library documents (656-byte
Main-KV rows, 8448-byte Indexer-K pages).  After the graph workload's timing
legs the replicas are checked for identity and one layer against the CPU oracle.

Printed: one JSON line with tokens/s (value), the store kernel's achieved HBM
bandwidth against the 8 TB/s peak (roofline), the fence cost per layer in its
three forms (release + acquire wait, release only, and the pages' earlier
two-launch fence with a host-held epoch), the plain-stream floor for the same
bytes, the prefill and heavy-tail store shapes, and the CPU oracle timed on a
bounded sample of the same workload (cpu_baseline).

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
READ_BYTES_PER_TOKEN = (512 + 64 + 128) * 2         # bf16 rows read
WRITE_BYTES_PER_TOKEN_PER_REPLICA = 656 + 128 + 4   # Main-KV row + Indexer-K codes + scale


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "store_kernel_graph_T4096_R2_traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "replicated_fp8_sparse_amd", "csrc", "store_kernel.hip")


def profile_record():
    """The committed rocprofv3 record of the store kernel (FETCH_SIZE / WRITE_SIZE and
    the kernel trace's durations), or (None, why) if the kernel source changed since."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_RECORD))
        src = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None, "no profile record"
    if rec.get("source_sha256") != src:
        return None, "the kernel source changed since the profile was taken"
    return rec, None


def measured_traffic():
    """(HBM bytes per store launch, how) from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE record, or (None, why) if the kernel source changed since."""
    rec, why = profile_record()
    if rec is None:
        return None, why
    cal = rec["calibration"]
    return rec["traffic_bytes_per_launch"], (
        f"bytes per launch: rocprofv3 FETCH_SIZE x{cal['fetch_factor']} + WRITE_SIZE x{cal['write_factor']}, "
        "the factors from the floor kernel moving the same bytes (profiles/store_kernel_graph_T4096_R2_traffic.json)")


def traced_durations():
    """The store kernel's rocprofv3 kernel-trace durations from the committed record
    (the roofline's launches: the store-only graph's timed replays), or None."""
    rec, _ = profile_record()
    if rec is None or "kernel_trace" not in rec:
        return None
    kt = rec["kernel_trace"]
    return {"mean_us": round(kt["timed_replays_mean_ns"] / 1e3, 3), "p50_us": round(kt["timed_replays_p50_ns"] / 1e3, 3),
            "dispatches": kt["dispatches"], "live_us_same_box": kt["live_us_same_box"],
            "how": "rocprofv3 --kernel-trace of this benchmark (" + kt["summary"] + "); the tracer leaves 3-4 us "
                   "between dispatches, so each one starts on an idle GPU (its XCDs start up to 1.4 us apart), "
                   "which back-to-back replays do not; live_us_same_box is this line's avg_launch_us measured "
                   "untraced on the box of the trace"}


def alg_bytes(valid_tokens, replicas):
    return valid_tokens * (READ_BYTES_PER_TOKEN + replicas * WRITE_BYTES_PER_TOKEN_PER_REPLICA)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the prefill / heavy-tail store-only figures")
    ap.add_argument("--no-vmm", action="store_true",
                    help="skip the heavy-tail store on VMM-backed replicas (hardware-counter passes use this)")
    ap.add_argument("--cpu-runs", type=int, default=5,
                    help="runs per CPU-baseline leg (the median is reported)")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (torch copy_) three times, so that "
                         "memory-traffic counters can be scaled by a kernel of known size")
    return ap.parse_args()


class Timer:
    """HIP events on a given torch stream."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.torch.cuda.synchronize()
        self.a.record(self.stream)
        return self

    def __exit__(self, *exc):
        self.b.record(self.stream)
        self.torch.cuda.synchronize()
        self.ms = self.a.elapsed_time(self.b)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the replicas of this path are buffers in one GPU's "
              "HBM, and publication across GPUs is not implemented; use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from replicated_fp8_sparse_amd import kvpub, workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    kvpub.load()
    dev_name = torch.cuda.get_device_name(0)
    if args.pmc_calibration:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    L, T = W.GRAPH_LAYERS, W.GRAPH_T
    layout = W.graph_layout()
    R = layout.replicas
    log(f"{dev_name}: graph workload {L} layers x T={T}, R={R}, pages={layout.num_pages}")

    main_bufs = [torch.empty(layout.main_bytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
    idx_bufs = [torch.empty(layout.idx_bytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
    for b in main_bufs:
        layout.fill_device(b, "main")
    for b in idx_bufs:
        layout.fill_device(b, "idx")
    mbp, ibp = [b.data_ptr() for b in main_bufs], [b.data_ptr() for b in idx_bufs]

    def context(flags=0):
        cfg = kvpub.kvpub_config_init(R, L, layout.num_pages)
        cfg.flags = flags
        st, c = kvpub.kvpub_create(cfg, mbp, ibp)
        kvpub.check(st, "kvpub_create")
        return c

    ctx = context()                                           # release + acquire-wait fence (default)
    ctx_rel = context(kvpub.KVPUB_CONFIG_FENCE_RELEASE_ONLY)  # release-only fence
    ctx_two = context()                                       # the two-launch host-epoch fence

    lat = torch.empty((L, T, 512), dtype=torch.bfloat16, device="cuda")
    rope = torch.empty((L, T, 64), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((L, T, 128), dtype=torch.bfloat16, device="cuda")
    W.graph_fill_inputs_device(lat, rope, idx, seed=5, replay=0)
    slots_np = W.graph_slots()
    slots = torch.from_numpy(slots_np).to("cuda")
    valid = int(((slots_np >= 0) & (slots_np < layout.capacity)).sum())

    ios = [kvpub.layer_io(lat[l].data_ptr(), rope[l].data_ptr(), idx[l].data_ptr(),
                          slots.data_ptr(), T, l) for l in range(L)]
    st, graph = kvpub.kvpub_graph_create(ctx, ios, 0)
    kvpub.check(st, "kvpub_graph_create")

    stream = torch.cuda.Stream()
    sh = stream.cuda_stream

    def store(c, l):
        kvpub.check(kvpub.kvpub_store(c, l, T, lat[l].data_ptr(), 512, rope[l].data_ptr(), 64,
                                      idx[l].data_ptr(), 128, slots.data_ptr(), sh))

    # --- the timed steps: K replays of the full store + fence graph -------------
    for _ in range(args.warmup):
        kvpub.check(kvpub.kvpub_graph_replay(graph, sh))
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done; timing {args.steps} steps")
    with Timer(torch, stream) as tm:
        for _ in range(args.steps):
            kvpub.kvpub_graph_replay(graph, sh)
    step_ms = tm.ms / args.steps
    st, epoch = kvpub.kvpub_epoch_read(ctx, 0)
    kvpub.check(st)
    assert epoch == L * (args.warmup + args.steps), epoch
    st, invalid, flags = kvpub.kvpub_error_read(ctx, False)
    kvpub.check(st)
    assert invalid == 0 and flags == 0
    tokens_per_s = valid * L / (step_ms * 1e-3)

    def graph_us(body, reps):
        """Average microseconds per replay of a torch graph of body()."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                body()
            for _ in range(2):
                g.replay()
            with Timer(torch, stream) as t:
                for _ in range(reps):
                    g.replay()
        return t.ms * 1e3 / reps, g

    reps = max(4, args.steps // 4)

    # --- store kernel alone: the same 61 stores captured without fences ---------
    us, _ = graph_us(lambda: [store(ctx, l) for l in range(L)], reps)
    store_us = us / L
    store_bytes = alg_bytes(valid, R)
    store_gbps = store_bytes / (store_us * 1e-6) / 1e9

    # --- the fence in its three forms ------------------------------------------
    fence_alone = {}
    fence_alone["acquire"], _ = graph_us(lambda: [kvpub.check(kvpub.kvpub_fence(ctx, 0, sh)) for _ in range(L)], reps)
    fence_alone["release"], _ = graph_us(
        lambda: [kvpub.check(kvpub.kvpub_fence(ctx_rel, 0, sh)) for _ in range(L)], reps)
    fence_alone["two_launch"], _ = graph_us(
        lambda: [kvpub.check(kvpub.kvpub_fence_host_epoch(ctx_two, 0, sh)) for _ in range(L)], reps)
    st, rel_graph = kvpub.kvpub_graph_create(ctx_rel, ios, 0)
    kvpub.check(st, "kvpub_graph_create (release only)")
    for _ in range(2):
        kvpub.check(kvpub.kvpub_graph_replay(rel_graph, sh))
    with Timer(torch, stream) as trel:
        for _ in range(args.steps):
            kvpub.kvpub_graph_replay(rel_graph, sh)
    rel_step_ms = trel.ms / args.steps
    kvpub.kvpub_graph_destroy(rel_graph)
    st, e_two0 = kvpub.kvpub_epoch_read(ctx_two, 0)
    kvpub.check(st)
    two_reps = reps
    two_us, _ = graph_us(lambda: [(store(ctx_two, l), kvpub.check(kvpub.kvpub_fence_host_epoch(ctx_two, 0, sh)))
                                  for l in range(L)], two_reps)
    st, e_two = kvpub.kvpub_epoch_read(ctx_two, 0)
    kvpub.check(st)
    for c in (ctx, ctx_rel, ctx_two):
        st, invalid, flags = kvpub.kvpub_error_read(c, False)
        kvpub.check(st)
        assert invalid == 0 and flags == 0
    per_layer = lambda ms: ms * 1e3 / L
    fence = {
        "form": "system-scope release RMW of the lane's epoch, then acquire loads of it (the default)",
        "in_step": round(per_layer(step_ms) - store_us, 3),
        "alone": round(fence_alone["acquire"] / L, 3),
        "layer_us": round(per_layer(step_ms), 3),
        "release_only": {"in_step": round(per_layer(rel_step_ms) - store_us, 3),
                         "alone": round(fence_alone["release"] / L, 3),
                         "layer_us": round(per_layer(rel_step_ms), 3),
                         "ms_per_step": round(rel_step_ms, 4)},
        "two_launch_host_epoch": {
            "in_step": round(two_us / L - store_us, 3),
            "alone": round(fence_alone["two_launch"] / L, 3),
            "layer_us": round(two_us / L, 3),
            "epoch_before_capture": e_two0,
            "epoch_after_replays": e_two,
            "replays": two_reps + 2,
            "epoch_if_replays_advanced_it": e_two0 + L * (two_reps + 2)},
        "how": "in_step = step time / 61 - store time per launch; alone = a graph of 61 fences / 61; "
               "two_launch_host_epoch = a publish kernel and a wait kernel per fence with the epoch counted on "
               "the host (the design the single-launch fence replaces), same 61-layer graph; its epoch stays "
               "at the value published at capture however often the graph is replayed",
    }

    # what the timed steps wrote (the later graphs of this section wrote the same bytes again)
    log("verifying the timed steps' output")
    check = verify_graph_output(torch, layout, main_bufs, idx_bufs, slots_np, layer=L // 2)

    gather = None if args.no_extras else aux_leg("gather", lambda: gather_line(torch, kvpub, ctx, slots, T, valid,
                                                                               stream))
    floor_graph = None if args.no_extras else aux_leg("floor", lambda: floor_graph_layer(torch, stream, L, T, valid,
                                                                                        R, store_us))

    extras = {}
    decode = fanout = None
    if not args.no_extras:
        extras = store_only_extras(torch, kvpub, W, stream, vmm=not args.no_vmm)
        decode = aux_leg("decode", lambda: decode_eager(torch, kvpub, W, stream))
        fanout = aux_leg("fan-out A/B", lambda: fanout_ab(torch, kvpub, W, stream))

    traffic, traffic_how = measured_traffic()
    result = {
        "metric": "cache-store tokens/sec and achieved HBM GB/s (% of peak); fence µs/layer",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "graph replay, model shape: 61 sparse layers x T=4096 tokens, R=2 replicas, "
                        "8192 pages x 64 slots per replica per layer-cache, store + fence per layer",
            "layers": L, "tokens_per_layer": T, "valid_tokens_per_layer": valid, "replicas": R,
            "pages": layout.num_pages, "inputs": "bf16 N(0,1), latent 512 + rope 64 + indexer 128",
            "cache": "e4m3fn codes + fp32 tile scales; 656 B Main-KV row, 8448 B Indexer-K page",
            "device": dev_name,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "store_kernel<2, true, false, true, 4>",
            "achieved": round(store_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(store_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_unit": traffic_how,
            "rocprof": traced_durations(),
            "alg_bytes_per_launch": store_bytes,
            "avg_launch_us": round(store_us, 3),
            "how": "HIP events around replays of a graph of the 61 store launches alone",
        },
        "fence_us_per_layer": fence,
        "store_us_per_layer": round(store_us, 3),
        "verified": check,
    }
    if floor_graph:
        result["roofline"]["floor"] = floor_graph
    if extras:
        result["store_only"] = extras
    if decode:
        result["decode_store_fence"] = decode
    if gather:
        result["gather"] = gather
    if fanout:
        result["fanout_ab"] = fanout

    kvpub.kvpub_graph_destroy(graph)

    if not args.no_cpu_baseline:
        def gpu_layer(l):
            """Replica 0's and replica R-1's bytes of layer l (Main-KV, Indexer-K) on the host."""
            ms, is_ = layout.main_layer_stride, layout.idx_layer_stride
            return [(b[l * ms:(l + 1) * ms].cpu().numpy(), c[l * is_:(l + 1) * is_].cpu().numpy())
                    for b, c in ((main_bufs[0], idx_bufs[0]), (main_bufs[-1], idx_bufs[-1]))]
        result["cpu_baseline"] = cpu_baseline(lat, rope, idx, slots_np, layout, args.cpu_runs, gpu_layer)

    for c in (ctx, ctx_rel, ctx_two):
        kvpub.check(kvpub.kvpub_destroy(c))
    print(json.dumps(result), flush=True)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def aux_leg(name, fn):
    """Run one auxiliary measurement (not the timed steps, their verification or the
    oracle comparison, which stay fatal).  An exception there is recorded in the
    line as {"error": ...} instead of losing the line."""
    try:
        return fn()
    except Exception as e:  # noqa: BLE001 -- reported, not hidden
        log(f"{name} failed: {type(e).__name__}: {e}")
        return {"error": f"{type(e).__name__}: {e}"}


def written_offsets(torch, layout, layer, slots_np):
    """Device byte offsets of the rows a store of `slots_np` writes in `layer`:
    (Main-KV [n, 656], Indexer-K codes [n, 128], Indexer-K scale [n, 4], valid mask)."""
    valid = (slots_np >= 0) & (slots_np < layout.capacity)
    s = torch.from_numpy(slots_np[valid]).to("cuda")
    p, o = s // 64, s % 64
    ar = lambda n: torch.arange(n, device="cuda", dtype=torch.int64)[None, :]
    mb = layer * layout.main_layer_stride + p * layout.main_page_stride + o * 656
    ib = layer * layout.idx_layer_stride + p * layout.idx_page_stride
    return mb[:, None] + ar(656), (ib + o * 128)[:, None] + ar(128), (ib + 8192 + o * 4)[:, None] + ar(4), valid


def verify_graph_output(torch, layout, main_bufs, idx_bufs, slots_np, layer):
    """After the graph workload's timing legs (which all write the bytes the timed
    steps wrote): every replica equals replica 0 (whole buffers); in
    `layer`, every byte outside the written rows still holds the fill pattern; the
    end canaries are intact.  (The written bytes are compared with the CPU oracle in
    the cpu_baseline leg, which runs the oracle on the same inputs.)"""
    from replicated_fp8_sparse_amd.workloads import FILL, GUARD, CANARY_BYTES
    torch.cuda.synchronize()
    for r in range(1, len(main_bufs)):
        assert torch.equal(main_bufs[r], main_bufs[0]), f"Main-KV replica {r} differs from replica 0"
        assert torch.equal(idx_bufs[r], idx_bufs[0]), f"Indexer-K replica {r} differs from replica 0"
    mo, co, so, valid = written_offsets(torch, layout, layer, slots_np)
    for buf, offs, lstride in ((main_bufs[0], (mo,), layout.main_layer_stride),
                               (idx_bufs[0], (co, so), layout.idx_layer_stride)):
        keep = torch.ones(lstride, dtype=torch.bool, device="cuda")
        for off in offs:
            keep[(off - layer * lstride).reshape(-1)] = False
        seg = buf[layer * lstride:(layer + 1) * lstride]
        assert bool((seg[keep] == FILL).all()), f"layer {layer}: a byte outside the written rows changed"
    for buf in main_bufs + idx_bufs:
        assert bool((buf[-CANARY_BYTES:] == GUARD).all()), "end-of-buffer canary changed"
    return {"replicas_identical": True, "untouched_bytes_layer": layer, "rows_written_per_layer": int(valid.sum()),
            "how": "after the graph workload's timing legs: torch.equal of every replica with replica 0, every byte outside one "
                   "layer's written rows against the fill pattern, the end canaries; the CPU oracle's bytes for "
                   "the last layer are compared in cpu_baseline (oracle_layer_check)"}


def floor_us(torch, stream, fl, inp, in_bytes, outs, out_bytes, n, policy, reps=8):
    """Average microseconds of floor launches over n rotated input / output regions
    (a torch graph of the n launches, replayed)."""
    sh = stream.cuda_stream
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                rc = fl.kvpub_floor_stream(inp.data_ptr() + i * in_bytes, in_bytes,
                                           [o.data_ptr() + i * out_bytes for o in outs], out_bytes, policy, sh)
                assert rc == 0, rc
        g.replay()
        with Timer(torch, stream) as t:
            for _ in range(reps):
                g.replay()
    del g
    return t.ms * 1e3 / (reps * n)


def floor_line(torch, stream, valid, R, n, store_us):
    """The plain-stream floor for the bytes of a store launch: read valid x 1408 B,
    write valid x 788 B to each of R outputs, n launches over distinct regions."""
    from replicated_fp8_sparse_amd import floor as fl
    in_bytes = valid * READ_BYTES_PER_TOKEN
    out_bytes = valid * WRITE_BYTES_PER_TOKEN_PER_REPLICA
    in_bytes, out_bytes = in_bytes - in_bytes % 16, out_bytes - out_bytes % 16
    inp = torch.empty(n * in_bytes, dtype=torch.uint8, device="cuda")
    inp.fill_(7)
    outs = [torch.empty(n * out_bytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
    res = {name: round(floor_us(torch, stream, fl, inp, in_bytes, outs, out_bytes, n, pol), 3)
           for name, pol in fl.POLICIES.items()}
    best = min(res.values())
    del inp, outs
    torch.cuda.empty_cache()
    return {"floor_us": best, "by_policy_us": res, "store_frac_of_floor": round(best / store_us, 4),
            "how": f"a trivial kernel reading {in_bytes} B and writing {out_bytes} B to each of {R} buffers as "
                   f"whole 16-B pieces, {n} launches over distinct regions in a replayed graph; the fastest store "
                   "policy"}


def empty_node_us(torch, stream, n, blocks, threads, reps=8):
    """Average microseconds per node of a replayed graph of n empty-kernel launches."""
    from replicated_fp8_sparse_amd import floor as fl
    sh = stream.cuda_stream
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for _ in range(n):
                rc = fl.kvpub_floor_empty(blocks, threads, sh)
                assert rc == 0, rc
        g.replay()
        with Timer(torch, stream) as t:
            for _ in range(reps):
                g.replay()
    del g
    return t.ms * 1e3 / (reps * n)


def floor_graph_layer(torch, stream, L, T, valid, R, store_us):
    """The floor for the graph layer's bytes, and the fixed cost of a launch of the
    store's shape (an empty kernel with its grid, per graph node)."""
    log("floor for the graph layer")
    out = floor_line(torch, stream, valid, R, L, store_us)
    empty = empty_node_us(torch, stream, L, (T + 15) // 16, 256)
    b = alg_bytes(valid, R)
    out["empty_node_us"] = round(empty, 3)
    out["store_less_empty_node_gbps"] = round(b / ((store_us - empty) * 1e-6) / 1e9, 1)
    out["frac_cap_at_this_size"] = round(b / ((empty + b / (HBM_PEAK_GBPS * 1e9) * 1e6) * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
    out["empty_how"] = (f"a replayed graph of {L} launches of an empty kernel with the store's grid "
                        f"({(T + 15) // 16} blocks of 256 threads): the fixed cost of each graph node; "
                        "store_less_empty_node_gbps = algorithmic bytes / (store time - that cost); "
                        "frac_cap_at_this_size = the fraction of peak a launch of these bytes would reach if its "
                        "work took exactly bytes / peak on top of the fixed cost")
    return out


def store_only_extras(torch, kvpub, W, stream, vmm=True):
    """Store-kernel bandwidth on the prefill (T=8192, R=4) and heavy-tail (T=32768, R=4)
    workloads.  Warm: a replayed graph of launches over rotated input copies and slot
    mappings that write disjoint page sets (16 prefill mappings in windows of 1024 pages,
    8 heavy mappings over successive 512-page blocks of one page permutation), so the
    bytes a replay touches (0.6 resp. 1.2 GB) exceed the 256 MB memory-side cache and the
    figure is one of HBM.  Cold: single launches, each after a 1 GiB read that leaves no
    dirty line behind.  The heavy shape runs again on VMM-backed replicas."""
    from replicated_fp8_sparse_amd import floor as _fl  # noqa: F401  (fails loudly if unbuilt)
    out = {}
    shapes = [("prefill_T8192_R4", W.prefill, False), ("heavy_T32768_R4", W.heavy, False)]
    if vmm:
        shapes.append(("heavy_T32768_R4_vmm", W.heavy, True))
    for name, fn, vmm in shapes:
        out[name] = aux_leg(f"store-only {name}", lambda: store_only_shape(torch, kvpub, W, stream, name, fn, vmm))
    return out


def store_only_shape(torch, kvpub, W, stream, name, fn, vmm):
    """One shape of store_only_extras: warm, same-slots and cold launch times, and
    (device allocations) the plain-stream floor for the same bytes."""
    sh = stream.cuda_stream
    layout, x = fn()
    rot = W.prefill_rotation_slots(16) if fn is W.prefill else W.heavy_rotation_slots(8)
    copies = len(rot)
    log(f"store-only {name}")
    R = layout.replicas
    cfg = kvpub.kvpub_config_init(R, 1, layout.num_pages)
    storage = None
    if vmm:
        # the store never reads the cache, so the VMM pages need no fill for timing
        st, storage, mbp, ibp = kvpub.kvpub_vmm_create(cfg, layout.num_pages)
        kvpub.check(st, "kvpub_vmm_create")
        mb = ib = None
    else:
        mb = [torch.empty(layout.main_bytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
        ib = [torch.empty(layout.idx_bytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
        for b in mb:
            layout.fill_device(b, "main")
        for b in ib:
            layout.fill_device(b, "idx")
        mbp, ibp = [b.data_ptr() for b in mb], [b.data_ptr() for b in ib]
    st, ctx = kvpub.kvpub_create(cfg, mbp, ibp)
    kvpub.check(st)
    T = x.slots.size
    lat = torch.from_numpy(x.latent.view(np.int16)).to("cuda").repeat(copies, 1, 1)
    rope = torch.from_numpy(x.rope.view(np.int16)).to("cuda").repeat(copies, 1, 1)
    idx = torch.from_numpy(x.indexer.view(np.int16)).to("cuda").repeat(copies, 1, 1)
    slots = torch.from_numpy(np.stack(rot)).to("cuda")
    same = torch.from_numpy(x.slots).to("cuda")
    valid = int(((x.slots >= 0) & (x.slots < layout.capacity)).sum())
    assert all(int(((s >= 0) & (s < layout.capacity)).sum()) == valid for s in rot)

    def launch(c, slot_ptr=None):
        return kvpub.kvpub_store(ctx, 0, T, lat[c].data_ptr(), 512, rope[c].data_ptr(), 64,
                                 idx[c].data_ptr(), 128, slots[c].data_ptr() if slot_ptr is None else slot_ptr, sh)

    def warm(body):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for c in range(copies):
                    kvpub.check(body(c))
            g.replay()
            reps = 8
            with Timer(torch, stream) as tm:
                for _ in range(reps):
                    g.replay()
        del g
        return tm.ms * 1e3 / (reps * copies)

    us = warm(launch)
    us_same = warm(lambda c: launch(c, same.data_ptr()))
    cold = cold_launch_us(torch, stream, launch, copies)
    b = alg_bytes(valid, R)
    gb = lambda t: b / (t * 1e-6) / 1e9
    res = {"avg_launch_us": round(us, 3), "alg_bytes": b,
                 "gbps": round(gb(us), 1), "frac": round(gb(us) / HBM_PEAK_GBPS, 4),
                 "tokens_per_s": round(valid / (us * 1e-6), 1),
                 "cold_launch_us": round(cold, 3), "cold_frac": round(gb(cold) / HBM_PEAK_GBPS, 4),
                 "same_slots_launch_us": round(us_same, 3),
                 "storage": "vmm" if vmm else "device allocations",
                 "how": f"warm: a replayed graph of {copies} launches over rotated input copies and slot "
                        "mappings writing disjoint page sets (bytes touched per replay exceed the 256 MB "
                        "memory-side cache); cold: median of single launches, each after reading a 1 GiB "
                        "buffer (no dirty lines left); same_slots: the warm graph with one slot mapping "
                        "(rewrites the same pages every launch)"}
    if not vmm:
        res["floor"] = floor_line(torch, stream, valid, R, copies, us)
    kvpub.check(kvpub.kvpub_destroy(ctx))
    if storage is not None:
        kvpub.check(kvpub.kvpub_vmm_destroy(storage), "kvpub_vmm_destroy")
    del mb, ib, lat, rope, idx
    torch.cuda.empty_cache()
    return res


def fanout_ab(torch, kvpub, W, stream):
    """The pages' A/B of the fan-out, on one GPU: one launch that reads each token's
    bf16 rows once and writes all R replicas, against R launches of single-replica
    contexts over the same buffers, each re-reading the rows (an insert per replica).
    Both write identical bytes; each is timed as replays of a captured graph over
    rotated input copies."""
    out = {}
    sh = stream.cuda_stream
    for name, fn in (("prefill_T8192_R4", W.prefill), ("heavy_T32768_R4", W.heavy)):
        layout, x = fn()
        print(f"[bench] fan-out A/B {name}", file=sys.stderr, flush=True)
        R, copies = layout.replicas, 4
        mb = [torch.empty(layout.main_bytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
        ib = [torch.empty(layout.idx_bytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
        cfg = kvpub.kvpub_config_init(R, 1, layout.num_pages)
        st, fused = kvpub.kvpub_create(cfg, [b.data_ptr() for b in mb], [b.data_ptr() for b in ib])
        kvpub.check(st)
        single = []
        for r in range(R):
            c1 = kvpub.kvpub_config_init(1, 1, layout.num_pages)
            st, c = kvpub.kvpub_create(c1, [mb[r].data_ptr()], [ib[r].data_ptr()])
            kvpub.check(st)
            single.append(c)
        T = x.slots.size
        lat = torch.from_numpy(x.latent.view(np.int16)).to("cuda").repeat(copies, 1, 1)
        rope = torch.from_numpy(x.rope.view(np.int16)).to("cuda").repeat(copies, 1, 1)
        idx = torch.from_numpy(x.indexer.view(np.int16)).to("cuda").repeat(copies, 1, 1)
        slots = torch.from_numpy(x.slots).to("cuda")
        valid = int(((x.slots >= 0) & (x.slots < layout.capacity)).sum())

        def store(ctx, c):
            kvpub.check(kvpub.kvpub_store(ctx, 0, T, lat[c].data_ptr(), 512, rope[c].data_ptr(), 64,
                                          idx[c].data_ptr(), 128, slots.data_ptr(), sh))

        def timed(body):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                with torch.cuda.graph(g, stream=stream):
                    for c in range(copies):
                        body(c)
                g.replay()
                reps = 8
                with Timer(torch, stream) as tm:
                    for _ in range(reps):
                        g.replay()
            return tm.ms * 1e3 / (reps * copies)

        fused_us = timed(lambda c: store(fused, c))
        split_us = timed(lambda c: [store(single[r], c) for r in range(R)])
        out[name] = {"fused_us": round(fused_us, 3), "per_replica_launches_us": round(split_us, 3),
                     "speedup": round(split_us / fused_us, 3), "fused_bytes": alg_bytes(valid, R),
                     "per_replica_bytes": R * alg_bytes(valid, 1)}
        for c in single:
            kvpub.check(kvpub.kvpub_destroy(c))
        kvpub.check(kvpub.kvpub_destroy(fused))
        del mb, ib, lat, rope, idx
        torch.cuda.empty_cache()
    out["how"] = ("one store launch writing all R replicas vs R single-replica store launches each re-reading "
                  "the bf16 rows, both captured in a graph over 4 rotated input copies and replayed; "
                  "microseconds per batch")
    return out


GATHER_READ_BYTES_PER_TOKEN = 656 + 128 + 4          # one replica's Main-KV row + Indexer-K
GATHER_WRITE_BYTES_PER_TOKEN = (512 + 64 + 128) * 2  # bf16 rows out


def gather_line(torch, kvpub, ctx, slots, T, valid, stream):
    """The reader side on the graph workload's layer: kvpub_gather of the T=4096
    slots from replica 0 back to bf16 rows, over the 61 layers.  Timed as replays of
    a graph of the 61 gathers (as the store is), eagerly back to back (host launch
    cost included), and cold (one launch after a 1 GiB read)."""
    sh = stream.cuda_stream
    L = 61
    lat = torch.empty((T, 512), dtype=torch.bfloat16, device="cuda")
    rope = torch.empty((T, 64), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((T, 128), dtype=torch.bfloat16, device="cuda")

    def launch(l):
        return kvpub.kvpub_gather(ctx, 0, l % L, T, slots.data_ptr(), lat.data_ptr(), 512, rope.data_ptr(), 64,
                                  idx.data_ptr(), 128, sh)

    for l in range(L):
        kvpub.check(launch(l))
    n = 4 * L
    with Timer(torch, stream) as tm:
        for i in range(n):
            launch(i)
    eager_us = tm.ms * 1e3 / n
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for l in range(L):
                kvpub.check(launch(l))
        for _ in range(2):
            g.replay()
        reps = 8
        with Timer(torch, stream) as tg:
            for _ in range(reps):
                g.replay()
    us = tg.ms * 1e3 / (reps * L)
    cold = cold_launch_us(torch, stream, launch, L)
    b = valid * (GATHER_READ_BYTES_PER_TOKEN + GATHER_WRITE_BYTES_PER_TOKEN)
    return {"kernel": "gather_kernel", "tokens": T, "avg_launch_us": round(us, 3), "alg_bytes": b,
            "gbps": round(b / (us * 1e-6) / 1e9, 1), "frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "tokens_per_s": round(valid / (us * 1e-6), 1), "eager_launch_us": round(eager_us, 3),
            "cold_launch_us": round(cold, 3),
            "how": "replays of a graph of 61 gathers over the 61 layer caches of replica 0 (avg), the same "
                   "launches eagerly back to back (eager, host launch cost included), and single launches "
                   "after a 1 GiB read (cold); bytes = 788 B read + 1408 B written per token",
            "decode": gather_decode(torch, kvpub, ctx, stream),
            "topk": gather_topk(torch, kvpub, ctx, stream)}


def graph_launch_us(torch, stream, launch, n, reps):
    """Average microseconds per launch of a replayed torch graph of launch(0..n-1)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                launch(i)
        for _ in range(2):
            g.replay()
        with Timer(torch, stream) as t:
            for _ in range(reps):
                g.replay()
    del g
    return t.ms * 1e3 / (reps * n)


def gather_outputs(torch, T):
    return (torch.empty((T, 512), dtype=torch.bfloat16, device="cuda"),
            torch.empty((T, 64), dtype=torch.bfloat16, device="cuda"),
            torch.empty((T, 128), dtype=torch.bfloat16, device="cuda"))


def gather_decode(torch, kvpub, ctx, stream):
    """The gather at a decode step's size: the decode workload's 64 slots (3 padded)
    from each of the 61 layer caches, beside an empty kernel of the same grid."""
    from replicated_fp8_sparse_amd import workloads as W
    sh = stream.cuda_stream
    sl = W.decode(layers=1)[1][0].slots
    T, L = sl.size, 61
    slots = torch.from_numpy(sl).to("cuda")
    lat, rope, idx = gather_outputs(torch, T)
    us = graph_launch_us(torch, stream, lambda l: kvpub.check(kvpub.kvpub_gather(
        ctx, 0, l, T, slots.data_ptr(), lat.data_ptr(), 512, rope.data_ptr(), 64, idx.data_ptr(), 128, sh)), L, 8)
    empty = empty_node_us(torch, stream, L, (T + 15) // 16, 256)
    return {"tokens": T, "avg_launch_us": round(us, 3), "empty_node_us": round(empty, 3),
            "how": "replays of a graph of 61 gathers of the decode workload's 64 slots (one per layer cache); "
                   "empty_node_us: the same graph of an empty kernel with the gather's grid (4 blocks of 256 threads)"}


def gather_topk(torch, kvpub, ctx, stream, layers=8):
    """The decode-time read pattern: 16 requests each selecting 2048 distinct slots of
    their own 512-page context (32,768 scattered rows), one launch per layer cache."""
    from replicated_fp8_sparse_amd import workloads as W
    sh = stream.cuda_stream
    sl = W.topk_slots()
    T = sl.size
    slots = torch.from_numpy(sl).to("cuda")
    lat, rope, idx = gather_outputs(torch, T)
    us = graph_launch_us(torch, stream, lambda l: kvpub.check(kvpub.kvpub_gather(
        ctx, 0, l, T, slots.data_ptr(), lat.data_ptr(), 512, rope.data_ptr(), 64, idx.data_ptr(), 128, sh)),
        layers, 4)
    b = T * (GATHER_READ_BYTES_PER_TOKEN + GATHER_WRITE_BYTES_PER_TOKEN)
    del lat, rope, idx
    torch.cuda.empty_cache()
    return {"tokens": T, "requests": 16, "k": 2048, "context_pages": 512, "avg_launch_us": round(us, 2),
            "alg_bytes": b, "gbps": round(b / (us * 1e-6) / 1e9, 1),
            "frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "how": f"replays of a graph of {layers} gathers, one per layer cache of replica 0, each reading the "
                   "32,768 rows of the top-k slot lists (each layer's 8192 pages covered by the 16 contexts)"}


def cold_launch_us(torch, stream, launch, copies, n=12):
    """Median duration of single launches, each after reading a 1 GiB buffer (which
    evicts the L2s and the memory-side cache and leaves no dirty line behind)."""
    scratch = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    times = []
    with torch.cuda.stream(stream):
        for i in range(n):
            sink = scratch.sum(dtype=torch.int64)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            launch(i % copies)
            b.record(stream)
            b.synchronize()
            times.append(a.elapsed_time(b) * 1e3)
    assert int(sink) == 1 << 28
    del scratch
    torch.cuda.empty_cache()
    return float(np.median(times))


def decode_eager(torch, kvpub, W, stream):
    """The decode shape (61 layers x T=64, R=2, 4096 pages): eager store + fence per
    layer, for context (a latency-bound case)."""
    layout, xs = W.decode()
    R = layout.replicas
    sh = stream.cuda_stream
    mb = [torch.empty(layout.main_bytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
    ib = [torch.empty(layout.idx_bytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
    for b in mb:
        layout.fill_device(b, "main")
    for b in ib:
        layout.fill_device(b, "idx")
    cfg = kvpub.kvpub_config_init(R, layout.layers, layout.num_pages)
    st, ctx = kvpub.kvpub_create(cfg, [b.data_ptr() for b in mb], [b.data_ptr() for b in ib])
    kvpub.check(st)
    dev = []
    for x in xs:
        dev.append((torch.from_numpy(x.latent.view(np.int16)).to("cuda"),
                    torch.from_numpy(x.rope.view(np.int16)).to("cuda"),
                    torch.from_numpy(x.indexer.view(np.int16)).to("cuda"),
                    torch.from_numpy(x.slots).to("cuda")))
    T = xs[0].slots.size

    def one_pass():
        for l, (a, r, i, s_) in enumerate(dev):
            kvpub.kvpub_store(ctx, l, T, a.data_ptr(), 512, r.data_ptr(), 64, i.data_ptr(), 128,
                              s_.data_ptr(), sh)
            kvpub.kvpub_fence(ctx, 0, sh)

    one_pass()
    reps = 5
    with Timer(torch, stream) as tm:
        for _ in range(reps):
            one_pass()
    eager = tm.ms * 1e3 / (reps * len(xs))
    ios = [kvpub.layer_io(a.data_ptr(), r.data_ptr(), i.data_ptr(), s_.data_ptr(), T, l)
           for l, (a, r, i, s_) in enumerate(dev)]
    st, graph = kvpub.kvpub_graph_create(ctx, ios, 0)
    kvpub.check(st, "kvpub_graph_create")
    for _ in range(3):
        kvpub.check(kvpub.kvpub_graph_replay(graph, sh))
    reps = 50
    with Timer(torch, stream) as tg:
        for _ in range(reps):
            kvpub.kvpub_graph_replay(graph, sh)
    replayed = tg.ms * 1e3 / (reps * len(xs))
    kvpub.check(kvpub.kvpub_graph_destroy(graph))
    kvpub.check(kvpub.kvpub_destroy(ctx))
    del mb, ib, dev
    torch.cuda.empty_cache()
    return {"us_per_layer": round(eager, 3), "graph_us_per_layer": round(replayed, 3),
            "how": "61 layers x T=64, R=2, 4096 pages, store + fence per layer: eager launches "
                   "(host launch cost included), and the same sequence captured once and replayed"}


def cpu_baseline(lat, rope, idx, slots_np, layout, runs, gpu_layer=None):
    """The CPU oracle (plain C, as it stands) on a bounded sample of the same workload:
    graph-workload layers one after another into host replicas of one layer-cache.
    Two legs, each run `runs` times (the median is reported, with the spread):
    single-threaded over 8 layers per run, and with one thread per host core (at most
    16) over contiguous token ranges of each of the 61 layers per run (race-free: a
    layer's valid slots are distinct; the C calls release the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    orc = oracle.get()
    L = lat.shape[0]
    m0, i0 = oracle_host_layer(layout)
    mains = [m0.copy() for _ in range(layout.replicas)]
    idxs = [i0.copy() for _ in range(layout.replicas)]
    valid_per_layer = int(((slots_np >= 0) & (slots_np < layout.capacity)).sum())
    T = slots_np.size
    u16 = lambda t: t.cpu().view(torch_int16()).numpy().view(np.uint16)
    host = [(u16(lat[l]), u16(rope[l]), u16(idx[l])) for l in range(L)]

    def store_range(x_l, x_r, x_i, a, b):
        orc.store(mains, idxs, num_pages=layout.num_pages,
                  main_page_stride=layout.main_page_stride, main_layer_stride=layout.main_layer_stride,
                  idx_page_stride=layout.idx_page_stride, idx_layer_stride=layout.idx_layer_stride,
                  layer=0, latent=x_l[a:b], rope=x_r[a:b], indexer=x_i[a:b], slot_mapping=slots_np[a:b])

    def run(threads, layers, ex):
        bounds = np.linspace(0, T, threads + 1).astype(int)
        t0 = time.perf_counter()
        for l in range(layers):
            x_l, x_r, x_i = host[l]
            if threads == 1:
                store_range(x_l, x_r, x_i, 0, T)
            else:
                list(ex.map(lambda ab: store_range(x_l, x_r, x_i, ab[0], ab[1]), zip(bounds[:-1], bounds[1:])))
        return valid_per_layer * layers / (time.perf_counter() - t0)

    def leg(threads, layers):
        with ThreadPoolExecutor(max_workers=threads) as ex:
            rates = [run(threads, layers, ex) for _ in range(runs)]
        return float(np.median(rates)), min(rates), max(rates)

    one_layers, many_layers = 8, L
    one = leg(1, one_layers)
    cores = max(1, min(os.cpu_count() or 1, 16))
    many = leg(cores, many_layers)
    # Every run ends with the last layer, and every layer uses the same slots, so the
    # host layer-cache now holds the oracle's encoding of the last layer's inputs:
    # compare it, written rows and untouched bytes alike, with that layer on the GPU.
    check = None
    if gpu_layer is not None:
        for r, (gm, gi) in enumerate(gpu_layer(L - 1)):
            assert np.array_equal(gm, mains[0][:gm.size]), f"GPU Main-KV layer {L - 1} differs from the oracle"
            assert np.array_equal(gi, idxs[0][:gi.size]), f"GPU Indexer-K layer {L - 1} differs from the oracle"
        check = {"layer": L - 1, "bytes_compared": int(2 * (gm.size + gi.size)), "equal": True,
                 "how": "the oracle's host layer-cache after the timed runs (the last layer's rows) against "
                        "that layer of the first and last GPU replicas, every byte"}
    return {"value": round(many[0], 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"graph workload layers (T=4096, R=2, 8192 pages) through the C oracle: {runs} runs of "
                      f"{many_layers} layers on {cores} threads (median reported) and {runs} runs of "
                      f"{one_layers} layers single-threaded",
            "runs": runs, "min": round(many[1], 1), "max": round(many[2], 1),
            "single_thread_value": round(one[0], 1),
            "single_thread_min": round(one[1], 1), "single_thread_max": round(one[2], 1),
            "gbps": round(alg_bytes(many[0], layout.replicas) / 1e9, 3),
            "single_thread_gbps": round(alg_bytes(one[0], layout.replicas) / 1e9, 3),
            "host_cpus": os.cpu_count(),
            "cpu_model": host_cpu_model(),
            "oracle_layer_check": check}


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def torch_int16():
    import torch
    return torch.int16


def oracle_host_layer(layout):
    from replicated_fp8_sparse_amd.workloads import CacheLayout
    one = CacheLayout(replicas=layout.replicas, layers=1, num_pages=layout.num_pages)
    return one.fill_host()


if __name__ == "__main__":
    main()
