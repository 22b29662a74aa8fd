"""Benchmark: the Gated DeltaNet speculative-verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one spec-decode round of one GDN layer on the 64-slot workload (64 slots, 16 key /
32 value heads, d = 128, K+1 = 16 bf16 tokens per slot, fp32 state and capture): gdn_verify
(conv, gate, delta rule, readout, norm/gate, per-position capture) followed by gdn_rollback_batch
with a random per-slot trim.  The same rounds as single gdn_verify_resume launches (each slot
starts from its accepted capture position instead of having it copied back; bit-identical
results) are timed beside it as step_resume.  Inputs are seeded synthetic data already resident in
HBM; input sets rotate, each with its own state and capture, so the 128 MiB state never sits in
the 256 MB Infinity Cache between its uses.

Prints one JSON line: tokens/s (value), the verify kernel's achieved HBM bandwidth against the
8 TB/s peak (roofline, timed with HIP events on the launch stream over the timed region), and
the CPU oracle's throughput on a bounded sample (cpu_baseline).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN verify tokens/s (64 slots, K+1=16) + achieved HBM GB/s vs peak"
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_FLOPS = 2.5e15  # dense bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_multi_slot_verify.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per verify launch from the committed rocprofv3 counter summary (FETCH_SIZE and
    WRITE_SIZE, each scaled by what it reads for the rollback copy kernel of known size), or None
    when the summary is missing or was taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("kernel_source_sha256_16") != source_digest(t["kernel_sources"]):
            return None
    except (OSError, ValueError, KeyError):
        return None
    return t.get("bytes_per_launch")


def counter_record(name: str):
    """The committed rocprofv3 counter summary profiles/counters_<name>.json, condensed, or None
    when it is missing or was taken on different kernel sources."""
    try:
        with open(os.path.join(ROOT, "profiles", f"counters_{name}.json")) as f:
            t = json.load(f)
        if t.get("kernel_source_sha256_16") != source_digest(t["kernel_sources"]):
            return None
    except (OSError, ValueError, KeyError):
        return None
    rec = {"file": f"profiles/counters_{name}.json", "hbm_bytes_per_call": t["hbm_bytes_per_call"]}
    if "traffic_over_algorithmic" in t:
        rec["traffic_over_algorithmic"] = t["traffic_over_algorithmic"]
    kern = {}
    busy = active = 0.0
    for k, e in t["kernels"].items():
        kern[k] = {"hbm_read_bytes": e["hbm_read_bytes"], "hbm_write_bytes": e["hbm_write_bytes"]}
        if "mfma_util" in e:
            kern[k]["mfma_util"] = e["mfma_util"]
            kern[k]["mfma_flops"] = e["mfma_bf16_flops"] + e["mfma_f32_flops"]
            busy += e["mfma_busy_cycles"]
            active += e["grbm_gui_active_per_xcd"] * 1024
    rec["kernels"] = kern
    if active:
        rec["mfma_util"] = busy / active  # MFMA busy cycles over active cycles x SIMDs, all kernels
    return rec


def cpu_baseline(shape, inp, target_s: float = 10.0) -> dict:
    """The fp64 oracle (test infrastructure, untuned) on the same workload: every (slot, value
    head) unit with capture, repeated until about target_s seconds of host time; the median
    repetition is reported."""
    from oracle import ref

    threads = ref.max_threads()
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    times = []
    t_all = time.perf_counter()
    while time.perf_counter() - t_all < target_s or len(times) < 3:
        t0 = time.perf_counter()
        ref.verify_units(shape, inp)
        times.append(time.perf_counter() - t0)
    times.sort()
    med = times[len(times) // 2]
    return {"value": shape.n_batch * shape.n_tok / med, "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": model, "host_cpus": os.cpu_count(),
            "sample": f"the whole call ({shape.n_batch} slots x {shape.n_vh} value heads x "
                      f"{shape.n_tok} tokens, fp64, with capture), {len(times)} repetitions in "
                      f"{sum(times):.1f} s, median {med * 1e3:.0f} ms"}


# Untimed launches before a component's timed ones, in seconds (see time_launches).
WARM_S = 0.25


def time_launches(fn, n: int, warmup: int = 20, warm_s=None) -> float:
    """Average duration in microseconds of fn() over n launches, HIP events on the current stream,
    after `warmup` untimed launches and then more untimed launches until `warm_s` seconds (default
    WARM_S) have passed or 1000 of them have run.  Each component starts after host-side input generation has left the GPU
    idle, and its first launches run slower for a few tens of milliseconds: the 1024-row
    in-projection took 155 us per launch over its first 70 launches and 133 us from about 30 ms of
    launches on, whatever its data.  The timed launches themselves are unchanged."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    span = WARM_S if warm_s is None else warm_s
    t0, extra = time.perf_counter(), 0
    while time.perf_counter() - t0 < span and extra < 1000:
        for _ in range(4):
            fn()
        extra += 4
        torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def components(args) -> dict:
    """Secondary timings of the other kernels on their own workloads (not part of the step)."""
    import numpy as np
    import torch

    from gated_deltanet_linear_verify_amd import bytemodel, device, gdn
    from gated_deltanet_linear_verify_amd import workloads as W

    out = {}
    # tree verify: 8 slots x 64-node trees
    s = W.TREE_VERIFY
    d = device.upload(s, W.make_tree_inputs(s, 0), mode=gdn.GDN_TREE, fill_capture=0.0)
    us = time_launches(lambda: device.verify_tree(d), 50)
    out["tree_verify"] = {"workload": "8 slots x 64-node trees, 16/32 heads, d=128, bf16",
                          "us": us, "tokens_per_s": s.n_batch * s.n_tok / (us * 1e-6),
                          "hbm_gbps": bytemodel.tree_bytes(s) / (us * 1e-6) / 1e9,
                          "algorithmic_bytes": bytemodel.tree_bytes(s),
                          "counters": counter_record("tree_8x64")}
    del d
    # single-slot verify: 1 slot x 16 tokens
    s = W.SINGLE_SLOT_VERIFY
    d = device.upload(s, W.make_inputs(s, 0), fill_capture=0.0)
    us = time_launches(lambda: device.verify(d), 200)
    out["single_slot_verify"] = {"workload": "1 slot x 16 tokens, 16/32 heads, d=128, bf16", "us": us,
                                 "tokens_per_s": s.n_tok / (us * 1e-6),
                                 "hbm_gbps": bytemodel.verify_bytes(s) / (us * 1e-6) / 1e9}
    # the same slot in the resume loop with the commit deferred: each round starts from the
    # previous round's accepted capture position
    device.verify(d)
    acc = torch.from_numpy(np.array([s.n_tok - 1 - int(W.make_inputs(s, 0)["trims"][0])], dtype=np.int32)).cuda()
    dims_defer = gdn.make_dims(s, flags=gdn.GDN_F_DEFER_COMMIT)
    us = time_launches(lambda: device.verify_resume(d, acc, dims=dims_defer), 200)
    out["single_slot_resume_deferred"] = {
        "workload": "1 slot x 16 tokens, 16/32 heads, d=128, bf16, gdn_verify_resume with GDN_F_DEFER_COMMIT",
        "us": us, "tokens_per_s": s.n_tok / (us * 1e-6),
        "hbm_gbps": bytemodel.verify_bytes(s, commit=False) / (us * 1e-6) / 1e9}
    del d
    # snapshot-and-replay rollback on the 64-slot workload (no per-position capture): a round is
    # snapshot + verify, plus restore + replay of the accepted tokens when some are rejected
    s = W.MULTI_SLOT_VERIFY
    d = device.upload(s, W.make_inputs(s, 0), capture=False)
    snap = {"state": torch.empty_like(d["state"]), "conv_state": torch.empty_like(d["conv_state"])}
    us_acc = time_launches(lambda: device.snapshot_replay_round(d, snap, s.n_tok), 50)
    us_rej = time_launches(lambda: device.snapshot_replay_round(d, snap, 1), 50)
    out["snapshot_replay"] = {"workload": "64 slots x 16 tokens, 16/32 heads, d=128, bf16, no capture",
                              "us_all_accepted": us_acc, "us_reject_after_first": us_rej,
                              "tokens_per_s_all_accepted": s.n_batch * s.n_tok / (us_acc * 1e-6),
                              "tokens_per_s_reject_after_first": s.n_batch * s.n_tok / (us_rej * 1e-6)}
    del d, snap
    # a spec-decode step over 48 GDN layers (the pages' model has 48 delta-net layers), 1 slot, 16
    # drafted tokens and plain 1-token decode: eager launches from the binding vs one replay of the
    # recorded HIP graph
    n_layers = 48
    for name, n_tok in (("graph_step_48_layers", 16), ("graph_step_48_layers_1_token", 1)):
        s = W.shape_with(W.SINGLE_SLOT_VERIFY, n_tok=n_tok)
        layers = [device.upload(s, W.make_inputs(s, 1000 + l), fill_capture=0.0) for l in range(n_layers)]
        slots = layers[0]["slot_ids"].clone()
        acc = torch.full((s.n_batch,), s.n_tok // 2, dtype=torch.int32, device="cuda")
        us_eager = time_launches(lambda: device.layers_step(layers, slots, acc), 20)
        g = device.layers_graph(layers, slots, acc)
        us_graph = time_launches(lambda: g.launch(), 20)
        g.close()
        step_bytes = n_layers * (bytemodel.verify_bytes(s) + bytemodel.rollback_bytes(s, s.n_batch))
        out[name] = {
            "workload": f"48 layers x (1 slot x {n_tok} token verify with capture) + one cross-layer rollback",
            "us_eager": us_eager, "us_graph": us_graph,
            "tokens_per_s_graph": s.n_tok / (us_graph * 1e-6),
            "hbm_gbps_graph": step_bytes / (us_graph * 1e-6) / 1e9}
        del layers, g
    # rollback of 48 layers x 64 slots: one cross-layer launch vs one batched launch per layer
    s = W.MULTI_SLOT_VERIFY
    dims = gdn.make_dims(s)
    C = s.conv_channels
    caps = []
    for _ in range(n_layers):
        st = torch.empty((s.n_pool, s.n_vh, s.d_v, s.d_k), dtype=torch.float32, device="cuda")
        cs = torch.empty((s.n_pool, 3, C), dtype=torch.float32, device="cuda")
        cap = torch.empty((s.n_pool, s.n_tok, s.n_vh, s.d_v, s.d_k), dtype=torch.float32, device="cuda")
        cc = torch.empty((s.n_pool, 3 + s.n_tok, C), dtype=torch.float32, device="cuda")
        caps.append(gdn.Capture(dims, cap, cc, st, cs, s.n_tok, gdn.GDN_CHAIN))
    slots = torch.randperm(s.n_pool, dtype=torch.int32).cuda()
    acc = torch.from_numpy((s.n_tok - 1 - W.make_inputs(s, 0)["trims"]).astype(np.int32)).cuda()
    us_one = time_launches(lambda: gdn.gdn_rollback_layers(caps, slots, acc, s.n_batch), 10)
    us_per_layer = time_launches(lambda: [gdn.gdn_rollback_batch(c, slots, acc, s.n_batch) for c in caps], 10)
    rb = n_layers * bytemodel.rollback_bytes(s, s.n_batch)
    n1 = 1  # the same rollback for one slot
    us_one_1 = time_launches(lambda: gdn.gdn_rollback_layers(caps, slots, acc, n1), 20)
    us_per_layer_1 = time_launches(lambda: [gdn.gdn_rollback_batch(c, slots, acc, n1) for c in caps], 20)
    out["rollback_48_layers"] = {"workload": "48 layers x 64 slots, 16/32 heads, d=128",
                                 "us_one_launch": us_one, "us_launch_per_layer": us_per_layer,
                                 "hbm_gbps_one_launch": rb / (us_one * 1e-6) / 1e9,
                                 "algorithmic_bytes": rb,
                                 "one_slot_us_one_launch": us_one_1,
                                 "one_slot_us_launch_per_layer": us_per_layer_1}
    del caps
    torch.cuda.empty_cache()
    # the whole GDN block: input projections (one gdn_linear), verify with capture, output
    # projection, at the model's width of 5120; 64 slots and 1 slot of 16 drafted tokens
    for name, nb in (("gdn_block_64_slots", 64), ("gdn_block_1_slot", 1)):
        s = W.shape_with(W.MULTI_SLOT_VERIFY, n_pool=nb, n_batch=nb)
        d = device.upload_block(s, W.make_block_inputs(s, W.HIDDEN, seed=3))
        M, C, Z, Hv = nb * s.n_tok, s.conv_channels, s.n_vh * s.d_v, s.n_vh
        n_in = C + Z + 2 * Hv
        segs = [(0, C, d["qkv"], C, 0), (C, C + Z, d["z"], Z, 0),
                (C + Z, C + Z + Hv, d["beta"], Hv, 1), (C + Z + Hv, n_in, d["alpha"], Hv, 0)]
        us_in = time_launches(lambda: gdn.gdn_linear(d["x"], d["w_in"], M, n_in, W.HIDDEN, segs), 20)
        us_ver = time_launches(lambda: device.verify(d), 20)
        us_out = time_launches(lambda: gdn.gdn_linear(d["out"], d["w_out"], M, W.HIDDEN, Z,
                                                      [(0, W.HIDDEN, d["y"], W.HIDDEN, 0)]), 20)
        us_all = time_launches(lambda: device.block_step(d), 20)
        f_in, f_out = 2.0 * M * n_in * W.HIDDEN, 2.0 * M * W.HIDDEN * Z
        out[name] = {
            "workload": f"{nb} slot(s) x 16 tokens, width 5120 -> qkv|z|beta|alpha ({n_in}) -> verify -> 5120",
            "us_block": us_all, "us_in_proj": us_in, "us_verify": us_ver, "us_out_proj": us_out,
            "tokens_per_s": M / (us_all * 1e-6),
            "in_proj_tflops": f_in / (us_in * 1e-6) / 1e12, "out_proj_tflops": f_out / (us_out * 1e-6) / 1e12,
            "in_proj_mfma_util_vs_bf16_peak": f_in / (us_in * 1e-6) / PEAK_BF16_FLOPS,
            "out_proj_mfma_util_vs_bf16_peak": f_out / (us_out * 1e-6) / PEAK_BF16_FLOPS}
        if nb == 64:
            out[name]["counters"] = counter_record("linear_block_64_slots")
        del d
    torch.cuda.empty_cache()
    # chunked prefill: one 8192-token sequence
    s = W.CHUNKED_PREFILL
    d = device.upload(s, W.make_inputs(s, 0), capture=False)
    # steady state: a process's first few dozen prefills run up to ~15% slower
    us = time_launches(lambda: device.prefill(d), 20, warmup=40)
    fl = bytemodel.prefill_flops(s)
    out["chunked_prefill"] = {"workload": "1 slot x 8192 tokens, 16/32 heads, d=128, bf16, chunk 64",
                              "timing": f"20 calls after 40 warm-up calls and {WARM_S} s (at most 1000 calls) of further untimed calls",
                              "us": us, "tokens_per_s": s.n_tok / (us * 1e-6),
                              "hbm_gbps": bytemodel.prefill_bytes(s) / (us * 1e-6) / 1e9,
                              "algorithmic_flops": fl, "tflops": fl / (us * 1e-6) / 1e12,
                              "mfma_util_vs_bf16_peak": fl / (us * 1e-6) / PEAK_BF16_FLOPS,
                              "counters": counter_record("prefill_8192")}
    del d
    torch.cuda.empty_cache()
    return out


COMPONENTS = ("prefill", "tree", "linear", "single_slot")


def component_only(name: str, steps: int, warmup: int) -> dict:
    """One secondary workload alone, for a profiler run: warmup + steps launches of its kernels,
    then the same count of the snapshot copy of 64 slots (a plain copy of known size, which
    calibrates byte counters), with the average launch time of each."""
    import torch

    from gated_deltanet_linear_verify_amd import bytemodel, device, gdn
    from gated_deltanet_linear_verify_amd import workloads as W

    global WARM_S
    WARM_S = 0.0  # exactly warmup + steps launches, so that counter passes see a known dispatch count
    n = warmup + steps
    res = {"component": name, "launches": n}
    if name == "prefill":
        s = W.CHUNKED_PREFILL
        d = device.upload(s, W.make_inputs(s, 0), capture=False)
        res["workload"] = "1 slot x 8192 tokens, 16/32 heads, d=128, bf16, chunk 64"
        res["us"] = time_launches(lambda: device.prefill(d), steps, warmup)
        res["algorithmic_flops"] = bytemodel.prefill_flops(s)
        res["algorithmic_bytes"] = bytemodel.prefill_bytes(s)
    elif name == "tree":
        s = W.TREE_VERIFY
        d = device.upload(s, W.make_tree_inputs(s, 0), mode=gdn.GDN_TREE, fill_capture=0.0)
        res["workload"] = "8 slots x 64-node trees, 16/32 heads, d=128, bf16"
        res["us"] = time_launches(lambda: device.verify_tree(d), steps, warmup)
        res["algorithmic_bytes"] = bytemodel.tree_bytes(s)
    elif name == "linear":
        s = W.MULTI_SLOT_VERIFY
        d = device.upload_block(s, W.make_block_inputs(s, W.HIDDEN, seed=3))
        M, C, Z, Hv = s.n_batch * s.n_tok, s.conv_channels, s.n_vh * s.d_v, s.n_vh
        n_in = C + Z + 2 * Hv
        segs = [(0, C, d["qkv"], C, 0), (C, C + Z, d["z"], Z, 0),
                (C + Z, C + Z + Hv, d["beta"], Hv, 1), (C + Z + Hv, n_in, d["alpha"], Hv, 0)]
        res["workload"] = f"64 slots x 16 tokens: {M} x {W.HIDDEN} -> {n_in} (in), {M} x {Z} -> {W.HIDDEN} (out), bf16"
        res["us_in_proj"] = time_launches(lambda: gdn.gdn_linear(d["x"], d["w_in"], M, n_in, W.HIDDEN, segs),
                                          steps, warmup)
        res["us_out_proj"] = time_launches(lambda: gdn.gdn_linear(d["out"], d["w_out"], M, W.HIDDEN, Z,
                                                                  [(0, W.HIDDEN, d["y"], W.HIDDEN, 0)]), steps, warmup)
        res["in_proj_flops"] = 2.0 * M * n_in * W.HIDDEN
        res["out_proj_flops"] = 2.0 * M * W.HIDDEN * Z
    elif name == "single_slot":
        s = W.SINGLE_SLOT_VERIFY
        d = device.upload(s, W.make_inputs(s, 0), fill_capture=0.0)
        res["workload"] = "1 slot x 16 tokens, 16/32 heads, d=128, bf16"
        res["us"] = time_launches(lambda: device.verify(d), steps, warmup)
        res["algorithmic_bytes"] = bytemodel.verify_bytes(s)
    del d
    torch.cuda.empty_cache()
    # calibration: snapshot of all 64 slots of the multi-slot pool, 2 x 140,509,184 B moved
    s = W.MULTI_SLOT_VERIFY
    dims = gdn.make_dims(s)
    st = torch.zeros((s.n_pool, s.n_vh, s.d_v, s.d_k), dtype=torch.float32, device="cuda")
    cs = torch.zeros((s.n_pool, 3, s.conv_channels), dtype=torch.float32, device="cuda")
    st2, cs2 = torch.empty_like(st), torch.empty_like(cs)
    slots = torch.arange(s.n_pool, dtype=torch.int32, device="cuda")
    res["calibration"] = {"kernel": "slot_copy_kernel (gdn_snapshot of 64 slots)",
                          "read_bytes": bytemodel.snapshot_bytes(s, s.n_pool) // 2 + 4 * s.n_pool,
                          "write_bytes": bytemodel.snapshot_bytes(s, s.n_pool) // 2,
                          "us": time_launches(lambda: gdn.gdn_snapshot(dims, st, cs, st2, cs2, slots, s.n_pool),
                                              steps, warmup)}
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=4, help="rotating input/state sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-components", action="store_true",
                    help="skip the secondary timings (tree verify, single-slot verify, rollback)")
    ap.add_argument("--component", choices=COMPONENTS,
                    help="profiling aid: run only this secondary workload (--warmup + --steps launches) "
                         "and a calibration copy, and print their launch times instead of the step's line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU code (got --gpus "
              f"{args.gpus})", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from gated_deltanet_linear_verify_amd import bytemodel, device, gdn
    from gated_deltanet_linear_verify_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    gdn.lib()
    torch.cuda.set_device(0)
    if args.component:
        print(json.dumps(component_only(args.component, args.steps, args.warmup)), flush=True)
        return 0
    shape = W.MULTI_SLOT_VERIFY
    B, T = shape.n_batch, shape.n_tok

    log(f"[bench] allocating {args.sets} input sets, each with its own capture, for {W.describe(shape)}")
    sets = []
    base = None
    for i in range(args.sets):
        inp = W.make_inputs(shape, seed=i)
        if base is None:
            base = inp
        d = device.upload(shape, inp, fill_capture=0.0)
        acc = (T - 1 - inp["trims"]).astype(np.int32)
        d["accepted"] = torch.from_numpy(acc).cuda()
        device.verify(d)  # the round before the first timed one: every capture position is written
        d["dims_defer"] = gdn.make_dims(shape, flags=gdn.GDN_F_DEFER_COMMIT)
        sets.append(d)
    stream = torch.cuda.current_stream()

    def step(i: int, ev=None):
        """One round: verify with capture, then the batched rollback copy."""
        d = sets[i % len(sets)]
        if ev is not None:
            ev[0].record(stream)
        device.verify(d, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        gdn.gdn_rollback_batch(d["capture"], d["slot_ids"], d["accepted"], B, stream)
        if ev is not None:
            ev[2].record(stream)

    def resume_step(key: str):
        def fn(i: int, ev=None):
            """The same round as one launch: the previous round's rollback folded into the verify."""
            d = sets[i % len(sets)]
            if ev is not None:
                ev[0].record(stream)
            device.verify_resume(d, d["accepted"], stream=stream, dims=d[key])
            if ev is not None:
                ev[1].record(stream)
                ev[2].record(stream)
        return fn

    def timed(fn, steps: int, warmup: int):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t_start.record(stream)
        for i in range(steps):
            fn(i, evs[i])
        t_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        verify_ms = [e[0].elapsed_time(e[1]) for e in evs]
        second_ms = [e[1].elapsed_time(e[2]) for e in evs]
        return t_start.elapsed_time(t_end) / steps, wall / steps, verify_ms, second_ms

    ms_step, wall_step, verify_ms, rollback_ms = timed(step, args.steps, args.warmup)
    rs_steps = max(20, args.steps // 2)
    rs_ms_step, _, rs_verify_ms, _ = timed(resume_step("dims"), rs_steps, min(args.warmup, 10))
    rd_ms_step, _, rd_verify_ms, _ = timed(resume_step("dims_defer"), rs_steps, min(args.warmup, 10))
    vb_defer = bytemodel.verify_bytes(shape, commit=False)
    r_avg = sum(rollback_ms) / len(rollback_ms)
    v_avg = sum(verify_ms) / len(verify_ms)
    vb = bytemodel.verify_bytes(shape)
    rb = bytemodel.rollback_bytes(shape, B)
    achieved = vb / (v_avg * 1e-3) / 1e9
    traffic = measured_traffic()
    log(f"[bench] {args.steps} steps: {ms_step * 1e3:.1f} us/step (wall {wall_step * 1e6:.1f} us), "
        f"verify {v_avg * 1e3:.1f} us avg, median {np.median(verify_ms) * 1e3:.1f} (p10 {np.percentile(verify_ms, 10) * 1e3:.1f}, "
        f"p90 {np.percentile(verify_ms, 90) * 1e3:.1f}) -> {achieved:.0f} GB/s, rollback {r_avg * 1e3:.1f} us; "
        f"step {(vb + rb) / (ms_step * 1e-3) / 1e9:.0f} GB/s; resume step {rs_ms_step * 1e3:.1f} us, "
        f"with the commit deferred {rd_ms_step * 1e3:.1f} us")

    result = {
        "metric": METRIC,
        "value": B * T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "multi_slot_verify", "slots": B, "tokens_per_slot": T,
                   "key_heads": shape.n_kh, "value_heads": shape.n_vh, "head_dim": shape.d_k,
                   "activations": "bf16", "state_and_capture": "f32",
                   "step": "gdn_verify + gdn_rollback_batch", "rotating_sets": args.sets},
        "hbm_gbps_step": (vb + rb) / (ms_step * 1e-3) / 1e9,
        "step_resume": {"step": "gdn_verify_resume (the previous round's rollback folded into the state load)",
                        "steps": rs_steps, "ms_per_step": rs_ms_step,
                        "tokens_per_s": B * T / (rs_ms_step * 1e-3),
                        "verify_us": sum(rs_verify_ms) / len(rs_verify_ms) * 1e3,
                        "hbm_gbps_step": vb / (rs_ms_step * 1e-3) / 1e9},
        "step_resume_deferred": {"step": "gdn_verify_resume with GDN_F_DEFER_COMMIT (the state stays in the capture)",
                                 "steps": rs_steps, "ms_per_step": rd_ms_step,
                                 "tokens_per_s": B * T / (rd_ms_step * 1e-3),
                                 "verify_us": sum(rd_verify_ms) / len(rd_verify_ms) * 1e3,
                                 "algorithmic_bytes": vb_defer,
                                 "hbm_gbps_step": vb_defer / (rd_ms_step * 1e-3) / 1e9},
        "rollback": {"us": r_avg * 1e3, "hbm_gbps": rb / (r_avg * 1e-3) / 1e9, "algorithmic_bytes": rb},
        "roofline": {"kernel": "verify_chain_kernel", "bound": "hbm", "achieved": achieved,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": vb,
                     "avg_launch_us": v_avg * 1e3,
                     "median_launch_us": float(np.median(verify_ms)) * 1e3,
                     "p10_launch_us": float(np.percentile(verify_ms, 10)) * 1e3,
                     "p90_launch_us": float(np.percentile(verify_ms, 90)) * 1e3,
                     "frac_at_median": vb / (float(np.median(verify_ms)) * 1e-3) / 1e9 / PEAK_HBM_GBPS},
    }
    sets.clear()  # 4 x 2.2 GB of state and capture, not needed by the components
    torch.cuda.empty_cache()
    if not args.no_components:
        result["components"] = components(args)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(shape, base)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
