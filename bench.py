#!/usr/bin/env python3
"""Benchmark of the KDA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--dtype f32|f16]
                    [--no-extras] [--no-cpu-baseline]

A step is one decode launch over the batched workload: 64 request slots
gathered by a random permutation from a 96-slot pool, one token each, H = 12
heads of K = V = 128 (fp32 pool by default, fp16 with --dtype f16).  Every
step's state is read from and written back to the pool in HBM.  Successive
steps rotate over enough distinct pool copies (>= 1 GiB in all) that the
256 MB last-level cache cannot hold the state between visits, as in a model
whose 69 KDA layers each stream their own pool.

Prints ONE JSON line.  value = state GB/s (state bytes read + written per
step / wall time per step, timed region bracketed by synchronisations);
roofline = algorithmic bytes of one launch / its average duration measured
with HIP events on the launch stream (the timed launches are replayed from
one HIP graph, back to back), against the 8 TB/s HBM peak; traffic =
hardware byte counters of the committed rocprofv3 summary when it was taken
on this kernel source, else null; cpu_baseline = the CPU oracle timed on a
bounded sample of the same workload.  Extra keys report the other workloads
(fp16 pool, 8 x 8 speculative rows, a 69-layer step) and a plain-copy
bandwidth probe.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # AMD MI355X published HBM3E bandwidth
PEAK_SOURCE = "AMD MI355X spec: 8 TB/s HBM3E"
# The pages' production kernel on this workload (fp32 state, H=12, K=V=128,
# N=64, at its fp32 V-block cap of 32): 24.6 us, i.e. 4092 GB/s of state.
PAGES_FP32_US = 24.6
PAGES_FP16_US = 16.1
KERNEL_SRC = os.path.join(ROOT, "kda_gated_delta_decode_amd", "csrc", "kda_decode.hip")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "kda_decode_tile_pmc_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    """The hash the committed counter summary records (decode kernel source
    and the csrc headers it is built with)."""
    from kda_gated_delta_decode_amd.profiling import kernel_hash as kh
    return kh(KERNEL_SRC)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--dtype", choices=["f32", "f16"], default="f32")
    ap.add_argument("--no-extras", action="store_true", help="skip the other workloads")
    ap.add_argument("--extras", choices=["all", "copy", "probes", "pmc", "layouts"], default="all",
                    help="'copy' runs only the plain-copy probe after the main workload, "
                         "'probes' only the bandwidth probes, 'pmc' the copies that calibrate "
                         "the byte counters (plain and nontemporal) and the 8 x 8 chained rows, "
                         "'layouts' only the launch shapes of chained rows and of the fused step side by "
                         "side (several minutes)")
    ap.add_argument("--eager", action="store_true",
                    help="launch eagerly instead of replaying a HIP graph (for profilers)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    return ap.parse_args()


class Workload:
    """Device buffers for one decode workload, with rotating pool copies."""

    def __init__(self, inp, min_rotation_bytes: int, torch):
        self.inp = inp
        dev = torch.device("cuda", 0)
        import numpy as np
        host_pool = inp.pool if inp.dtype == "f32" else inp.pool.view(np.float16)
        pool_bytes = host_pool.nbytes
        n_copies = max(1, math.ceil(min_rotation_bytes / pool_bytes))
        first = torch.from_numpy(host_pool).to(dev)
        self.pools = [first] + [first.clone() for _ in range(n_copies - 1)]
        self.ids = torch.from_numpy(inp.slot_ids).to(dev)
        self.q, self.k, self.v, self.g, self.b = (torch.from_numpy(getattr(inp, n)).to(dev)
                                                  for n in ("q", "k", "v", "g", "b"))
        R, H, V = inp.slot_ids.size, inp.pool.shape[1], inp.pool.shape[3]
        self.out = torch.empty((R, H, V), dtype=torch.float32, device=dev)
        self.rotation_bytes = pool_bytes * n_copies

    def launch(self, i: int, B):
        B.kda_decode_step(self.pools[i % len(self.pools)], self.ids, self.q, self.k, self.v,
                          self.g, self.b, self.out, n_rows_per_slot=self.inp.n_rows,
                          scale=self.inp.scale)


EAGER = False
ROT = 1 << 30  # bytes of pool copies each timed workload rotates over (> the 256 MiB MALL)


def time_launches(fn, steps: int, warmup: int, torch):
    """Time `steps` calls of fn(i) (each enqueues one step on the current
    stream) replayed from a HIP graph, after `warmup` calls replayed the same
    way.  Graph replay is how a serving step is launched; it takes the
    Python binding's per-call overhead off the GPU's timeline, so the event
    region measures the kernels back to back.  Returns per-step times."""
    if EAGER:
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(steps):
            fn(warmup + i)
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end)
        return {"ms_per_step": ms / steps, "host_ms_per_step": ms / steps, "launch_ms_mean": ms / steps}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)                       # one eager call before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g_warm = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_warm):
        for i in range(warmup):
            fn(i)
    g_timed = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_timed):
        for i in range(steps):
            fn(warmup + i)
    g_warm.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    g_timed.replay()
    end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    region_ms = start.elapsed_time(end)
    del g_warm, g_timed
    # Graph-replayed launches run back to back, so the event region divided
    # by the step count is the mean step (and, at one launch per step, the
    # mean launch) duration.
    return {"ms_per_step": region_ms / steps, "host_ms_per_step": wall_ms / steps,
            "launch_ms_mean": region_ms / steps}


def pmc_traffic(expected_launch_key: str):
    """Traffic from the committed counter summary, if it was taken on the
    current kernel source for this launch; else None."""
    try:
        with open(PMC_SUMMARY) as f:
            s = json.load(f)
    except (OSError, ValueError):
        return None
    entry = s.get("launches", {}).get(expected_launch_key)
    if entry is None or s.get("kernel_source_sha256_16") != kernel_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_baseline(inp, seconds: float):
    """Time the CPU oracle (fp32 loop, one thread) on a bounded sample of the
    workload: whole oracle launches over the first 8 requests, repeated until
    `seconds` have passed."""
    from oracle import kda_oracle
    n_req = min(8, inp.n_req)
    rows = n_req * inp.n_rows
    sel = slice(0, rows)
    pool = inp.pool.copy()
    calls = 0
    t0 = time.perf_counter()
    while True:
        kda_oracle.step_f32(pool, inp.slot_ids[sel], inp.q[sel], inp.k[sel], inp.v[sel],
                            inp.g[sel], inp.b[sel], n_rows=inp.n_rows, scale=inp.scale)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    H, K, V = inp.pool.shape[1:]
    elem = 4 if inp.dtype == "f32" else 2
    state_bytes = calls * n_req * H * K * V * elem * (1 + inp.n_rows)
    return {
        "value": state_bytes / el / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "%d oracle launches of %d of the %d requests x %d heads (%s pool, %d row(s)), %.1f s"
                  % (calls, n_req, inp.n_req, H, inp.dtype, inp.n_rows, el),
        "us_per_full_step": el / calls * (inp.n_req / n_req) * 1e6,
        "host_cpus_available": len(os.sched_getaffinity(0)),
        "host_cpus_online": os.cpu_count(),
        "cpu_model": cpu_model(),
        "parallel": cpu_baseline_parallel(inp, min(seconds, 6.0)),
        "other_configs": cpu_other_configs(min(seconds / 6.0, 2.0)),
    }


def cpu_model() -> str:
    """The host CPU's model name (Linux), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_other_configs(seconds: float):
    """The same oracle (one thread) on the other workloads: the batched step
    on both pool dtypes, the 8 x 8 chained rows on an fp16 pool (whole oracle
    launches, repeated for about `seconds` each), and one pass of the 69-layer
    fp32 step (69 oracle launches of 64 requests; one pool serves every layer,
    since the oracle's time does not depend on the values)."""
    from oracle import kda_oracle
    import kda_inputs
    res = {}

    def timed(inp, secs):
        pool = inp.pool.copy()
        calls, t0 = 0, time.perf_counter()
        while True:
            kda_oracle.step_f32(pool, inp.slot_ids, inp.q, inp.k, inp.v, inp.g, inp.b,
                                n_rows=inp.n_rows, scale=inp.scale)
            calls += 1
            el = time.perf_counter() - t0
            if el >= secs:
                return el / calls
    for name, inp in (("batched_f32", kda_inputs.batched_f32(0)), ("batched_f16", kda_inputs.batched_f16(0)),
                      ("spec_verify_f16", kda_inputs.spec_verify_f16(0))):
        per = timed(inp, seconds)
        res[name] = {"us_per_step": round(per * 1e6, 1),
                     "state_GB/s": round(inp.state_bytes() / per / 1e9, 2)}
    inp = kda_inputs.layer_step(0, "f32")
    per = timed(inp, 0.0) * 69
    res["layers69_f32_one_pass"] = {"us_per_step": round(per * 1e6, 1),
                                    "state_GB/s": round(69 * inp.state_bytes() / per / 1e9, 2)}
    return res


def cpu_baseline_parallel(inp, seconds: float, max_threads: int = 16):
    """The same oracle, one thread per available core (at most 16): each
    thread runs whole oracle launches over its own 2 requests on its own
    copy of the pool (the C oracle releases the GIL while it runs), for
    about `seconds`.  A reported baseline, not tuned."""
    import threading
    from oracle import kda_oracle
    n_threads = max(1, min(max_threads, len(os.sched_getaffinity(0)), inp.n_req // 2))
    done = [0] * n_threads
    stop = time.perf_counter() + seconds

    def work(i):
        sel = slice(2 * i * inp.n_rows, 2 * (i + 1) * inp.n_rows)
        pool = inp.pool.copy()
        while time.perf_counter() < stop:
            kda_oracle.step_f32(pool, inp.slot_ids[sel], inp.q[sel], inp.k[sel], inp.v[sel],
                                inp.g[sel], inp.b[sel], n_rows=inp.n_rows, scale=inp.scale)
            done[i] += 1
    t0 = time.perf_counter()
    threads = [threading.Thread(target=work, args=(i,)) for i in range(n_threads)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    el = time.perf_counter() - t0
    H, K, V = inp.pool.shape[1:]
    elem = 4 if inp.dtype == "f32" else 2
    state_bytes = sum(done) * 2 * H * K * V * elem * (1 + inp.n_rows)
    return {"value": state_bytes / el / 1e9, "unit": "GB/s", "cores": n_threads,
            "sample": "%d threads x whole oracle launches of 2 requests x %d heads, %.1f s"
                      % (n_threads, H, el)}


def main():
    args = parse()
    global EAGER
    EAGER = args.eager
    if args.gpus != 1:
        print("bench.py measures one GPU: this path has no cross-GPU exchange and this build "
              "runs on a single MI355X; --gpus %d is not supported (use --gpus 1)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kda_inputs
    from kda_gated_delta_decode_amd import binding as B

    B.library()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("no GPU visible: bench.py needs an MI355X", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    dev_name = torch.cuda.get_device_name(0)

    main_inp = kda_inputs.batched_f32(0) if args.dtype == "f32" else kda_inputs.batched_f16(0)
    wl = Workload(main_inp, ROT, torch)
    log("workload:", main_inp.name, "rotation copies:", len(wl.pools))
    t = time_launches(lambda i: wl.launch(i, B), args.steps, args.warmup, torch)
    state_bytes = main_inp.state_bytes()
    alg_bytes = state_bytes + main_inp.io_bytes()
    value = state_bytes / (t["ms_per_step"] * 1e-3) / 1e9
    achieved = alg_bytes / (t["launch_ms_mean"] * 1e-3) / 1e9
    desc = B.kda_describe_launch(main_inp.n_req, main_inp.n_rows, main_inp.pool.shape[1], main_inp.dtype)
    launch_key = "%s_n%d_rows%d" % (main_inp.dtype, main_inp.n_req, main_inp.n_rows)
    pages_us = PAGES_FP32_US if args.dtype == "f32" else PAGES_FP16_US
    pages_gbs = state_bytes / (pages_us * 1e-6) / 1e9

    rec = {
        "metric": "KDA decode state GB/s (% of HBM peak) + us/step, H=12 K=V=128 N=64 fp16/fp32",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / pages_gbs, 3),
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {
            "workload": "batched KDA decode: 64 of 96 slots, 1 token each, H=12, K=V=128, %s state pool, "
                        "pools rotated over %.2f GiB" % ("fp32" if args.dtype == "f32" else "fp16",
                                                          wl.rotation_bytes / 2 ** 30),
            "n_req": main_inp.n_req, "rows_per_req": main_inp.n_rows, "heads": 12, "K": 128, "V": 128,
            "pool_slots": int(main_inp.pool.shape[0]), "state_dtype": args.dtype,
            "launch": desc,
        },
        "us_per_step": round(t["ms_per_step"] * 1e3, 3),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "updates_per_s": main_inp.n_req * main_inp.n_rows * 12 / (t["ms_per_step"] * 1e-3),
        "vs_baseline_basis": "the pages' production fused gating kernel at this workload: %.1f us "
                             "(%.0f GB/s of state), MI355X context" % (pages_us, pages_gbs),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": pmc_traffic(launch_key),
            "kernel": "kda_decode_tile",
            "algorithmic_bytes_per_launch": alg_bytes,
            "launch_us_mean": round(t["launch_ms_mean"] * 1e3, 3),
            "timing": ("HIP events around %d eager launches" % args.steps) if args.eager else
                      ("HIP events around one HIP-graph replay of the %d launches" % args.steps),
            "peak_source": PEAK_SOURCE,
        },
        "device": dev_name,
    }

    if not args.no_extras and args.extras == "layouts":
        rec["extras"] = {"chained_layouts": chained_layouts(B, torch), "fused_layouts": fused_layouts(B, torch)}
    if not args.no_extras and args.extras != "layouts":
        extras = {}
        # plain copies: the achievable streaming read+write bandwidth at
        # 1 GiB, and a copy moving the same bytes as one decode step; the
        # latter rotates over >= 1 GiB of buffer pairs like the decode pools
        for label, nbytes in (("copy_probe_1GiB", 1 << 30),
                              ("copy_probe_same_bytes", (state_bytes // 2) // 16 * 16)):
            if args.extras == "probes":
                break
            pairs = max(1, math.ceil((1 << 30) / (2 * nbytes)))
            bufs = [(torch.empty(nbytes, dtype=torch.uint8, device="cuda"),
                     torch.empty(nbytes, dtype=torch.uint8, device="cuda")) for _ in range(pairs)]
            for src, _ in bufs:
                src.fill_(1)
            tc = time_launches(lambda i: B.kda_copy_probe(bufs[i % pairs][1], bufs[i % pairs][0]),
                               max(20, 2 * pairs), 3, torch)
            extras[label] = {"bytes_copied": nbytes, "buffer_pairs_rotated": pairs,
                             "GB/s_read_plus_write": round(2 * nbytes / (tc["launch_ms_mean"] * 1e-3) / 1e9, 1),
                             "us": round(tc["launch_ms_mean"] * 1e3, 2)}
            del bufs
        if args.extras == "pmc":
            # the nontemporal copy (the decode's state traffic carries the
            # hint) at the step's bytes and at 1 GiB, then the chained rows
            for label, nbytes in (("copy_nt_v1_1GiB", 1 << 29), ("copy_nt_v1_step_bytes", state_bytes // 2)):
                nbytes = nbytes // 16 * 16
                src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
                dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
                tc = time_launches(lambda i: B.kda_bw_probe(dst, src, nbytes, B.KDA_PROBE_COPY, 1, True), 5, 1, torch)
                extras[label] = {"bytes_copied": nbytes, "us": round(tc["launch_ms_mean"] * 1e3, 2)}
                del src, dst
            inp = kda_inputs.spec_verify_f16(0)
            w = Workload(inp, ROT, torch)
            extras["spec_verify_f16"] = summarize(inp, time_launches(lambda i: w.launch(i, B), 20, 2, torch))
            del w
        if args.extras in ("all", "probes"):
            probes = bandwidth_probes(B, torch, state_bytes)
            extras["bandwidth_probes"] = probes
            best = max(v["GB/s"] for k, v in probes.items() if k.startswith("copy_") and "1GiB" in k)
            rec["achievable_copy_GB/s"] = best
            rec["pct_of_copy_bandwidth"] = round(100.0 * achieved / best, 2)
            tp = probes.get("tile_pattern_" + args.dtype)
            if tp is not None:
                rec["pct_of_tile_pattern"] = round(100.0 * tp["us"] / (t["launch_ms_mean"] * 1e3), 2)
        elif "copy_probe_1GiB" in extras:
            rec["pct_of_copy_bandwidth"] = round(
                100.0 * achieved / extras["copy_probe_1GiB"]["GB/s_read_plus_write"], 2)
        other = () if args.extras in ("copy", "probes", "pmc") else (
                        ("batched_f16" if args.dtype == "f32" else "batched_f32",
                          kda_inputs.batched_f16 if args.dtype == "f32" else kda_inputs.batched_f32),
                         ("spec_verify_f16", kda_inputs.spec_verify_f16),
                         ("single_slot_f32", kda_inputs.single_slot_f32))
        for name, fn in other:
            inp = fn(0)
            w = Workload(inp, ROT, torch)
            tt = time_launches(lambda i: w.launch(i, B), max(50, args.steps // 2), 10, torch)
            extras[name] = summarize(inp, tt)
            if name == "spec_verify_f16":
                # counter-derived HBM bytes of the chained-rows kernel (null
                # unless the committed summary matches the kernel source)
                extras[name]["traffic"] = pmc_traffic("%s_n64_rows1_spec_verify_8x8" % args.dtype)
            del w
        rp = extras.get("bandwidth_probes", {}).get("rows_pattern_f16_8x8")
        if rp is not None and "spec_verify_f16" in extras:
            sv = extras["spec_verify_f16"]
            sv["rows_pattern_us"] = rp["us"]
            sv["pct_of_rows_pattern"] = round(100.0 * rp["us"] / sv["us_per_step"], 2)
        if args.extras == "all":
            # the same batched step out of place: each request reads slot A
            # and writes slot B of a 128-slot pool (init_slot_ids), as a
            # runtime that ping-pongs two slots per request would
            inp = kda_inputs.make_inputs("batched decode N=64, out of place (128-slot pool), %s pool"
                                         % args.dtype, 128, 64, 1, args.dtype, seed=0)
            inp.slot_ids[:] = np.arange(64, 128, dtype=np.int32)
            w = Workload(inp, ROT, torch)
            init_d = torch.arange(64, dtype=torch.int32, device="cuda")

            def pingpong(i):
                B.kda_decode_step(w.pools[i % len(w.pools)], w.ids, w.q, w.k, w.v, w.g, w.b, w.out,
                                  scale=inp.scale, init_slot_ids=init_d)
            tt = time_launches(pingpong, max(50, args.steps // 2), 10, torch)
            extras["batched_%s_out_of_place" % args.dtype] = summarize(inp, tt)
            del w
        if args.extras == "all":
            # informational: the main workload on one pool, no rotation, so the
            # state can stay in the 256 MiB last-level cache between launches
            # (never the reported value)
            w = Workload(main_inp, 0, torch)
            tt = time_launches(lambda i: w.launch(i, B), max(50, args.steps // 2), 10, torch)
            hot = summarize(main_inp, tt)
            hot["workload"] = main_inp.name + ", one pool, not rotated (cache-resident state)"
            extras["batched_%s_hot_pool" % args.dtype] = hot
            del w
        if args.extras == "all":
            for name, (n_req, n_rows, dt) in (("batched_%s_fused_conv" % args.dtype, (64, 1, args.dtype)),
                                              ("spec_verify_f16_fused_conv", (8, 8, "f16"))):
                extras[name] = fused_conv(n_req, n_rows, dt, B, torch, max(50, args.steps // 2))
        if args.extras == "all":
            extras["prefill_" + args.dtype] = prefill_extra(args.dtype, B, torch, 20)
        if args.extras == "all":
            extras["long_run_8192"] = long_run_extra(B, torch)
        # a 69-layer decode step: 69 independent 64-slot pools, one launch each
        for dt in (("f32", "f16") if args.extras == "all" else ()):
            extras["layers69_" + dt] = layers69(dt, B, torch, steps=10, warmup=2)
        rec["extras"] = extras
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(main_inp, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def bandwidth_probes(B, torch, step_state_bytes):
    """What this GPU reaches on plain traffic, measured like the decode
    (graph replay, buffers rotated over >= 1 GiB where one is smaller):
    streaming copies (plain or nontemporal, 1, 2 or 4 16-byte vectors per
    thread) at 1 GiB, the best of them at 100 MB and 4 GiB, read-only and
    write-only streams at 1 GiB and at one decode step's bytes, and the decode
    launch's own tile traffic (kda_tile_probe: same grid, layout and
    nontemporal loads and stores, no arithmetic) on the batched workloads'
    rotated pools, and the 8 x 8 chained rows' own traffic (kda_rows_probe)
    on the spec-verify workload's.  GB/s counts every byte read plus every
    byte written."""
    import kda_inputs
    GiB = 1 << 30
    res = {}

    def run(label, mode, v, nt, nbytes):
        nbytes = nbytes // 16 * 16
        moved = nbytes * (2 if mode == B.KDA_PROBE_COPY else 1)
        sets = max(1, math.ceil(GiB / moved))
        bufs = []
        for _ in range(sets):
            src = None
            if mode != B.KDA_PROBE_WRITE:
                src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
                src.fill_(1)
            dst = torch.empty(nbytes if mode != B.KDA_PROBE_READ else 16, dtype=torch.uint8, device="cuda")
            bufs.append((src, dst))
        tc = time_launches(lambda i: B.kda_bw_probe(bufs[i % sets][1], bufs[i % sets][0], nbytes, mode, v, nt),
                           max(20, 2 * sets), 3, torch)
        us = tc["launch_ms_mean"] * 1e3
        res[label] = {"bytes_moved": moved, "buffer_sets_rotated": sets, "us": round(us, 2),
                      "GB/s": round(moved / us / 1e3, 1)}
        del bufs
        torch.cuda.empty_cache()

    C, R, W = B.KDA_PROBE_COPY, B.KDA_PROBE_READ, B.KDA_PROBE_WRITE
    for v in (1, 2, 4):
        run("copy_nt_v%d_1GiB" % v, C, v, True, GiB // 2)
        run("copy_plain_v%d_1GiB" % v, C, v, False, GiB // 2)
    best_v = max((1, 2, 4), key=lambda v: res["copy_nt_v%d_1GiB" % v]["GB/s"])
    run("copy_nt_v%d_100MB" % best_v, C, best_v, True, 50 * 10 ** 6)
    run("copy_nt_v%d_4GiB" % best_v, C, best_v, True, 2 * GiB)
    for nt, tag in ((True, "nt"), (False, "plain")):
        run("read_%s_v4_1GiB" % tag, R, 4, nt, GiB)
        run("write_%s_v4_1GiB" % tag, W, 4, nt, GiB)
    half = step_state_bytes // 2
    run("read_nt_v4_step_bytes", R, 4, True, half)
    run("write_nt_v4_step_bytes", W, 4, True, half)
    run("copy_nt_v%d_step_bytes" % best_v, C, best_v, True, half)
    # the 8 x 8 chained rows' snapshot stores alone: 8 snapshots of 96 fp16
    # (request, head) states, 25.2 MB
    run("write_nt_v1_spec_verify_snapshot_bytes", W, 1, True, 8 * 96 * 128 * 128 * 2)
    for dtype, fn in (("f32", kda_inputs.batched_f32), ("f16", kda_inputs.batched_f16)):
        inp = fn(0)
        w = Workload(inp, ROT, torch)
        tc = time_launches(lambda i: B.kda_tile_probe(w.pools[i % len(w.pools)], w.ids), 100, 10, torch)
        us = tc["launch_ms_mean"] * 1e3
        res["tile_pattern_" + dtype] = {"bytes_moved": inp.state_bytes(), "pools_rotated": len(w.pools),
                                        "us": round(us, 2), "GB/s": round(inp.state_bytes() / us / 1e3, 1)}
        del w
        torch.cuda.empty_cache()
    # the 8 x 8 chained rows' own traffic (kda_rows_probe: the matrix-core
    # block form's grid, layout, slot id loads, state loads and snapshot
    # stores, no arithmetic) on the spec-verify workload's rotated pools; then
    # the same traffic in the tiles the block form was weighed against: 32 and
    # 128 columns over 8 waves, and the fused convolution's whole heads (128
    # columns, two halves of 8 waves)
    inp = kda_inputs.spec_verify_f16(0)
    w = Workload(inp, ROT, torch)
    for name, cols, nw in (("rows_pattern_f16_8x8", 0, 0), ("rows_pattern_f16_8x8_cols32", 32, 8),
                           ("rows_pattern_f16_8x8_cols128", 128, 8),
                           ("rows_pattern_f16_8x8_cols128_waves16", 128, 16)):
        tc = time_launches(lambda i, cols=cols, nw=nw: B.kda_rows_probe(
            w.pools[i % len(w.pools)], w.ids, inp.n_rows, tile_cols=cols, waves=nw), 100, 10, torch)
        us = tc["launch_ms_mean"] * 1e3
        res[name] = {"bytes_moved": inp.state_bytes(), "pools_rotated": len(w.pools), "tile_cols": cols or 64,
                     "waves": nw or 8, "us": round(us, 2), "GB/s": round(inp.state_bytes() / us / 1e3, 1)}
    del w
    torch.cuda.empty_cache()
    return res


def summarize(inp, tt):
    sb, ab = inp.state_bytes(), inp.state_bytes() + inp.io_bytes()
    us = tt["ms_per_step"] * 1e3
    return {"workload": inp.name, "us_per_step": round(us, 3),
            "state_GB/s": round(sb / us / 1e3, 1),
            "algorithmic_GB/s": round(ab / us / 1e3, 1),
            "frac_of_peak": round(ab / us / 1e3 / HBM_PEAK_GBS, 4)}


def fused_conv(n_req, n_rows, dtype, B, torch, steps, **launch):
    """Time the decode step with the short convolution fused in front
    (kda_decode_step_conv, with pair counters: kda_decode_step_conv_ws) on a
    96-slot pool; state pools and conv pools both rotate over >= 1 GiB.
    Algorithmic bytes add to the plain step's the raw q|k|v rows, the taps,
    and the conv history (3 bf16 entries of 3*H*128 channels) read once per
    request and written once per row."""
    import kda_inputs
    ci = kda_inputs.make_conv_inputs("fused conv + decode, %d req x %d rows, %s pool, H=12"
                                     % (n_req, n_rows, dtype), 96, n_req, n_rows, dtype, seed=0)
    inp = ci.dec
    w = Workload(inp, ROT, torch)
    conv0 = torch.from_numpy(ci.conv).cuda().view(torch.bfloat16)
    convs = [conv0] + [conv0.clone() for _ in range(len(w.pools) - 1)]
    x = torch.from_numpy(ci.x).cuda()
    cw = torch.from_numpy(ci.w).cuda()
    launch.setdefault("pair_counts", B.conv_pair_counts(n_req, inp.pool.shape[1], x.device))

    def step(i):
        B.kda_decode_step_conv(w.pools[i % len(w.pools)], convs[i % len(convs)], w.ids, x, cw,
                               w.g, w.b, w.out, n_rows_per_slot=n_rows, scale=inp.scale, **launch)
    tt = time_launches(step, steps, 10, torch)
    R, H = inp.slot_ids.size, inp.pool.shape[1]
    hist = 3 * 3 * H * 128 * 2
    extra = R * 3 * H * 128 * 4 + 3 * H * 128 * 4 * 4 + hist * (n_req + R) \
        - R * H * 128 * 3 * 4  # x replaces q, k, v
    us = tt["ms_per_step"] * 1e3
    ab = inp.state_bytes() + inp.io_bytes() + extra
    del w, convs
    return {"workload": inp.name, "us_per_step": round(us, 3),
            "algorithmic_GB/s": round(ab / us / 1e3, 1),
            "frac_of_peak": round(ab / us / 1e3 / HBM_PEAK_GBS, 4)}


def chained_layouts(B, torch):
    """Chained rows' launch shapes side by side, in us per launch (graph
    replay, pools rotated over >= 1 GiB, median of 3 interleaved runs): the
    matrix-core block form, the K split and (fp16) whole K per wave."""
    import kda_inputs
    import statistics
    shapes = {"f16": [(1, 2), (4, 2), (8, 2), (16, 2), (48, 2), (1, 4), (4, 4), (8, 4), (16, 4), (24, 4), (8, 6),
                      (8, 8), (12, 8), (20, 8), (24, 8), (32, 8)],
              "f32": [(1, 2), (4, 2), (8, 2), (16, 2), (1, 4), (4, 4), (8, 4), (16, 4), (8, 6), (1, 8), (4, 8),
                      (8, 8), (12, 8), (20, 8), (32, 8)]}
    out = {}
    for dt in ("f16", "f32"):
        forms = {"block": B.KDA_ROWS_MATRIX, "k_split": B.KDA_ROWS_K_SPLIT}
        if dt == "f16":
            forms["whole_k"] = B.KDA_ROWS_WAVE_K
        res = {}
        for n_req, n_rows in shapes[dt]:
            inp = kda_inputs.make_inputs("chained layouts", max(96, n_req * n_rows + 8), n_req, n_rows, dt, seed=1)
            w = Workload(inp, ROT, torch)
            t = {f: [] for f in forms}
            for _ in range(3):
                for f, layout in forms.items():
                    def step(i, layout=layout):
                        B.kda_decode_step(w.pools[i % len(w.pools)], w.ids, w.q, w.k, w.v, w.g, w.b, w.out,
                                          n_rows_per_slot=n_rows, scale=inp.scale, rows_layout=layout)
                    t[f].append(time_launches(step, 60, 10, torch)["launch_ms_mean"] * 1e3)
            res["%dx%d" % (n_req, n_rows)] = {f: round(statistics.median(v), 2) for f, v in t.items()}
            print("chained layouts %s %dx%d %s" % (dt, n_req, n_rows, res["%dx%d" % (n_req, n_rows)]),
                  file=sys.stderr, flush=True)
            del w
            torch.cuda.empty_cache()
        out[dt] = res
    return out


def fused_layouts(B, torch):
    """The fused step's launch shapes side by side, in us per launch (graph
    replay, state and history pools rotated over >= 1 GiB, median of 3
    interleaved runs): chained rows in 64-column halves (with pair counters),
    as whole heads and in the K split; one row per request over 2, 4 and 8
    waves per tile."""
    import kda_inputs
    import statistics
    M, KS = B.KDA_ROWS_MATRIX, B.KDA_ROWS_K_SPLIT
    chained = {"f16": [(1, 2), (8, 2), (16, 2), (48, 2), (1, 4), (8, 4), (12, 4), (16, 4), (24, 4), (8, 6),
                       (1, 8), (8, 8), (12, 8), (16, 8), (20, 8), (32, 8)],
               "f32": [(1, 2), (4, 2), (8, 2), (1, 4), (4, 4), (8, 4), (12, 4), (8, 6), (1, 8), (4, 8),
                       (8, 8), (12, 8)]}
    out = {}
    for dt in ("f16", "f32"):
        res = {}
        for n_req, n_rows in chained[dt] + [(n, 1) for n in (16, 32, 64, 96)]:
            ci = kda_inputs.make_conv_inputs("fused layouts", max(96, n_req * n_rows + 8), n_req, n_rows, dt, seed=2)
            inp = ci.dec
            w = Workload(inp, ROT, torch)
            conv0 = torch.from_numpy(ci.conv).cuda().view(torch.bfloat16)
            convs = [conv0] + [conv0.clone() for _ in range(len(w.pools) - 1)]
            x = torch.from_numpy(ci.x).cuda()
            cw = torch.from_numpy(ci.w).cuda()
            if n_rows > 1:
                counts = B.conv_pair_counts(n_req, inp.pool.shape[1], x.device)
                forms = {"halves": dict(rows_layout=M, pair_counts=counts), "whole_heads": dict(rows_layout=M),
                         "k_split": dict(rows_layout=KS)}
            else:
                forms = {"waves_%d" % nw: dict(waves_per_tile=nw) for nw in (2, 4, 8)}
            t = {f: [] for f in forms}
            for _ in range(3):
                for f, o in forms.items():
                    def step(i, o=o):
                        B.kda_decode_step_conv(w.pools[i % len(w.pools)], convs[i % len(convs)], w.ids, x, cw,
                                               w.g, w.b, w.out, n_rows_per_slot=n_rows, scale=inp.scale, **o)
                    t[f].append(time_launches(step, 60, 10, torch)["launch_ms_mean"] * 1e3)
            res["%dx%d" % (n_req, n_rows)] = {f: round(statistics.median(v), 2) for f, v in t.items()}
            print("fused layouts %s %dx%d %s" % (dt, n_req, n_rows, res["%dx%d" % (n_req, n_rows)]),
                  file=sys.stderr, flush=True)
            del w, convs
            torch.cuda.empty_cache()
        out[dt] = res
    return out


MFMA_F32_PEAK_TFLOPS = 157.3  # AMD MI355X spec: dense fp32 matrix throughput
# Algorithmic flops of the prefill per (token, head): the recurrence's own
# work, 7 K V (decay, the two column sums over K, the rank-1 update, the
# read-out).  The chunked form the kernel runs does more, 122,880 per (token,
# head) at 32-token chunks (the three state contractions plus the block
# couplings, solve and P Delta); the roofline credits only the method's.
PREFILL_FLOP_PER_TOKEN_HEAD = 7 * 128 * 128
PREFILL_CHUNKED_FLOP_PER_TOKEN_HEAD = (3 * 2 * 32 * 128 * 128 + 2 * 3 * 2 * 16 * 16 * 128
                                       + 2 * 3 * 2 * 16 * 16 * 128) // 32


def prefill_extra(dtype, B, torch, steps):
    """Time kda_prefill on the prefill workload (32 ragged prompts, ~34K
    tokens, H = 12): launches replayed from a HIP graph; the roofline is the
    fp32 matrix-core peak (the contractions run as fp32 MFMA)."""
    import numpy as np
    import kda_inputs
    inp = kda_inputs.prefill_batch(dtype)
    dev = torch.device("cuda", 0)
    pool = torch.from_numpy(inp.pool if dtype == "f32" else inp.pool.view(np.float16)).to(dev)
    t = {n: torch.from_numpy(getattr(inp, n)).to(dev) for n in ("q", "k", "v", "g", "b")}
    init = torch.from_numpy(inp.init_slot_ids).to(dev)
    cu = torch.from_numpy(inp.cu_seqlens).to(dev)
    out = torch.empty((inp.q.shape[0], 12, 128), device=dev)

    def step(_i):
        B.kda_prefill(pool, init, cu, t["q"], t["k"], t["v"], t["g"], t["b"], out, scale=inp.scale)
    tt = time_launches(step, steps, 3, torch)
    us = tt["ms_per_step"] * 1e3
    flops = inp.n_tokens * 12 * PREFILL_FLOP_PER_TOKEN_HEAD
    tfs = flops / (us * 1e-6) / 1e12
    chunked = inp.n_tokens * 12 * PREFILL_CHUNKED_FLOP_PER_TOKEN_HEAD
    res = {"workload": inp.name, "tokens": inp.n_tokens, "us_per_launch": round(us, 1),
           "chunked_form_TFLOP/s": round(chunked / (us * 1e-6) / 1e12, 2),
           "tokens_per_s": round(inp.n_tokens / (us * 1e-6)),
           "roofline": {"bound": "mfma", "achieved": round(tfs, 2), "peak": MFMA_F32_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tfs / MFMA_F32_PEAK_TFLOPS, 4),
                        "traffic": None, "algorithmic_flops_per_launch": flops},
           "hbm_GB/s": round(inp.io_bytes() / (us * 1e-6) / 1e9, 1)}
    del pool, t, out
    return res


def long_run_extra(B, torch, n_tokens=8192, chunk=1024):
    """The long single-slot run (H = 12, fresh seeded inputs per token, one
    launch per token), fp32 and fp16 pools.  Timing: the n_tokens launches
    replayed from one HIP graph, us per token.  Drift: the same run launched
    token by token, each token's stored state kept, against the fp64 oracle
    run from the same initial state (ROCm/ATOM PR #2130, Note on the default:
    long-context error is offline numerics), reported per chunk of 1024
    tokens as max abs and RMS state error; the comparison runs on the GPU
    in fp64 on the oracle's trajectory."""
    import numpy as np
    import kda_inputs
    from oracle import kda_oracle
    H = 12
    s0, q, k, v, g, b = kda_inputs.drift_tokens(n_tokens, seed=0, H=H)
    dev = torch.device("cuda", 0)
    d = {n: torch.from_numpy(a).to(dev) for n, a in zip("qkvgb", (q, k, v, g, b))}
    ids = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.empty((n_tokens, H, 128), device=dev)
    pools = {"f32": torch.from_numpy(s0.copy()).to(dev),
             "f16": torch.from_numpy(s0.astype(np.float16)).to(dev)}

    def step(pool, t):
        sl = slice(t, t + 1)
        B.kda_decode_step(pool, ids, d["q"][sl], d["k"][sl], d["v"][sl], d["g"][sl], d["b"][sl],
                          out[sl])

    res = {"tokens": n_tokens, "heads": H, "chunk": chunk}
    for dt, pool in pools.items():
        tt = time_launches(lambda i, pool=pool: step(pool, i % n_tokens), n_tokens, 64, torch)
        res["us_per_token_" + dt] = round(tt["launch_ms_mean"] * 1e3, 3)
    # drift: fresh pools, token by token, each token's state kept per chunk
    pools = {"f32": torch.from_numpy(s0.copy()).to(dev),
             "f16": torch.from_numpy(s0.astype(np.float16)).to(dev)}
    ref_state = s0[0].astype(np.float64)
    chain = np.arange(1, chunk + 1, dtype=np.int32)
    curves = {dt: [] for dt in pools}
    for c0 in range(0, n_tokens, chunk):
        sl = slice(c0, c0 + chunk)
        traj = {dt: torch.empty((chunk, H, 128, 128), dtype=p.dtype, device=dev) for dt, p in pools.items()}
        for t in range(c0, c0 + chunk):
            for dt, p in pools.items():
                step(p, t)
                traj[dt][t - c0].copy_(p[0])
        p64 = np.empty((chunk + 1, H, 128, 128), dtype=np.float64)
        p64[1] = ref_state
        kda_oracle.step_f64(p64, chain, q[sl], k[sl], v[sl], g[sl], b[sl], n_rows=chunk)
        ref_state = p64[-1].copy()
        ref = torch.from_numpy(p64[1:]).to(dev)
        del p64
        for dt in pools:
            diff = traj[dt].double() - ref
            curves[dt].append({"tokens": [c0, c0 + chunk],
                               "max_abs": float(diff.abs().max()),
                               "rms": float(diff.square().mean().sqrt())})
            del diff
        del ref, traj
        torch.cuda.empty_cache()
    for dt in pools:
        res["drift_vs_fp64_" + dt] = curves[dt]
        res["max_abs_" + dt] = max(c["max_abs"] for c in curves[dt])
    del pools, d, out
    torch.cuda.empty_cache()
    return res


def layers69(dtype, B, torch, steps, warmup, n_layers=69):
    """Time 69 back-to-back launches (one per layer: its own pool of 64
    slots and its own row inputs, one token each) as one decode step."""
    import kda_inputs
    H, n = 12, 64
    tdt = torch.float32 if dtype == "f32" else torch.float16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    pools = []
    for _ in range(n_layers):
        p = torch.randn((n, H, 128, 128), generator=gen, device="cuda", dtype=torch.float32)
        pools.append((p * 0.05).to(tdt))
        del p
    inp = kda_inputs.make_inputs("row inputs", n, n, 1, "f32", H=1, seed=0)  # only for ids
    ids = torch.from_numpy(inp.slot_ids).cuda()
    # every layer its own row inputs and outputs, as in a model (no layer
    # reads another's q, k, v, g, b from cache)
    rows = []
    for _ in range(n_layers):
        rows.append((torch.randn((n, H, 128), generator=gen, device="cuda"),
                     torch.randn((n, H, 128), generator=gen, device="cuda"),
                     torch.randn((n, H, 128), generator=gen, device="cuda"),
                     -torch.nn.functional.softplus(torch.randn((n, H, 128), generator=gen, device="cuda")),
                     torch.randn((n, H), generator=gen, device="cuda"),
                     torch.empty((n, H, 128), device="cuda")))

    def one_step(_i):
        for p, (q, k, v, g, b, out) in zip(pools, rows):
            B.kda_decode_step(p, ids, q, k, v, g, b, out)
    tt = time_launches(one_step, steps, warmup, torch)
    elem = 4 if dtype == "f32" else 2
    state = n_layers * n * H * 128 * 128 * elem * 2
    io = n_layers * n * H * (3 * 128 + 2 * 128 + 1) * 4
    res = {"us_per_step": round(tt["ms_per_step"] * 1e3, 1),
           "state_GB/s": round(state / (tt["ms_per_step"] * 1e-3) / 1e9, 1),
           "algorithmic_bytes": state + io,
           "frac_of_peak": round((state + io) / (tt["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del pools, rows
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
