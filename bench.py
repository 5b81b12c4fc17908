"""Benchmark of the quantized paged KV-cache hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = one pass of every operation of the path, each over its full
synthetic workload, inputs resident in HBM:

  1. nvfp4_ds_mla write      524288 tokens into 8192 x 64 x 352 B (pre-fill)
  2. fp8_ds_mla write        1048576 tokens into 16384 x 64 x 656 B (pre-fill)
  3. nvfp4_ds_mla gather     16 requests, L ~ U[1024, 32768], from seq_starts
  4. per-head NVFP4 write    8192 tokens x 8 heads x 128 (1% padding)
  5. fp8_ds_mla gather       32 requests, L ~ U[512, 16384], from seq_starts
  6. per-head NVFP4 gather   every written token back to bf16 K and V

(writes and the gathers over their caches are interleaved so that a gather
does not find its freshly written cache in the 256 MB last-level cache).

Prints ONE JSON line.  `value` is the metric: the algorithmic bytes of the
NVFP4 DS-MLA write (op 1) and gather-upconvert (op 3) over their kernel time,
both kernels timed live inside the timed region by HIP events bound to their
own begin and end (gcache_time_next_launch: no enqueue gap, so the figures
agree with rocprofv3's kernel durations); `roofline` is the gather's,
`roofline_write` the write's.  Also: the whole step's throughput (all six
ops' bytes / wall time per step), per-kernel durations of every op from a
separate pass of K steps, every op against the HBM roofline, and the CPU
oracle's throughput on a bounded sample of the same workloads.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
NV, F8 = 352, 656
PAIR = ("nvfp4_ds_mla_write", "nvfp4_ds_mla_gather")   # the metric's two kernels


class KernelTimer:
    """Kernel-bound HIP events: arm(i) makes the library's next launch bind a
    start/stop event pair of slot i to that kernel's own begin and end
    (gcache_time_next_launch, hipExtLaunchKernel), so ms(i) is the kernel's
    duration without the enqueue gap that events recorded around a call add
    (a few microseconds per pair on this machine)."""
    _hip = None

    def __init__(self, gc):
        import ctypes
        self.gc = gc
        self.ev = {}
        if KernelTimer._hip is None:
            # the HIP runtime torch and libgcache.so already share (never a second copy)
            hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_NOW)
            hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            hip.hipEventCreate.restype = hip.hipEventElapsedTime.restype = hip.hipEventDestroy.restype = ctypes.c_int
            KernelTimer._hip = hip

    def _pair(self, i):
        import ctypes
        if i not in self.ev:
            pair = []
            for _ in range(2):
                e = ctypes.c_void_p()
                rc = KernelTimer._hip.hipEventCreate(ctypes.byref(e))
                if rc != 0:
                    raise RuntimeError(f"hipEventCreate failed ({rc})")
                pair.append(e.value)
            self.ev[i] = tuple(pair)
        return self.ev[i]

    def arm(self, i):
        self.gc.time_next_launch(*self._pair(i))

    def close(self):
        """Destroy the events (after their last read)."""
        for pair in self.ev.values():
            for e in pair:
                KernelTimer._hip.hipEventDestroy(e)
        self.ev = {}

    def ms(self, i):
        import ctypes
        t = ctypes.c_float()
        a, b = self.ev[i]
        rc = KernelTimer._hip.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(t.value)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # ~60 ms of back-to-back steps: after an idle gap the first tens of
    # milliseconds of work run measurably slower (clocks ramping back up).
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=40.0,
                    help="approximate CPU seconds for the oracle baseline sample")
    ap.add_argument("--cold", action="store_true",
                    help="also time every kernel once per run after evicting the caches")
    ap.add_argument("--only", default=None, help="comma list of op names to run (profiling aid)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the extras measured after the timed step (BF16 comparator, chunked "
                         "context, sparse index conversion)")
    ap.add_argument("--extras-only", action="store_true",
                    help="profiling aid: fill the nvfp4 cache once, run only the extras, print them")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain elementwise kernel reading and writing MIB MiB, three "
                         "times, outside the timed region, so HBM counters can be scaled against "
                         "known bytes")
    ap.add_argument("--traffic-from", nargs=2, default=None, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="host only: turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then "
                         "WRITE_SIZE, each with --copy-calibration) into profiles/traffic.json")
    ap.add_argument("--stats-from", default=None, metavar="PROF_DIR",
                    help="host only: turn a rocprofv3 --kernel-trace --stats run of this script "
                         "(--steps 20 --warmup 3) into profiles/prefill_pass_all_kernels_stats.md")
    ap.add_argument("--bench-json", default=None, metavar="FILE",
                    help="with --stats-from: a bench.py output line of the same build, tabulated beside")
    ap.add_argument("--stats-extras", action="store_true",
                    help="with --stats-from: the run was --extras-only; write profiles/extras_kernels_stats.md")
    ap.add_argument("--decode-write-only", action="store_true",
                    help="profiling aid: run only the decode-batch writes (4096 tokens at random slots, both "
                         "DS-MLA formats), --steps times each, then the --copy-calibration kernel; print their "
                         "device times")
    ap.add_argument("--decode-traffic-from", nargs=2, default=None, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="host only: turn two rocprofv3 --pmc runs of --decode-write-only (FETCH_SIZE, then "
                         "WRITE_SIZE, each with --copy-calibration) into profiles/decode_write_hbm_traffic_pmc.md")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# Workloads and their algorithmic bytes
# ---------------------------------------------------------------------------
def build_workloads():
    import synth
    w3 = synth.nvfp4_prefill_write()
    g3 = synth.nvfp4_prefill_gather()
    w4 = synth.fp8_prefill_write()
    g4 = synth.fp8_prefill_gather()
    w5, g5 = synth.perhead_write_gather()
    return w3, g3, w4, g4, w5, g5


def ds_write_bytes(w, entry):
    valid = int((w.slot_mapping >= 0).sum())
    return valid * (512 * 2 + 64 * 2 + entry) + w.num_tokens * 8


def ds_gather_bytes(g, entry):
    return g.total_tokens * (entry + 576 * 2)


def kv_write_bytes(w):
    T, H, hs = w.key.shape
    valid = int((w.slot_mapping >= 0).sum())
    return valid * 2 * H * (hs * 2 + hs // 2 + hs // 16) + T * 8


def kv_gather_bytes(g, H, hs):
    return g.total_tokens * 2 * H * (hs * 2 + hs // 2 + hs // 16)


# ---------------------------------------------------------------------------
def main():
    args = parse()
    if args.traffic_from:
        write_traffic(*args.traffic_from)
        return
    if args.stats_from:
        write_stats(args.stats_from, args.bench_json, args.stats_extras)
        return
    if args.decode_traffic_from:
        write_decode_traffic(*args.decode_traffic_from)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(every op is token-parallel with no exchange between tokens, so one GPU's share at its real "
              "shape is what it times).", file=sys.stderr)
        sys.exit(2)
    import torch
    import gather_concat_cache_amd as gc

    def dev_bf16(a):          # bf16 bits (uint16) -> device bfloat16, bit for bit
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    def dev_arr(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    torch.cuda.init()
    if args.decode_write_only:
        decode_write_only(torch, gc, args)
        return
    dname = torch.cuda.get_device_name(0)
    t0 = time.time()
    w3, g3, w4, g4, w5, g5 = build_workloads()
    gen_s = time.time() - t0

    H, hs = w5.key.shape[1], w5.key.shape[2]
    fd = hs // 2 + hs // 16
    # ---- device-resident inputs and outputs
    d = {}
    d["kv3"], d["pe3"], d["sl3"] = dev_bf16(w3.kv_c), dev_bf16(w3.k_pe), dev_arr(w3.slot_mapping)
    d["cache3"] = torch.zeros((w3.num_blocks, w3.block_size, NV), dtype=torch.uint8, device="cuda")
    d["bt3"], d["ws3"], d["ss3"] = dev_arr(g3.block_table), dev_arr(g3.workspace_starts), dev_arr(g3.seq_starts)
    d["dst3"] = torch.empty((g3.total_tokens, 576), dtype=torch.bfloat16, device="cuda")
    d["kv4"], d["pe4"], d["sl4"] = dev_bf16(w4.kv_c), dev_bf16(w4.k_pe), dev_arr(w4.slot_mapping)
    d["cache4"] = torch.zeros((w4.num_blocks, w4.block_size, F8), dtype=torch.uint8, device="cuda")
    d["bt4"], d["ws4"], d["ss4"] = dev_arr(g4.block_table), dev_arr(g4.workspace_starts), dev_arr(g4.seq_starts)
    d["dst4"] = torch.empty((g4.total_tokens, 576), dtype=torch.bfloat16, device="cuda")
    d["k5"], d["v5"], d["sl5"] = dev_bf16(w5.key), dev_bf16(w5.value), dev_arr(w5.slot_mapping)
    d["cache5"] = torch.zeros((w5.num_blocks, 2, w5.block_size, H, fd), dtype=torch.uint8, device="cuda")
    d["ks5"] = torch.tensor([w5.k_scale], dtype=torch.float32, device="cuda")
    d["vs5"] = torch.tensor([w5.v_scale], dtype=torch.float32, device="cuda")
    d["bt5"], d["ws5"], d["ss5"] = dev_arr(g5.block_table), dev_arr(g5.workspace_starts), dev_arr(g5.seq_starts)
    d["ko5"] = torch.empty((g5.total_tokens, H, hs), dtype=torch.bfloat16, device="cuda")
    d["vo5"] = torch.empty((g5.total_tokens, H, hs), dtype=torch.bfloat16, device="cuda")

    ops = [
        ("nvfp4_ds_mla_write", ds_write_bytes(w3, NV), w3.num_tokens,
         lambda: gc.cache_write_nvfp4_ds_mla(d["kv3"], d["pe3"], d["cache3"], d["sl3"])),
        ("fp8_ds_mla_write", ds_write_bytes(w4, F8), w4.num_tokens,
         lambda: gc.cache_write_fp8_ds_mla(d["kv4"], d["pe4"], d["cache4"], d["sl4"])),
        ("nvfp4_ds_mla_gather", ds_gather_bytes(g3, NV), g3.total_tokens,
         lambda: gc.cache_gather_upconvert_nvfp4_ds_mla(d["cache3"], d["dst3"], d["bt3"], d["ws3"], d["ss3"])),
        ("nvfp4_kv_write", kv_write_bytes(w5), w5.slot_mapping.shape[0],
         lambda: gc.reshape_and_cache_nvfp4(d["k5"], d["v5"], d["cache5"], d["sl5"], d["ks5"], d["vs5"])),
        ("fp8_ds_mla_gather", ds_gather_bytes(g4, F8), g4.total_tokens,
         lambda: gc.cache_gather_upconvert_fp8_ds_mla(d["cache4"], d["dst4"], d["bt4"], d["ws4"], d["ss4"])),
        ("nvfp4_kv_gather", kv_gather_bytes(g5, H, hs), g5.total_tokens,
         lambda: gc.gather_upconvert_nvfp4_kv(d["cache5"], d["ko5"], d["vo5"], d["bt5"], d["ws5"], d["ks5"],
                                              d["vs5"], seq_starts=d["ss5"])),
    ]
    if args.extras_only:
        ops[0][3]()                                  # the nvfp4 pre-fill the extras read
        torch.cuda.synchronize()
        print(json.dumps({"extras": measure_extras(torch, gc, g3, args.steps, dev_arr, d["cache3"],
                                                   (w5, g5, d))}), flush=True)
        return
    if args.only:
        keep = set(args.only.split(","))
        ops = [o for o in ops if o[0] in keep]
    step_bytes = sum(o[1] for o in ops)

    pair = [i for i, o in enumerate(ops) if o[0] in PAIR]

    def step(timer=None, timed=()):
        """One pass of the ops; the kernels of the ops in `timed` carry
        kernel-bound HIP events of `timer` (gcache_time_next_launch)."""
        for i, (_, _, _, fn) in enumerate(ops):
            if i in timed:
                timer.arm(i)
            fn()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- per-kernel pass (not the timed region): K steps with every kernel's
    # own begin and end bound to HIP events on its launch stream
    kern = {i: [] for i in range(len(ops))}
    kt = KernelTimer(gc)
    for _ in range(args.steps):
        step(kt, timed=range(len(ops)))
        torch.cuda.synchronize()
        for i in range(len(ops)):
            kern[i].append(kt.ms(i))
    kern_ms = {ops[i][0]: float(np.mean(v)) for i, v in kern.items()}

    # ---- timed region: exactly K steps of the whole pass; the two NVFP4
    # DS-MLA kernels (the metric's write and gather) carry kernel-bound HIP
    # events, read after the region
    live = {i: [] for i in pair}
    timers = [KernelTimer(gc) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        step(timers[k], timed=pair)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    for k in range(args.steps):
        for i in pair:
            live[i].append(timers[k].ms(i))
    ms_per_step = wall * 1e3 / args.steps
    live_ms = {ops[i][0]: float(np.mean(v)) for i, v in live.items()}
    for t in timers + [kt]:
        t.close()

    kernels = {}
    for name, nbytes, units, _ in ops:
        ms = kern_ms[name]
        kernels[name] = {"ms": round(ms, 5), "bytes": nbytes, "units": units,
                         "units_per_s": round(units / (ms * 1e-3), 1),
                         "GB_per_s": round(nbytes / (ms * 1e6), 1),
                         "frac_of_hbm_peak": round(nbytes / (ms * 1e6) / HBM_PEAK_GBS, 4)}

    extras = None if args.no_extras else measure_extras(torch, gc, g3, args.steps, dev_arr, d["cache3"],
                                                        (w5, g5, d))
    if extras is not None:
        mix = {"nvfp4_ds_mla_write": (w3.num_tokens, 1152, NV), "fp8_ds_mla_write": (w4.num_tokens, 1152, F8),
               "nvfp4_ds_mla_gather": (g3.total_tokens, NV, 1152), "fp8_ds_mla_gather": (g4.total_tokens, F8, 1152)}
        extras["same_mix_ceilings"] = measure_ceilings(torch, [o for o in ops if o[0] in mix], mix)
        extras["empty_grid_floor_us"] = measure_launch_floor(torch, gc)
        extras["gather_streaming_rate"] = measure_gather_streaming(torch, gc, [
            ("nvfp4_ds_mla_gather", g3.total_tokens, NV,
             lambda n: gc.cache_gather_upconvert_nvfp4_ds_mla(d["cache3"], d["dst3"][:n], d["bt3"], d["ws3"],
                                                             d["ss3"])),
            ("fp8_ds_mla_gather", g4.total_tokens, F8,
             lambda n: gc.cache_gather_upconvert_fp8_ds_mla(d["cache4"], d["dst4"][:n], d["bt4"], d["ws4"],
                                                           d["ss4"]))])

    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)

    cold = None
    if args.cold:
        cold = measure_cold(torch, ops)

    # every op against the same HBM roofline (per-kernel pass durations), with
    # the measured HBM bytes per launch where the counters match this build
    roofline_by_op = {name: {"bound": "hbm", "achieved": round(nbytes / (kern_ms[name] * 1e6), 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(nbytes / (kern_ms[name] * 1e6) / HBM_PEAK_GBS, 4),
                             "algorithmic_bytes": nbytes, "traffic": traffic_for(name)}
                      for name, nbytes, _, _ in ops}

    def live_roofline(name):
        nbytes = next(o[1] for o in ops if o[0] == name)
        achieved = nbytes / (live_ms[name] * 1e6)
        return {"kernel": name, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "ms": round(live_ms[name], 5),
                "algorithmic_bytes": nbytes, "traffic": traffic_for(name)}

    roofline = live_roofline("nvfp4_ds_mla_gather")
    roofline_write = live_roofline("nvfp4_ds_mla_write")

    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_budget_s, w3, g3, w4, g4, w5, g5)

    pair_bytes = sum(ops[i][1] for i in pair)
    pair_ms = sum(live_ms[ops[i][0]] for i in pair)
    value = pair_bytes / (pair_ms * 1e6)
    step_value = step_bytes / (ms_per_step * 1e6)
    out = {
        "metric": "effective HBM GB/s (% of peak) for NVFP4 DS-MLA cache write and gather-upconvert",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16->e2m1/e4m3 (u8) and back", "data": "synthetic (seeded, see synth/)",
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "config": {"workload": f"nvfp4_ds_mla pre-fill write ({w3.num_tokens} tokens into {w3.num_blocks} x "
                               f"{w3.block_size} x 352 B) + prefill gather-upconvert ({len(g3.workspace_starts)} "
                               f"requests from seq_starts, {g3.total_tokens} rows), each timed by its own kernel "
                               "events inside a pass of all six ops of the path",
                   "value_bytes": pair_bytes, "value_ms": round(pair_ms, 5),
                   "step": "nvfp4_ds_mla write 524288 tok + gather 16 req; fp8_ds_mla write 1048576 tok + "
                           f"gather 32 req ({g4.total_tokens} rows); per-head nvfp4 write 8192 tok x 8 heads x "
                           f"128 + gather {g5.total_tokens} rows",
                   "step_bytes": step_bytes, "ops": [o[0] for o in ops], "device": dname},
        "step_throughput": {"value": round(step_value, 1), "unit": "GB/s",
                            "frac_of_hbm_peak": round(step_value / HBM_PEAK_GBS, 4),
                            "what": "algorithmic bytes of all six ops / wall time per step over the timed region"},
        "kernels": kernels,
        "roofline": roofline,
        "roofline_write": roofline_write,
        "roofline_by_op": roofline_by_op,
        "cpu_baseline": cpu,
        "extras": extras,
        "input_generation_s": round(gen_s, 2),
    }
    if cold is not None:
        out["kernels_cold"] = cold
    print(json.dumps(out), flush=True)


def device_ms(torch, fn, steps, spin_cycles=300_000):
    """Mean device time of fn() over `steps` launches.  Each launch is queued
    behind a short spin kernel, so the HIP events around it (on the launch
    stream) see only GPU work: the host's per-call overhead cannot leave the
    GPU idle between the first event and the kernel."""
    fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        torch.cuda._sleep(spin_cycles)
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def kernel_ms(torch, gc, fn, steps, cold=False):
    """Mean duration of the one library kernel that fn() launches, from HIP
    events bound to that kernel's own begin and end (gcache_time_next_launch),
    so no enqueue gap is counted (the figure rocprofv3 reports).  cold: each
    launch follows a 2 GiB write that evicts L2 and the 256 MB MALL."""
    fn()
    flush = torch.empty(2 << 30, dtype=torch.uint8, device="cuda") if cold else None
    timer = KernelTimer(gc)
    for k in range(steps):
        if cold:
            flush.zero_()
        timer.arm(k)
        fn()
    torch.cuda.synchronize()
    ms = float(np.mean([timer.ms(k) for k in range(steps)]))
    timer.close()
    del flush
    return ms


def _extra(ms, nbytes, units, workload, **more):
    return {"ms": round(ms, 5), "bytes": nbytes, "units": units, **more,
            "GB_per_s": round(nbytes / (ms * 1e6), 1),
            "frac_of_hbm_peak": round(nbytes / (ms * 1e6) / HBM_PEAK_GBS, 4), "workload": workload}


def measure_extras(torch, gc, g3, steps, dev_arr, cache3, perhead):
    """Outside the timed step, kernel durations (kernel_ms: events bound to
    the kernel's own begin and end) of:
    (1) the BF16 comparator gather (same walk, 1152-byte bf16 entries copied)
        over the nvfp4 prefill gather's requests and cache geometry -- what a
        walk-driven gather of full rows reaches on this device;
    (2) the chunked-context driver gathering every request's whole nvfp4
        context (the prefill requests' lengths, from position 0) through a
        65536-row workspace (several launches and a metadata upload, so
        device time between events around the pass, see device_ms), and the
        same pass's wall time on an idle GPU;
    (3) the sparse index conversion, 4096 rows x top-2048;
    (4) the per-head workload under the split layout and under reading B
        (interleaved [data | scale] rows);
    (5) the decode-batch nvfp4 write (4096 tokens, lognormal magnitudes with
        outliers, 2% padding) and the per-head pair, warm (back to back) and
        cold (each launch after a 2 GiB write that evicts L2 and the MALL).
        These launches move a few to a few tens of MB: launch and ramp, not
        HBM bandwidth, set their time."""
    import synth
    out = {}
    nb, bs = g3.num_blocks, g3.block_size
    cache = torch.from_numpy(synth.normal_bf16_rows(1013, 0, nb * bs, 576).view(np.int16)) \
        .view(torch.bfloat16).reshape(nb, bs, 576).cuda()
    dst = torch.empty((g3.total_tokens, 576), dtype=torch.bfloat16, device="cuda")
    bt, ws, ss = dev_arr(g3.block_table), dev_arr(g3.workspace_starts), dev_arr(g3.seq_starts)
    ms = kernel_ms(torch, gc, lambda: gc.cache_gather_bf16(cache, dst, bt, ws, ss), steps)
    out["bf16_gather_comparator"] = _extra(
        ms, g3.total_tokens * 2 * 1152, g3.total_tokens,
        f"{g3.total_tokens} rows of the nvfp4 prefill gather over a bf16 cache {nb} x {bs} x 1152 B "
        "(1152 B read + 1152 B written per row)", rows_per_s=round(g3.total_tokens / (ms * 1e-3), 1))
    del cache, dst

    lens = np.asarray(g3.lengths, np.int32)
    ws_rows = 65536
    workspace = torch.empty((ws_rows, 576), dtype=torch.bfloat16, device="cuda")
    _, plan = gc.context_chunks(lens, ws_rows, bs)
    rows = int(sum(t for _, _, t in plan))

    def chunked():
        for _ in gc.gather_context_chunked(gc.cache_gather_upconvert_nvfp4_ds_mla, cache3, workspace, bt, lens):
            pass
    busy = device_ms(torch, chunked, steps, spin_cycles=2_000_000)
    wall_t = []
    for _ in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        chunked()
        b.record()
        torch.cuda.synchronize()
        wall_t.append(a.elapsed_time(b))
    wall = float(np.mean(wall_t))
    nbytes = rows * (NV + 1152)
    out["chunked_context_nvfp4_gather"] = _extra(
        busy, nbytes, rows,
        f"whole contexts of the {lens.shape[0]} prefill requests ({rows} positions) gathered in {len(plan)} "
        f"chunks through a {ws_rows}-row workspace; ms = device time of the pass (metadata upload included), "
        "wall_ms = the pass on an idle GPU, host call overhead included",
        chunks=len(plan), wall_ms=round(wall, 5), wall_GB_per_s=round(nbytes / (wall * 1e6), 1))
    del workspace

    req, idx, sbt, sbs, snb = synth.sparse_index_case()
    req_d, idx_d, sbt_d = dev_arr(req), dev_arr(idx), dev_arr(sbt)
    sout = torch.empty_like(idx_d)
    ms = kernel_ms(torch, gc, lambda: gc.convert_req_index_to_global_index(req_d, idx_d, sbt_d, sbs, snb, out=sout),
                   steps)
    out["sparse_index_conversion"] = _extra(
        ms, idx.size * 8 + req.size * 4, int(idx.size),
        f"{idx.shape[0]} token rows x top-{idx.shape[1]} positions over {sbt.shape[0]} requests "
        "(4 B read + 4 B written per index; block-table reads not counted)")

    w5, g5, d = perhead
    H, hs = w5.key.shape[1], w5.key.shape[2]
    fd = hs // 2 + hs // 16
    bs5 = w5.block_size
    layouts = {
        "split_rows": gc.nvfp4_kv_split_layout(bs5, H, hs),
        "interleaved_rows": gc.NvFp4KvLayout(
            data_offset=0, data_token_stride=H * fd, data_head_stride=fd, scale_offset=hs // 2,
            scale_token_stride=H * fd, scale_head_stride=fd, side_stride=bs5 * H * fd,
            block_stride=2 * bs5 * H * fd)}
    cache5 = torch.zeros((w5.num_blocks, 2, bs5, H, fd), dtype=torch.uint8, device="cuda")
    gp5 = synth.perhead_prefill_gather()
    ko_p = torch.empty((gp5.total_tokens, H, hs), dtype=torch.bfloat16, device="cuda")
    vo_p = torch.empty_like(ko_p)
    bt_p, ws_p, ss_p = dev_arr(gp5.block_table), dev_arr(gp5.workspace_starts), dev_arr(gp5.seq_starts)
    for lname, L in layouts.items():
        what = ("the default split layout" if lname == "split_rows" else
                f"each (token, head) cache row laid out as [{hs // 2} data | {hs // 16} scale] bytes")
        ms = kernel_ms(torch, gc, lambda: gc.reshape_and_cache_nvfp4(d["k5"], d["v5"], cache5, d["sl5"], d["ks5"],
                                                                     d["vs5"], layout=L), steps)
        out[f"perhead_write_{lname}"] = _extra(ms, kv_write_bytes(w5), w5.slot_mapping.shape[0],
                                               f"the per-head write workload, {what}")
        ms = kernel_ms(torch, gc, lambda: gc.gather_upconvert_nvfp4_kv(cache5, d["ko5"], d["vo5"], d["bt5"], d["ws5"],
                                                                       d["ks5"], d["vs5"], seq_starts=d["ss5"],
                                                                       layout=L), steps)
        out[f"perhead_gather_{lname}"] = _extra(ms, kv_gather_bytes(g5, H, hs), g5.total_tokens,
                                                f"the per-head gather workload, {what}")
        ms = kernel_ms(torch, gc, lambda: gc.gather_upconvert_nvfp4_kv(cache5, ko_p, vo_p, bt_p, ws_p, d["ks5"],
                                                                       d["vs5"], seq_starts=ss_p, layout=L), steps)
        out[f"perhead_gather_prefill_walk_{lname}"] = _extra(
            ms, kv_gather_bytes(gp5, H, hs), gp5.total_tokens,
            f"per-head gather on a prefill walk: {len(gp5.workspace_starts)} requests, L ~ U[512, 6144] from "
            f"seq_starts ~ U[0, L/2], {gp5.total_tokens} rows over the per-head cache's {w5.num_blocks} blocks, {what}")
    del cache5

    w2 = synth.decode_batch_write()
    kv2, pe2 = (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
                for a in (w2.kv_c, w2.k_pe))
    sl2 = dev_arr(w2.slot_mapping)
    cache2 = torch.zeros((w2.num_blocks, w2.block_size, NV), dtype=torch.uint8, device="cuda")
    small = [("decode_batch_nvfp4_write", ds_write_bytes(w2, NV), w2.num_tokens,
              lambda: gc.cache_write_nvfp4_ds_mla(kv2, pe2, cache2, sl2),
              f"{w2.num_tokens} decode tokens (lognormal magnitudes, 1% x50 outliers, "
              f"{int((w2.slot_mapping < 0).sum())} padding slots) into {w2.num_blocks} x {w2.block_size} x 352 B"),
             ("perhead_write_cold_warm", kv_write_bytes(w5), w5.slot_mapping.shape[0],
              lambda: gc.reshape_and_cache_nvfp4(d["k5"], d["v5"], d["cache5"], d["sl5"], d["ks5"], d["vs5"]),
              "the per-head write workload, default split layout"),
             ("perhead_gather_cold_warm", kv_gather_bytes(g5, H, hs), g5.total_tokens,
              lambda: gc.gather_upconvert_nvfp4_kv(d["cache5"], d["ko5"], d["vo5"], d["bt5"], d["ws5"], d["ks5"],
                                                   d["vs5"], seq_starts=d["ss5"]),
              "the per-head gather workload, default split layout")]
    for name, nbytes, units, fn, what in small:
        warm = kernel_ms(torch, gc, fn, steps)
        cold = kernel_ms(torch, gc, fn, steps, cold=True)
        out[name] = _extra(warm, nbytes, units, what + "; ms = warm (back to back), cold_ms = after evicting "
                           "L2 and the MALL", cold_ms=round(cold, 5), cold_GB_per_s=round(nbytes / (cold * 1e6), 1))
    del cache2
    return out


def measure_launch_floor(torch, gc, reps=21):
    """Median duration between kernel-bound events of launches whose waves
    exit without touching memory (gcache_bench_empty_grid in
    libgcache_bench.so), for grids of 1 to 262144 workgroups: the cost any
    kernel of that grid pays before and after its work.  The cache kernels'
    grids: nvfp4 write 262144 x 64 lanes, fp8 write 262144 x 128, DS-MLA
    gathers 10111 / 13705 x 256, per-head ops about 2048 x 256."""
    import ctypes
    from gather_concat_cache_amd import build
    lib = ctypes.CDLL(build.BENCH_LIB)
    fn = lib.gcache_bench_empty_grid
    fn.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    stream = torch.cuda.current_stream().cuda_stream
    timer = KernelTimer(gc)
    out = {}
    for threads in (64, 128, 256):
        for groups in (1, 2048, 10111, 40444, 262144):
            t = []
            for k in range(reps):
                a, b = timer._pair(k)
                rc = fn(groups, threads, a, b, stream)
                if rc != 0:
                    raise RuntimeError(f"gcache_bench_empty_grid returned {rc}")
            torch.cuda.synchronize()
            t = [timer.ms(k) for k in range(reps)]
            out[f"{groups}x{threads}"] = round(float(np.median(t)) * 1e3, 2)
    timer.close()
    return out


def measure_ceilings(torch, ops, mix, reps=21):
    """For each DS-MLA op: the same-mix row copy of libgcache_bench.so (rows
    of the op's read bytes in, its write bytes out, contiguous, staged
    through LDS in groups of rows, no walk and no conversion) in several
    workgroup shapes, and the op itself, all cold (each launch after a 2 GiB
    write that evicts L2 and the MALL).  The fastest shape is the ceiling:
    what a plain stream with the op's byte pattern reaches on this device."""
    import ctypes
    from gather_concat_cache_amd import build
    lib = ctypes.CDLL(build.BENCH_LIB)
    fn = lib.gcache_bench_copy_mix
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    shapes = [(16, 256), (8, 256), (4, 128), (2, 64)]     # (rows per workgroup, threads)
    op_cold = measure_cold(torch, ops, reps)
    out = {}
    for name, nbytes, _, _ in ops:
        rows, rb, wb = mix[name]
        src = torch.empty(rows * rb, dtype=torch.uint8, device="cuda").fill_(0x3C)
        dst = torch.empty(rows * wb, dtype=torch.uint8, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        cbytes = rows * (rb + wb)
        per_shape = {}
        for g, nt in shapes:
            def copy(g=g, nt=nt):
                rc = fn(src.data_ptr(), dst.data_ptr(), rows, rb, wb, g, nt, stream)
                if rc != 0:
                    raise RuntimeError(f"gcache_bench_copy_mix returned {rc}")
            per_shape[f"{g}x{nt}"] = measure_cold(torch, [(name, cbytes, rows, copy)], reps)[name]
        best = min(per_shape, key=lambda k: per_shape[k]["ms"])
        ceil = per_shape[best]
        op_gbs = op_cold[name]["GB_per_s"]
        out[name] = {"rows": rows, "read_bytes": rb, "write_bytes": wb, "ceiling_ms": ceil["ms"],
                     "ceiling_GB_per_s": ceil["GB_per_s"], "ceiling_shape": best,
                     "shapes_GB_per_s": {k: v["GB_per_s"] for k, v in per_shape.items()},
                     "op_cold_ms": op_cold[name]["ms"], "op_cold_GB_per_s": op_gbs,
                     "frac_of_ceiling": round(op_gbs / ceil["GB_per_s"], 4)}
        del src, dst
    return out


def measure_gather_streaming(torch, gc, cases, reps=21):
    """Each DS-MLA gather over all of its workspace rows and over the first
    half of them (the same requests, cut at half the rows), both cold.  The
    difference gives the rate at which the kernel streams once running
    (bytes of the second half / extra time) and the fixed cost of a launch
    (the full time less the full bytes at that rate; it includes the few
    microseconds a HIP event pair adds)."""
    out = {}
    for name, rows, entry, run in cases:
        half = rows // 2
        per_row = entry + 1152
        t = measure_cold(torch, [("full", rows * per_row, rows, lambda: run(rows)),
                                 ("half", half * per_row, half, lambda: run(half))], reps)
        extra_ms = t["full"]["ms"] - t["half"]["ms"]
        rate = (rows - half) * per_row / (extra_ms * 1e6) if extra_ms > 0 else float("nan")
        out[name] = {"rows": rows, "ms_full": t["full"]["ms"], "ms_half": t["half"]["ms"],
                     "streaming_GB_per_s": round(rate, 1), "streaming_frac_of_hbm_peak": round(rate / HBM_PEAK_GBS, 4),
                     "fixed_ms": round(t["full"]["ms"] - rows * per_row / (rate * 1e6), 5)}
    return out


def measure_cold(torch, ops, reps=21):
    """Each kernel alone after writing a 2 GiB buffer (evicts L2 and the
    256 MB MALL); median over reps."""
    flush = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    res = {}
    for name, nbytes, _, fn in ops:
        t = []
        for _ in range(reps):
            flush.zero_()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            t.append(a.elapsed_time(b))
        ms = float(np.median(t))
        res[name] = {"ms": round(ms, 5), "GB_per_s": round(nbytes / (ms * 1e6), 1)}
    del flush
    return res


def traffic_for(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, when
    it was taken on the current kernel source (else null)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            t = json.load(f)
        from gather_concat_cache_amd.build import source_digest
        if t.get("source_digest") != source_digest():
            return None
        return t["kernels"].get(kernel, {}).get("hbm_bytes_per_launch")
    except Exception:
        return None


# kernel symbol (prefix up to the parameter list, or up to the template
# argument list of the write kernels) -> op name used above
KERNEL_OPS = {
    "void gcache::k_write_nvfp4_ds_mla": "nvfp4_ds_mla_write",
    "void gcache::k_write_fp8_ds_mla": "fp8_ds_mla_write",
    "void gcache::k_gather_ds_mla<true>": "nvfp4_ds_mla_gather",
    "void gcache::k_reshape_and_cache_nvfp4<true>": "nvfp4_kv_write",      # staged (split or row layouts)
    "void gcache::k_reshape_and_cache_nvfp4<false>": "nvfp4_kv_write",     # direct (other layouts)
    "void gcache::k_gather_ds_mla<false>": "fp8_ds_mla_gather",
    "void gcache::k_gather_nvfp4_kv<true>": "nvfp4_kv_gather",
    "void gcache::k_gather_nvfp4_kv<false>": "nvfp4_kv_gather",
}
CALIBRATION_KERNEL = "CUDAFunctorOnSelf_add"


def kernel_op(name):
    """Op name of a demangled kernel symbol, or None."""
    return next((op for k, op in KERNEL_OPS.items()
                 if name.startswith(k + "(") or (not k.endswith(">") and name.startswith(k + "<"))), None)


def write_traffic(fetch_dir, write_dir):
    """Scale the per-dispatch FETCH_SIZE and WRITE_SIZE counters (KiB) of each
    kernel by what the same counter reads for the calibration kernel, an
    elementwise add that reads and writes exactly --copy-calibration MiB each,
    and store the mean HBM bytes per launch with the current library digest."""
    import csv
    import glob
    from gather_concat_cache_amd.build import source_digest

    def per_kernel(d, counter):
        (path,) = glob.glob(os.path.join(d, "*counter_collection.csv"))
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = kernel_op(name)
            if key is None and CALIBRATION_KERNEL in name:
                key = "calibration"
            if key is not None:
                vals.setdefault(key, []).append(float(r["Counter_Value"]))
        return vals

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    cal_mib = 1024
    cal_kib = cal_mib * 1024.0
    f_scale = cal_kib / float(np.mean(fetch["calibration"]))
    w_scale = cal_kib / float(np.mean(write["calibration"]))
    w3, g3, w4, g4, w5, g5 = build_workloads()
    H, hs = w5.key.shape[1], w5.key.shape[2]
    algo = {"nvfp4_ds_mla_write": ds_write_bytes(w3, NV), "fp8_ds_mla_write": ds_write_bytes(w4, F8),
            "nvfp4_ds_mla_gather": ds_gather_bytes(g3, NV), "nvfp4_kv_write": kv_write_bytes(w5),
            "fp8_ds_mla_gather": ds_gather_bytes(g4, F8), "nvfp4_kv_gather": kv_gather_bytes(g5, H, hs)}
    out = {"source_digest": source_digest(), "calibration_mib": cal_mib,
           "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5), "kernels": {}}
    for op in KERNEL_OPS.values():
        fb = float(np.mean(fetch[op])) * 1024 * f_scale
        wb = float(np.mean(write[op])) * 1024 * w_scale
        out["kernels"][op] = {"dispatches": [len(fetch[op]), len(write[op])],
                              "fetch_kib_raw": round(float(np.mean(fetch[op])), 1),
                              "write_kib_raw": round(float(np.mean(write[op])), 1),
                              "hbm_bytes_per_launch": int(round(fb + wb)),
                              "algorithmic_bytes": algo[op],
                              "traffic_over_algorithmic": round((fb + wb) / algo[op], 4)}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    cal_f = ", ".join(f"{v:,.0f}" for v in fetch["calibration"])
    cal_w = ", ".join(f"{v:,.0f}" for v in write["calibration"])
    run = ("timeout -s KILL 120 rocprofv3 --pmc {c} --kernel-trace -f csv -d $R/{d} -o bench -- python3 "
           "$R/bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-extras --copy-calibration 1024")
    md = ["# HBM traffic per launch — all six kernels, prefill-context pass workload", "",
          "Two counter runs (one counter each), run from /tmp on an MI355X machine with the repository at $R, "
          "then the host-side summary:", "", "```",
          run.format(c="FETCH_SIZE", d=os.path.relpath(fetch_dir, ROOT)),
          run.format(c="WRITE_SIZE", d=os.path.relpath(write_dir, ROOT)),
          f"python3 bench.py --traffic-from {os.path.relpath(fetch_dir, ROOT)} "
          f"{os.path.relpath(write_dir, ROOT)}", "```", "",
          f"Kernel sources: library digest {out['source_digest']}. Calibration: torch's elementwise add "
          f"over {cal_mib} MiB (reads and writes {cal_kib:,.0f} KiB each); FETCH_SIZE read {cal_f} KiB "
          f"and WRITE_SIZE {cal_w} KiB per dispatch, so fetch counts are scaled by {out['fetch_scale']} "
          f"and write counts by {out['write_scale']}. Each kernel: mean over its dispatches "
          "(1 warm-up + 3 timed steps).", "",
          "| Kernel op | FETCH_SIZE (KiB, raw) | WRITE_SIZE (KiB, raw) | HBM bytes / launch (scaled) "
          "| Algorithmic bytes | Ratio |", "|---|---|---|---|---|---|"]
    for k, v in out["kernels"].items():
        md.append(f"| {k} | {v['fetch_kib_raw']:,} | {v['write_kib_raw']:,} | {v['hbm_bytes_per_launch']:,} "
                  f"| {v['algorithmic_bytes']:,} | {v['traffic_over_algorithmic']:.4f} |")
    md += ["", "Kernel symbols: " + ", ".join(f"{op} = `{k}`" for k, op in KERNEL_OPS.items()) + "."]
    with open(os.path.join(ROOT, "profiles", "all_kernels_hbm_traffic_pmc.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print(json.dumps(out, indent=1))


def write_stats(prof_dir, bench_json, extras=False):
    """Markdown summary of a rocprofv3 --stats run of this script, with the
    HIP-event figures of a bench.py line of the same build when given
    (extras=True: a run with --extras-only)."""
    import csv
    import glob
    from gather_concat_cache_amd.build import source_digest
    (path,) = glob.glob(os.path.join(prof_dir, "*kernel_stats.csv"))
    rows = list(csv.DictReader(open(path)))
    flags = "--extras-only" if extras else "--no-cpu-baseline --no-extras"
    cmd = ("rocprofv3 --kernel-trace --stats -f csv -d $R/" + os.path.relpath(prof_dir, ROOT) +
           f" -o bench -- python3 $R/bench.py --steps 20 --warmup 3 {flags}")
    title = ("the bench extras (BF16 comparator, chunked context, sparse index conversion, per-head layouts)" if extras
             else "all six kernels, prefill-context pass workload")
    what = ("20 timed repetitions of each extra after one nvfp4 pre-fill write. The chunked-context pass "
            "launches the nvfp4 gather once per chunk (8 chunks), so its calls share that kernel's name; "
            "the spin kernel holds the queue while the chunk launches are enqueued." if extras else
            "3 warm-up steps, 20 steps of the per-kernel event pass and 20 timed steps (43 calls per kernel). Workloads: nvfp4_ds_mla write 524288 tokens, "
            "fp8_ds_mla write 1048576 tokens, nvfp4 gather 161766 rows, fp8 gather 219273 rows, per-head "
            "write 8192 tokens x 8 heads x 128, per-head gather 8110 rows.")
    md = [f"# rocprofv3 kernel statistics — {title}", "",
          "Command (run from /tmp on an MI355X machine, repository at $R), then the host-side summary:", "",
          "```", cmd, f"python3 bench.py --stats-from {os.path.relpath(prof_dir, ROOT)}"
          + (" --stats-extras" if extras else "")
          + (f" --bench-json {os.path.relpath(bench_json, ROOT)}" if bench_json else ""), "```", "",
          f"{what} Library digest {source_digest()}.",
          "", "| Kernel | Calls | Average (ns) | Min (ns) | Max (ns) | % of GPU time |",
          "|---|---|---|---|---|---|"]
    for r in rows:
        n = r["Name"] if len(r["Name"]) <= 72 else r["Name"][:72] + "…"
        md.append(f"| `{n}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} "
                  f"| {float(r['Percentage']):.2f} |")
    if bench_json:
        b = json.load(open(bench_json))
        if extras:
            md += ["", "Same-build figures from an unprofiled `python bench.py --extras-only` run: kernel "
                   "durations from HIP events bound to each kernel's own begin and end (gcache_time_next_launch), "
                   "except the chunked-context pass (events around the whole pass of several launches):", "",
                   "| Extra | ms | GB/s | % of 8 TB/s |", "|---|---|---|---|"]
            for k, v in b["extras"].items():
                md.append(f"| {k} | {v['ms']:.5f} | {v['GB_per_s']:.0f} | {100 * v['frac_of_hbm_peak']:.1f} |")
        else:
            md += ["", "Same-build figures from an unprofiled `python bench.py` run (inside the profiled run "
                   "the same events read longer than rocprofv3's own durations), all from "
                   "HIP events bound to each kernel's own begin and end (gcache_time_next_launch), so they "
                   f"measure what rocprofv3 measures. Per-kernel pass of {b['steps']} steps:", "",
                   "| Kernel op | ms | GB/s | % of 8 TB/s |", "|---|---|---|---|"]
            for k, v in b["kernels"].items():
                md.append(f"| {k} | {v['ms']:.5f} | {v['GB_per_s']:.0f} | {100 * v['frac_of_hbm_peak']:.1f} |")
            md += ["", f"Inside the {b['steps']} timed steps: nvfp4_ds_mla write {b['roofline_write']['ms']:.5f} ms "
                   f"({100 * b['roofline_write']['frac']:.1f} %), gather {b['roofline']['ms']:.5f} ms "
                   f"({100 * b['roofline']['frac']:.1f} %); the metric's value (the pair's bytes over the pair's "
                   f"kernel time) {b['value']} GB/s, {100 * b['frac_of_hbm_peak']:.1f} % of 8 TB/s; whole six-op step "
                   f"{b['step_throughput']['value']} GB/s."]
    traces = glob.glob(os.path.join(prof_dir, "*kernel_trace.csv"))
    if not extras and traces:
        # the profiled command runs 3 warm-up steps, 20 per-kernel-pass steps and 20 timed steps
        trace = list(csv.DictReader(open(traces[0])))
        phases = []
        for op, prefix in (("nvfp4_ds_mla write", "void gcache::k_write_nvfp4_ds_mla"),
                           ("nvfp4_ds_mla gather", "void gcache::k_gather_ds_mla<true>")):
            ds = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in trace
                        if r["Kernel_Name"].startswith(prefix))
            if len(ds) == 43:
                us = [(e - st) / 1e3 for st, e in ds]
                phases.append(f"{op} {np.mean(us[:3]):.2f} / {np.mean(us[3:23]):.2f} / {np.mean(us[23:]):.2f} µs")
        if phases:
            md += ["", "rocprofv3's own durations of the metric's two kernels by phase of the profiled run "
                   "(its kernel trace; warm-up / per-kernel pass / timed steps): " + "; ".join(phases) + ". "
                   "The profiler times every dispatch; inside the timed steps bench.py binds events to these "
                   "two kernels only, and those durations read a few per cent longer than the profiler's "
                   "(a kernel after an unarmed neighbour carries part of that neighbour's tail)."]
    name = "extras_kernels_stats.md" if extras else "prefill_pass_all_kernels_stats.md"
    with open(os.path.join(ROOT, "profiles", name), "w") as f:
        f.write("\n".join(md) + "\n")


def copy_calibration(torch, mib):
    """A plain elementwise kernel that reads and writes exactly `mib` MiB
    each, three times (torch's copy_ of two device buffers goes to a DMA
    engine instead), so HBM counters can be scaled against known bytes."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(3):
        torch.add(src, 1, out=dst)
    torch.cuda.synchronize()
    del src, dst


def decode_write_only(torch, gc, args):
    """The decode-batch write workload alone (4096 tokens with lognormal
    magnitudes into 4096 random slots of a 1024 x 64 cache, 82 padding), in
    both DS-MLA formats: --steps launches each, then the calibration kernel.
    Random single-token slots leave entries that start inside 128-byte lines,
    so the counters show how much partial-line traffic the hardware adds."""
    import synth
    w2 = synth.decode_batch_write()
    kv = torch.from_numpy(np.ascontiguousarray(w2.kv_c).view(np.int16)).view(torch.bfloat16).cuda()
    pe = torch.from_numpy(np.ascontiguousarray(w2.k_pe).view(np.int16)).view(torch.bfloat16).cuda()
    sl = torch.from_numpy(np.ascontiguousarray(w2.slot_mapping)).cuda()
    out = {}
    for name, eb, fn in (("decode_batch_nvfp4_write", NV, gc.cache_write_nvfp4_ds_mla),
                         ("decode_batch_fp8_write", F8, gc.cache_write_fp8_ds_mla)):
        cache = torch.zeros((w2.num_blocks, w2.block_size, eb), dtype=torch.uint8, device="cuda")
        ms = kernel_ms(torch, gc, lambda: fn(kv, pe, cache, sl), max(1, args.steps))
        out[name] = _extra(ms, ds_write_bytes(w2, eb), w2.num_tokens,
                           f"{w2.num_tokens} decode tokens into {w2.num_blocks} x {w2.block_size} x {eb} B, "
                           f"{int((w2.slot_mapping < 0).sum())} padding slots")
        del cache
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
    print(json.dumps({"decode_writes": out}), flush=True)


def write_decode_traffic(fetch_dir, write_dir):
    """HBM bytes per launch of the decode-batch writes from two counter runs
    of --decode-write-only (scaled by the calibration kernel, as for the
    prefill pass) against their algorithmic bytes."""
    import csv
    import glob
    import synth
    from gather_concat_cache_amd.build import source_digest

    names = {"nvfp4_ds_mla_write": "decode_batch_nvfp4_write", "fp8_ds_mla_write": "decode_batch_fp8_write"}

    def per_kernel(d, counter):
        (path,) = glob.glob(os.path.join(d, "*counter_collection.csv"))
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = names.get(kernel_op(r["Kernel_Name"]))
            if key is None and CALIBRATION_KERNEL in r["Kernel_Name"]:
                key = "calibration"
            if key is not None:
                vals.setdefault(key, []).append(float(r["Counter_Value"]))
        return vals

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    cal_kib = 1024 * 1024.0
    f_scale = cal_kib / float(np.mean(fetch["calibration"]))
    w_scale = cal_kib / float(np.mean(write["calibration"]))
    w2 = synth.decode_batch_write()
    valid = int((w2.slot_mapping >= 0).sum())
    run = ("timeout -s KILL 120 rocprofv3 --pmc {c} --kernel-trace -f csv -d $R/{d} -o bench -- python3 "
           "$R/bench.py --decode-write-only --steps 20 --copy-calibration 1024")
    md = ["# HBM traffic per launch — decode-batch writes (4096 tokens at random slots)", "",
          "Two counter runs, run from /tmp on an MI355X machine with the repository at $R, then the host-side summary:",
          "", "```", run.format(c="FETCH_SIZE", d=os.path.relpath(fetch_dir, ROOT)),
          run.format(c="WRITE_SIZE", d=os.path.relpath(write_dir, ROOT)),
          f"python3 bench.py --decode-traffic-from {os.path.relpath(fetch_dir, ROOT)} "
          f"{os.path.relpath(write_dir, ROOT)}", "```", "",
          f"Kernel sources: library digest {source_digest()}. Workload: {w2.num_tokens} tokens ({valid} valid, "
          f"{w2.num_tokens - valid} padding) into {w2.num_blocks} x {w2.block_size} entries at slots drawn "
          "without replacement from all 65536, so most entries start inside a 128-byte line whose other "
          "bytes belong to entries this launch does not write. Counters are scaled as for the prefill pass "
          f"(fetch x{f_scale:.5f}, write x{w_scale:.5f}, from torch's elementwise add over 1 GiB in the same "
          "run); each kernel: mean over its dispatches (20 launches each, plus the first call).", "",
          "| Kernel op | Dispatches | FETCH_SIZE (KiB, raw) | WRITE_SIZE (KiB, raw) | Read bytes (scaled) "
          "| Algorithmic read | Written bytes (scaled) | Entry bytes | Write ratio |",
          "|---|---|---|---|---|---|---|---|---|"]
    for key, eb in (("decode_batch_nvfp4_write", NV), ("decode_batch_fp8_write", F8)):
        fr, wr = float(np.mean(fetch[key])), float(np.mean(write[key]))
        rb, wb = fr * 1024 * f_scale, wr * 1024 * w_scale
        algo_r = valid * 1152 + w2.num_tokens * 8
        algo_w = valid * eb
        md.append(f"| {key} | {len(fetch[key])} / {len(write[key])} | {fr:,.1f} | {wr:,.1f} | {rb:,.0f} | "
                  f"{algo_r:,} | {wb:,.0f} | {algo_w:,} | {wb / algo_w:.3f} |")
    with open(os.path.join(ROOT, "profiles", "decode_write_hbm_traffic_pmc.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))

# ---------------------------------------------------------------------------
def _cpu_threads():
    """Host threads for the all-cores oracle run: the process's CPU share
    (OMP_NUM_THREADS where the launcher sets it, else the usable cores),
    at most 16."""
    n = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    if n <= 0:
        n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def _request_shards(ws, total, n, parts):
    """Split workspace rows [0, n) at request boundaries into about `parts`
    runs of requests: (b0, b1, row0, row1) with rows [row0, row1) belonging
    to requests b0 .. b1-1."""
    B = ws.shape[0]
    ends = np.append(ws[1:].astype(np.int64), total)
    out, b0 = [], 0
    target = max(1, -(-n // parts))
    while b0 < B and ws[b0] < n:
        b1 = b0 + 1
        while b1 < B and ws[b1] < n and min(int(ends[b1 - 1]), n) - int(ws[b0]) < target:
            b1 += 1
        out.append((b0, b1, int(ws[b0]), min(int(ends[b1 - 1]), n)))
        b0 = b1
    return out


def cpu_baseline(budget_s, w3, g3, w4, g4, w5, g5):
    """The oracle, as it stands, on a bounded sample of each workload.  Each op
    is first timed on a small slice to size its sample to about budget_s / 6
    seconds on one thread (capped at the whole workload).  Write samples: the
    first n tokens of each pre-fill; gather samples: the first n rows of each
    gather, reading a cache that holds the oracle's own output for the
    sampled tokens (other entries zero; the decode cost does not depend on
    the bytes).  The same samples are then run again split over the host's
    threads (writes by token ranges, gathers by runs of whole requests; the
    oracle calls release the GIL), which gives the reported value; the
    single-thread figures are kept beside it.  GB/s from the same
    algorithmic byte counts as the GPU figures."""
    import concurrent.futures as cf
    import oracle
    per_op = budget_s / 6.0
    threads = _cpu_threads()
    H, hs = w5.key.shape[1], w5.key.shape[2]
    L = oracle.kv_layout_split(w5.block_size, H, hs)
    c3 = np.zeros(w3.num_blocks * w3.block_size * NV, np.uint8)
    c4 = np.zeros(w4.num_blocks * w4.block_size * F8, np.uint8)
    c5 = np.zeros(w5.num_blocks * L.block_stride, np.uint8)
    kv_row = 2 * H * (2 * hs + hs // 2 + hs // 16)

    def ds_write(w, cache, fn, entry):
        def run(a, b):
            fn(w.kv_c[a:b], w.k_pe[a:b], cache, w.slot_mapping[a:b], w.num_blocks, w.block_size)
        return run, lambda n: n * (1152 + entry + 8)

    def kv_write_run(a, b):
        oracle.reshape_and_cache_nvfp4(np.ascontiguousarray(w5.key[a:b]), np.ascontiguousarray(w5.value[a:b]),
                                       c5, w5.slot_mapping[a:b], w5.num_blocks, w5.block_size, L, w5.k_scale,
                                       w5.v_scale)

    def kv_write_bytes_n(n):
        return int((w5.slot_mapping[:n] >= 0).sum()) * kv_row + n * 8

    def ds_gather(g, cache, fn):
        def run(b0, b1, r0, r1, dst):
            ws = (g.workspace_starts[b0:b1] - g.workspace_starts[b0]).astype(np.int32)
            fn(cache, r1 - r0, g.block_table[b0:b1], ws, g.seq_starts[b0:b1], g.num_blocks, g.block_size,
               dst=dst[r0:r1])
        return run, lambda n: np.zeros((n, 576), np.uint16)

    def kv_gather_run(b0, b1, r0, r1, dst):
        ws = (g5.workspace_starts[b0:b1] - g5.workspace_starts[b0]).astype(np.int32)
        oracle.gather_upconvert_nvfp4_kv(c5, r1 - r0, g5.block_table[b0:b1], ws, g5.seq_starts[b0:b1], H, hs,
                                         w5.num_blocks, w5.block_size, L, w5.k_scale, w5.v_scale)

    nv_w, nv_wb = ds_write(w3, c3, oracle.write_nvfp4_ds_mla, NV)
    f8_w, f8_wb = ds_write(w4, c4, oracle.write_fp8_ds_mla, F8)
    nv_g, nv_dst = ds_gather(g3, c3, oracle.gather_nvfp4_ds_mla)
    f8_g, f8_dst = ds_gather(g4, c4, oracle.gather_fp8_ds_mla)
    plan = [  # name, kind, units available, run, algorithmic bytes of n units, gather case, dst(n)
        ("nvfp4_ds_mla_write", "write", w3.num_tokens, nv_w, nv_wb, None, None),
        ("nvfp4_ds_mla_gather", "gather", g3.total_tokens, nv_g, lambda n: n * (NV + 1152), g3, nv_dst),
        ("fp8_ds_mla_write", "write", w4.num_tokens, f8_w, f8_wb, None, None),
        ("fp8_ds_mla_gather", "gather", g4.total_tokens, f8_g, lambda n: n * (F8 + 1152), g4, f8_dst),
        ("nvfp4_kv_write", "write", w5.slot_mapping.shape[0], kv_write_run, kv_write_bytes_n, None, None),
        ("nvfp4_kv_gather", "gather", g5.total_tokens, kv_gather_run, lambda n: n * kv_row, g5,
         lambda n: np.zeros((n, 1), np.uint16)),
    ]

    def once(kind, run, g, dst_of, n):
        if kind == "write":
            run(0, n)
        else:
            dst = dst_of(n)
            for sh in _request_shards(g.workspace_starts, g.total_tokens, n, 1):
                run(*sh, dst)

    def parallel(pool, kind, run, g, dst_of, n):
        if kind == "write":
            cuts = np.linspace(0, n, threads + 1).astype(np.int64)
            futs = [pool.submit(run, int(a), int(b)) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
        else:
            dst = dst_of(n)
            futs = [pool.submit(run, *sh, dst) for sh in _request_shards(g.workspace_starts, g.total_tokens,
                                                                          n, threads)]
        for f in futs:
            f.result()

    res, desc = {}, []
    tot_bytes, tot_1, tot_mt = 0, 0.0, 0.0
    with cf.ThreadPoolExecutor(max_workers=threads) as pool:
        for name, kind, avail, run, nbytes_of, g, dst_of in plan:
            n0 = min(avail, 64)
            while True:                          # calibrate on >= 0.1 s of work
                t = time.perf_counter()
                once(kind, run, g, dst_of, n0)
                el = time.perf_counter() - t
                if el >= 0.1 or n0 >= avail:
                    break
                n0 = min(avail, n0 * 4)
            per_unit = max(el / n0, 1e-9)
            n = int(min(avail, max(n0, per_op / per_unit)))
            t = time.perf_counter()
            once(kind, run, g, dst_of, n)
            sec1 = time.perf_counter() - t
            t = time.perf_counter()
            parallel(pool, kind, run, g, dst_of, n)
            secm = time.perf_counter() - t
            nbytes = nbytes_of(n)
            res[name] = {"units": n, "s_1_thread": round(sec1, 3), f"s_{threads}_threads": round(secm, 3),
                         "GB_per_s_1_thread": round(nbytes / sec1 / 1e9, 4),
                         "GB_per_s": round(nbytes / secm / 1e9, 4), "bytes": nbytes}
            tot_bytes += nbytes
            tot_1 += sec1
            tot_mt += secm
            desc.append(f"{name} {n}/{avail}")
    pb = sum(res[n]["bytes"] for n in PAIR)
    pm = sum(res[n][f"s_{threads}_threads"] for n in PAIR)
    p1 = sum(res[n]["s_1_thread"] for n in PAIR)
    return {"value": round(pb / pm / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "the metric's pair: the first tokens of the nvfp4_ds_mla pre-fill write and the first "
                      "workspace rows of its prefill gather (" + ", ".join(d for d in desc if d.split()[0] in PAIR)
                      + "), the C oracle (gcc -O2) unchanged, on " f"{threads} host threads (writes split by "
                      f"token ranges, gathers by runs of whole requests): {pm:.1f} s wall ({p1:.1f} s on one "
                      "thread); value = their algorithmic bytes over that time.  The other four ops' samples ("
                      + ", ".join(d for d in desc if d.split()[0] not in PAIR) + ") are in per_op and in "
                      f"value_all_ops ({tot_mt:.1f} s wall for all six)",
            "value_1_thread": round(pb / p1 / 1e9, 4),
            "value_all_ops": round(tot_bytes / tot_mt / 1e9, 4),
            "value_all_ops_1_thread": round(tot_bytes / tot_1 / 1e9, 4),
            "per_op": res, "host_cpu": _cpu_name()}


def _cpu_name():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
