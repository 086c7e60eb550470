"""Benchmark: position-split decode attention on one MI355X.

Workload (the headline configuration): a Qwen2.5-14B-shaped decode layer --
1 query token, 40 query heads / 8 KV heads, head_dim 128, n_kv = 65536 keys
of f16 K and V drawn N(0,1) with 1 % of the (KV head, dim) channels scaled by
8 -- split by key position into a device window [0, 49152) and a 16384-key
tail [49152, 65536) (also device-resident); 48 independent layers run back to
back.  One step = for every layer one rkv_attend_split call over the two
segments: the split-K kernel attends window and tail tiles in one launch
(Q staging, K/V tile reads, in-register conversion, scores, online softmax,
PV accumulation, per-split partials) and the fixed-order merge kernel turns
the partials of both segments into the combined O and LSE.  The metric is
effective KV bytes/s: the K+V bytes the step must read (48 x 268.4 MB) over
the step time.

Beside it (each in the form a caller runs it): the tiny f32 call, the q8_0
head_dim-512 softcap layer, the shared-prefix fan-out, the streamed tail
through the ring with its free-zone sweep, an 8-row verify step and the
write path; the read ceiling of a plain streaming-read kernel; and the
binary64 oracle timed per configuration on the host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
    python bench.py --only c3      # one workload alone (profiling runs)

Prints one JSON line on stdout (progress on stderr).  Only one GPU is used;
--gpus above 1 exits.  --copy-probe adds one plain 1 GiB device copy (torch)
before the workload, whose hardware counters calibrate the FETCH_SIZE /
WRITE_SIZE readings of the attention kernels.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X published dense f16 matrix-core rate

# Sources whose content decides the attention kernels: figures taken from
# hardware counters are valid only for the kernels they were taken on.
KERNEL_SOURCES = ["attend_kernel.h", "attend_shd.h", "attend_rgs.h", "attend_inst.hip", "attend.hip", "common.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "position_split_kv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# Figures from rocprofv3 --pmc runs of `bench.py --only ...` (profiles/ holds
# the summaries and commands), each with the kernel-source hash it was taken
# on; a figure whose hash differs from the current sources is reported as null.
#   c2_split_traffic: HBM bytes (FETCH_SIZE, then WRITE_SIZE, each scaled by the
#     same counter's reading for a plain 1 GiB copy) per split-kernel launch.
#   c3_counters / c5_counters / c4_window_counters / tbq3_window_counters /
#     verify_counters: SQ figures of the workload's attention kernel (VALU and MFMA busy fractions,
#     instructions per wave; profiles/rkv_split_kernels_sq_counters.md).
MEASURED = {
    "c2_split_traffic": {"src": "8c18b6b1c1b901a0", "fetch_bytes": 268994319, "write_bytes": 5570675, "bytes": 274564994},
    "c3_counters": {"valu_busy": 0.4682, "mfma_busy": 0.1145, "valu_per_wave": 20938, "mfma_per_wave": 1280, "salu_per_wave": 3895, "lds_per_wave": 1708, "wait_frac": 0.347, "issue_frac": 0.378, "lds_conflict_per_lds_active": 1.82, "src": "8c18b6b1c1b901a0"},
    "c5_counters": {"valu_busy": 0.3753, "mfma_busy": 0.1549, "valu_per_wave": 6202, "mfma_per_wave": 640, "salu_per_wave": 1592, "lds_per_wave": 982, "wait_frac": 0.361, "issue_frac": 0.421, "lds_conflict_per_lds_active": 0.555, "src": "8c18b6b1c1b901a0"},
    "c4_window_counters": {"valu_busy": 0.3964, "mfma_busy": 0.096, "valu_per_wave": 5283, "mfma_per_wave": 320, "salu_per_wave": 1232, "lds_per_wave": 358, "wait_frac": 0.301, "issue_frac": 0.425, "lds_conflict_per_lds_active": 1.461, "src": "8c18b6b1c1b901a0"},
    "tbq3_window_counters": {"valu_busy": 0.3287, "mfma_busy": 0.0777, "valu_per_wave": 5416, "mfma_per_wave": 320, "salu_per_wave": 1109, "lds_per_wave": 550, "wait_frac": 0.305, "issue_frac": 0.431, "lds_conflict_per_lds_active": 1.778, "src": "8c18b6b1c1b901a0"},
    "verify_counters": {"valu_busy": 0.3131, "mfma_busy": 0.1628, "valu_per_wave": 5908, "mfma_per_wave": 768, "salu_per_wave": 2330, "lds_per_wave": 582, "wait_frac": 0.455, "issue_frac": 0.359, "lds_conflict_per_lds_active": 0.703, "src": "8c18b6b1c1b901a0"},
}


def measured(name):
    m = MEASURED.get(name)
    return m if m and m.get("src") == kernel_source_hash() else None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def pct(xs, p):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(p / 100.0 * (len(xs) - 1)))))]


def timed(f, reps=20, warm=3):
    """Mean time of f() over reps calls on the current stream (HIP events), after warm calls."""
    import torch

    for _ in range(warm):
        f()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        f()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=48)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU work of the oracle sample")
    ap.add_argument("--no-oracle-configs", action="store_true", help="skip the per-configuration oracle timing")
    ap.add_argument("--copy-probe", action="store_true", help="run one plain 1 GiB copy first (counter calibration)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the three-call comparison and the read-ceiling probe (profiling runs)")
    ap.add_argument("--no-streamed", action="store_true", help="skip the streamed-tail measurement")
    ap.add_argument("--no-others", action="store_true", help="skip the tiny, softcap-q8_0 and shared-prefix timings")
    ap.add_argument("--only", choices=["c1", "c2", "c3", "c4", "c4-sweep", "c4-window", "tbq3", "c5", "verify",
                                       "append", "ceiling"],
                    help="run one workload alone and print its figures (profiling runs)")
    ap.add_argument("--reps", type=int, default=20, help="timed calls per workload of the other workloads")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); sharding across GPUs is described, "
              "not built", file=sys.stderr)
        sys.exit(2)

    import torch

    import position_split_kv_amd as P
    import synth

    torch.cuda.init()
    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log("bench: copy probe: 1073741824 bytes read, 1073741824 bytes written")
        del a, b

    if args.only and args.only != "c2":
        fn = {"c1": lambda: tiny_f32(P, synth, args.reps), "c3": lambda: softcap_q8_d512(P, synth, args.reps),
              "c5": lambda: shared_prefix(P, synth, args.reps), "verify": lambda: verify_rows(P, synth, args.reps),
              "append": lambda: append_path(P, synth, args.reps),
              "c4": lambda: streamed_tail(P, synth, quick=True),
              "c4-sweep": lambda: streamed_tail(P, synth),
              "c4-window": lambda: window_q8q4(P, synth, args.reps),
              "tbq3": lambda: window_q8q4(P, synth, args.reps, synth.TBQ3),
              "ceiling": lambda: read_ceiling(None)}[args.only]
        print(json.dumps({args.only: fn(), "kernel_src": kernel_source_hash()}), flush=True)
        return

    L, S, Hq, Hkv, D, n, wc = args.layers, 1, 40, 8, 128, 65536, 49152
    scale = 1.0 / math.sqrt(D)
    outliers = round(0.01 * Hkv * D)
    log(f"bench: building {L} layers of K/V [{n}][{Hkv}][{D}] f16 ({outliers} outlier channels x8)")
    layers = []
    for li in range(L):
        kc = synth.make_cache(n, Hkv, D, synth.F16, synth.stream_seed(2, 1, li), "cuda", outlier_channels=outliers,
                              channels_seed=synth.stream_seed(2, 7, li))
        vc = synth.make_cache(n, Hkv, D, synth.F16, synth.stream_seed(2, 2, li), "cuda", outlier_channels=outliers,
                              channels_seed=synth.stream_seed(2, 7, li))
        q = synth.make_query(S, Hq, D, synth.stream_seed(2, 3, li), "cuda")
        layers.append((kc, vc, q))
    torch.cuda.synchronize()
    desc = P.Desc(S, Hq, Hkv, D, scale)
    segs = [[P.view_of_cache(kc, vc, 0, wc), P.view_of_cache(kc, vc, wc, n)] for kc, vc, _ in layers]
    ws = P.workspace(P.rkv_attend_split_workspace_bytes(desc, segs[0]))
    # one workspace per layer for the phase timing (partials of all 48 layers
    # are live between the two phases)
    ws_l = [P.workspace(P.rkv_attend_split_workspace_bytes(desc, segs[0])) for _ in range(L)]
    outs = [(torch.empty(S, Hq, D, device="cuda"), torch.empty(S, Hq, device="cuda")) for _ in range(L)]
    stream = torch.cuda.current_stream()

    def step():
        for li in range(L):
            P.rkv_attend_split(desc, layers[li][2], segs[li], outs[li][0], outs[li][1], ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps

    kv_bytes_layer = 2 * n * Hkv * D * 2
    step_bytes = L * kv_bytes_layer
    gbs = step_bytes / dt / 1e9

    # The dominant kernel: each rkv_attend_split call is the split kernel over
    # all 65536 keys (268.4 MB of K+V) followed by the small partial-merge
    # kernel.  HIP events on the launch stream bracket each step of 48 calls
    # (the average launch is the step time over 48; an event pair around every
    # call would add its own ~2 us); a second pass brackets single calls for
    # the distribution (p10 / p50 / p90).
    reps = max(2, args.steps // 2)
    ev_step = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev_step:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    call_s = sum(a.elapsed_time(b) for a, b in ev_step) * 1e-3 / (reps * L)
    call_gbs = kv_bytes_layer / call_s / 1e9

    # The unsplit run (one segment [0, n), i.e. wc = n_kv), timed the same way:
    # the split overhead is the two-segment call's time minus this one's.
    segs1 = [[P.view_of_cache(kc, vc, 0, n)] for kc, vc, _ in layers]
    ws1 = P.workspace(P.rkv_attend_split_workspace_bytes(desc, segs1[0]))

    def step1():
        for li in range(L):
            P.rkv_attend_split(desc, layers[li][2], segs1[li], outs[li][0], outs[li][1], ws1, stream)

    step1()
    for a, b in ev_step:
        a.record(stream)
        step1()
        b.record(stream)
    torch.cuda.synchronize()
    unsplit_s = sum(a.elapsed_time(b) for a, b in ev_step) * 1e-3 / (reps * L)
    del ws1
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(L)]
    times = []
    for _ in range(reps):
        for li in range(L):
            ev[li][0].record(stream)
            P.rkv_attend_split(desc, layers[li][2], segs[li], outs[li][0], outs[li][1], ws, stream)
            ev[li][1].record(stream)
        torch.cuda.synchronize()
        times += [a.elapsed_time(b) * 1e-3 for a, b in ev]

    # The dominant kernel alone: the same 48 calls cut at the phase boundary,
    # HIP events around each step of 48 split-kernel launches (first phase),
    # then around 48 merges (second phase); each phase's work is unchanged.
    ev_ph = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(2 * reps)]
    for r in range(reps):
        a, b = ev_ph[2 * r]
        a.record(stream)
        for li in range(L):
            P.rkv_attend_split_partials(desc, layers[li][2], segs[li], outs[li][0], outs[li][1], ws_l[li], stream)
        b.record(stream)
        a, b = ev_ph[2 * r + 1]
        a.record(stream)
        for li in range(L):
            P.rkv_attend_split_merge(desc, segs[li], outs[li][0], outs[li][1], ws_l[li], stream)
        b.record(stream)
    torch.cuda.synchronize()
    split_s = sum(ev_ph[2 * r][0].elapsed_time(ev_ph[2 * r][1]) for r in range(reps)) * 1e-3 / (reps * L)
    merge_s = sum(ev_ph[2 * r + 1][0].elapsed_time(ev_ph[2 * r + 1][1]) for r in range(reps)) * 1e-3 / (reps * L)
    split_gbs = kv_bytes_layer / split_s / 1e9
    if args.only == "c2":
        print(json.dumps({"c2": {"us_per_layer": round(dt / L * 1e6, 3), "split_us": round(split_s * 1e6, 3),
                                 "merge_us": round(merge_s * 1e6, 3), "call_us": round(call_s * 1e6, 3)},
                          "kernel_src": kernel_source_hash()}), flush=True)
        return

    three_us = ceiling = None
    if not args.no_extras:
        three_us = three_calls(P, desc, layers, segs, outs, stream, S, Hq, D, L)
        ceiling = read_ceiling(layers)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(layers, desc, args.cpu_seconds)

    others = None
    if not args.no_others:
        others = {"tiny_f32": tiny_f32(P, synth, args.reps), "softcap_q8_d512": softcap_q8_d512(P, synth, args.reps),
                  "window_q8q4": window_q8q4(P, synth, args.reps),
                  "window_q8_tbq3": window_q8q4(P, synth, args.reps, synth.TBQ3),
                  "shared_prefix": shared_prefix(P, synth, args.reps),
                  "verify_8_rows_f16": verify_rows(P, synth, args.reps), **append_path(P, synth, args.reps)}

    del layers, segs, outs, ws, ws_l
    torch.cuda.empty_cache()
    streamed = None
    if not args.no_streamed:
        streamed = streamed_tail(P, synth)
    if cpu is not None and not args.no_oracle_configs:
        cpu["per_config"] = oracle_per_config(synth)

    traffic = measured("c2_split_traffic")
    out = {
        "metric": "decode attention effective KV GB/s & us/layer vs HBM peak; tail-hidden fraction",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 K/V, f32 accumulate",
        "data": "synthetic, seeded N(0,1) f16 K/V with 1% outlier channels x8; f32 Q",
        "config": {
            "workload": "Qwen2.5-14B-shaped decode attention: 1 token, 40 q heads / 8 KV heads, head_dim 128, "
                        "n_kv 65536 = window 49152 + tail 16384 (device), f16 K/V, 48 layers back to back",
            "layers": L, "n_kv": n, "wc": wc, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": D,
            "us_per_layer": round(dt / L * 1e6, 3),
            "us_per_layer_call_p10_p50_p90": [round(pct(times, p) * 1e6, 2) for p in (10, 50, 90)],
            "us_per_layer_three_calls": three_us and round(three_us, 3),
            "us_per_layer_unsplit": round(unsplit_s * 1e6, 3),
            "split_overhead_us": round((call_s - unsplit_s) * 1e6, 3),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "read_ceiling": ceiling,
            "frac_of_read_ceiling": ceiling and round(gbs / ceiling["per_layer_kv_GBs"], 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "rkv_split_kernel<f16,f16,128,5> (the attention kernel of one rkv_attend_split call, "
                      "timed alone through rkv_attend_split_partials)",
            "achieved": round(split_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(split_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic and traffic["bytes"],
            "traffic_kernel_src": traffic and traffic["src"],
            "kernel_src": kernel_source_hash(),
            "algorithmic_bytes_per_launch": kv_bytes_layer,
            "avg_launch_us": round(split_s * 1e6, 3),
            "frac_of_read_ceiling": ceiling and round(split_gbs / ceiling["per_layer_kv_GBs"], 4),
            "merge_avg_launch_us": round(merge_s * 1e6, 3),
            "call_avg_us": round(call_s * 1e6, 3),
            "call_GBs": round(call_gbs, 2),
            "call_frac": round(call_gbs / HBM_PEAK_GBS, 4),
            "median_single_call_us": round(statistics.median(times) * 1e6, 3),
        },
        "cpu_baseline": cpu,
        "streamed_tail": streamed,
        "other_workloads": others,
    }
    if streamed is not None:
        out["config"]["tail_hidden_fraction"] = streamed["tail_hidden_fraction_in_free_zone"]
    print(json.dumps(out), flush=True)


def three_calls(P, desc, layers, segs, outs, stream, S, Hq, D, L):
    """The same layers through the three-call form (window, tail, combine)."""
    import torch

    dev = "cuda"
    ow, lw = torch.empty(S, Hq, D, device=dev), torch.empty(S, Hq, device=dev)
    ot, lt = torch.empty_like(ow), torch.empty_like(lw)
    ws_w = P.workspace(P.rkv_attend_workspace_bytes(desc, segs[0][0]))
    ws_t = P.workspace(P.rkv_attend_workspace_bytes(desc, segs[0][1]))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for it in range(2):
        if it == 1:
            e0.record(stream)
        for li in range(L):
            P.rkv_attend_segment(desc, layers[li][2], segs[li][0], ow, lw, ws_w, stream)
            P.rkv_attend_segment(desc, layers[li][2], segs[li][1], ot, lt, ws_t, stream)
            P.rkv_lse_combine([ow, ot], [lw, lt], outs[li][0], outs[li][1], D, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / L


def read_ceiling(layers):
    """The read rate of a plain streaming-read kernel (librkvprobe.so: 16-byte
    non-temporal loads, every byte once, nothing written), as the ceiling the
    attention kernels are compared with:
      linear: one 4 GiB buffer per launch;
      per_layer_kv: the 48 layers' K and V (2 x 128 MiB each, the headline
        workload's buffers) one layer per launch, 48 launches back to back,
        i.e. the same bytes per launch as one attention call.
    Each figure is the best over a few grid sizes (workgroups of 256 threads)."""
    import torch

    from position_split_kv_amd import build as B

    L = ctypes.CDLL(B.PROBE_LIB)
    L.rkv_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p]
    L.rkv_probe_read.restype = ctypes.c_int
    stream = torch.cuda.current_stream()
    sink = torch.zeros(1 << 15, dtype=torch.int32, device="cuda")
    ev = lambda: torch.cuda.Event(enable_timing=True)
    grids = (1024, 2048, 4096, 8192)

    def launch(a, na, b, nb, blocks):
        rc = L.rkv_probe_read(a, na, b, nb, blocks, sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"rkv_probe_read failed: {rc}")

    big = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    lin = {}
    for g in grids:
        launch(big.data_ptr(), big.numel(), None, 0, g)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(5):
            launch(big.data_ptr(), big.numel(), None, 0, g)
        e1.record(stream)
        torch.cuda.synchronize()
        lin[g] = 5 * big.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del big
    res = {"kernel": "rkv_probe_read_kernel (16-byte nt loads, read once)",
           "linear_4GiB_GBs": round(max(lin.values()), 1), "linear_by_grid": {str(k): round(v, 1) for k, v in lin.items()}}
    if layers:
        nb = layers[0][0].data.numel() * layers[0][0].data.element_size()
        per = {}
        for g in grids:
            for kc, vc, _ in layers[:2]:
                launch(kc.data.data_ptr(), nb, vc.data.data_ptr(), nb, g)
            torch.cuda.synchronize()
            e0, e1 = ev(), ev()
            e0.record(stream)
            for _ in range(3):
                for kc, vc, _ in layers:
                    launch(kc.data.data_ptr(), nb, vc.data.data_ptr(), nb, g)
            e1.record(stream)
            torch.cuda.synchronize()
            per[g] = 3 * len(layers) * 2 * nb / (e0.elapsed_time(e1) * 1e-3) / 1e9
        best = max(per, key=per.get)
        res.update({"per_layer_kv_GBs": round(per[best], 1), "per_layer_kv_us": round(2 * nb / per[best] / 1e3, 3),
                    "per_layer_by_grid": {str(k): round(v, 1) for k, v in per.items()}})
    return res


def tiny_f32(P, synth, reps):
    """f32, 8/2 heads, D 128, window 3072 + tail 1024: cache-resident, launch-latency bound."""
    import torch

    kc = synth.make_cache(4096, 2, 128, synth.F32, synth.stream_seed(1, 1), "cuda")
    vc = synth.make_cache(4096, 2, 128, synth.F32, synth.stream_seed(1, 2), "cuda")
    q = synth.make_query(1, 8, 128, synth.stream_seed(1, 3), "cuda")
    d = P.Desc(1, 8, 2, 128, 1 / math.sqrt(128))
    segs = [P.view_of_cache(kc, vc, 0, 3072), P.view_of_cache(kc, vc, 3072, 4096)]
    ws = P.workspace(P.rkv_attend_split_workspace_bytes(d, segs))
    o, l = torch.empty(1, 8, 128, device="cuda"), torch.empty(1, 8, device="cuda")
    t = timed(lambda: P.rkv_attend_split(d, q, segs, o, l, ws), reps)
    return {"us": round(t * 1e6, 2), "GBs": round(2 * 4096 * 2 * 512 / t / 1e9, 1),
            "note": "8.4 MB, cache-resident: launch-latency bound"}


def softcap_q8_d512(P, synth, reps):
    """q8_0 K and V, 16/2 heads, D 512, 262144 keys = 196608 + 65536, softcap 30:
    one rkv_attend_split call, two cache instances alternated (1.14 GB, past the
    256 MB last-level cache).  The roofline object is the attention kernel alone
    (the call's first phase, rkv_attend_split_partials)."""
    import torch

    inst = []
    for i in range(2):
        inst.append((synth.make_cache(262144, 2, 512, synth.Q8_0, synth.stream_seed(3, 1, i), "cuda"),
                     synth.make_cache(262144, 2, 512, synth.Q8_0, synth.stream_seed(3, 2, i), "cuda")))
    q = synth.make_query(1, 16, 512, synth.stream_seed(3, 3), "cuda")
    d = P.Desc(1, 16, 2, 512, 1 / math.sqrt(512), 30.0)
    segs = [[P.view_of_cache(kc, vc, 0, 196608), P.view_of_cache(kc, vc, 196608, 262144)] for kc, vc in inst]
    ws = P.workspace(P.rkv_attend_split_workspace_bytes(d, segs[0]))
    o, l = torch.empty(1, 16, 512, device="cuda"), torch.empty(1, 16, device="cuda")
    k = [0]

    def call():
        P.rkv_attend_split(d, q, segs[k[0] % 2], o, l, ws)
        k[0] += 1

    def part():
        P.rkv_attend_split_partials(d, q, segs[k[0] % 2], o, l, ws)
        k[0] += 1
    t = timed(call, reps)
    tk = timed(part, reps)
    b = 2 * 262144 * 2 * 544
    flops = 2 * 2 * 16 * 262144 * 512  # QK^T and PV, 16 query rows
    res = {"us": round(t * 1e6, 2), "GBs": round(b / t / 1e9, 1), "frac_of_hbm_peak": round(b / t / 1e9 / HBM_PEAK_GBS, 4),
           "bytes": b,
           "roofline": {"bound": "hbm", "kernel": "rkv_split_kernel<q8_0,q8_0,128,8,4> (4 dim slices of 128)",
                        "achieved": round(b / tk / 1e9, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(b / tk / 1e9 / HBM_PEAK_GBS, 4), "avg_launch_us": round(tk * 1e6, 2),
                        "algorithmic_flops": flops,
                        "mfma_frac_algorithmic": round(flops / tk / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}}
    c = measured("c3_counters")
    res["roofline"]["sq_counters"] = c
    return res


def window_q8q4(P, synth, reps, vt=None):
    """The window of the streamed-tail layers: q8_0 K / q4_0 V, 40/8 heads, D 128,
    65536 keys (109 MB), one rkv_attend_segment call; four cache instances
    alternated (436 MB, past the 256 MB last-level cache).  The roofline object
    is the attention kernel alone (rkv_attend_split_partials over the one
    segment).  vt: another value type (TBQ3: the 3-bit tier, 98.6 MB, whose
    call also turns the output back from the rotated space)."""
    import torch

    Hq, Hkv, D, n = 40, 8, 128, 65536
    vt = synth.Q4_0 if vt is None else vt
    inst = []
    for i in range(4):
        inst.append((synth.make_cache(n, Hkv, D, synth.Q8_0, synth.stream_seed(6, 1, i), "cuda"),
                     synth.make_cache(n, Hkv, D, vt, synth.stream_seed(6, 2, i), "cuda")))
    q = synth.make_query(1, Hq, D, synth.stream_seed(6, 3), "cuda")
    d = P.Desc(1, Hq, Hkv, D, 1 / math.sqrt(D))
    segs = [P.view_of_cache(kc, vc) for kc, vc in inst]
    ws = P.workspace(max(P.rkv_attend_workspace_bytes(d, segs[0]), P.rkv_attend_split_workspace_bytes(d, segs[:1])))
    o, l = torch.empty(1, Hq, D, device="cuda"), torch.empty(1, Hq, device="cuda")
    k = [0]

    def call():
        P.rkv_attend_segment(d, q, segs[k[0] % 4], o, l, ws)
        k[0] += 1

    def part():
        P.rkv_attend_split_partials(d, q, [segs[k[0] % 4]], o, l, ws)
        k[0] += 1
    t = timed(call, reps)
    tk = timed(part, reps)
    b = n * (inst[0][0].pos_stride + inst[0][1].pos_stride)  # 8 heads x (136 + 72 or 52) B per key
    res = {"us": round(t * 1e6, 2), "GBs": round(b / t / 1e9, 1), "frac_of_hbm_peak": round(b / t / 1e9 / HBM_PEAK_GBS, 4),
           "bytes": b,
           "roofline": {"bound": "hbm", "kernel": f"rkv_split_kernel<q8_0,{synth.TYPE_NAMES[vt]},128,5,1>",
                        "achieved": round(b / tk / 1e9, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(b / tk / 1e9 / HBM_PEAK_GBS, 4), "avg_launch_us": round(tk * 1e6, 2)}}
    res["roofline"]["sq_counters"] = measured("tbq3_window_counters" if vt == synth.TBQ3 else "c4_window_counters")
    return res


def shared_prefix(P, synth, reps):
    """15 sequences x 32/8 heads, D 128, a 32768-key q8_0 / q4_0 prefix stored
    once + a private 2048-key f16 suffix per sequence: one rkv_attend_split
    call over both (the shared-decode launch over the prefix, the suffix
    launch, one merge), the three-call form (segment, segment, combine) and
    the prefix launch alone; two instances alternated.  Bytes: the prefix is
    counted once.  The roofline object is the prefix (shared-decode) kernel:
    HBM bytes and matrix-core work (60 rows x 32768 keys x 128 per KV head,
    QK^T and PV)."""
    import torch

    S, Hq, Hkv, D, npre, nsuf = 15, 32, 8, 128, 32768, 2048
    inst = []
    for i in range(2):
        pk = synth.make_cache(npre, Hkv, D, synth.Q8_0, synth.stream_seed(5, 1, i), "cuda")
        pv = synth.make_cache(npre, Hkv, D, synth.Q4_0, synth.stream_seed(5, 2, i), "cuda")
        sk = synth.make_cache(S * nsuf, Hkv, D, synth.F16, synth.stream_seed(5, 4, i), "cuda")
        sv = synth.make_cache(S * nsuf, Hkv, D, synth.F16, synth.stream_seed(5, 5, i), "cuda")
        inst.append((P.view_of_cache(pk, pv),
                     P.view_of_cache(sk, sv, 0, nsuf, nsuf * sk.pos_stride, nsuf * sv.pos_stride), pk, pv, sk, sv))
    q = synth.make_query(S, Hq, D, synth.stream_seed(5, 3), "cuda")
    d = P.Desc(S, Hq, Hkv, D, 1 / math.sqrt(D))
    wsp = P.workspace(P.rkv_attend_workspace_bytes(d, inst[0][0]))
    wss = P.workspace(P.rkv_attend_workspace_bytes(d, inst[0][1]))
    op, lp = torch.empty(S, Hq, D, device="cuda"), torch.empty(S, Hq, device="cuda")
    os_, ls = torch.empty_like(op), torch.empty_like(lp)
    oo, lo = torch.empty_like(op), torch.empty_like(lp)
    k = [0]

    def c5three():
        pv_, sv_ = inst[k[0] % 2][:2]
        k[0] += 1
        P.rkv_attend_segment(d, q, pv_, op, lp, wsp)
        P.rkv_attend_segment(d, q, sv_, os_, ls, wss)
        P.rkv_lse_combine([op, os_], [lp, ls], oo, lo, D)

    def c5prefix():
        P.rkv_attend_split_partials(d, q, [inst[k[0] % 2][0]], op, lp, wsp)
        k[0] += 1
    wsc = P.workspace(P.rkv_attend_split_workspace_bytes(d, list(inst[0][:2])))

    def c5one():
        P.rkv_attend_split(d, q, list(inst[k[0] % 2][:2]), oo, lo, wsc)
        k[0] += 1
    t = timed(c5one, reps)
    t3 = timed(c5three, reps)
    tp = timed(c5prefix, reps)
    pre_b = npre * Hkv * (136 + 72)
    b = pre_b + S * nsuf * Hkv * 2 * 256
    flops = 2 * 2 * (S * Hq) * npre * D  # QK^T and PV of all 480 rows over the prefix
    res = {"us": round(t * 1e6, 2), "GBs": round(b / t / 1e9, 1), "frac_of_hbm_peak": round(b / t / 1e9 / HBM_PEAK_GBS, 4),
           "bytes": b, "three_call_us": round(t3 * 1e6, 2), "prefix_only_us": round(tp * 1e6, 2),
           "roofline": {"bound": "mfma", "kernel": "rkv_split_shd_kernel<q8_0,q4_0> (the prefix launch alone)",
                        "achieved": round(flops / tp / 1e12, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(flops / tp / 1e12 / MFMA_F16_PEAK_TFLOPS, 4), "algorithmic_flops": flops,
                        "hbm_GBs": round(pre_b / tp / 1e9, 1), "hbm_frac": round(pre_b / tp / 1e9 / HBM_PEAK_GBS, 4),
                        "avg_launch_us": round(tp * 1e6, 2), "sq_counters": measured("c5_counters")}}
    return res


def verify_rows(P, synth, reps):
    """Several query rows under the causal mask: a verify step of 8 draft tokens
    (positions 65528 .. 65535) over the 40/8-head, head_dim 128 f16 cache of
    65536 keys (window 49152 + tail 16384, one call); two instances
    alternated.  Bytes: the K/V read once."""
    import torch

    Hq, Hkv, D, n, wc, nq = 40, 8, 128, 65536, 49152, 8
    inst = [(synth.make_cache(n, Hkv, D, synth.F16, synth.stream_seed(2, 1, i), "cuda"),
             synth.make_cache(n, Hkv, D, synth.F16, synth.stream_seed(2, 2, i), "cuda")) for i in range(2)]
    q = synth.make_query(nq, Hq, D, synth.stream_seed(2, 9), "cuda")
    d = P.Desc(nq, Hq, Hkv, D, 1 / math.sqrt(D), q_pos=list(range(n - nq, n)))
    segs = [[P.view_of_cache(kc, vc, 0, wc), P.view_of_cache(kc, vc, wc, n)] for kc, vc in inst]
    ws = P.workspace(P.rkv_attend_split_workspace_bytes(d, segs[0]))
    o, l = torch.empty(nq, Hq, D, device="cuda"), torch.empty(nq, Hq, device="cuda")
    k = [0]

    def ver():
        P.rkv_attend_split(d, q, segs[k[0] % 2], o, l, ws)
        k[0] += 1

    def part():
        P.rkv_attend_split_partials(d, q, segs[k[0] % 2], o, l, ws)
        k[0] += 1
    t = timed(ver, reps)
    tk = timed(part, reps)
    b = 2 * n * Hkv * D * 2
    return {"us": round(t * 1e6, 2), "GBs": round(b / t / 1e9, 1), "frac_of_hbm_peak": round(b / t / 1e9 / HBM_PEAK_GBS, 4),
            "bytes": b, "rows_per_kv_head": nq * Hq // Hkv,
            "roofline": {"bound": "hbm", "kernel": "rkv_split_rgs_kernel (f16, 40 rows per KV head: each tile staged once "
                                                   "per head)",
                         "achieved": round(b / tk / 1e9, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(b / tk / 1e9 / HBM_PEAK_GBS, 4), "avg_launch_us": round(tk * 1e6, 2),
                         "sq_counters": measured("verify_counters")}}


def append_path(P, synth, reps):
    """The write path: new binary32 rows quantised on append (q8_0 K, q4_0 V),
    8 KV heads x head_dim 128.  decode: one token into each of 48 layers'
    windows (latency per call); prefill: a 4096-token chunk that crosses from
    the window into the tail of one layer (bytes = f32 rows read + stored rows
    written)."""
    Hkv, D, wc, tc = 8, 128, 49152, 16384
    win = [(synth.make_cache(wc, Hkv, D, synth.Q8_0, synth.stream_seed(6, 1, i), "cuda"),
            synth.make_cache(wc, Hkv, D, synth.Q4_0, synth.stream_seed(6, 2, i), "cuda")) for i in range(48)]
    tail = (synth.make_cache(tc, Hkv, D, synth.Q8_0, synth.stream_seed(6, 3), "cuda"),
            synth.make_cache(tc, Hkv, D, synth.Q4_0, synth.stream_seed(6, 4), "cuda"))
    wv = [P.view_of_cache(kc, vc) for kc, vc in win]
    tv = P.view_of_cache(*tail)
    x1 = synth.append_rows(1, Hkv, D, synth.stream_seed(6, 5), "cuda", large=False)
    k = [0]

    def dec():
        P.rkv_append_kv(Hkv, D, 1, 1000 + k[0] % 4096, 0, x1, x1, wv[k[0] % 48], tv)
        k[0] += 1
    t = timed(dec, reps)
    res = {"append_decode": {"us_per_call": round(t * 1e6, 2),
                             "note": "one token, 8 KV heads x 128, q8_0 K / q4_0 V, 48 layers' windows in turn"}}
    nch = 4096
    xk = synth.append_rows(nch, Hkv, D, synth.stream_seed(6, 6), "cuda", large=False)
    xv = synth.append_rows(nch, Hkv, D, synth.stream_seed(6, 7), "cuda", large=False)
    t = timed(lambda: P.rkv_append_kv(Hkv, D, nch, wc - nch // 2, 0, xk, xv, wv[0], tv), reps)
    b = 2 * nch * Hkv * D * 4 + nch * Hkv * (136 + 72)
    res["append_prefill_4096"] = {"us": round(t * 1e6, 2), "GBs": round(b / t / 1e9, 1),
                                  "frac_of_hbm_peak": round(b / t / 1e9 / HBM_PEAK_GBS, 4), "bytes": b}
    return res


# The free-zone sweep: window 65536 fixed, tails of these many keys per layer,
# each with one tile per layer (tile = min(8192, tail)) and with 1024-key tiles.
SWEEP_TAILS = (1024, 2048, 4096, 6144)


def streamed_tail(P, synth, L=48, steps=3, quick=False):
    """The streamed-tail workload: 40 q heads / 8 KV heads, head_dim 128, q8_0 K and
    q4_0 V, 131072 keys per layer: window [0, 65536) in HBM, tail [65536, 131072) in
    pinned host memory, streamed in 8192-key tiles through a 3-slot device ring on
    a copy stream; between layers a dense-FFN stand-in (a 14336 x 4096 f16 GEMV,
    48 distinct matrices, repeated r times to about 0.2 ms).

    T_c: the step with the tails already in HBM (the same ring step with
    device-resident tails, attended in place: the same tile cut, launches and
    merge; no copies).  T_d: the tile copies alone on
    the copy stream.  T_p: the pipelined step through the ring.  Tail-hidden
    fraction h = (T_c + T_d - T_p) / T_d (clipped to [0, 1]); link fraction =
    (tail bytes / T_p) / R_link, with R_link the measured pinned H2D rate.
    quick: the whole tail and one free-zone point only (profiling runs)."""
    import torch

    dev = "cuda"
    Hq, Hkv, D, n, wc, tile, B = 40, 8, 128, 131072, 65536, 8192, 3
    desc = P.Desc(1, Hq, Hkv, D, 1.0 / math.sqrt(D))
    log(f"streamed: building {L} layers (q8_0 K / q4_0 V, {n} keys; tail {n - wc} keys in pinned host memory)")
    lay = []
    for li in range(L):
        kc = synth.make_cache(n, Hkv, D, synth.Q8_0, synth.stream_seed(4, 1, li), dev)
        vc = synth.make_cache(n, Hkv, D, synth.Q4_0, synth.stream_seed(4, 2, li), dev)
        q = synth.make_query(1, Hq, D, synth.stream_seed(4, 3, li), dev)
        kh = torch.empty(kc.data[wc:].shape, dtype=kc.data.dtype, pin_memory=True)
        vh = torch.empty(vc.data[wc:].shape, dtype=vc.data.dtype, pin_memory=True)
        kh.copy_(kc.data[wc:])
        vh.copy_(vc.data[wc:])
        lay.append(dict(kc=kc, vc=vc, q=q, kh=synth.Cache(kh, kc.dtype, n - wc, Hkv, D),
                        vh=synth.Cache(vh, vc.dtype, n - wc, Hkv, D)))
    W = [torch.randn(14336, 4096, device=dev, dtype=torch.float16, generator=torch.Generator(dev).manual_seed(900 + i))
         for i in range(L)]
    x = torch.randn(4096, device=dev, dtype=torch.float16)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    # FFN stand-in calibration
    for _ in range(3):
        torch.mv(W[0], x)
    e0, e1 = ev(), ev()
    e0.record(stream)
    for i in range(20):
        torch.mv(W[i % L], x)
    e1.record(stream)
    torch.cuda.synchronize()
    t_gemv = e0.elapsed_time(e1) * 1e-3 / 20
    reps = max(1, round(200e-6 / t_gemv))
    reps_ffn = reps

    # every GEMV of the stand-in reads a different matrix, as the calibration
    # did (a matrix read again right after would come from the last-level
    # cache and the FFN would be shorter than the 0.2 ms it stands for)
    def ffn(li):
        for r in range(reps):
            torch.mv(W[(li * reps + r) % L], x)

    # pinned H2D rate (256 MiB, non-blocking stream)
    cs = torch.cuda.Stream()
    hbuf = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    dbuf = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    with torch.cuda.stream(cs):
        dbuf.copy_(hbuf, non_blocking=True)
        a, b = ev(), ev()
        a.record(cs)
        for _ in range(4):
            dbuf.copy_(hbuf, non_blocking=True)
        b.record(cs)
    torch.cuda.synchronize()
    r_link = 4 * hbuf.numel() / (a.elapsed_time(b) * 1e-3) / 1e9
    del hbuf, dbuf

    outs = [(torch.empty(1, Hq, D, device=dev), torch.empty(1, Hq, device=dev)) for _ in range(L)]
    o_w, l_w = torch.empty(1, Hq, D, device=dev), torch.empty(1, Hq, device=dev)
    ws_w = P.workspace(P.rkv_attend_workspace_bytes(desc, P.view_of_cache(lay[0]["kc"], lay[0]["vc"], 0, wc)))

    def measure(tail_keys, tile_keys, reps=steps):
        """T_c, T_d, T_p of one (tail, tile) setting.  The three kinds of step
        ('resident': the tiles attended from HBM, no copies; 'copy': the tile
        copies alone on the copy stream; 'stream': the pipelined step through
        the ring) are set up once and run interleaved, rep after rep, so that
        slow drifts of the part's clocks hit all three alike; each figure is
        the median over the reps (after one untimed rep)."""
        n_t = (tail_keys + tile_keys - 1) // tile_keys
        kc0, vc0 = lay[0]["kc"], lay[0]["vc"]
        # the ring's device memory stays that of 3 slots of 8192 keys: shorter
        # tiles get more slots (at most 16)
        nb = min(16, B * tile // tile_keys)
        ring = P.Ring(nb, tile_keys * kc0.pos_stride, tile_keys * vc0.pos_stride)
        ring_r = P.Ring(nb, tile_keys * kc0.pos_stride, tile_keys * vc0.pos_stride)
        tails = {"stream": [P.view_of_cache(l_["kh"], l_["vh"], 0, tail_keys, pos0=wc) for l_ in lay],
                 "resident": [P.view_of_cache(l_["kc"], l_["vc"], wc, wc + tail_keys) for l_ in lay]}
        rings = {"stream": ring, "resident": ring_r}
        slots = [(torch.empty(tile_keys * kc0.pos_stride, dtype=torch.uint8, device=dev),
                  torch.empty(tile_keys * vc0.pos_stride, dtype=torch.uint8, device=dev)) for _ in range(nb)]
        ws_s = [None]

        def step(mode):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            if mode == "copy":
                with torch.cuda.stream(cs):
                    j = 0
                    for l_ in lay:
                        kb, vb = l_["kh"].data.view(-1), l_["vh"].data.view(-1)
                        for t in range(n_t):
                            a0, a1 = t * tile_keys, min(tail_keys, (t + 1) * tile_keys)
                            sk, sv = slots[j % nb]
                            sk[: (a1 - a0) * kc0.pos_stride].copy_(kb[a0 * kc0.pos_stride: a1 * kc0.pos_stride], non_blocking=True)
                            sv[: (a1 - a0) * vc0.pos_stride].copy_(vb[a0 * vc0.pos_stride: a1 * vc0.pos_stride], non_blocking=True)
                            j += 1
                cs.synchronize()
            else:
                rg = rings[mode]
                rg.rkv_ring_begin_step(tails[mode], tile_keys)
                if ws_s[0] is None:
                    ws_s[0] = P.workspace(rg.rkv_stream_tail_workspace_bytes(0, desc))
                for li, l_ in enumerate(lay):
                    P.rkv_attend_segment(desc, l_["q"], P.view_of_cache(l_["kc"], l_["vc"], 0, wc), o_w, l_w, ws_w, stream)
                    rg.rkv_stream_tail(li, desc, l_["q"], o_w, l_w, outs[li][0], outs[li][1], ws_s[0], stream)
                    ffn(li)
                rg.rkv_ring_end_step()
                torch.cuda.synchronize()
            return time.perf_counter() - t0

        times = {"resident": [], "copy": [], "stream": []}
        try:
            for rep in range(reps + 1):
                for mode in ("resident", "copy", "stream"):
                    dt = step(mode)
                    if rep > 0:
                        times[mode].append(dt)
        finally:
            ring.close()
            ring_r.close()
        t_c, t_d, t_p = (statistics.median(times[m]) for m in ("resident", "copy", "stream"))
        tail_bytes = L * tail_keys * (kc0.pos_stride + vc0.pos_stride)
        h = min(1.0, max(0.0, (t_c + t_d - t_p) / t_d))
        # The residency planner on the measured terms: the device memory this
        # layout uses (L windows + the ring), the measured link rate and
        # per-layer compute, the FFN weights the step reads; its window, tile,
        # slots and bounded-win prediction beside the measurement.
        bpk = kc0.pos_stride + vc0.pos_stride
        plan = P.rkv_plan_residency(L, wc + tail_keys, bpk, L * wc * bpk + nb * tile_keys * bpk,
                                    L * reps_ffn * 14336 * 4096 * 2, HBM_PEAK_GBS * 1e9, r_link * 1e9, 0.0, 0.0,
                                    t_c / L)
        return {"tail_keys": tail_keys, "tile_keys": tile_keys, "n_slots": nb, "reps": reps, "T_c_ms": round(t_c * 1e3, 3),
                "T_d_ms": round(t_d * 1e3, 3), "T_p_ms": round(t_p * 1e3, 3), "tail_hidden_fraction": round(h, 4),
                "tail_GBs": round(tail_bytes / t_p / 1e9, 2), "link_fraction": round(tail_bytes / t_p / 1e9 / r_link, 4),
                "free_zone_keys_per_layer": round(t_c * r_link * 1e9 / L / bpk),
                "planner": {"window_keys": plan["window_keys"], "tail_keys": plan["tail_keys"],
                            "tile_keys": plan["tile_keys"], "n_slots": plan["n_slots"],
                            "tactic": ["resident", "stream", "quantize"][plan["tactic"]],
                            "predicted_step_ms": round(plan["predicted_step_s"] * 1e3, 3),
                            "predicted_hidden": round(plan["predicted_hidden"], 4),
                            "t_star_MB": round(plan["t_star_bytes"] / 1e6, 1)}}

    log(f"streamed: FFN stand-in {reps} x GEMV ({t_gemv * 1e6:.1f} us each); pinned H2D {r_link:.1f} GB/s")
    main = measure(n - wc, tile)
    res = dict(main)
    res.update({"workload": "q8_0 K / q4_0 V, 40/8 heads, D 128, 131072 keys = window 65536 (HBM) + tail 65536 "
                            "(pinned host, 8192-key tiles, 3-slot ring), 48 layers, 0.2 ms FFN GEMV stand-in",
                "R_link_GBs": round(r_link, 2), "ffn_gemv_reps": reps, "ffn_ms": round(reps * t_gemv * 1e3, 4)})
    # The same layers with shorter tails (same window): the free-zone sweep,
    # each tail with one tile per layer and with 1024-key tiles; the figure
    # reported is the worst point inside the free zone.  Two longer tails at
    # 8192-key tiles show the edge of the zone.
    if quick:
        pts = [(4096, 4096)]
    else:
        pts = [(t, min(8192, t)) for t in SWEEP_TAILS] + [(t, 1024) for t in SWEEP_TAILS if t > 1024]
        pts += [(8192, 8192), (12288, 8192)]
    fz = [measure(t, tk, reps=9) for t, tk in pts]
    res["free_zone_points"] = fz
    inside = [x["tail_hidden_fraction"] for x in fz
              if x["tail_keys"] in SWEEP_TAILS and x["tail_keys"] <= x["free_zone_keys_per_layer"]]
    res["tail_hidden_fraction_in_free_zone"] = min(inside) if inside else None
    return res


def cpu_baseline(layers, desc, seconds):
    """The binary64 oracle (as it stands) on the host cores, on a bounded
    sample of the same workload: whole layers (all 40 query heads over all
    65536 keys, unsplit) cycling over the first four layers until about
    `seconds` of work; reported as effective K+V GB/s."""
    import oracle

    threads = oracle.max_threads()
    oracle.set_threads(threads)
    host = []
    for kc, vc, q in layers[:4]:
        host.append((kc.to("cpu"), vc.to("cpu"), q.cpu().numpy()))
    Hkv = desc.c.n_kv_heads
    t0 = time.perf_counter()
    done = 0
    while True:
        kh, vh, qh = host[done % len(host)]
        oracle.attend(qh, [oracle.view_of(kh, vh)], Hkv, desc.c.scale)
        done += 1
        if time.perf_counter() - t0 >= seconds or done >= 400:
            break
    dt = time.perf_counter() - t0
    kc, vc, _ = layers[0]
    layer_bytes = kc.data.numel() * kc.data.element_size() + vc.data.numel() * vc.data.element_size()
    return {
        "value": round(done * layer_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} whole layers (40 q heads x 65536 keys, f16 K/V, unsplit, binary64, cycling over "
                  f"4 layers) in {dt:.1f} s",
        "us_per_layer": round(dt / done * 1e6, 1),
        "cpu_model": cpu_model(),
        "nproc": os.cpu_count(),
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_per_config(synth):
    """The oracle timed on each of the five configurations, single-threaded and
    on all the threads it is given, each on a bounded sample of query rows (every
    sampled row attends every key of its call; the oracle is unsplit attention,
    so a call's time is the per-row time times its rows); reported as us per
    call (a layer) and effective K+V GB/s."""
    import numpy as np

    import oracle

    all_t = oracle.max_threads()
    out = {"threads_all": all_t}

    def run(name, q, views, hkv, scale, softcap, n_rows_call, bytes_call, rows1, rows_all):
        res = {}
        for label, threads, rows in (("1_thread", 1, rows1), ("all_threads", all_t, rows_all)):
            oracle.set_threads(threads)
            t0 = time.perf_counter()
            oracle.attend(q, views, hkv, scale, softcap=softcap, rows=rows)
            dt = time.perf_counter() - t0
            per_call = dt / len(rows) * n_rows_call
            res[label] = {"threads": threads, "rows_sampled": len(rows), "s": round(dt, 3),
                          "us_per_call": round(per_call * 1e6, 1), "GBs": round(bytes_call / per_call / 1e9, 4)}
        out[name] = res
        log(f"oracle {name}: 1 thread {res['1_thread']['us_per_call']:.0f} us/call, "
            f"{all_t} threads {res['all_threads']['us_per_call']:.0f} us/call")

    def host_pair(n, hkv, d, kt, vt, seed, outliers=0):
        kc = synth.make_cache(n, hkv, d, kt, synth.stream_seed(seed, 1), "cuda", outlier_channels=outliers,
                              channels_seed=synth.stream_seed(seed, 7))
        vc = synth.make_cache(n, hkv, d, vt, synth.stream_seed(seed, 2), "cuda", outlier_channels=outliers,
                              channels_seed=synth.stream_seed(seed, 7))
        return kc.to("cpu"), vc.to("cpu")

    spread = lambda n_rows, k: [int(x) for x in np.linspace(0, n_rows - 1, k).round()]
    # C1: f32 8/2 heads D 128, 4096 keys: the whole call both ways
    kc, vc = host_pair(4096, 2, 128, synth.F32, synth.F32, 1)
    q = synth.make_query(1, 8, 128, synth.stream_seed(1, 3)).numpy()
    run("c1_tiny_f32", q, [oracle.view_of(kc, vc)], 2, 1 / math.sqrt(128), 0.0, 8, 2 * 4096 * 2 * 512,
        list(range(8)), list(range(8)))
    # C2: one f16 layer, 40/8 heads, 65536 keys
    kc, vc = host_pair(65536, 8, 128, synth.F16, synth.F16, 2, outliers=10)
    q = synth.make_query(1, 40, 128, synth.stream_seed(2, 3)).numpy()
    run("c2_f16_layer", q, [oracle.view_of(kc, vc)], 8, 1 / math.sqrt(128), 0.0, 40, 268435456,
        spread(40, 2), spread(40, 2 * all_t))
    del kc, vc
    # C3: q8_0 D512, 16/2 heads, 262144 keys, softcap 30
    kc, vc = host_pair(262144, 2, 512, synth.Q8_0, synth.Q8_0, 3)
    q = synth.make_query(1, 16, 512, synth.stream_seed(3, 3)).numpy()
    run("c3_q8_d512_softcap", q, [oracle.view_of(kc, vc)], 2, 1 / math.sqrt(512), 30.0, 16, 570425344,
        [0], list(range(min(16, all_t))))
    del kc, vc
    # C4: one layer's 131072 q8_0 / q4_0 keys (window and tail attended as one), 40/8 heads
    kc, vc = host_pair(131072, 8, 128, synth.Q8_0, synth.Q4_0, 4)
    q = synth.make_query(1, 40, 128, synth.stream_seed(4, 3)).numpy()
    run("c4_q8q4_layer", q, [oracle.view_of(kc, vc)], 8, 1 / math.sqrt(128), 0.0, 40, 131072 * 8 * (136 + 72),
        spread(40, 2), spread(40, min(40, 2 * all_t)))
    del kc, vc
    # C5: 15 sequences x 32/8 heads over a 32768-key q8_0 / q4_0 prefix + 2048 private f16 keys each
    S, Hq, npre, nsuf = 15, 32, 32768, 2048
    pk, pv = host_pair(npre, 8, 128, synth.Q8_0, synth.Q4_0, 5)
    sk, sv = host_pair(S * nsuf, 8, 128, synth.F16, synth.F16, 55)
    q = synth.make_query(S, Hq, 128, synth.stream_seed(5, 3)).numpy()
    views = [oracle.view_of(pk, pv), oracle.view_of(sk, sv, 0, nsuf, nsuf * sk.pos_stride, nsuf * sv.pos_stride)]
    run("c5_shared_prefix", q, views, 8, 1 / math.sqrt(128), 0.0, S * Hq, npre * 8 * 208 + S * nsuf * 8 * 512,
        spread(S * Hq, 4), spread(S * Hq, 4 * all_t))
    oracle.set_threads(all_t)
    return out


if __name__ == "__main__":
    main()
