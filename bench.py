#!/usr/bin/env python3
"""Benchmark of the MoE token layout -> dispatch -> combine hot path on one GPU.

One step is one pass of the whole path over one synthetic batch already
resident in HBM: moe_layout, moe_dispatch, the identity expert (the combine
reads the dispatched buffer), moe_combine. The default workload is the
DeepSeek-V3-shaped layer (T=4096, D=7168, E=256, top-8, bf16, Zipf(1.1)
routing). Prints one JSON line. `value` and `ms_per_step` time K plain
steps; the per-kernel times (and the roofline of the dominant kernel) come
from a second pass of K steps with HIP events around each call (events
created without the system-scope fence by default; a third pass with torch's
default events is reported beside them).

The line also carries, under "expert_step", the expert step between dispatch
and combine (moe_grouped_gemm: one linear map per expert driven by the
device-side offsets) at the workload's expert shape, timed over its own
launches; it is not part of the step above. Under "configs" it carries the
metric's other configurations timed the same way (tiny; the padded shape at
T=3 and T=2047 of a 2048-token capacity; both 32k-token prefills; the graph
shape at T=8192, eager and as a hipGraph replay), and under "cpu_baseline"
the oracle on every host CPU the process may use ("host" gives the count).

    python bench.py [--steps K] [--warmup W] [--workload dsv3] [--expert-iters N]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E peak, GB/s
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "combine_moe_layout_05_amd", "csrc")
KERNEL_SOURCES = {
    "dispatch": ["dispatch.hip", "moe_lanes.h", "moe_kernels.h"],
    "combine": ["combine.hip", "moe_lanes.h", "moe_kernels.h"],
    "layout": ["layout.hip", "moe_kernels.h"],
    "grouped_gemm": ["grouped_gemm.hip", "moe_lanes.h", "moe_kernels.h"],
}
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 matrix-core peak
METRIC = ("dispatch+combine tokens/s and achieved HBM GB/s (% of peak), "
          "T=4096 D=7168 E=256 k=8")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class FenceFreeEvent:
    """A HIP timing event created with hipEventDisableSystemFence.

    A default event's record carries a system-scope release and acquire: the
    command processor writes back and invalidates the caches at the marker,
    and that work lands inside the interval being timed. HIP documents this
    flag for events used only for timing. The event is recorded on torch's
    current stream, the one every library call is launched on, through the
    HIP runtime torch has already loaded.
    """
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes

            import torch
            path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
            cls._hip = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so")
        return cls._hip

    def __init__(self):
        import ctypes
        self._c = ctypes
        self.ev = ctypes.c_void_p()
        rc = self._runtime().hipEventCreateWithFlags(ctypes.byref(self.ev),
                                                      ctypes.c_uint(self.DISABLE_SYSTEM_FENCE))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        import torch
        stream = self._c.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = self._runtime().hipEventRecord(self.ev, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end: "FenceFreeEvent") -> float:
        """Milliseconds from this event to `end` (both complete)."""
        ms = self._c.c_float()
        rc = self._runtime().hipEventElapsedTime(self._c.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="dsv3")
    p.add_argument("--cold-iters", type=int, default=10,
                   help="iterations of the cache-flushed per-kernel measurement (0 = skip)")
    p.add_argument("--graph-replays", type=int, default=20,
                   help="timed replays of the step captured in a hipGraph (0 = skip)")
    p.add_argument("--events", choices=["fence_free", "system"], default="fence_free",
                   help="per-kernel timing events: created with hipEventDisableSystemFence "
                        "(default) or torch's default events (system-scope fence at each record)")
    p.add_argument("--fused-steps", type=int, default=0,
                   help="also time the step with moe_layout_dispatch (0 = skip, the default: "
                        "it does not beat the separate calls on MI355X)")
    p.add_argument("--copy-reference", type=int, default=1,
                   help="1: also time a plain 1 GiB device write and copy (0 = skip)")
    p.add_argument("--cpu-single-seconds", type=float, default=3.0,
                   help="budget of the single-threaded oracle sample (0 = skip)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="budget of the oracle CPU baseline (0 = skip)")
    p.add_argument("--dispatch-segments", type=int, default=0)
    p.add_argument("--combine-segments", type=int, default=0)
    p.add_argument("--dispatch-nontemporal", type=int, default=-1,
                   help="1/0 forces dispatch's streaming stores on/off; -1 keeps the default")
    p.add_argument("--combine-nontemporal", type=int, default=-1,
                   help="1/0 forces combine's streaming loads on/off; -1 keeps the default")
    p.add_argument("--dispatch-block-waves", type=int, default=0)
    p.add_argument("--combine-block-waves", type=int, default=0)
    p.add_argument("--combine-store-nontemporal", type=int, default=-1,
                   help="1/0: streaming or ordinary stores of the combine output (-1: library default)")
    p.add_argument("--layout-launches", type=int, default=0, choices=[-1, 0, 1, 2],
                   help="1/2: force the one- or two-launch layout; -1 or 0: by size (default)")
    p.add_argument("--dispatch-store-burst", type=int, default=0, choices=[0, 1, 2],
                   help="1/2: back-to-back or paced dispatch stores; 0: library default (paced)")
    p.add_argument("--combine-backward-store", type=int, default=0, choices=[0, 1, 2],
                   help="stores of dL/dy_e in moe_combine_backward: 1 streaming, 2 ordinary, "
                        "0 the library's choice (streaming when the buffer exceeds the "
                        "last-level cache)")
    p.add_argument("--dispatch-x-nontemporal", type=int, default=0, choices=[0, 1, 2],
                   help="loads of x in dispatch: 1 streaming, 2 ordinary, 0 the library's choice "
                        "(streaming when the expert buffer is 1-4x the last-level cache)")
    p.add_argument("--backward", type=int, default=0,
                   help="also time moe_combine_backward and moe_dispatch_backward (steps)")
    p.add_argument("--expert-iters", type=int, default=10,
                   help="time the expert step (grouped GEMM) over this many launches; 0 skips")
    p.add_argument("--ceiling-iters", type=int, default=20,
                   help="time the combine beside its no-arithmetic traffic probes (0 = skip)")
    p.add_argument("--configs", type=int, default=1,
                   help="1: also time the other configurations of the metric (tiny, padded "
                        "T=3 and 2047, both 32k prefills, the graph shape eager and replayed)")
    p.add_argument("--config-steps", type=int, default=20,
                   help="timed steps (and replays) per configuration")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="only run plain device write/read/copy of this size (HBM ceiling, "
                        "counter scaling)")
    return p.parse_args()


def bytes_per_token(w, kind: str) -> int:
    """Algorithmic HBM bytes per token (every routed slot has an expert).
    layout:   read ids (4K), write row_map (4K) and src_map (4K)
    dispatch: read x row, row_map (4K), scores (4K); write K rows, s_e (4K)
    combine:  read K rows, row_map (4K), scores (4K); write one row"""
    eb = 2 if w.dtype == "bf16" else 4
    row = w.D * eb
    K = w.K
    return {"layout": 12 * K,
            "dispatch": row * (K + 1) + 12 * K,
            "combine": row * (K + 1) + 8 * K,
            # read dL/dy row and K expert rows, write K scaled rows; row_map,
            # scores in, dL/dscores out
            "combine_backward": row * (2 * K + 1) + 12 * K,
            # read K rows, write one; row_map in
            "dispatch_backward": row * (K + 1) + 4 * K}[kind]


def source_digest(kind: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_traffic(kind: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this kernel and workload, or None when there is none or the kernel
    source changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{kind}_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != source_digest(kind):
        return None
    return rec.get("hbm_bytes_per_launch")


def device_copy_rates(mib: int = 1024, reps: int = 10) -> dict:
    """Rates of a plain device write (torch fill_) and copy (HIP copyBuffer
    through torch copy_) of `mib` MiB, timed like the path's kernels: a
    reference for what a plain streaming kernel reaches on this GPU."""
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    res = {"bytes": n}
    for name, fn, nbytes in (("write", lambda: a.fill_(3), n), ("copy", lambda: b.copy_(a), 2 * n)):
        e0, e1 = FenceFreeEvent(), FenceFreeEvent()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        res[f"{name}_gbps"] = round(nbytes / (us * 1e-6) / 1e9, 1)
    del a, b
    torch.cuda.empty_cache()
    return res


def calibrate_copy(mib: int) -> None:
    """Plain device write, read and copy of `mib` MiB through torch's own
    kernels: the rates a streaming kernel can reach on this GPU, and (under
    rocprofv3 counters) the bytes the counters report for a known size."""
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    b.fill_(2)
    torch.cuda.synchronize()
    res = {"calibration": "device write/read/copy", "bytes": n}
    ops = {"write": (lambda: a.fill_(3), n),
           "read": (lambda: a.view(torch.float32).sum(), n),
           "copy": (lambda: b.copy_(a), 2 * n)}
    for name, (fn, nbytes) in ops.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        res[name] = {"us": round(us, 2), "gbps": round(nbytes / (us * 1e-6) / 1e9, 1)}
    print(json.dumps(res), flush=True)


def expert_algorithmic_bytes(counts, k_in: int, n_out: int) -> int:
    """Algorithmic HBM bytes of one expert-step launch: the weights of every
    expert with rows (each read once), the rows in (k_in bf16) and out (n_out
    bf16), and the offsets."""
    used = int((counts > 0).sum())
    total = int(counts.sum())
    return used * n_out * k_in * 2 + total * (k_in + n_out) * 2 + (counts.size + 1) * 4


def time_expert_step(args, w, disp, ids, x, s, ntpr, dev) -> dict:
    import numpy as np
    import torch

    import workloads
    from combine_moe_layout_05_amd import grouped_gemm, round_up4, tile_expert_weights

    sh = workloads.EXPERT_SHAPES[w.name]
    k_in, n_out = sh["k_in"], sh["n_out"]
    log(f"expert step: {w.E} experts {k_in} -> {n_out}, weights {w.E * n_out * k_in * 2 / 1e9:.1f} GB")
    wts = workloads.expert_weights(w.E, n_out, k_in, sh["seed"])
    wd = torch.from_numpy(wts.view(np.int16)).to(dev).view(torch.bfloat16)
    del wts
    # the weights are static: tiled once for the matrix cores, outside the timing
    wt = tile_expert_weights(wd)
    del wd
    lay = disp.layout(ids, ntpr)
    disp.dispatch(x, s, ids, lay.counts, num_tokens_per_rank=ntpr)
    rows = round_up4(ntpr) * w.K
    x_e = disp.x_e[:rows]
    out = torch.empty((rows, n_out), dtype=torch.bfloat16, device=dev)
    for _ in range(2):
        grouped_gemm(x_e, wt, lay.offsets, out)
    stream = torch.cuda.current_stream(dev)        # the stream the launches go to
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.expert_iters + 1)]
    ev[0].record(stream)
    for i in range(args.expert_iters):
        grouped_gemm(x_e, wt, lay.offsets, out)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    us = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(args.expert_iters)])) * 1e3
    counts = lay.counts.cpu().numpy()
    per_launch = expert_algorithmic_bytes(counts, k_in, n_out)
    flops = 2.0 * int(counts.sum()) * k_in * n_out
    achieved = per_launch / (us * 1e-6) / 1e9
    tflops = flops / (us * 1e-6) / 1e12
    del wt, out
    torch.cuda.empty_cache()
    log(f"expert step {us:.1f} us: {achieved:.0f} GB/s, {tflops:.0f} TFLOP/s")
    # Bound by arithmetic intensity against the ridge peak_flops / peak_bytes.
    if flops / per_launch > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9):
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                "algorithmic_flops_per_launch": flops}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4)}
    roof.update({"traffic": counter_traffic("grouped_gemm", w.name), "kernel": "grouped_gemm",
                 "algorithmic_bytes_per_launch": per_launch})
    return {
        "workload": f"{w.name} experts: {w.E} x ({k_in} -> {n_out}) bf16, "
                    f"{int(counts.sum())} routed rows in {int((counts > 0).sum())} experts",
        "weights": "tiled (moe_tile_expert_weights, once, untimed)",
        "launches": args.expert_iters,
        "avg_launch_us": round(us, 2),
        "roofline": roof,
        "hbm_gbps": round(achieved, 1),
        "tflops": round(tflops, 1),
        "frac_of_bf16_dense_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
    }


def load_batch(w, dev, T=None):
    """Seeded synthetic batch of workload w on the device: (x, ids, scores,
    host batch). With T, the first T rows of the workload's batch."""
    import numpy as np
    import torch

    import workloads
    b = workloads.make_batch(w)
    if T is not None:
        b = {k: v[:T] for k, v in b.items()}
    if w.dtype == "bf16":
        x = torch.from_numpy(np.ascontiguousarray(b["x"]).view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        x = torch.from_numpy(np.ascontiguousarray(b["x"])).to(dev)
    ids = torch.from_numpy(np.ascontiguousarray(b["ids"])).to(dev)
    s = torch.from_numpy(np.ascontiguousarray(b["scores"])).to(dev)
    return x, ids, s, b


def make_step(disp, x, ids, s, ntpr):
    """One pass of the path: layout, dispatch, identity expert, combine. With
    a list of 4 events, each call is bracketed by event records."""
    def step(ev=None):
        if ev is not None:
            ev[0].record()
        lay = disp.layout(ids, ntpr)
        if ev is not None:
            ev[1].record()
        disp.dispatch(x, s, ids, lay.counts, num_tokens_per_rank=ntpr)
        if ev is not None:
            ev[2].record()
        disp.combine(disp.x_e, lay.row_map, s, num_tokens_per_rank=ntpr)
        if ev is not None:
            ev[3].record()
    return step


def time_plain(step, steps: int) -> float:
    """Milliseconds per step over `steps` back-to-back steps, no events."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def time_events(step, steps: int, make_event):
    """Per-kernel milliseconds (layout, dispatch, combine lists) and the
    wall milliseconds per step of a pass with events around each call."""
    import torch
    events = [[make_event() for _ in range(4)] for _ in range(steps)]
    t_ev = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    per_step = (time.perf_counter() - t_ev) * 1e3 / steps
    return ([e[0].elapsed_time(e[1]) for e in events],
            [e[1].elapsed_time(e[2]) for e in events],
            [e[2].elapsed_time(e[3]) for e in events], per_step)


def time_graph(step, replays: int, dev, steps_per_graph: int = 1) -> float:
    """Microseconds per step of a hipGraph holding `steps_per_graph` steps,
    over `replays` replays (warmed up on a side stream first, as capture
    requires). Each graph launch costs a fixed few microseconds on the host
    and the GPU, which a graph holding more work pays once."""
    import torch
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps_per_graph):
            step()
    g.replay()
    torch.cuda.synchronize()
    t_g = time.perf_counter()
    for _ in range(replays):
        g.replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t_g) * 1e6 / (replays * steps_per_graph)
    del g
    return us


# The five configurations of the metric, each timed in the same run as the
# headline: (key, workload, materialized T or None for the workload's T,
# whether a graph replay is timed too, whether the roofline fraction means
# anything at that size).
CONFIGS = (
    ("tiny", "tiny", None, False, False),
    ("padded_T3", "padded", 3, False, False),
    ("padded_T2047", "padded", 2047, False, True),
    ("prefill32k_uniform", "prefill32k_uniform", None, False, True),
    ("prefill32k_zipf", "prefill32k_zipf", None, False, True),
    ("graph_T8192", "graph", None, True, True),
)


def measure_config(key, wname, T, graph, meaningful, steps, warmup, dev, make_event) -> dict:
    """Tokens/s, per-kernel times and dispatch+combine GB/s (and fraction of
    the HBM peak) of one configuration, timed like the headline."""
    import gc

    import numpy as np
    import torch

    import workloads
    from combine_moe_layout_05_amd import MoeDispatcher

    w = workloads.WORKLOADS[wname]
    T = w.T if T is None else T
    log(f"config {key}: T={T} ntpr={w.ntpr} nmax={w.nmax} D={w.D} E={w.E} K={w.K} {w.dtype}")
    x, ids, s, _ = load_batch(w, dev, T if T != w.T else None)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    disp = MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=dt, device=dev)
    step = make_step(disp, x, ids, s, w.ntpr)
    for _ in range(warmup):
        step()
    ms = time_plain(step, steps)
    lay_ms, dis_ms, com_ms, _ = time_events(step, steps, make_event)
    kus = {"layout": float(np.mean(lay_ms)) * 1e3, "dispatch": float(np.mean(dis_ms)) * 1e3,
           "combine": float(np.mean(com_ms)) * 1e3}
    dc_us = kus["dispatch"] + kus["combine"]
    dc_bytes = (bytes_per_token(w, "dispatch") + bytes_per_token(w, "combine")) * T
    out = {"workload": wname, "T": T, "num_tokens_per_rank": w.ntpr,
           "num_max_tokens_per_rank": w.nmax, "D": w.D, "E": w.E, "K": w.K, "dtype": w.dtype,
           "routing": w.routing + (f"(s={w.zipf_s})" if w.routing == "zipf" else ""),
           "steps": steps, "step_us": round(ms * 1e3, 2),
           "tokens_per_s": round(T / (ms * 1e-3), 1),
           "kernels_us": {k: round(v, 2) for k, v in kus.items()},
           "dispatch_combine_us": round(dc_us, 2),
           "dispatch_combine_bytes": dc_bytes}
    if meaningful:
        gbps = dc_bytes / (dc_us * 1e-6) / 1e9
        out["dispatch_combine_gbps"] = round(gbps, 1)
        out["frac_of_peak"] = round(gbps / PEAK_HBM_GBPS, 4)
    else:
        out["note"] = "latency-bound size: microseconds only, no roofline fraction"
    if graph:
        g_us = time_graph(step, steps, dev)
        out["graph_replay_us"] = round(g_us, 2)
        out["graph_tokens_per_s"] = round(T / (g_us * 1e-6), 1)
    # Ten steps per graph: the per-launch cost amortized, as in a captured
    # layer; at the small shapes this is the GPU-side step latency.
    g10 = time_graph(step, max(2, steps // 5), dev, steps_per_graph=10)
    out["graph_10_steps_us_per_step"] = round(g10, 2)
    log(f"config {key}: step {out['step_us']:.1f} us, dispatch+combine {dc_us:.1f} us"
        + (f" ({out['frac_of_peak'] * 100:.1f} % of peak)" if meaningful else "")
        + (f", graph replay {out['graph_replay_us']:.1f} us" if graph else ""))
    del disp, x, ids, s, step
    gc.collect()
    torch.cuda.empty_cache()
    return out


def combine_ceiling(disp, x, ids, s, w, dev, make_event, iters: int) -> dict:
    """The combine beside kernels that move its exact HBM traffic with no
    arithmetic (libmoe_traffic_probe.so): the gather-copy (same reads, same
    launch shape, the XOR of the K rows stored), the same reads with no
    store, the same read:write byte ratio in sequential order, and a plain
    sequential read of the same bytes; and dispatch beside a sequential
    stream of its own byte ratio (1 read : 8 written). Each is
    timed by fence-free events both right after layout + dispatch (the
    step's context: dispatch's writes are still draining) and after a 1 GiB
    read has evicted the caches ("cold")."""
    import ctypes

    import numpy as np
    import torch

    from combine_moe_layout_05_amd._paths import PROBE_LIB_PATH

    if not os.path.exists(PROBE_LIB_PATH):
        raise RuntimeError(f"{PROBE_LIB_PATH} is not built")
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.probe_gather_copy.argtypes = [vp, vp, i32, i32, i32, i64, vp, vp, ctypes.c_int, vp]
    lib.probe_stream.argtypes = [ctypes.c_int, vp, vp, i64, vp, vp]
    ntpr = w.ntpr
    rows = (w.ntpr + 3) // 4 * 4 * w.K
    chunks = w.D * (2 if w.dtype == "bf16" else 4) // 16
    out = torch.empty((w.T, w.D), dtype=disp.dtype, device=dev)
    sink = torch.full((4,), 0x7FC17FC1, dtype=torch.int32, device=dev)
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sinkf = torch.empty((), dtype=torch.float32, device=dev)
    stream = lambda: torch.cuda.current_stream(dev).cuda_stream  # noqa: E731
    lay = disp.layout(ids, ntpr)

    def gather(store):
        rc = lib.probe_gather_copy(disp.x_e.data_ptr(), lay.row_map.data_ptr(), w.T, w.K, chunks,
                                   rows, out.data_ptr(), sink.data_ptr(), store, stream())
        if rc != 0:
            raise RuntimeError(f"probe_gather_copy failed ({rc})")

    read_bytes = w.T * w.K * chunks * 16

    def streaming(kind):
        rc = lib.probe_stream(kind, disp.x_e.data_ptr(), out.data_ptr(), read_bytes,
                              sink.data_ptr(), stream())
        if rc != 0:
            raise RuntimeError(f"probe_stream failed ({rc})")

    kernels = {
        "combine": lambda: disp.combine(disp.x_e, lay.row_map, s, num_tokens_per_rank=ntpr),
        "gather_copy": lambda: gather(1),
        "gather_read": lambda: gather(0),
        "sequential_mix": lambda: streaming(2),
        "sequential_read": lambda: streaming(0),
    }
    res = {}
    for name, fn in kernels.items():
        for where in ("step", "cold"):
            us = []
            for i in range(iters + 2):
                if where == "step":
                    lay2 = disp.layout(ids, ntpr)
                    disp.dispatch(x, s, ids, lay2.counts, num_tokens_per_rank=ntpr)
                else:
                    torch.sum(scratch, dim=0, out=sinkf)
                e0, e1 = make_event(), make_event()
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                if i >= 2:
                    us.append(e0.elapsed_time(e1) * 1e3)
            res[f"{name}_{where}_us"] = round(float(np.median(us)), 2)
    # Dispatch beside the same bytes in sequential order (one 1 KiB read
    # written to eight consecutive KiB): in a step it follows the previous
    # step's combine and this step's layout.
    x_bytes = w.T * chunks * 16

    def seq_1to8():
        rc = lib.probe_stream(3, x.data_ptr(), disp.x_e.data_ptr(), x_bytes, sink.data_ptr(),
                              stream())
        if rc != 0:
            raise RuntimeError(f"probe_stream failed ({rc})")

    dkernels = {"dispatch": lambda: disp.dispatch(x, s, ids, lay.counts, num_tokens_per_rank=ntpr),
                "sequential_1to8": seq_1to8}
    for name, fn in dkernels.items():
        for where in ("step", "cold"):
            us = []
            for i in range(iters + 2):
                if where == "step":
                    disp.combine(disp.x_e, lay.row_map, s, num_tokens_per_rank=ntpr)
                    disp.layout(ids, ntpr)
                else:
                    disp.layout(ids, ntpr)
                    torch.sum(scratch, dim=0, out=sinkf)
                e0, e1 = make_event(), make_event()
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                if i >= 2:
                    us.append(e0.elapsed_time(e1) * 1e3)
            res[f"{name}_{where}_us"] = round(float(np.median(us)), 2)
    res["combine_over_gather_copy_step"] = round(res["combine_step_us"] / res["gather_copy_step_us"], 4)
    res["combine_over_gather_copy_cold"] = round(res["combine_cold_us"] / res["gather_copy_cold_us"], 4)
    res["dispatch_over_sequential_1to8_step"] = round(
        res["dispatch_step_us"] / res["sequential_1to8_step_us"], 4)
    res["dispatch_over_sequential_1to8_cold"] = round(
        res["dispatch_cold_us"] / res["sequential_1to8_cold_us"], 4)
    res["bytes"] = {"combine_and_gather_copy": bytes_per_token(w, "combine") * w.T,
                    "gather_read": read_bytes, "sequential_mix": read_bytes + read_bytes // 8,
                    "sequential_read": read_bytes, "dispatch": bytes_per_token(w, "dispatch") * w.T,
                    "sequential_1to8": 9 * x_bytes}
    del out, scratch
    torch.cuda.empty_cache()
    return res


def host_cores() -> dict:
    """Host CPUs this process may run on, with the cgroup CPU quota if one
    is set (cgroup v2 cpu.max)."""
    rec = {"affinity": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count(),
           "cgroup_quota_cpus": None}
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        if quota != "max":
            rec["cgroup_quota_cpus"] = round(int(quota) / int(period), 2)
    except (OSError, ValueError):
        pass
    return rec


def main() -> int:
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); this path has no multi-GPU mode.", file=sys.stderr, flush=True)
        return 2
    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib)
        return 0

    import numpy as np
    import torch

    import workloads
    from combine_moe_layout_05_amd import MoeDispatcher, load

    load()                                   # fails loudly if the library is not built
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda", 0)
    w = workloads.WORKLOADS[args.workload]
    log(f"workload {w.name}: T={w.T} D={w.D} E={w.E} K={w.K} {w.dtype} {w.routing}")
    x, ids, s, b = load_batch(w, dev)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    disp = MoeDispatcher(w.nmax, w.D, w.E, w.K, dtype=dt, device=dev,
                         backward=args.backward > 0)
    disp.set_tuning(args.dispatch_segments, args.combine_segments,
                    bool(args.dispatch_nontemporal) if args.dispatch_nontemporal >= 0 else None,
                    bool(args.combine_nontemporal) if args.combine_nontemporal >= 0 else None,
                    args.dispatch_block_waves, args.combine_block_waves,
                    bool(args.combine_store_nontemporal) if args.combine_store_nontemporal >= 0
                    else None, args.layout_launches, args.dispatch_store_burst,
                    args.combine_backward_store, args.dispatch_x_nontemporal)
    tuning = disp.get_tuning()
    ntpr = w.ntpr
    step = make_step(disp, x, ids, s, ntpr)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The timed region: K steps exactly as a caller runs them, no
    # instrumentation. The per-kernel times come from a second pass of K
    # steps with HIP events recorded around each call on the launch stream
    # (the event records add a few microseconds per step, so that pass is
    # reported separately and does not set `value`).
    K = args.steps
    log(f"timed {K} steps")
    elapsed = time_plain(step, K) * K * 1e-3

    def timed_pass(make_event):
        return time_events(step, K, make_event)

    def torch_event():
        return torch.cuda.Event(enable_timing=True)

    main_event, other_event = ((FenceFreeEvent, torch_event) if args.events == "fence_free"
                               else (torch_event, FenceFreeEvent))
    log(f"{K} steps with per-kernel events ({args.events})")
    lay_ms, dis_ms, com_ms, ms_per_step_events = timed_pass(main_event)
    # The same pass with the other kind of event, reported for comparison.
    o_lay, o_dis, o_com, o_step = timed_pass(other_event)
    other_kind = "system" if args.events == "fence_free" else "fence_free"
    other_events = {"events": other_kind, "step_us": round(o_step * 1e3, 2),
                    "kernels_us": {"layout": round(float(np.mean(o_lay)) * 1e3, 2),
                                   "dispatch": round(float(np.mean(o_dis)) * 1e3, 2),
                                   "combine": round(float(np.mean(o_com)) * 1e3, 2)}}
    ms_per_step = elapsed * 1e3 / K
    value = w.T * K / elapsed
    avg = {"layout": float(np.mean(lay_ms)), "dispatch": float(np.mean(dis_ms)),
           "combine": float(np.mean(com_ms))}
    gbps = {k: bytes_per_token(w, k) * w.T / (avg[k] * 1e-3) / 1e9 for k in avg}
    dc_ms = avg["dispatch"] + avg["combine"]
    dc_bytes = (bytes_per_token(w, "dispatch") + bytes_per_token(w, "combine")) * w.T
    log(f"step {ms_per_step * 1e3:.1f} us; layout {avg['layout'] * 1e3:.1f} us, "
        f"dispatch {avg['dispatch'] * 1e3:.1f} us ({gbps['dispatch']:.0f} GB/s), "
        f"combine {avg['combine'] * 1e3:.1f} us ({gbps['combine']:.0f} GB/s)")

    # The same step captured once into a hipGraph and replayed: the launch
    # gaps between the kernels disappear.
    graph_us = graph10_us = None
    if args.graph_replays > 0:
        log(f"graph capture of one step, {args.graph_replays} timed replays")
        graph_us = time_graph(step, args.graph_replays, dev)
        graph10_us = time_graph(step, max(2, args.graph_replays // 5), dev, steps_per_graph=10)
        log(f"graph replay {graph_us:.1f} us per step; ten steps per graph {graph10_us:.1f} us per step")

    # The same step with the layout fused into dispatch (moe_layout_dispatch:
    # two launches instead of three), timed the same way; reported beside the
    # separate calls, which remain the measured step.
    fused = None
    if args.fused_steps > 0:
        log(f"fused layout+dispatch step, {args.fused_steps} timed steps")

        def fused_step():
            lay, dsp = disp.layout_dispatch(x, s, ids, num_tokens_per_rank=ntpr)
            disp.combine(dsp.x_e, lay.row_map, s, num_tokens_per_rank=ntpr)

        for _ in range(args.warmup):
            fused_step()
        torch.cuda.synchronize()
        t_f = time.perf_counter()
        for _ in range(args.fused_steps):
            fused_step()
        torch.cuda.synchronize()
        fused_us = (time.perf_counter() - t_f) * 1e6 / args.fused_steps
        fused = {"step_us": round(fused_us, 2),
                 "vs_separate_step": round(fused_us / (ms_per_step * 1e3), 4)}
        # the separate calls once more, right after, against drift
        t_s = time.perf_counter()
        for _ in range(args.fused_steps):
            step()
        torch.cuda.synchronize()
        fused["separate_step_us_after"] = round((time.perf_counter() - t_s) * 1e6 /
                                                args.fused_steps, 2)
        log(f"fused step {fused_us:.1f} us")

    # Cold-cache per-kernel times: a 1 GiB read evicts L2 and the MALL
    # before each timed kernel (outside the timed interval); a read leaves
    # clean lines, so no write-back of the flush lands in the timed kernel.
    cold = None
    if args.cold_iters > 0:
        log(f"cold-cache per-kernel timing, {args.cold_iters} iterations")
        scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        sink = torch.empty((), dtype=torch.float32, device=dev)
        cd, cc = [], []
        for i in range(args.cold_iters):
            lay = disp.layout(ids, ntpr)
            torch.sum(scratch, dim=0, out=sink)
            e0, e1 = main_event(), main_event()
            e0.record()
            disp.dispatch(x, s, ids, lay.counts, num_tokens_per_rank=ntpr)
            e1.record()
            torch.sum(scratch, dim=0, out=sink)
            e2, e3 = main_event(), main_event()
            e2.record()
            disp.combine(disp.x_e, lay.row_map, s, num_tokens_per_rank=ntpr)
            e3.record()
            torch.cuda.synchronize()
            cd.append(e0.elapsed_time(e1))
            cc.append(e2.elapsed_time(e3))
        del scratch
        cold = {"dispatch_us": float(np.median(cd)) * 1e3,
                "combine_us": float(np.median(cc)) * 1e3}
        cold["dispatch_gbps"] = bytes_per_token(w, "dispatch") * w.T / (cold["dispatch_us"] * 1e-6) / 1e9
        cold["combine_gbps"] = bytes_per_token(w, "combine") * w.T / (cold["combine_us"] * 1e-6) / 1e9
        log(f"cold: dispatch {cold['dispatch_us']:.1f} us, combine {cold['combine_us']:.1f} us")

    backward = None
    if args.backward > 0:
        log(f"backward: {args.backward} timed steps")
        gy = torch.randn((w.T, w.D), generator=torch.Generator(device=dev).manual_seed(5),
                         device=dev).to(dt)
        lay = disp.layout(ids, ntpr)
        disp.dispatch(x, s, ids, lay.counts, num_tokens_per_rank=ntpr)
        bev = [[main_event() for _ in range(3)]
               for _ in range(args.backward + 2)]
        for e in bev:
            e[0].record()
            g_e, _ = disp.combine_backward(gy, disp.x_e, lay.row_map, s, num_tokens_per_rank=ntpr)
            e[1].record()
            disp.dispatch_backward(g_e, lay.row_map, w.T, num_tokens_per_rank=ntpr)
            e[2].record()
        torch.cuda.synchronize()
        cb = float(np.mean([e[0].elapsed_time(e[1]) for e in bev[2:]])) * 1e3
        db = float(np.mean([e[1].elapsed_time(e[2]) for e in bev[2:]])) * 1e3
        backward = {"combine_backward_us": round(cb, 2), "dispatch_backward_us": round(db, 2),
                    "both_us": round(cb + db, 2),
                    "combine_backward_store": "streaming" if tuning["combine_backward_store"] == 1
                    else "ordinary",
                    "combine_backward_gbps": round(bytes_per_token(w, "combine_backward") * w.T
                                                   / (cb * 1e-6) / 1e9, 1),
                    "dispatch_backward_gbps": round(bytes_per_token(w, "dispatch_backward") * w.T
                                                    / (db * 1e-6) / 1e9, 1)}
        log(f"backward: combine_backward {cb:.1f} us, dispatch_backward {db:.1f} us")

    ceiling = None
    if args.ceiling_iters > 0:
        log(f"combine beside its traffic probes, {args.ceiling_iters} iterations each")
        ceiling = combine_ceiling(disp, x, ids, s, w, dev, main_event, args.ceiling_iters)
        log(f"combine {ceiling['combine_step_us']:.1f} us against the gather-copy "
            f"{ceiling['gather_copy_step_us']:.1f} us in the step, "
            f"{ceiling['combine_cold_us']:.1f} / {ceiling['gather_copy_cold_us']:.1f} us cold")

    expert = None
    if args.expert_iters > 0 and w.name in workloads.EXPERT_SHAPES:
        expert = time_expert_step(args, w, disp, ids, x, s, ntpr, dev)

    dominant = "dispatch" if avg["dispatch"] >= avg["combine"] else "combine"
    per_launch = bytes_per_token(w, dominant) * w.T
    achieved = per_launch / (avg[dominant] * 1e-3) / 1e9
    traffic = counter_traffic(dominant, w.name)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                "traffic": traffic, "kernel": dominant,
                "algorithmic_bytes_per_launch": per_launch,
                "avg_launch_us": round(avg[dominant] * 1e3, 2)}

    def oracle_rate(threads: int, budget_s: float) -> dict:
        import oracle
        log(f"oracle CPU baseline on {threads} thread(s), ~{budget_s:.0f} s")
        n, t_start = 0, time.perf_counter()
        while True:
            oracle.run_pipeline(b["x"], b["ids"], b["scores"], w.T, ntpr, w.E, w.K,
                                nthreads=threads)
            n += 1
            if time.perf_counter() - t_start >= budget_s:
                break
        cpu_s = time.perf_counter() - t_start
        rate = w.T * n / cpu_s
        return {"value": round(rate, 1), "unit": "tokens/s", "cores": threads,
                "kind": "oracle",
                "gbps": round(rate * (bytes_per_token(w, "dispatch") +
                                      bytes_per_token(w, "combine")) / 1e9, 2),
                "sample": f"{n} full {w.name} batches (T={w.T}) through the oracle's "
                          f"layout+dispatch+combine, {cpu_s:.1f} s; gbps counts the "
                          f"dispatch+combine algorithmic bytes"}

    ref = None
    if args.copy_reference:
        log("device write/copy reference, 1 GiB")
        ref = device_copy_rates()
        ref["dispatch_combine_over_copy"] = round(
            dc_bytes / (dc_ms * 1e-3) / 1e9 / ref["copy_gbps"], 4)

    # The five configurations, each timed like the headline (the headline's
    # own workload is the line's top level).
    configs = None
    if args.configs:
        configs = {}
        for key, wname, T, graph, meaningful in CONFIGS:
            if wname == w.name and T is None:
                continue
            configs[key] = measure_config(key, wname, T, graph, meaningful, args.config_steps,
                                          args.warmup, dev, main_event)

    host = host_cores()
    cpu = None
    if args.cpu_seconds > 0:
        # every host CPU this process may run on
        cpu = oracle_rate(max(1, host["affinity"]), args.cpu_seconds)
    cpu_single = oracle_rate(1, args.cpu_single_seconds) if args.cpu_single_seconds > 0 else None

    def interval_stats(ms) -> dict:
        us = np.asarray(ms, dtype=np.float64) * 1e3
        return {"mean": round(float(us.mean()), 2), "median": round(float(np.median(us)), 2),
                "min": round(float(us.min()), 2), "p90": round(float(np.percentile(us, 90)), 2)}

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "D": w.D, "E": w.E, "K": w.K,
                   "num_tokens_per_rank": w.ntpr, "num_max_tokens_per_rank": w.nmax,
                   "routing": w.routing + (f"(s={w.zipf_s})" if w.routing == "zipf" else ""),
                   "scores": w.scores, "parallelism": "single-gpu", "tuning": tuning},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_baseline_single_thread": cpu_single,
        "kernels_us": {k: round(v * 1e3, 2) for k, v in avg.items()},
        "kernels_gbps": {k: round(v, 1) for k, v in gbps.items()},
        "kernels_us_stats": {"layout": interval_stats(lay_ms), "dispatch": interval_stats(dis_ms),
                             "combine": interval_stats(com_ms)},
        "dispatch_combine": {
            "us": round(dc_ms * 1e3, 2),
            "tokens_per_s": round(w.T / (dc_ms * 1e-3), 1),
            "gbps": round(dc_bytes / (dc_ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(dc_bytes / (dc_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        },
        "cold_cache": cold,
        "device_copy_reference": ref,
        "graph_replay_us_per_step": None if graph_us is None else round(graph_us, 2),
        "graph_10_steps_us_per_step": None if graph10_us is None else round(graph10_us, 2),
        "ms_per_step_with_kernel_events": round(ms_per_step_events, 4),
        "kernel_events": args.events,
        "kernels_with_other_events": other_events,
        "fused_layout_dispatch": fused,
        "backward": backward,
        "expert_step": expert,
        "combine_ceiling": ceiling,
        "configs": configs,
        "host": host,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
