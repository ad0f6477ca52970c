"""Benchmark of the GDN spec-verify layer step on one MI355X.

One step = one gdn_spec_attention call (conv + ring roll, gates, norms, the
gated delta rule with per-token state snapshots) over the Qwen3-Next-shaped
batch: 64 spec rows, K=3 tokens each, 16 k-heads / 32 v-heads, dk=dv=128,
fp32 states in a 512-slot pool.  Steps cycle over several independent layers
(each with its own pools and inputs, as consecutive GDN layers of a model
have), so no step finds the previous step's states in the last-level cache.

Prints one JSON line: tokens/s, us per layer, achieved HBM bandwidth of the
kernel against the 8 TB/s MI355X peak, and the CPU oracle timed on a bounded
sample of the same workload (one thread, then all the host's threads).
Each timed region starts behind a short GPU spin queued after the
synchronisation: the host launches the first steps while the GPU spins, so
the region holds the steps' GPU time and not the host's latency to launch
the first one onto an idle stream (on a 20-step region that latency adds
about 1.5 us to every step).  The same steps timed from an idle stream are
reported beside it.
Beside the headline mean over the timed region: the median, p10 and p90 of
one series of the same steps (an event between consecutive calls), a
labelled "hot" series (one layer back to back), and a measured same-GPU
ceiling for the step's state traffic (a kernel that only reads each row's
state blocks and writes them to the store slots, on the same layers and
metadata).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN layer tokens/sec + us/layer + % HBM peak, spec verify K=3, batch 64"
HBM_PEAK_GBS = 8000.0
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_gdn_rows_qwen3next_k3_b64.json")


DEFAULT_WORKLOAD = "qwen3next_k3_b64"
# Spin queued ahead of a timed region's first event (GPU clock cycles; about
# 0.4 ms at 2.4 GHz, far longer than the host needs to launch one step).
LEAD_CYCLES = 1_000_000


def algorithmic_bytes(case) -> int:
    """Bytes the spec step must move, counted from the batch's metadata."""
    d, sp = case["dims"], case["spec"]
    Hk, Hv, dk, dv, W, L = d["Hk"], d["Hv"], d["dk"], d["dv"], d["W"], d["L"]
    C = 2 * Hk * dk + Hv * dv
    T = sp["num_spec_tokens"]
    tile = Hv * dv * dk * 4
    total = T * C * 2 + 2 * T * Hv * 2 + T * Hv * dv * 2      # qkv, a+b, out
    total += C * W * 2 + 2 * Hv * 4                            # conv weight, A_log, dt_bias
    sq, ssi, nacc = sp["spec_query_start_loc"], sp["spec_state_indices"], sp["num_accepted_tokens"]
    for b in range(sp["num_spec_decodes"]):
        Tb = int(sq[b + 1] - sq[b])
        n = int(nacc[b])
        cs = int(sp["spec_cache_indices"][b]) if sp.get("spec_cache_indices") is not None \
            else int(ssi[b][0])
        if d.get("conv_layout", 0) == 1:
            # per-token slots: the window of slot ssi[n-1], a window per stored token
            if ssi[b][n - 1] > 0:
                total += (W - 1) * C * 2
            total += sum((W - 1) * C * 2 for t in range(Tb) if ssi[b][t] > 0)
        elif cs > 0:
            read_cols = set(range(n - 1, n - 1 + W - 1)) | set(range(n, n + max(L - Tb, 0)))
            total += (len(read_cols) + L) * C * 2               # ring read + rewrite
        if ssi[b][n - 1] > 0:
            total += tile                                       # state load
        total += sum(tile for t in range(Tb) if ssi[b][t] > 0)  # per-token stores
    total += 4 * (sp["num_spec_decodes"] + 1) + 4 * ssi.size + 4 * sp["num_spec_decodes"]
    if sp.get("spec_token_indx") is not None:
        total += 4 * T
    return int(total)


def nonspec_bytes(case) -> int:
    """Bytes the non-spec rows must move (decodes and prefills): inputs,
    gates and outputs of their tokens, ring read/rewrite, the initial state
    when it is read and the final state."""
    d, ns = case["dims"], case["nonspec"]
    Hk, Hv, dk, dv, W, L = d["Hk"], d["Hv"], d["dk"], d["dv"], d["W"], d["L"]
    C = 2 * Hk * dk + Hv * dv
    tile = Hv * dv * dk * 4
    T = ns["num_non_spec_tokens"]
    total = T * C * 2 + 2 * T * Hv * 2 + T * Hv * dv * 2 + 4 * T
    qsl, slots = ns["query_start_loc"], ns["cache_indices"]
    his = ns.get("has_initial_state")
    for i in range(ns["num_decodes"] + ns["num_prefills"]):
        Ti = int(qsl[i + 1] - qsl[i])
        c = int(slots[i])
        init = (his is None or his[i]) and c > 0
        if c > 0:
            total += ((W - 1 + max(L - Ti, 0)) if init else 0) * C * 2 + L * C * 2 + tile
        if init:
            total += tile
    return int(total)


def chunked_flops(case) -> int:
    """Multiply-adds x 2 of the chunked prefill form (64-token chunks)."""
    d, ns = case["dims"], case["nonspec"]
    Hv, dk, dv = d["Hv"], d["dk"], d["dv"]
    qsl = ns["query_start_loc"]
    total = 0
    for i in range(ns["num_decodes"], ns["num_decodes"] + ns["num_prefills"]):
        nch = -(-int(qsl[i + 1] - qsl[i]) // 64)
        # K K^T, Q K^T, W, U~ (prep); W S^T, Q S^T, P U, state update (state pass)
        per = 2 * 64 * 64 * dk + 64 * 64 * (dk + dv) + 64 * dk * dv * 3 + 64 * 64 * dv
        total += 2 * nch * Hv * per
    return int(total)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _host_threads():
    """Threads this process may use: its CPU affinity (else the CPU count),
    capped by OMP_NUM_THREADS when that is set (the host's share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    return max(1, min(n, int(cap))) if cap and cap.isdigit() else n


def oracle_row_blocks(case, nthreads):
    """The spec metadata split into ``nthreads`` contiguous blocks of rows
    (each keeping its tokens' global rows)."""
    from tests.gpu_util import sub_spec
    sp = case["spec"]
    bounds = np.linspace(0, sp["num_spec_decodes"], nthreads + 1).astype(int)
    return [sub_spec(sp, list(range(bounds[i], bounds[i + 1]))) for i in range(nthreads)]


def oracle_threaded(dims, c, parts, out):
    """One oracle step with one thread per block of rows, in place on the
    pools of ``c`` and on ``out`` (the blocks touch disjoint slots and rows)."""
    import threading

    import oracle  # test infrastructure: the baseline leg only
    ts = [threading.Thread(target=oracle.spec_step, args=(dims, c, p, out)) for p in parts]
    for t in ts:
        t.start()
    for t in ts:
        t.join()


def cpu_baseline(case, seconds=(8.0, 8.0)):
    """The oracle (C, fp64) on the whole batch, repeated for a bounded time:
    first on one thread, then on N threads, each taking a contiguous block of
    rows (rows use disjoint slots and token rows; ctypes releases the GIL
    during each call).  Results are the same bits at any thread count."""
    import oracle  # test infrastructure: the baseline leg only
    from tests.helpers import clone
    c = clone(case)
    sp = case["spec"]
    out = np.zeros((case["num_actual_tokens"], case["dims"]["Hv"], case["dims"]["dv"]), np.uint16)
    nrows = sp["num_spec_decodes"]
    nthreads = max(1, min(_host_threads(), nrows))
    parts = oracle_row_blocks(case, nthreads)

    def run(limit, n):
        reps, t0 = 0, time.perf_counter()
        while True:
            if n == 1:
                oracle.spec_step(case["dims"], c, sp, out)
            else:
                oracle_threaded(case["dims"], c, parts, out)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= limit:
                return reps, dt

    r1, t1 = run(seconds[0], 1)
    rn, tn = run(seconds[1], nthreads)
    tok = sp["num_spec_tokens"]
    return {"value": rn * tok / tn, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"the whole batch ({nrows} rows, {tok} tokens) {rn} times in {tn:.1f} s on "
                      f"{nthreads} threads (a block of rows each)",
            "one_thread": {"value": r1 * tok / t1, "unit": "tokens/s", "cores": 1,
                           "sample": f"the whole batch {r1} times in {t1:.1f} s on one thread"},
            "us_per_layer": tn / rn * 1e6, "us_per_layer_one_thread": t1 / r1 * 1e6,
            "host_cpu": _cpu_model(), "host_threads": _host_threads()}


def profiled_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counters, if they
    were taken on this workload and on the current kernel source."""
    import hashlib
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    with open(PROFILE_TRAFFIC) as f:
        rec = json.load(f)
    if rec.get("workload") != workload:
        return None
    src = os.path.join(ROOT, "speculative_decoding_causal_amd", "csrc", "gdn_rows.hip")
    with open(src, "rb") as f:
        cur = hashlib.sha256(f.read()).hexdigest()[:16]
    return rec.get("bytes_per_launch") if rec.get("source_sha256_16") == cur else None


def state_bytes(case) -> int:
    """The state part of the algorithmic bytes: load and per-token stores."""
    d, sp = case["dims"], case["spec"]
    tile = d["Hv"] * d["dv"] * d["dk"] * 4
    sq, ssi, nacc = sp["spec_query_start_loc"], sp["spec_state_indices"], sp["num_accepted_tokens"]
    total = 0
    for b in range(sp["num_spec_decodes"]):
        Tb = int(sq[b + 1] - sq[b])
        total += tile * (int(ssi[b][int(nacc[b]) - 1] > 0) + int((ssi[b][:Tb] > 0).sum()))
    return int(total)


def _bench_lib():
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "speculative_decoding_causal_amd", "libgdn_bench.so"))
    lib.gdn_bench_state_fanout.argtypes = [ctypes.c_void_p] + [ctypes.c_int32] * 7 + \
        [ctypes.c_void_p] * 4
    lib.gdn_bench_state_fanout.restype = ctypes.c_int
    return lib


def state_fanout_ceiling(case, layers, meta, stream, steps, achieved_gbs):
    """The step's state traffic alone (gdn_bench_state_fanout: each row's
    state blocks read from the load slot and written to every store slot, no
    arithmetic) on the same layers and metadata, timed the same way: a
    measured ceiling for the access pattern on this GPU."""
    lib = _bench_lib()
    d, sp = case["dims"], case["spec"]

    def call(i):
        L = layers[i % len(layers)]
        rc = lib.gdn_bench_state_fanout(L["ssm"].data_ptr(), d["num_slots"], d["Hk"], d["Hv"],
                                        d["dk"], d["dv"], sp["num_spec_decodes"], sp["K"],
                                        meta["sqsl"].data_ptr(), meta["ssi"].data_ptr(),
                                        meta["nacc"].data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"gdn_bench_state_fanout failed ({rc})")

    for i in range(5):
        call(i)
    series = time_series(call, steps, stream, start=5, block=len(layers))
    sb = state_bytes(case)
    gbs = sb / (series["mean_us"] * 1e-6) / 1e9
    return {"kernel": "gdn_bench_state_fanout (state load + per-token stores, no arithmetic)",
            "state_bytes_per_launch": sb, "series_us": series, "achieved_GBs": gbs,
            "frac_of_peak": gbs / HBM_PEAK_GBS, "frac_of_ceiling": achieved_gbs / gbs}


def lead(stream):
    """Queue a GPU spin on ``stream`` ahead of a timed region's first event,
    so that the host has launched the region's first steps by the time the
    spin ends and the events see no launch gap."""
    import torch
    with torch.cuda.stream(stream):
        torch.cuda._sleep(LEAD_CYCLES)


def time_region(fn, n, stream, start=0, led=True):
    """Mean time per call of ``n`` calls back to back, bracketed by one pair
    of events and synchronised on both sides."""
    import torch
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if led:
        lead(stream)
    t_begin.record(stream)
    for i in range(n):
        fn(start + i)
    t_end.record(stream)
    torch.cuda.synchronize()
    return t_begin.elapsed_time(t_end) / n


def time_series(fn, n, stream, start=0, block=8):
    """n calls back to back in blocks of ``block`` calls with one event
    between consecutive blocks: each sample is a block's time per call (the
    events' own cost spread over the block), the samples sum to the whole
    region, and their median, p10 and p90 describe the same series as the
    mean."""
    import torch
    nb = max(n // block, 1)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    torch.cuda.synchronize()
    lead(stream)
    ev[0].record(stream)
    for i in range(nb):
        for j in range(block):
            fn(start + i * block + j)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    us = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 / block for i in range(nb)])
    return {"mean_us": float(us.mean()), "median_us": float(np.median(us)),
            "p10_us": float(np.percentile(us, 10)), "p90_us": float(np.percentile(us, 90)),
            "samples": int(nb), "calls_per_sample": int(block)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--qkv-layout", choices=("grouped", "per_k_head"), default="grouped",
                    help="channel order of mixed_qkv (per_k_head: reorder_input=False; the "
                         "same values repacked)")
    ap.add_argument("--conv-layout", choices=("rolled", "per_token"), default="rolled",
                    help="conv contract of spec rows (per_token: a window per token slot, "
                         "state_len = conv_width - 1)")
    ap.add_argument("--no-turns", action="store_true",
                    help="call without turn counters: one row-kernel workgroup per "
                         "(row, k-head) on every batch")
    ap.add_argument("--graph", action="store_true",
                    help="capture each layer's step in a HIP graph and time graph replays")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB ten times "
                         "(the reference kernel for scaling the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the GDN step shards heads and rows with no "
              "exchange, so there is no multi-GPU path to time here", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 10}), flush=True)
        return

    import speculative_decoding_causal_amd as gdn
    import synth
    from tests.gpu_util import bf, f32, i32, u8

    over = {}
    if args.conv_layout == "per_token":
        over["L"] = synth.CONFIGS[args.workload]["W"] - 1
    case = synth.make_case(args.workload, seed=args.seed, **over)
    d, sp, ns = case["dims"], case["spec"], case.get("nonspec")
    if args.conv_layout == "per_token":
        if ns is not None:
            raise SystemExit("--conv-layout per_token applies to spec-only workloads")
        d["conv_layout"] = 1
    if args.qkv_layout == "per_k_head":
        from tests.test_layout import per_k_head
        case["mixed_qkv"] = per_k_head(case["mixed_qkv"], d["Hk"], d["Hv"], d["dk"], d["dv"])
    cfg = gdn.GdnConfig(d["Hk"], d["Hv"], d["dk"], d["dv"], d["W"], d["activation"],
                        d["use_qk_l2norm"], d["eps"], d["scale"],
                        reorder_input=args.qkv_layout == "grouped",
                        conv_layout=int(d.get("conv_layout", 0)))
    dev = torch.device("cuda:0")
    T_spec = sp["num_spec_tokens"]
    T_all = case["num_actual_tokens"]
    meta = dict(sqsl=i32(sp["spec_query_start_loc"]), ssi=i32(sp["spec_state_indices"]),
                nacc=i32(sp["num_accepted_tokens"]), tix=i32(sp.get("spec_token_indx")),
                cache=i32(sp.get("spec_cache_indices")))
    if ns is not None:
        meta.update(qsl=i32(ns["query_start_loc"]), nsi=i32(ns["cache_indices"]),
                    his=u8(ns.get("has_initial_state")), ntix=i32(ns.get("token_indx")))
        ws_bytes = gdn.gdn_workspace_bytes(cfg, d["L"], d["num_slots"],
                                           ns["num_non_spec_tokens"], ns["num_prefills"])
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    conv0, ssm0 = bf(case["conv_state"]), f32(case["ssm_state"])
    w, A_log, dt_bias = bf(case["conv_weight"]), f32(case["A_log"]), f32(case["dt_bias"])
    layers = []
    g = torch.Generator(device="cpu").manual_seed(args.seed)
    for li in range(args.layers):
        perm = torch.randperm(T_all, generator=g)
        qkv = bf(case["mixed_qkv"])[perm.to(dev)].contiguous()
        layers.append(dict(qkv=qkv, a=bf(case["a"]), b=bf(case["b"]),
                           conv=conv0.clone(), ssm=ssm0.clone(),
                           out=torch.empty(T_all, d["Hv"], d["dv"],
                                           dtype=torch.bfloat16, device=dev),
                           turns=None if args.no_turns
                           else gdn.conv_turns(cfg, d["num_slots"], dev)))
    del conv0, ssm0
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step(i):
        L = layers[i % len(layers)]
        if ns is None:
            gdn.gdn_spec_attention(cfg, L["qkv"], L["a"], L["b"], w, None, A_log, dt_bias,
                                   L["conv"], L["ssm"], meta["sqsl"], meta["ssi"], meta["nacc"],
                                   L["out"], spec_cache_indices=meta["cache"],
                                   spec_token_indx=meta["tix"], num_spec_tokens=T_spec,
                                   conv_turns=L["turns"], stream=stream)
        else:
            gdn.gdn_attention(cfg, L["qkv"], L["a"], L["b"], w, None, A_log, dt_bias,
                              L["conv"], L["ssm"], L["out"], num_decodes=ns["num_decodes"],
                              num_prefills=ns["num_prefills"],
                              num_non_spec_tokens=ns["num_non_spec_tokens"],
                              query_start_loc=meta["qsl"], non_spec_state_indices=meta["nsi"],
                              has_initial_state=meta["his"], non_spec_token_indx=meta["ntix"],
                              spec_query_start_loc=meta["sqsl"], spec_state_indices=meta["ssi"],
                              num_accepted_tokens=meta["nacc"], spec_cache_indices=meta["cache"],
                              spec_token_indx=meta["tix"], num_spec_tokens=T_spec,
                              workspace=workspace, conv_turns=L["turns"], stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if args.graph:
        # one graph per layer, captured on a side stream after the warm-up;
        # a step is then one replay on the launch stream
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        for li in range(len(layers)):
            g_ = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_, stream=side):
                call_stream = torch.cuda.current_stream()
                eager, stream = stream, call_stream
                step(li)
                stream = eager
            graphs.append(g_)
        torch.cuda.synchronize()
        eager_step = step

        def step(i):  # noqa: F811 (the timed step replays the layer's graph)
            graphs[i % len(graphs)].replay()
        del eager_step
    # Timed region: exactly `steps` layer steps, synchronised on both sides,
    # behind the lead spin.
    ms_per_step = time_region(step, args.steps, stream, start=args.warmup)
    # The same steps from an idle stream (no lead): the host's latency to
    # launch the first step counted in.
    idle_ms = time_region(step, args.steps, stream, start=args.warmup, led=False)
    # The same steps again with an event after every block of `layers` calls
    # (layers cycled: cold states): median, p10 and p90 of one series.
    cold = time_series(step, args.steps, stream, start=args.warmup, block=args.layers)
    # Hot: one layer called back to back, so its states may sit in the
    # last-level cache between calls (labelled; not the headline).
    hot = time_series(lambda i: step(0), args.steps, stream, block=args.layers)
    # Kernel time per launch over the timed region (one launch per step for
    # the spec workload).
    avg_launch_s = ms_per_step * 1e-3
    nbytes = algorithmic_bytes(case) + (nonspec_bytes(case) if ns is not None else 0)
    achieved = nbytes / avg_launch_s / 1e9
    default_variant = (args.qkv_layout, args.conv_layout, args.graph) == ("grouped", "rolled", False)
    traffic = profiled_traffic(args.workload) if ns is None and default_variant else None
    tokens = T_all if ns is not None else T_spec

    result = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "us_per_layer": ms_per_step * 1e3,
        "hbm_frac_of_peak": achieved / HBM_PEAK_GBS,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": args.workload, "spec_rows": sp["num_spec_decodes"], "K": sp["K"],
                   "tokens_per_step": tokens, "num_k_heads": d["Hk"], "num_v_heads": d["Hv"],
                   "head_k_dim": d["dk"], "head_v_dim": d["dv"], "conv_width": d["W"],
                   "state_len": d["L"], "num_slots": d["num_slots"],
                   "layers_cycled": args.layers, "parallelism": "single GPU",
                   "qkv_layout": args.qkv_layout, "conv_layout": args.conv_layout,
                   "hip_graph": bool(args.graph),
                   "conv_turns": not args.no_turns},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "gdn_rows_kernel (dk=dv=128)",
                     "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": avg_launch_s * 1e6,
                     "idle_start_us": idle_ms * 1e3,
                     "series_us": cold, "hot_series_us": hot},
    }
    if ns is None:
        result["roofline"]["same_box"] = state_fanout_ceiling(case, layers, meta, stream,
                                                              args.steps, achieved)
    if ns is None and args.workload != DEFAULT_WORKLOAD:
        # the headline metric names its own batch; other spec batches say theirs
        result["metric"] = (f"GDN layer tokens/sec + us/layer + % HBM peak, spec verify "
                            f"K={sp['K']}, batch {sp['num_spec_decodes']}")
    if ns is not None:
        result["metric"] = "GDN layer tokens/sec on a mixed spec/decode/prefill batch"
        result["config"].update(decode_rows=ns["num_decodes"], prefill_rows=ns["num_prefills"],
                                non_spec_tokens=ns["num_non_spec_tokens"])
        result["roofline"]["kernel"] = "whole step (6 kernels); see the rocprofv3 profile"
        result["chunked_prefill_gflop"] = chunked_flops(case) / 1e9
    if not args.no_cpu_baseline and ns is None:
        result["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
