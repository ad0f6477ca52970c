"""Benchmark of the GDN spec-verify layer step on one MI355X.

One step = one gdn_spec_attention call (conv + ring roll, gates, norms, the
gated delta rule with per-token state snapshots) over the Qwen3-Next-shaped
batch: 64 spec rows, K=3 tokens each, 16 k-heads / 32 v-heads, dk=dv=128,
fp32 states in a 512-slot pool.  Steps cycle over several independent layers
(each with its own pools and inputs, as consecutive GDN layers of a model
have), so no step finds the previous step's states in the last-level cache.

Prints one JSON line: tokens/s, us per layer, achieved HBM bandwidth of the
kernel against the 8 TB/s MI355X peak, and the CPU oracle timed on a bounded
sample of the same workload.
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
        if cs > 0:
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


def cpu_baseline(case, min_seconds=10.0):
    """The oracle (single-threaded C, fp64) on the whole batch, repeated until
    at least ``min_seconds`` of CPU time has been spent."""
    import oracle  # test infrastructure: the baseline leg only
    from tests.helpers import clone
    c = clone(case)
    sp = case["spec"]
    out = np.zeros((case["num_actual_tokens"], case["dims"]["Hv"], case["dims"]["dv"]), np.uint16)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.spec_step(case["dims"], c, sp, out)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": reps * sp["num_spec_tokens"] / dt, "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"the whole batch ({sp['num_spec_decodes']} rows, {sp['num_spec_tokens']} "
                      f"tokens) {reps} times in a row on one thread, {dt:.1f} s"}


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


def same_box_ceilings(stream, achieved_gbs, mib=256, reps=20):
    """Plain torch copy and fill rates on this GPU (context for the HBM peak:
    what streaming kernels with no arithmetic reach here), timed with events
    on the launch stream."""
    import torch
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    rates = {}
    for name, fn, moved in (("copy", lambda: dst.copy_(src), 2 * n * 4),
                            ("fill", lambda: dst.fill_(1.0), n * 4)):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        rates[name] = moved * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    # one read per three writes, as the spec step moves its state: a copy of
    # a quarter of the bytes (read + write) and a fill of the other half, run
    # one after the other
    mix = 1.0 / (0.5 / rates["copy"] + 0.5 / rates["fill"])
    return {"copy_GBs": rates["copy"], "fill_GBs": rates["fill"], "mix_1r3w_GBs": mix,
            "frac_of_copy": achieved_gbs / rates["copy"],
            "frac_of_fill": achieved_gbs / rates["fill"],
            "frac_of_mix_1r3w": achieved_gbs / mix,
            "what": f"torch copy_ of {mib} MiB (read + write counted) and fill_ of {mib} MiB, "
                    f"{reps} each"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    case = synth.make_case(args.workload, seed=args.seed)
    d, sp, ns = case["dims"], case["spec"], case.get("nonspec")
    cfg = gdn.GdnConfig(d["Hk"], d["Hv"], d["dk"], d["dv"], d["W"], d["activation"],
                        d["use_qk_l2norm"], d["eps"], d["scale"])
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
                                           dtype=torch.bfloat16, device=dev)))
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
                                   stream=stream)
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
                              workspace=workspace, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Timed region: exactly `steps` layer steps, synchronised on both sides.
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_begin.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_begin.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    # Per-launch kernel durations: events on the launch stream around each call.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    launch_ms = np.array([a.elapsed_time(b) for a, b in ev])
    # Kernel time per launch over the timed region (one launch per step for
    # the spec workload); the per-launch event pairs give the spread.
    avg_launch_s = ms_per_step * 1e-3
    nbytes = algorithmic_bytes(case) + (nonspec_bytes(case) if ns is not None else 0)
    achieved = nbytes / avg_launch_s / 1e9
    traffic = profiled_traffic(args.workload) if ns is None else None
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
                   "layers_cycled": args.layers, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "gdn_rows_kernel (dk=dv=128)",
                     "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": avg_launch_s * 1e6,
                     "p10_launch_us": float(np.percentile(launch_ms, 10)) * 1e3,
                     "p90_launch_us": float(np.percentile(launch_ms, 90)) * 1e3},
    }
    result["roofline"]["same_box"] = same_box_ceilings(stream, achieved)
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
