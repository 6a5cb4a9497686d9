"""Benchmark of the CQS attention forward on one MI355X.

A step is one pass of the whole hot path over the workload: the masked attention
partials of every CQS task followed by the merge into O and LSE.  The default
workload is N=57344 tokens, 8 heads, d=128, bf16, CQS l=3 (7 chunks of 8192),
Q/K/V resident in HBM (inputs are resident before the timed region starts).

Prints one JSON line: useful attention TFLOP/s (4 N^2 d H per step), the fraction
of the bf16 dense MFMA peak, the roofline of the partial kernel (its average launch
duration measured with HIP events on the stream it runs on), the fp64 oracle timed
on a bounded sample of host cores, and the host-pinned streamed run of the
N=212992, 16-head workload under a 16 GiB budget (PCIe-inclusive, reported beside
the value, never as it).
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0
METRIC = "useful attention TFLOP/s + % bf16 MFMA peak, CQS-streamed fwd at fixed mem budget"
GiB = 1 << 30

WORKLOADS = {
    # name: (N, H, d, levels, budget, residency description)
    "device_n57344": (57344, 8, 128, [3], 0, "device"),
    "pinned_n212992": (212992, 16, 128, [4], 16 * GiB, "host_pinned"),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    """sha256 (first 16 hex) of the partial kernel's sources: kernels.hip then device_common.hpp."""
    h = hashlib.sha256()
    for name in ("kernels.hip", "device_common.hpp"):
        with open(os.path.join(ROOT, "memory_bounded_streaming_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_hash, units_per_launch):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it matches this kernel."""
    path = TRAFFIC_RECORD
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "attn_partial_bf16_d128_n57344_h8_l3_traffic.json")


def traffic_record(fetch_csv, write_csv, kernel_hash):
    """HBM traffic record of the partial and merge kernels from two rocprofv3 counter runs.

    fetch_csv / write_csv: `run_counter_collection.csv` of a `--pmc FETCH_SIZE` and of a
    `--pmc WRITE_SIZE` run of this script with --calib-copy (KiB per dispatch).  Each
    counter is scaled by what it reads for the 1 GiB calibration copy (1 GiB read and
    1 GiB written), then averaged over the launches of each kernel.
    """
    import csv

    def per_kernel(path, counter):
        calib, part, merge = [], [], []
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                value, name = float(row["Counter_Value"]), row["Kernel_Name"]
                if "copyBuffer" in name and value > 1000.0:
                    calib.append(value)
                elif "attn_partial_bf16<128>" in name:
                    part.append(value)
                elif "merge_partials<128" in name:
                    merge.append(value)
        if not calib or not part or not merge:
            raise ValueError(f"{path}: needs the calibration copy and both kernels under {counter}")
        return calib[0], part, merge

    cf, fetch, mfetch = per_kernel(fetch_csv, "FETCH_SIZE")
    cw, write, mwrite = per_kernel(write_csv, "WRITE_SIZE")
    fscale, wscale = GiB / (cf * 1024.0), GiB / (cw * 1024.0)
    mean = lambda xs: sum(xs) / len(xs)  # noqa: E731
    read_b = mean(fetch) * 1024.0 * fscale
    write_b = mean(write) * 1024.0 * wscale
    merge_b = mean(mfetch) * 1024.0 * fscale + mean(mwrite) * 1024.0 * wscale
    return {
        "kernel": "attn_partial_bf16<128>",
        "workload": "N=57344, H=8, d=128, bf16, CQS l=3, device-resident (one launch per step)",
        "kernel_source_sha256_16": kernel_hash,
        "fetch_size_kib_per_launch": fetch,
        "write_size_kib_per_launch": write,
        "calibration": {"kernel": "__amd_rocclr_copyBuffer (1 GiB device copy: 1 GiB read, 1 GiB written)",
                        "fetch_size_kib": cf, "write_size_kib": cw,
                        "fetch_scale": round(fscale, 5), "write_scale": round(wscale, 5)},
        "hbm_bytes_read_per_launch": int(round(read_b)),
        "hbm_bytes_written_per_launch": int(round(write_b)),
        "hbm_bytes_per_launch": int(round(read_b + write_b)),
        "merge": {"fetch_size_kib": mfetch, "write_size_kib": mwrite, "hbm_bytes_per_launch": int(round(merge_b))},
    }


def cpu_baseline(rows_wanted=1024):
    """The fp64 oracle on a bounded sample of the N=57344, 8-head workload (all keys, sampled query rows)."""
    from memory_bounded_streaming_amd.inputs import gen_qkv, sample_rows
    from oracle.attention import attention_fp64
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = len(os.sched_getaffinity(0))
    n, h, d = 57344, 8, 128
    q, k, v = gen_qkv(0, n, h, d, "bf16")
    rows = sample_rows(n, rows_wanted, 0)
    t0 = time.perf_counter()
    attention_fp64(q, k, v, rows=rows, dtype="bf16")
    dt = time.perf_counter() - t0
    flop = 4.0 * rows.size * n * d * h
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows.size} sampled query rows x {h} heads of the N={n}, d={d} workload against all "
                      f"{n} keys, fp64 two-pass softmax; {dt:.1f} s wall; rate = 4*rows*N*d*H / time",
            "sample_wall_s": round(dt, 2),
            "extrapolated_full_n_s": round(dt * n / rows.size, 1),
            "extrapolation": f"sample wall x N/rows = time for all {n} query rows (not measured)"}


def run_device(args, torch, cqsa):
    from memory_bounded_streaming_amd.inputs import gen_qkv
    n, h, d, levels, _, _ = WORKLOADS["device_n57344"]
    q, k, v = gen_qkv(args.seed, n, h, d, "bf16")
    dev = [torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() for x in (q, k, v)]
    plan = cqsa.Plan(n, h, d, cqsa.CQSA_BF16, levels)
    V = plan.info["visits"]
    ws_n = torch.empty((V, n, h, d), dtype=torch.float32, device="cuda")
    ws_ml = torch.empty((V, n, h, 2), dtype=torch.float32, device="cuda")
    o = torch.empty((n, h, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((h, n), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        plan.partials(*dev, ws_n, ws_ml, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        plan.merge(ws_n, ws_ml, o, lse, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    attn_ms = [e[0].elapsed_time(e[1]) for e in evs]
    merge_ms = [e[1].elapsed_time(e[2]) for e in evs]
    flop = plan.info["useful_flop"]
    ms = total_ms / args.steps
    attn_avg = float(np.mean(attn_ms))
    merge_avg = float(np.mean(merge_ms))
    merge_bytes = n * h * ((d + 2) * 4 * V + d * 2 + 4)  # read V partial triples, write O (bf16) + LSE
    out = {
        "plan": plan.info,
        "ms_per_step": ms,
        "value": flop / (ms / 1e3) / 1e12,
        "attn_ms": attn_avg,
        "attn_tflops": flop / (attn_avg / 1e3) / 1e12,
        "merge_ms": merge_avg,
        "merge_gbs": merge_bytes / (merge_avg / 1e3) / 1e9,
        "merge_bytes": merge_bytes,
    }
    plan.close()
    return out


def run_backward(args, torch, cqsa):
    """The backward of the device-resident workload: one cqsa_backward call per step
    (Delta/transposes, dK/dV and dQ kernels, slot sums), timed with HIP events on its
    stream; O and LSE come from one forward beforehand."""
    from memory_bounded_streaming_amd.inputs import gen_qkv, gen_tensor
    n, h, d, levels, _, _ = WORKLOADS["device_n57344"]
    q, k, v = gen_qkv(args.seed, n, h, d, "bf16")
    do = gen_tensor(args.seed, 3, n, h, d, "bf16")
    dev = [torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() for x in (q, k, v, do)]
    plan = cqsa.Plan(n, h, d, cqsa.CQSA_BF16, levels)
    o = torch.empty((n, h, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((h, n), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    plan.forward(dev[0], dev[1], dev[2], o, lse, stream=stream)
    grads = [torch.empty((n, h, d), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    ws = torch.empty(plan.backward_workspace_size(), dtype=torch.uint8, device="cuda")
    args_ = (dev[0], dev[1], dev[2], o, lse, dev[3], *grads)
    for _ in range(args.warmup):
        plan.backward(*args_, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream)
        plan.backward(*args_, workspace=ws, stream=stream)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    st = plan.backward(*args_, workspace=ws, stream=stream, stats=True)
    useful = 10.0 * n * n * d * h
    executed = 14.0 * n * n * d * h  # S and dP are formed in both gradient kernels
    plan.close()
    return {
        "workload": f"backward of the N={n}, H={h}, d={d} bf16 l={levels[0]} workload (device-resident)",
        "ms_per_step": round(ms, 4),
        "tflops_useful": round(useful / (ms / 1e3) / 1e12, 3),
        "useful_flop": useful,
        "grad_kernels_ms": round(st["t_attn_ms"], 4),
        "grad_kernels_tflops_executed": round(executed / (st["t_attn_ms"] / 1e3) / 1e12, 3),
        "executed_flop": executed,
        "elementwise_ms": round(st["t_merge_ms"], 4),
        "fwd_bwd_ratio_note": "ms_per_step here / the forward step's ms_per_step",
    }


def run_streamed_backward(args, torch, cqsa):
    """Backward of the host-pinned N=212992, 16-head workload under 16 GiB: Q, K, V, O, dO
    and LSE in pinned memory, gradients written to pinned memory (one warm call, one timed)."""
    from memory_bounded_streaming_amd.inputs import gen_tensor
    n, h, d, levels, budget, _ = WORKLOADS["pinned_n212992"]
    ts = []
    for i in range(4):  # Q, K, V, dO
        t = torch.empty((n, h, d), dtype=torch.int16, pin_memory=True)
        gen_tensor(args.seed, i, n, h, d, "bf16", out=t.numpy().view(np.uint16))
        ts.append(t)
    o = torch.empty((n, h, d), dtype=torch.int16, pin_memory=True)
    lse = torch.empty((h, n), dtype=torch.float32, pin_memory=True)
    grads = [torch.empty((n, h, d), dtype=torch.int16, pin_memory=True) for _ in range(3)]
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, levels, budget_bytes=budget) as plan:
        plan.forward(ts[0], ts[1], ts[2], o, lse, residency=cqsa.CQSA_RES_HOST_PINNED)
        need = plan.backward_workspace_size(cqsa.CQSA_RES_HOST_PINNED)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        call = (ts[0], ts[1], ts[2], o, lse, ts[3], *grads)
        plan.backward(*call, residency=cqsa.CQSA_RES_HOST_PINNED, workspace=ws)  # warm-up
        t0 = time.perf_counter()
        st = plan.backward(*call, residency=cqsa.CQSA_RES_HOST_PINNED, workspace=ws, stats=True)
        wall = time.perf_counter() - t0
        useful = 2.5 * plan.info["useful_flop"]
    return {
        "workload": f"backward of N={n}, H={h}, d={d}, bf16, CQS l={levels[0]}, pinned host memory, "
                    f"device budget {budget // GiB} GiB",
        "wall_s": wall,
        "tflops_pcie_inclusive": useful / wall / 1e12,
        "grad_kernels_tflops_executed": 14.0 / 10.0 * useful / (st["t_attn_ms"] / 1e3) / 1e12,
        "bytes_h2d": st["bytes_h2d"],
        "bytes_d2h": st["bytes_d2h"],
        "peak_device_bytes": st["peak_device_bytes"],
        "budget_bytes": budget,
    }


def pcie_achievable(torch, nbytes=512 << 20, reps=5):
    """Plain pinned-memory copies of 512 MiB in each direction: the achievable PCIe rate."""
    h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = {}
    for name, fn in (("h2d_gbs", lambda: d.copy_(h, non_blocking=True)), ("d2h_gbs", lambda: h.copy_(d, non_blocking=True))):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        out[name] = reps * nbytes / (time.perf_counter() - t0) / 1e9
    return out


def run_streamed(args, torch, cqsa):
    from memory_bounded_streaming_amd.inputs import gen_tensor
    n, h, d, levels, budget, _ = WORKLOADS["pinned_n212992"]
    ts = []
    for i in range(3):
        t = torch.empty((n, h, d), dtype=torch.int16, pin_memory=True)
        gen_tensor(args.seed, i, n, h, d, "bf16", out=t.numpy().view(np.uint16))
        ts.append(t)
    o = torch.empty((n, h, d), dtype=torch.int16, pin_memory=True)
    lse = torch.empty((h, n), dtype=torch.float32, pin_memory=True)
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, levels, budget_bytes=budget) as plan:
        ws = torch.empty(plan.workspace_size(cqsa.CQSA_RES_HOST_PINNED), dtype=torch.uint8, device="cuda")
        plan.forward(*ts, o, lse, residency=cqsa.CQSA_RES_HOST_PINNED, workspace=ws)  # warm-up
        t0 = time.perf_counter()
        st = plan.forward(*ts, o, lse, residency=cqsa.CQSA_RES_HOST_PINNED, workspace=ws, stats=True)
        wall = time.perf_counter() - t0
        flop = plan.info["useful_flop"]
        pcie = pcie_achievable(torch)
        h2d = st["bytes_h2d"] / (st["t_h2d_ms"] / 1e3) / 1e9 if st["t_h2d_ms"] else None
        d2h = st["bytes_d2h"] / (st["t_d2h_ms"] / 1e3) / 1e9 if st["t_d2h_ms"] else None
        return {
            "workload": f"N={n}, H={h}, d={d}, bf16, CQS l={levels[0]} (c=13), Q/K/V in pinned host memory, "
                        f"device budget {budget // GiB} GiB",
            "mode": cqsa.MODE_NAMES[plan.info["stream_mode"]],
            "tflops_pcie_inclusive": flop / wall / 1e12,
            "wall_s": wall,
            "attn_tflops": flop / (st["t_attn_ms"] / 1e3) / 1e12,
            "h2d_gbs": h2d,
            "d2h_gbs": d2h,
            "h2d_achievable_gbs": pcie["h2d_gbs"],
            "d2h_achievable_gbs": pcie["d2h_gbs"],
            "h2d_frac_of_achievable": h2d / pcie["h2d_gbs"] if h2d else None,
            "d2h_frac_of_achievable": d2h / pcie["d2h_gbs"] if d2h else None,
            "merge_ms": st["t_merge_ms"],
            "attn_ms": st["t_attn_ms"],
            "bytes_h2d": st["bytes_h2d"],
            "bytes_d2h": st["bytes_d2h"],
            "bytes_d2d_chunk_reuse": st["bytes_d2d"],
            "peak_device_bytes": st["peak_device_bytes"],
            "budget_bytes": budget,
        }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-streamed", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-streamed-backward", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=8192)
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one plain device copy of 1 GiB first (reference for HBM traffic counters)")
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic record from two rocprofv3 counter CSVs and exit (no GPU use)")
    args = ap.parse_args()
    if args.traffic_record:
        rec = traffic_record(args.traffic_record[0], args.traffic_record[1], kernel_source_hash())
        with open(TRAFFIC_RECORD, "w") as f:
            json.dump(rec, f, indent=2)
            f.write("\n")
        print(json.dumps(rec))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from memory_bounded_streaming_amd import cqsa
    cqsa.load()
    torch.cuda.set_device(0)

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("bench: calibration copy of 1 GiB done")
    log("bench: device-resident workload")
    dres = run_device(args, torch, cqsa)
    log(f"bench: {dres['value']:.1f} TFLOP/s end-to-end, partial kernel {dres['attn_tflops']:.1f} TFLOP/s")
    bwd = None
    if not args.no_backward:
        log("bench: backward of the device-resident workload")
        bwd = run_backward(args, torch, cqsa)
        bwd["fwd_bwd_ratio"] = round((bwd["ms_per_step"] + dres["ms_per_step"]) / dres["ms_per_step"], 3)
        bwd.pop("fwd_bwd_ratio_note")
        log(f"bench: backward {bwd['tflops_useful']:.1f} useful TFLOP/s, {bwd['ms_per_step']:.2f} ms")
    stream_res = None
    if not args.no_streamed:
        log("bench: host-pinned streamed workload")
        stream_res = run_streamed(args, torch, cqsa)
        log(f"bench: streamed {stream_res['tflops_pcie_inclusive']:.1f} TFLOP/s PCIe-inclusive")
    sbwd = None
    if not args.no_streamed and not args.no_streamed_backward:
        log("bench: host-pinned streamed backward")
        sbwd = run_streamed_backward(args, torch, cqsa)
        log(f"bench: streamed backward {sbwd['tflops_pcie_inclusive']:.1f} useful TFLOP/s PCIe-inclusive")
    dry = None
    if stream_res is not None:
        # the billion-token case priced with this run's measured rates (plan-only, no data)
        rates = {"attn_tflops": dres["attn_tflops"], "merge_gbs": dres["merge_gbs"],
                 "h2d_gbs": stream_res["h2d_achievable_gbs"], "d2h_gbs": stream_res["d2h_achievable_gbs"]}
        dry = []
        for budget in (16 * GiB, 2 * GiB):
            e = cqsa.cqsa_plan_estimate(1 << 30, 1, 128, cqsa.CQSA_BF16, [3], n_levels=0, budget_bytes=budget,
                                        flags=cqsa.CQSA_FLAG_PAD, rates=rates)
            dry.append({"n_tokens": 1 << 30, "heads": 1, "head_dim": 128, "budget_bytes": budget,
                        "levels": e["l"], "task_tokens": e["task_tokens"],
                        "mode": cqsa.MODE_NAMES[e["stream_mode"]], "stream_workspace_bytes": e["stream_workspace_bytes"],
                        "host_pinned_bytes": e["host_pinned_bytes"], "bytes_h2d": e["bytes_h2d"],
                        "bytes_d2h": e["bytes_d2h"], "est_hours": round(e["t_est_s"] / 3600, 2),
                        "attn_hours": round(e["t_attn_s"] / 3600, 2), "h2d_hours": round(e["t_h2d_s"] / 3600, 2)})
            if sbwd is not None:
                # not a plan of the backward: the forward estimate scaled by the streamed backward's
                # measured time over the streamed forward's on the 16 GiB workload
                ratio = sbwd["wall_s"] / stream_res["wall_s"]
                dry[-1]["bwd_hours_by_ratio"] = round(e["t_est_s"] * ratio / 3600, 1)
                dry[-1]["bwd_ratio_note"] = (f"extrapolation: forward estimate x {ratio:.2f}, the measured streamed "
                                             "backward / forward time of the N=212992, 16-head workload")
    cpu = None
    if not args.no_cpu_baseline:
        log("bench: oracle cpu baseline")
        cpu = cpu_baseline(args.cpu_rows)

    n, h, d, levels, _, _ = WORKLOADS["device_n57344"]
    flop = dres["plan"]["useful_flop"]
    khash = kernel_source_hash()
    traffic = measured_traffic(khash, 1)
    line = {
        "metric": METRIC,
        "value": round(dres["value"], 3),
        "unit": "TFLOP/s",
        "pct_bf16_mfma_peak": round(100.0 * dres["value"] / BF16_MFMA_PEAK_TFLOPS, 3),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dres["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: Q/K/V i.i.d. N(0,1) rounded to bf16, seed %d" % args.seed,
        "config": {"workload": f"N={n} tokens, {h} heads, d={d}, bf16, non-causal, CQS l={levels[0]} "
                               f"(c=7 chunks of 8192), Q/K/V device-resident",
                   "n_tokens": n, "heads": h, "head_dim": d, "levels": levels, "residency": "device"},
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_partial_bf16<128>",
            "achieved": round(dres["attn_tflops"], 3),
            "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(dres["attn_tflops"] / BF16_MFMA_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "flop_per_launch": flop,
            "avg_launch_ms": round(dres["attn_ms"], 4),
        },
        "merge": {"bound": "hbm", "achieved": round(dres["merge_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(dres["merge_gbs"] / HBM_PEAK_GBS, 4), "bytes_per_launch": dres["merge_bytes"],
                  "avg_launch_ms": round(dres["merge_ms"], 4)},
        "streamed": stream_res,
        "backward": bwd,
        "streamed_backward": sbwd,
        "dry_run_1b_tokens": dry,
        "cpu_baseline": cpu,
        "kernel_source_sha256_16": khash,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
