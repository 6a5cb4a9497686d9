"""Benchmark of the CQS-streamed attention forward on one MI355X.

A step is one call of the whole hot path on the 8 GiB streamed workload: N=1,376,256
tokens, 8 heads, d=128, bf16, CQS l=5 (21 chunks of 65,536), Q/K/V/O/LSE in pinned host
memory and a device-memory budget of 8 GiB.  Every step gathers each task's K/V segments
and Q blocks into device staging (hipMemcpyAsync, double buffered), runs the masked
attention partials, merges them into the accumulator (kept in pinned host memory under
this budget, with round trips) and returns O and LSE -- the inputs are resident in host
memory before the timed region starts, as the method keeps them.

Prints one JSON line: useful attention TFLOP/s (4 N^2 d H per step) and its fraction of
the bf16 dense MFMA peak, the roofline of the partial kernel (its launches timed with HIP
events on the stream it runs on, inside the timed calls), the stream phases' rates while
copying against the pinned-copy rate measured on the box, the merge kernel against HBM,
peak device memory (modelled and observed) against the budget, the forward error on
sampled rows against the fp64 oracle, and the oracle itself timed on those rows on the
host's cores.  Secondary keys: the device-resident N=57,344 workload, its backward, the
16 GiB streamed workload (N=212,992, 16 heads) and its backward, and the billion-token
dry run priced with this run's rates.  For reference, measured on the same box after the
timed calls: a device copy and the vendor bf16 GEMM (`ceilings`), and the vendor's fused
attention (torch scaled_dot_product_attention) on the device-resident workload's inputs.
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
    "pinned_n1376256": (1376256, 8, 128, [5], 8 * GiB, "host_pinned"),
    "pinned_n12845056": (12845056, 1, 128, [3, 3], 2 * GiB, "host_pinned"),
}
HEADLINE = "pinned_n1376256"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    """sha256 (first 16 hex) of the partial kernel's sources: kernels.hip then device_common.hpp."""
    h = hashlib.sha256()
    for name in ("kernels.hip", "device_common.hpp"):
        with open(os.path.join(ROOT, "memory_bounded_streaming_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_hash, record):
    """HBM bytes per launch from a committed rocprofv3 PMC record, if it matches this kernel."""
    path = TRAFFIC_RECORDS[record]
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


TRAFFIC_RECORDS = {
    "device_n57344": os.path.join(ROOT, "profiles", "attn_partial_bf16_d128_n57344_h8_l3_traffic.json"),
    "pinned_n1376256": os.path.join(ROOT, "profiles", "attn_partial_bf16_d128_n1376256_h8_l5_traffic.json"),
}
TRAFFIC_WORKLOADS = {
    "device_n57344": "N=57344, H=8, d=128, bf16, CQS l=3, device-resident (one launch per step)",
    "pinned_n1376256": "N=1376256, H=8, d=128, bf16, CQS l=5, pinned host memory, 8 GiB budget "
                       "(105 launches per step, one per (task, query unit))",
}


def traffic_record(fetch_csv, write_csv, kernel_hash, workload=TRAFFIC_WORKLOADS["device_n57344"]):
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
        "workload": workload,
        "launches": len(fetch),
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


def copy_summary(trace_csv, streams=None):
    """Host-to-device and device-to-host busy time from a rocprofv3 memory-copy trace.

    For each direction: the number of copies, the union of their [start, end] intervals
    (copies on several streams at once count once) and the span from the first start to
    the last end, in ms.  Byte counts are not in the trace; the engine's counters give them.
    streams: if given, only copies on these rocprofv3 stream ids count (the engine's copy
    streams, leaving out the bench's own set-up and pinned-rate copies on other streams).
    """
    import csv
    iv = {"h2d": [], "d2h": []}
    with open(trace_csv) as f:
        for row in csv.DictReader(f):
            direction = (row.get("Direction") or "").upper()
            key = "h2d" if "HOST_TO_DEVICE" in direction else "d2h" if "DEVICE_TO_HOST" in direction else None
            if key is None or (streams is not None and row.get("Stream_Id") not in streams):
                continue
            iv[key].append((int(row["Start_Timestamp"]), int(row["End_Timestamp"])))
    out = {}
    for key, xs in iv.items():
        xs.sort()
        busy, cb, ce = 0, None, None
        for b, e in xs:
            if ce is not None and b <= ce:
                ce = max(ce, e)
                continue
            if ce is not None:
                busy += ce - cb
            cb, ce = b, e
        if ce is not None:
            busy += ce - cb
        out[key] = {"copies": len(xs), "busy_ms": busy / 1e6,
                    "span_ms": (xs[-1][1] - xs[0][0]) / 1e6 if xs else 0.0}
    return out


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        return len(os.sched_getaffinity(0))


def oracle_check(q, k, v, o_bits, lse, rows_wanted, seed):
    """The fp64 oracle on sampled rows of a workload (all keys): its time on the host's
    cores (the cpu_baseline) and the GPU output's error on those rows."""
    from memory_bounded_streaming_amd.inputs import bf16_bits_to_f32, sample_rows
    from oracle.attention import attention_fp64
    from oracle.tolerance import error_report
    n, h, d = q.shape
    rows = sample_rows(n, rows_wanted, seed)
    t0 = time.perf_counter()
    o_ref, lse_ref = attention_fp64(q, k, v, rows=rows, dtype="bf16")
    dt = time.perf_counter() - t0
    flop = 4.0 * rows.size * n * d * h
    cpu = {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads()), "kind": "oracle",
           "sample": f"{rows.size} seeded sampled query rows x {h} heads of the N={n}, d={d} workload against "
                     f"all {n} keys, fp64 two-pass softmax; {dt:.1f} s wall; rate = 4*rows*N*d*H / time",
           "sample_wall_s": round(dt, 2),
           "extrapolated_full_n_s": round(dt * n / rows.size, 1),
           "extrapolation": f"sample wall x N/rows = time for all {n} query rows (not measured)"}
    rep = error_report(bf16_bits_to_f32(o_bits[rows]).astype(np.float64), o_ref)
    err = {"rows": int(rows.size), "heads": h, "reference": "dense fp64 oracle on the same bf16 inputs",
           "max_abs": rep["max_abs"], "mean_abs": rep["mean_abs"], "rowwise_rel": rep["rowwise_rel"],
           "lse_max_abs": float(np.abs(lse[:, rows] - lse_ref).max())}
    return cpu, err


def run_device(args, torch, cqsa, causal=False):
    """The device-resident workload (N=57344, H=8, d=128, l=3): partials then merge per
    step, each timed with HIP events on its stream.  causal=True runs the plan with
    CQSA_FLAG_CAUSAL (row i attends keys j <= i; useful FLOP 2 N (N+1) d H)."""
    from memory_bounded_streaming_amd.inputs import gen_qkv
    n, h, d, levels, _, _ = WORKLOADS["device_n57344"]
    q, k, v = gen_qkv(args.seed, n, h, d, "bf16")
    dev = [torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() for x in (q, k, v)]
    plan = cqsa.Plan(n, h, d, cqsa.CQSA_BF16, levels, flags=cqsa.CQSA_FLAG_CAUSAL if causal else 0)
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


def box_ceilings(torch, reps=10):
    """What plain library work reaches on this machine, beside the published peaks: a 1 GiB
    device-to-device copy (bytes read + written per second), and the best of two large
    bf16 matrix products through torch.matmul (the vendor GEMM, fp32 accumulation) on
    N(0,1) data, contiguous operands: 16384 x 16384 x 16384 and 8192 x 8192 x 32768."""
    out = {}
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    out["hbm_copy_gbs"] = reps * 2 * (1 << 30) / (time.perf_counter() - t0) / 1e9
    del src, dst
    g = torch.Generator(device="cuda").manual_seed(0)
    best = {}
    for m, n, k in ((16384, 16384, 16384), (8192, 8192, 32768)):
        a = torch.randn((m, k), device="cuda", generator=g).to(torch.bfloat16).contiguous()
        b = torch.randn((k, n), device="cuda", generator=g).to(torch.bfloat16).contiguous()
        for _ in range(3):
            c = torch.matmul(a, b)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            c = torch.matmul(a, b)
        torch.cuda.synchronize()
        rate = reps * 2.0 * m * n * k / (time.perf_counter() - t0) / 1e12
        if rate > best.get("tflops", 0.0):
            best = {"tflops": rate, "shape": f"{m}x{n}x{k}"}
        del a, b, c
    out["bf16_gemm_tflops"] = best["tflops"]
    out["bf16_gemm_shape"] = best["shape"]
    out["note"] = ("measured on this box after the timed calls: 1 GiB device copy (read + written bytes); "
                   "best torch.matmul rate of two large contiguous bf16 products on N(0,1) data")
    return out


def vendor_attention(args, torch, reps=5):
    """The vendor's fused attention on the device-resident workload's inputs (the same
    seeded bf16 Q/K/V, N=57344, 8 heads, d=128, scale 1/sqrt(d)): torch's
    scaled_dot_product_attention restricted to its flash backend (else its memory-efficient
    one; never the unfused math path), non-causal and causal, timed with HIP events.  A
    reference measured on the same box, like the GEMM ceiling: undivided attention with no
    memory budget, so it bounds nothing about the CQS path and is not part of it."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    from memory_bounded_streaming_amd.inputs import gen_qkv
    n, h, d, _, _, _ = WORKLOADS["device_n57344"]
    q, k, v = gen_qkv(args.seed, n, h, d, "bf16")
    # [N, H, d] -> [1, H, N, d], contiguous, outside the timed region
    dev = [torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda().view(n, h, d).permute(1, 0, 2)
           .contiguous().unsqueeze(0) for x in (q, k, v)]
    sdpa = torch.nn.functional.scaled_dot_product_attention
    out = {"workload": "N=57344, 8 heads, d=128, bf16, the device-resident workload's inputs, undivided",
           "call": "torch.nn.functional.scaled_dot_product_attention"}
    for name, causal in (("noncausal", False), ("causal", True)):
        res = None
        for backend in (SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION):
            try:
                with sdpa_kernel([backend]):
                    o = sdpa(*dev, is_causal=causal)
                    torch.cuda.synchronize()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(reps):
                        o = sdpa(*dev, is_causal=causal)
                    e1.record()
                    torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / reps
                flop = 2.0 * n * (n + 1) * d * h if causal else 4.0 * n * n * d * h
                res = {"backend": backend.name.lower(), "ms": round(ms, 4), "tflops": round(flop / (ms / 1e3) / 1e12, 1)}
                del o
                break
            except RuntimeError as ex:
                res = {"error": f"{backend.name.lower()}: {str(ex)[:160]}"}
        out[name] = res
    del dev
    torch.cuda.empty_cache()
    return out


def vendor_ratio(value, vendor, key):
    """A whole CQS forward step's useful TFLOP/s over the vendor attention's on the same
    inputs (None when the vendor call was not measured)."""
    if not vendor or "error" in vendor or not vendor.get(key) or "tflops" not in vendor[key]:
        return None
    return round(value / vendor[key]["tflops"], 3)


def runtime_first_use(torch):
    """Make the HIP runtime's one-time device set-up of this process happen before any
    measured call: it takes device memory at the process's first device allocation, copy
    and kernel, whoever makes them (about 150 MiB on this image), and would otherwise be
    counted in the observed memory of the headline's first call.  Returns the free device
    memory it took; the line reports it on its own."""
    free0, _ = torch.cuda.mem_get_info()
    x = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    x.copy_(torch.ones(1 << 20, dtype=torch.uint8).pin_memory())
    x.copy_(torch.ones(1 << 20, dtype=torch.uint8))
    x.fill_(2)
    ok = int(x.cpu()[0]) == 2
    del x
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    if not ok:
        raise RuntimeError("device set-up copy or fill returned a wrong value")
    return max(0, free0 - free1)


def pinned_inputs(torch, seed, n, h, d, count=3):
    """Q, K, V (and dO for count=4) drawn straight into pinned host memory."""
    from memory_bounded_streaming_amd.inputs import gen_tensor
    ts = []
    for i in range(count):
        t = torch.empty((n, h, d), dtype=torch.int16, pin_memory=True)
        gen_tensor(seed, i, n, h, d, "bf16", out=t.numpy().view(np.uint16))
        ts.append(t)
    return ts


def phase_rates(st, pcie):
    """Rates of the stream phases while copying (bytes / busy time) and their fraction of the
    pinned-copy rate measured on the box."""
    h2d = st["bytes_h2d"] / (st["t_h2d_ms"] / 1e3) / 1e9 if st["t_h2d_ms"] else None
    d2h = st["bytes_d2h"] / (st["t_d2h_ms"] / 1e3) / 1e9 if st["t_d2h_ms"] else None
    return {
        "h2d_gbs": h2d, "d2h_gbs": d2h,
        "h2d_busy_ms": st["t_h2d_ms"], "d2h_busy_ms": st["t_d2h_ms"],
        "h2d_achievable_gbs": pcie["h2d_gbs"], "d2h_achievable_gbs": pcie["d2h_gbs"],
        "h2d_frac_of_achievable": h2d / pcie["h2d_gbs"] if h2d else None,
        "d2h_frac_of_achievable": d2h / pcie["d2h_gbs"] if d2h else None,
        "bytes_h2d": st["bytes_h2d"], "bytes_d2h": st["bytes_d2h"], "bytes_d2d_chunk_reuse": st["bytes_d2d"],
        "copies_h2d": st["n_h2d_copies"], "copies_d2h": st["n_d2h_copies"],
        "rate_note": "bytes / union of the phase's event-timed copy intervals over its streams",
    }


def run_headline(args, torch, cqsa, runtime_bytes=None):
    """The streamed forward at a fixed budget (args.workload: by default the 8 GiB one):
    warm-up calls, then exactly args.steps timed calls of cqsa_forward (synchronous) with
    Q/K/V resident in pinned host memory.  The first call runs on a fresh plan with a
    library-allocated workspace, so its observed peak covers every device byte the call
    holds."""
    n, h, d, levels, budget, _ = WORKLOADS[args.workload]
    log(f"bench: drawing the N={n} workload into pinned memory")
    q, k, v = pinned_inputs(torch, args.seed, n, h, d)
    o = torch.empty((n, h, d), dtype=torch.int16, pin_memory=True)
    lse = torch.empty((h, n), dtype=torch.float32, pin_memory=True)
    plan = cqsa.Plan(n, h, d, cqsa.CQSA_BF16, levels, budget_bytes=budget)
    info = plan.info

    def call():
        return plan.forward(q, k, v, o, lse, residency=cqsa.CQSA_RES_HOST_PINNED, stats=True)

    first = None
    for i in range(args.warmup):
        st = call()
        first = first or st
        log(f"bench: warm-up call {i + 1}/{args.warmup}: {st['t_total_ms'] / 1e3:.2f} s")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    timed = []
    for i in range(args.steps):
        timed.append(call())
        log(f"bench: timed call {i + 1}/{args.steps}: {timed[-1]['t_total_ms'] / 1e3:.2f} s")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    first = first or timed[0]
    flop = info["useful_flop"]
    ms = wall / args.steps * 1e3
    attn_ms = float(np.mean([st["t_attn_ms"] for st in timed]))
    merge_ms = float(np.mean([st["t_merge_ms"] for st in timed]))
    launches = timed[0]["n_attn_launches"]
    est = cqsa.cqsa_plan_estimate(n, h, d, cqsa.CQSA_BF16, levels, budget_bytes=budget,
                                  rates={"attn_tflops": 1.0, "merge_gbs": 1.0, "h2d_gbs": 1.0, "d2h_gbs": 1.0})
    merge_bytes = est["merge_bytes"]
    pcie = pcie_achievable(torch)
    last = timed[-1]
    rates = phase_rates(last, pcie)
    rates["h2d_gbs_mean"] = float(np.mean([st["bytes_h2d"] / st["t_h2d_ms"] / 1e6 for st in timed]))
    rates["d2h_gbs_mean"] = float(np.mean([st["bytes_d2h"] / st["t_d2h_ms"] / 1e6 for st in timed]))
    out = {
        "plan": info, "ms_per_step": ms, "value": flop / (ms / 1e3) / 1e12,
        "attn_ms": attn_ms, "attn_launches": launches, "attn_tflops": flop / (attn_ms / 1e3) / 1e12,
        "merge_ms": merge_ms, "merge_bytes": merge_bytes, "merge_gbs": merge_bytes / (merge_ms / 1e3) / 1e9,
        "merge_launches": timed[0]["n_merge_launches"], "stream": rates,
        "memory": {"budget_bytes": budget, "peak_device_bytes_modelled": first["peak_device_bytes"],
                   "peak_device_bytes_observed": first["observed_peak_bytes"],
                   "device_free_at_entry": first["device_free_at_entry"],
                   "stream_workspace_bytes": info["stream_workspace_bytes"],
                   "host_accumulator_bytes": info["host_acc_bytes"],
                   "observed_note": "hipMemGetInfo free memory at entry minus its minimum over the first call "
                                    "(fresh plan, library-allocated workspace)",
                   "runtime_first_use_bytes": runtime_bytes,
                   "runtime_note": "device memory the HIP runtime took for its one-time set-up of this process "
                                   "(first device allocation, copy and kernel, made before the timed calls): "
                                   "not the library's and outside any budget"},
        "calls_s": [round(st["t_total_ms"] / 1e3, 3) for st in timed],
    }
    if not args.no_cpu_baseline:
        log(f"bench: oracle on {args.cpu_rows} sampled rows of the N={n} workload")
        qn, kn, vn = (t.numpy().view(np.uint16) for t in (q, k, v))
        out["cpu_baseline"], out["error"] = oracle_check(qn, kn, vn, o.numpy().view(np.uint16), lse.numpy(),
                                                         args.cpu_rows, args.seed)
    plan.close()
    return out


def run_streamed(args, torch, cqsa):
    n, h, d, levels, budget, _ = WORKLOADS["pinned_n212992"]
    ts = pinned_inputs(torch, args.seed, n, h, d)
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
        return {
            "workload": f"N={n}, H={h}, d={d}, bf16, CQS l={levels[0]} (c=13), Q/K/V in pinned host memory, "
                        f"device budget {budget // GiB} GiB",
            "mode": cqsa.MODE_NAMES[plan.info["stream_mode"]],
            "tflops_pcie_inclusive": flop / wall / 1e12,
            "wall_s": wall,
            "attn_tflops": flop / (st["t_attn_ms"] / 1e3) / 1e12,
            "merge_ms": st["t_merge_ms"],
            "attn_ms": st["t_attn_ms"],
            "stream": phase_rates(st, pcie),
            "peak_device_bytes": st["peak_device_bytes"],
            "budget_bytes": budget,
        }


def guarded(name, fn):
    """Run a secondary leg; its failure is recorded in the line instead of ending the run."""
    try:
        return fn()
    except Exception as exc:  # noqa: BLE001 -- any failure of a secondary leg is reported, not raised
        log(f"bench: {name} failed: {exc}")
        return {"error": f"{type(exc).__name__}: {exc}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-device", action="store_true", help="skip the device-resident N=57344 leg")
    ap.add_argument("--no-streamed", action="store_true", help="skip the N=212992 streamed leg")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-streamed-backward", action="store_true")
    ap.add_argument("--headline-only", action="store_true", help="run the headline workload and nothing else")
    ap.add_argument("--device-only", action="store_true",
                    help="run only the device-resident N=57344 leg (its kernel trace and counters)")
    ap.add_argument("--with-ceilings", action="store_true",
                    help="with --device-only: also run the box ceilings (device copy, vendor bf16 GEMMs)")
    ap.add_argument("--workload", default=HEADLINE, choices=[w for w in WORKLOADS if w.startswith("pinned_")],
                    help="streamed workload the line is measured on (default: the 8 GiB one, N=1376256)")
    ap.add_argument("--cpu-rows", type=int, default=256)
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one plain device copy of 1 GiB first (reference for HBM traffic counters)")
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic record from two rocprofv3 counter CSVs and exit (no GPU use)")
    ap.add_argument("--traffic-workload", default=HEADLINE, choices=sorted(TRAFFIC_RECORDS),
                    help="which workload's record --traffic-record writes")
    ap.add_argument("--copy-summary", metavar="TRACE_CSV",
                    help="print the copy busy times of a rocprofv3 memory-copy trace and exit (no GPU use)")
    ap.add_argument("--copy-streams", metavar="IDS",
                    help="with --copy-summary: comma-separated rocprofv3 stream ids to count (default: all)")
    args = ap.parse_args()
    if args.traffic_record:
        rec = traffic_record(args.traffic_record[0], args.traffic_record[1], kernel_source_hash(),
                             TRAFFIC_WORKLOADS[args.traffic_workload])
        with open(TRAFFIC_RECORDS[args.traffic_workload], "w") as f:
            json.dump(rec, f, indent=2)
            f.write("\n")
        print(json.dumps(rec))
        return
    if args.copy_summary:
        streams = set(args.copy_streams.split(",")) if args.copy_streams else None
        print(json.dumps(copy_summary(args.copy_summary, streams)))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    if args.headline_only:
        args.no_device = args.no_streamed = args.no_backward = args.no_streamed_backward = True
    if args.steps < 1 or args.warmup < 0:
        print("need --steps >= 1 and --warmup >= 0", file=sys.stderr)
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
    if args.device_only:
        log("bench: device-resident workload only")
        dres = run_device(args, torch, cqsa)
        out = {"device_resident": dres}
        if args.with_ceilings:
            out["ceilings"] = box_ceilings(torch)
        print(json.dumps(out), flush=True)
        return

    runtime_bytes = runtime_first_use(torch)
    log(f"bench: runtime first-use set-up took {runtime_bytes / (1 << 20):.0f} MiB of device memory")
    log(f"bench: headline, the streamed workload {args.workload}")
    head = run_headline(args, torch, cqsa, runtime_bytes)
    log(f"bench: {head['value']:.1f} TFLOP/s end-to-end, partial kernel {head['attn_tflops']:.1f} TFLOP/s")
    ceil = guarded("box ceilings", lambda: box_ceilings(torch))
    if "error" not in ceil:
        log(f"bench: box ceilings {ceil['bf16_gemm_tflops']:.1f} TFLOP/s bf16 GEMM, "
            f"{ceil['hbm_copy_gbs']:.1f} GB/s device copy")
    dres = None
    if not args.no_device:
        log("bench: device-resident workload")
        dres = guarded("device-resident leg", lambda: run_device(args, torch, cqsa))
        if "error" in dres:
            dres = None
        else:
            log(f"bench: device-resident {dres['value']:.1f} TFLOP/s, partial kernel "
                f"{dres['attn_tflops']:.1f} TFLOP/s")
    dcausal = None
    if not args.no_device:
        log("bench: device-resident workload, causal")
        dcausal = guarded("device-resident causal leg", lambda: run_device(args, torch, cqsa, causal=True))
        if "error" not in dcausal:
            log(f"bench: device-resident causal {dcausal['value']:.1f} useful TFLOP/s, partial kernel "
                f"{dcausal['attn_tflops']:.1f}")
    vendor = None
    if not args.no_device:
        log("bench: vendor fused attention on the device-resident workload's inputs")
        vendor = guarded("vendor attention", lambda: vendor_attention(args, torch))
        if "error" not in vendor:
            log("bench: vendor attention " + ", ".join(
                f"{k} {vendor[k].get('tflops', vendor[k].get('error'))}" for k in ("noncausal", "causal")))
    bwd = None
    if not args.no_backward and dres is not None:
        log("bench: backward of the device-resident workload")
        bwd = guarded("backward leg", lambda: run_backward(args, torch, cqsa))
        if "error" not in bwd:
            bwd["fwd_bwd_ratio"] = round((bwd["ms_per_step"] + dres["ms_per_step"]) / dres["ms_per_step"], 3)
            bwd.pop("fwd_bwd_ratio_note")
            log(f"bench: backward {bwd['tflops_useful']:.1f} useful TFLOP/s, {bwd['ms_per_step']:.2f} ms")
    stream_res = None
    if not args.no_streamed:
        log("bench: host-pinned streamed N=212992 workload")
        stream_res = guarded("streamed 16 GiB leg", lambda: run_streamed(args, torch, cqsa))
        if "error" not in stream_res:
            log(f"bench: streamed {stream_res['tflops_pcie_inclusive']:.1f} TFLOP/s PCIe-inclusive")
    sbwd = None
    if not args.no_streamed and not args.no_streamed_backward:
        log("bench: host-pinned streamed backward")
        sbwd = guarded("streamed backward leg", lambda: run_streamed_backward(args, torch, cqsa))
        if "error" not in sbwd:
            log(f"bench: streamed backward {sbwd['tflops_pcie_inclusive']:.1f} useful TFLOP/s PCIe-inclusive")
    dry = None
    if stream_res is not None:
        # the billion-token case priced with this run's measured rates (plan-only, no data)
        rates = {"attn_tflops": head["attn_tflops"], "merge_gbs": head["merge_gbs"],
                 "h2d_gbs": head["stream"]["h2d_achievable_gbs"], "d2h_gbs": head["stream"]["d2h_achievable_gbs"]}
        dry = []
        for budget in (16 * GiB, 2 * GiB):
            def one(budget=budget):
                e = cqsa.cqsa_plan_estimate(1 << 30, 1, 128, cqsa.CQSA_BF16, [3], n_levels=0, budget_bytes=budget,
                                            flags=cqsa.CQSA_FLAG_PAD, rates=rates)
                return {"n_tokens": 1 << 30, "heads": 1, "head_dim": 128, "budget_bytes": budget,
                        "levels": e["l"], "task_tokens": e["task_tokens"],
                        "mode": cqsa.MODE_NAMES[e["stream_mode"]], "stream_workspace_bytes": e["stream_workspace_bytes"],
                        "host_pinned_bytes": e["host_pinned_bytes"], "bytes_h2d": e["bytes_h2d"],
                        "bytes_d2h": e["bytes_d2h"], "est_hours": round(e["t_est_s"] / 3600, 2),
                        "attn_hours": round(e["t_attn_s"] / 3600, 2), "h2d_hours": round(e["t_h2d_s"] / 3600, 2),
                        "t_est_s": e["t_est_s"],
                        "backward_footprint": {
                            "levels": e["bwd_levels"], "task_tokens": e["bwd_task_tokens"],
                            "mode": cqsa.MODE_NAMES.get(e["bwd_stream_mode"]),
                            "stats_in_host_memory": bool(e["bwd_host_stats"]),
                            "stream_workspace_bytes": e["bwd_stream_workspace_bytes"],
                            "note": "device workspace of the host-pinned backward under this budget, at the "
                                    "fewest levels of l=3 where one of its layouts fits (plan-only)"}}
            dry.append(guarded(f"dry run at {budget // GiB} GiB", one))
            ok = "error" not in dry[-1]
            if ok and sbwd is not None and "error" not in sbwd and "error" not in stream_res:
                # not a plan of the backward: the forward estimate scaled by the streamed backward's
                # measured time over the streamed forward's on the 16 GiB workload
                ratio = sbwd["wall_s"] / stream_res["wall_s"]
                dry[-1]["bwd_hours_by_ratio"] = round(dry[-1]["t_est_s"] * ratio / 3600, 1)
                dry[-1]["bwd_ratio_note"] = (f"extrapolation: forward estimate x {ratio:.2f}, the measured streamed "
                                             "backward / forward time of the N=212992, 16-head workload")

    n, h, d, levels, budget, _ = WORKLOADS[args.workload]
    cs = [l * (l - 1) + 1 for l in levels]
    units = int(np.prod(cs))
    khash = kernel_source_hash()
    flop = head["plan"]["useful_flop"]
    device_resident = None
    if dres is not None:
        device_resident = {
            "workload": "N=57344, 8 heads, d=128, bf16, CQS l=3 (c=7 chunks of 8192), Q/K/V device-resident",
            "tflops": round(dres["value"], 3), "ms_per_step": round(dres["ms_per_step"], 4),
            "roofline": {"bound": "mfma", "kernel": "attn_partial_bf16<128>",
                         "achieved": round(dres["attn_tflops"], 3), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(dres["attn_tflops"] / BF16_MFMA_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic(khash, "device_n57344"),
                         "flop_per_launch": dres["plan"]["useful_flop"], "avg_launch_ms": round(dres["attn_ms"], 4),
                         "frac_of_measured_ceiling": (round(dres["attn_tflops"] / ceil["bf16_gemm_tflops"], 4)
                                                      if "error" not in ceil else None)},
            "merge": {"bound": "hbm", "achieved": round(dres["merge_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(dres["merge_gbs"] / HBM_PEAK_GBS, 4), "bytes_per_launch": dres["merge_bytes"],
                      "avg_launch_ms": round(dres["merge_ms"], 4)},
            "vs_vendor_attention": vendor_ratio(dres["value"], vendor, "noncausal"),
        }
    device_causal = None
    if dcausal is not None:
        device_causal = dcausal if "error" in dcausal else {
            "workload": "the N=57344, 8-head, d=128 bf16 l=3 device-resident workload with CQSA_FLAG_CAUSAL "
                        "(row i attends keys j <= i)",
            "tflops_useful": round(dcausal["value"], 3), "ms_per_step": round(dcausal["ms_per_step"], 4),
            "useful_flop": dcausal["plan"]["useful_flop"],
            "roofline": {"bound": "mfma", "kernel": "attn_partial_bf16<128>",
                         "achieved": round(dcausal["attn_tflops"], 3), "peak": BF16_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(dcausal["attn_tflops"] / BF16_MFMA_PEAK_TFLOPS, 4),
                         "avg_launch_ms": round(dcausal["attn_ms"], 4),
                         "note": "achieved = useful FLOP 2 N (N+1) d H / partial-kernel time"},
            "vs_vendor_attention": vendor_ratio(dcausal["value"], vendor, "causal"),
        }
    line = {
        "metric": METRIC,
        "value": round(head["value"], 3),
        "unit": "TFLOP/s",
        "pct_bf16_mfma_peak": round(100.0 * head["value"] / BF16_MFMA_PEAK_TFLOPS, 3),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: Q/K/V i.i.d. N(0,1) rounded to bf16, seed %d" % args.seed,
        "config": {"workload": f"N={n} tokens, {h} heads, d={d}, bf16, non-causal, "
                               + (f"CQS l={levels[0]} (c={cs[0]} chunks of {n // cs[0]})" if len(levels) == 1 else
                                  f"CQS l=({','.join(map(str, levels))}) ({'x'.join(map(str, cs))} = {units} units "
                                  f"of {n // units})")
                               + f", Q/K/V/O/LSE in pinned host memory, "
                               f"device budget {budget // GiB} GiB (CQS-streamed forward)",
                   "n_tokens": n, "heads": h, "head_dim": d, "levels": levels, "residency": "host_pinned",
                   "budget_bytes": budget, "stream_mode": cqsa.MODE_NAMES[head["plan"]["stream_mode"]]},
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_partial_bf16<128>",
            "achieved": round(head["attn_tflops"], 3),
            "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(head["attn_tflops"] / BF16_MFMA_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(khash, args.workload) if args.workload in TRAFFIC_RECORDS else None,
            "launches_per_step": head["attn_launches"],
            "flop_per_launch": flop / head["attn_launches"],
            "avg_launch_ms": round(head["attn_ms"] / head["attn_launches"], 4),
            "measured_ceiling": round(ceil["bf16_gemm_tflops"], 1) if "error" not in ceil else None,
            "frac_of_measured_ceiling": (round(head["attn_tflops"] / ceil["bf16_gemm_tflops"], 4)
                                         if "error" not in ceil else None),
        },
        "merge": {"bound": "hbm", "achieved": round(head["merge_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(head["merge_gbs"] / HBM_PEAK_GBS, 4), "bytes_per_step": head["merge_bytes"],
                  "launches_per_step": head["merge_launches"],
                  "avg_launch_ms": round(head["merge_ms"] / head["merge_launches"], 4),
                  "measured_ceiling": round(ceil["hbm_copy_gbs"], 1) if "error" not in ceil else None,
                  "frac_of_measured_ceiling": (round(head["merge_gbs"] / ceil["hbm_copy_gbs"], 4)
                                               if "error" not in ceil else None)},
        "ceilings": ceil,
        "vendor_attention": vendor,
        "stream": head["stream"],
        "memory": head["memory"],
        "error": head.get("error"),
        "cpu_baseline": head.get("cpu_baseline"),
        "calls_s": head["calls_s"],
        "device_resident": device_resident,
        "device_resident_causal": device_causal,
        "streamed_16gib": stream_res,
        "backward": bwd,
        "streamed_backward": sbwd,
        "dry_run_1b_tokens": dry,
        "kernel_source_sha256_16": khash,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
