"""Full-size host-pinned workloads on the GPU, checked on seeded sampled rows.

* N=212992, H=16, d=128, bf16, l=4 (c=13), device budget 16 GiB
* N=1376256, H=8, d=128, bf16, l=5 (c=21), device budget 8 GiB (accumulator on host)
* N=12845056, H=1, d=128, bf16, two levels l=(3,3), device budget 2 GiB

Q/K/V are drawn straight into pinned host memory; the call streams every task through
the budget; the oracle evaluates the sampled rows (plus every unit's first and last
token) in fp64.  The bound is 2e-2 row-wise relative error.
"""
import os
import time

import numpy as np
import pytest

from memory_bounded_streaming_amd import cqsa
from memory_bounded_streaming_amd.inputs import sample_rows
from oracle.plan import make_plan
from oracle.stream_bytes import stream_traffic
from oracle.tolerance import BF16_LSE_TOL, BF16_REL_TOL, error_report

from gpu_util import as_f64, init_device_runtime, log, oracle_rows, pinned, pinned_qkv

pytestmark = pytest.mark.gpu
GiB = 1 << 30

WORKLOADS = {
    "n212992_h16_l4_16GiB": (212992, 16, 128, [4], 16 * GiB, 4096, 1),
    "n1376256_h8_l5_8GiB": (1376256, 8, 128, [5], 8 * GiB, 4096, 2),
    "n12845056_h1_l3x3_2GiB": (12845056, 1, 128, [3, 3], 2 * GiB, 1024, 4),
}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(WORKLOADS))
def test_streamed_workload_sampled_rows(name):
    torch = pytest.importorskip("torch")
    n, h, d, levels, budget, r_count, mode = WORKLOADS[name]
    os.environ["CQSA_PROGRESS"] = "1"
    # the runtime's one-time device set-up is not the call's: make it happen first, so the
    # observed peak below is the call's own whichever case runs first in the process
    log(f"{name}: runtime first-use set-up took {init_device_runtime() / (1 << 20):.0f} MiB")
    log(f"{name}: drawing inputs into pinned memory")
    t0 = time.time()
    (tq, tk, tv), (q, k, v) = pinned_qkv(0, n, h, d, "bf16")
    to, oa = pinned((n, h, d), "bf16")
    tl = torch.empty((h, n), dtype=torch.float32, pin_memory=True)
    log(f"  inputs ready in {time.time() - t0:.1f} s")
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, levels, budget_bytes=budget) as p:
        info = p.info
        assert info["stream_mode"] == mode
        assert info["stream_workspace_bytes"] <= budget
        free0, _ = torch.cuda.mem_get_info()
        t0 = time.time()
        st = p.forward(tq, tk, tv, to, tl, residency=cqsa.CQSA_RES_HOST_PINNED, stats=True)
        wall = time.time() - t0
        free1, _ = torch.cuda.mem_get_info()
    log(f"  forward {wall:.1f} s: {info['useful_flop'] / wall / 1e12:.1f} TFLOP/s end-to-end, "
        f"partial kernel {info['useful_flop'] / (st['t_attn_ms'] / 1e3) / 1e12:.1f} TFLOP/s, "
        f"peak device {st['peak_device_bytes'] / GiB:.3f} GiB modelled, "
        f"{st['observed_peak_bytes'] / GiB:.3f} GiB observed, of {budget / GiB:.0f} GiB; "
        f"H2D {st['bytes_h2d'] / st['t_h2d_ms'] / 1e6:.1f} GB/s, D2H {st['bytes_d2h'] / st['t_d2h_ms'] / 1e6:.1f} GB/s "
        f"while copying")
    assert st["peak_device_bytes"] <= budget
    # observed with hipMemGetInfo over the call (fresh plan, library-allocated workspace:
    # every device byte the call holds is in it)
    assert 0 < st["observed_peak_bytes"] <= budget
    # the allocator may serve part of the workspace from memory it already held
    assert st["observed_peak_bytes"] >= info["stream_workspace_bytes"] - (64 << 20)
    assert st["replans"] == 0 and st["levels_used"] == len(levels)
    assert abs(free1 - free0) < (256 << 20)
    e = 2
    visits = info["visits"]
    assert st["bytes_h2d"] + st["bytes_d2d"] >= 3 * visits * n * h * d * e
    # the dry run predicts the copies exactly; its time uses this run's measured rates
    rates = {"attn_tflops": info["useful_flop"] / (st["t_attn_ms"] / 1e3) / 1e12,
             "merge_gbs": 5000.0, "h2d_gbs": st["bytes_h2d"] / (st["t_h2d_ms"] / 1e3) / 1e9,
             "d2h_gbs": st["bytes_d2h"] / (st["t_d2h_ms"] / 1e3) / 1e9}
    est = cqsa.cqsa_plan_estimate(n, h, d, cqsa.CQSA_BF16, levels, budget_bytes=budget, rates=rates)
    assert (est["bytes_h2d"], est["bytes_d2h"], est["bytes_d2d"]) == (st["bytes_h2d"], st["bytes_d2h"], st["bytes_d2d"])
    # and the oracle's walk of the plan, which is pinned to the closed forms
    walk = stream_traffic(make_plan(n, levels), h, d, e, host_acc=info["stream_mode"] in (2, 4),
                          kv_buffers=info["kv_buffers"])
    assert (walk["bytes_h2d"], walk["bytes_d2h"], walk["bytes_d2d"]) == (st["bytes_h2d"], st["bytes_d2h"], st["bytes_d2d"])
    log(f"  dry run: {est['t_est_s']:.2f} s estimated vs {wall:.2f} s measured")
    rows = sample_rows(n, r_count, 0, unit_tokens=info["unit_tokens"])
    log(f"  oracle on {rows.size} rows")
    t0 = time.time()
    o_ref, lse_ref = oracle_rows(q, k, v, rows, "bf16")
    log(f"  oracle {time.time() - t0:.1f} s")
    rep = error_report(as_f64(oa[rows], "bf16"), o_ref)
    log(f"  {rep}")
    assert rep["rowwise_rel"] <= BF16_REL_TOL
    assert np.abs(tl.numpy()[:, rows] - lse_ref).max() <= BF16_LSE_TOL
