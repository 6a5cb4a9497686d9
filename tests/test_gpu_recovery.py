"""GPU tests of the out-of-memory recovery and the debugging aids of the host-pinned
forward (needs an MI355X).

* An allocation failure (injected: the library's next device allocations report out of
  memory) makes the call re-plan one CQS Divide level deeper and finish inside the same
  call ("Stream-CQSA: Exact Out-of-Memory Recovery for Attention", abstract: a
  memory-capacity failure becomes a recoverable execution path; "The Recursive Benefit"
  section of the wispaper explainer).  The deeper plan computes the same attention, so
  the output meets the oracle's tolerance; the division differs, so bits may differ.
* A plan whose budget is the device's free memory minus a margin, with the depth chosen
  automatically.
* CQSA_SYNC=1 (every step waited for) and CQSA_CANARY=1 (guard words around every
  workspace piece) give the same bits as a plain call.
"""
import os

import numpy as np
import pytest

from memory_bounded_streaming_amd import cqsa
from memory_bounded_streaming_amd.inputs import gen_qkv
from oracle.attention import attention_fp64
from oracle.tolerance import BF16_LSE_TOL, BF16_REL_TOL, rowwise_rel_err

from gpu_util import as_f64, init_device_runtime, log, pinned

pytestmark = pytest.mark.gpu
MiB = 1 << 20


def _pinned_inputs(q, k, v, n, h, d):
    import torch
    ts = []
    for a in (q, k, v):
        t, view = pinned((n, h, d), "bf16")
        view[...] = a
        ts.append(t)
    to, oa = pinned((n, h, d), "bf16")
    tl = torch.empty((h, n), dtype=torch.float32, pin_memory=True)
    return ts, to, oa, tl


def _check(oa, tl, q, k, v):
    o_ref, lse_ref = attention_fp64(q, k, v, dtype="bf16")
    err = rowwise_rel_err(as_f64(oa, "bf16"), o_ref)
    lse_err = float(np.abs(tl.numpy() - lse_ref).max())
    log(f"  row-wise rel err {err:.3e}, lse abs err {lse_err:.3e}")
    assert err <= BF16_REL_TOL and lse_err <= BF16_LSE_TOL


@pytest.mark.parametrize("fails,levels_after", [(1, 2), (2, 3)])
def test_injected_allocation_failure_replans_deeper(fails, levels_after):
    pytest.importorskip("torch")
    n, h, d = 7 * 256, 2, 128
    log(f"recovery: N={n} l=3, {fails} injected device allocation failure(s)")
    q, k, v = gen_qkv(5, n, h, d, "bf16")
    (tq, tk, tv), to, oa, tl = _pinned_inputs(q, k, v, n, h, d)
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [3]) as p:
        cqsa.cqsa_debug_fail_allocations(fails)
        try:
            st = p.forward(tq, tk, tv, to, tl, residency=cqsa.CQSA_RES_HOST_PINNED, stats=True)
        finally:
            cqsa.cqsa_debug_fail_allocations(0)
        assert st["replans"] == fails
        assert st["levels_used"] == levels_after
        assert p.info["levels"] == 1  # the caller's plan is unchanged
    _check(oa, tl, q, k, v)


def test_injected_failure_with_a_caller_workspace_is_reported():
    torch = pytest.importorskip("torch")
    n, h, d = 7 * 256, 2, 128
    q, k, v = gen_qkv(6, n, h, d, "bf16")
    (tq, tk, tv), to, oa, tl = _pinned_inputs(q, k, v, n, h, d)
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [3]) as p:
        ws = torch.empty(p.workspace_size(cqsa.CQSA_RES_HOST_PINNED), dtype=torch.uint8, device="cuda")
        cqsa.cqsa_debug_fail_allocations(1)  # the descriptor tables' first upload fails
        try:
            with pytest.raises(cqsa.CqsaError) as e:
                p.forward(tq, tk, tv, to, tl, residency=cqsa.CQSA_RES_HOST_PINNED, workspace=ws)
        finally:
            cqsa.cqsa_debug_fail_allocations(0)
        assert e.value.status == -6
        # nothing is left behind: the same call succeeds now
        p.forward(tq, tk, tv, to, tl, residency=cqsa.CQSA_RES_HOST_PINNED, workspace=ws)
    _check(oa, tl, q, k, v)


def test_budget_from_free_device_memory():
    torch = pytest.importorskip("torch")
    n, h, d = 7 * 2048, 4, 128
    q, k, v = gen_qkv(8, n, h, d, "bf16")
    (tq, tk, tv), to, oa, tl = _pinned_inputs(q, k, v, n, h, d)
    init_device_runtime()  # the runtime's one-time device set-up is not the call's
    torch.cuda.synchronize()
    free, _ = torch.cuda.mem_get_info()
    margin = free - 64 * MiB  # leaves a 64 MiB budget: the undivided plan does not fit
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [3], n_levels=0, budget_bytes=margin,
                   flags=cqsa.CQSA_FLAG_FREE_BUDGET) as p:
        info = p.info
        log(f"free-memory budget {info['budget_bytes'] / MiB:.1f} MiB: levels {info['l']}, "
            f"mode {cqsa.MODE_NAMES[info['stream_mode']]}")
        assert abs(info["budget_bytes"] - 64 * MiB) < 32 * MiB
        assert info["l"][0] == 3 and info["stream_workspace_bytes"] <= info["budget_bytes"]
        st = p.forward(tq, tk, tv, to, tl, residency=cqsa.CQSA_RES_HOST_PINNED, stats=True)
        assert st["observed_peak_bytes"] <= info["budget_bytes"]
    _check(oa, tl, q, k, v)


@pytest.mark.parametrize("env", ["CQSA_SYNC", "CQSA_CANARY"])
def test_debug_modes_give_the_same_bits(env):
    pytest.importorskip("torch")
    n, h, d = 13 * 192, 2, 128
    q, k, v = gen_qkv(9, n, h, d, "bf16")
    (tq, tk, tv), to, oa, tl = _pinned_inputs(q, k, v, n, h, d)
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [4], flags=cqsa.CQSA_FLAG_HOST_ACC) as p:
        p.forward(tq, tk, tv, to, tl, residency=cqsa.CQSA_RES_HOST_PINNED)
        o1, l1 = oa.copy(), tl.numpy().copy()
        os.environ[env] = "1"
        try:
            p.forward(tq, tk, tv, to, tl, residency=cqsa.CQSA_RES_HOST_PINNED)
        finally:
            del os.environ[env]
        assert np.array_equal(oa, o1) and np.array_equal(tl.numpy(), l1)
    _check(oa, tl, q, k, v)
